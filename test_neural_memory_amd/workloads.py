"""Seeded synthetic workloads for the memory kernels (inputs only).

This module draws inputs; it holds none of the memory's arithmetic.  Both the
HIP path (tests, bench) and the float64 oracle consume exactly these arrays:
bf16 inputs are rounded once here (round-to-nearest-even, via torch) and the
oracle reads the rounded values upcast to float64.

The five workloads (shapes, value distributions, chunk sizes):

1. tiny linear memory, float32: B=1 H=1 T=64 d=16 b=8; q, k, v ~ N(0,1) with
   q and k L2-normalised per token; theta ~ U[0.01, 0.1], eta ~ U[0.8, 0.95],
   alpha ~ U[0, 0.05]; M0 = S0 = 0.
2. TTT-Linear-style: B=8 H=12 T=2048 d=64 b=16, bf16 q, k, v as above;
   theta = 0.05, eta = 0, alpha = 0; M0 ~ N(0, 0.02^2) drawn per head and
   shared by the batch; S0 = 0.
3. Titans linear memory: B=4 H=16 T=8192 d=128 b=64, bf16 q, k, v as above;
   theta = 0.1 sigmoid(N(0,1)), eta = sigmoid(N(2, 0.5)), alpha =
   0.05 sigmoid(N(-1,1)) per token (second argument of N is the variance);
   M0 = S0 = 0.
4. long-context carry: B=1 H=32 T=131072 d=128 b=64, distributions of 3.
5. deep (2-layer MLP) memory: B=4 H=8 T=4096 d=64 hidden=256 b=16, bf16 q, k,
   v as above; theta = 0.02, eta = 0.9, alpha = 0.01; W1 ~ N(0, 1/64),
   W2 ~ N(0, 1/256) per head shared by the batch; momenta 0.

Seeds: ``numpy.random.default_rng(1000 + id)``; draw order q, k, v, theta,
eta, alpha, then initial states.  Any size can be overridden (for parity cases
small enough for the oracle) while keeping the distributions.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_cotangents", "to_numpy64"]


@dataclasses.dataclass(frozen=True)
class Workload:
    id: int
    name: str
    B: int
    H: int
    T: int
    d: int
    b: int
    dtype: str            # "f32" or "bf16" (q, k, v)
    gates: str            # "uniform", "const" or "titans"
    theta: float = 0.0
    eta: float = 0.0
    alpha: float = 0.0
    m0_std: float = 0.0   # per-head N(0, m0_std^2) initial memory, 0 = zeros
    hidden: int = 0       # > 0: deep (MLP) memory

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    1: Workload(1, "tiny-linear-f32", 1, 1, 64, 16, 8, "f32", "uniform"),
    2: Workload(2, "ttt-linear-style", 8, 12, 2048, 64, 16, "bf16", "const", theta=0.05, eta=0.0, alpha=0.0,
                m0_std=0.02),
    3: Workload(3, "titans-linear", 4, 16, 8192, 128, 64, "bf16", "titans"),
    4: Workload(4, "long-context-carry", 1, 32, 131072, 128, 64, "bf16", "titans"),
    5: Workload(5, "deep-mlp-memory", 4, 8, 4096, 64, 16, "bf16", "const", theta=0.02, eta=0.9, alpha=0.01,
                hidden=256),
}


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _unit_rows(x):
    # L2-normalise each token vector (input featurisation, not the memory).
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / np.maximum(n, 1e-30)).astype(np.float32)


def _normal(rng, shape, chunk=1 << 26):
    """float32 N(0,1) draws, generated in slices to bound host memory."""
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1)
    for s in range(0, flat.size, chunk):
        flat[s:s + chunk] = rng.standard_normal(min(chunk, flat.size - s), dtype=np.float32)
    return out


def make_inputs(w: Workload, seed: int | None = None) -> dict:
    """Draw one workload's inputs as CPU torch tensors.

    Returns a dict with ``q, k, v`` ([B,H,T,d], float32 or bfloat16), ``theta,
    eta, alpha`` ([B,H,T] float32) and ``M0, S0`` ([B,H,d,d] float32 or None)
    -- for the deep memory ``W1`` ([B,H,d,hid]), ``W2`` ([B,H,hid,d]) and
    ``S1, S2`` (None) instead of ``M0, S0``.
    """
    rng = np.random.default_rng(1000 + w.id if seed is None else seed)
    B, H, T, d = w.B, w.H, w.T, w.d
    shape = (B, H, T, d)
    q = _unit_rows(_normal(rng, shape))
    k = _unit_rows(_normal(rng, shape))
    v = _normal(rng, shape)
    gshape = (B, H, T)
    if w.gates == "uniform":
        theta = rng.uniform(0.01, 0.1, gshape)
        eta = rng.uniform(0.8, 0.95, gshape)
        alpha = rng.uniform(0.0, 0.05, gshape)
    elif w.gates == "const":
        theta = np.full(gshape, w.theta)
        eta = np.full(gshape, w.eta)
        alpha = np.full(gshape, w.alpha)
    elif w.gates == "titans":
        theta = 0.1 * _sigmoid(rng.standard_normal(gshape))
        eta = _sigmoid(rng.normal(2.0, np.sqrt(0.5), gshape))
        alpha = 0.05 * _sigmoid(rng.normal(-1.0, 1.0, gshape))
    else:
        raise ValueError(w.gates)
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    out = {
        "q": torch.from_numpy(q).to(tdt),
        "k": torch.from_numpy(k).to(tdt),
        "v": torch.from_numpy(v).to(tdt),
        "theta": torch.from_numpy(theta.astype(np.float32)),
        "eta": torch.from_numpy(eta.astype(np.float32)),
        "alpha": torch.from_numpy(alpha.astype(np.float32)),
    }
    if w.hidden:
        W1 = rng.standard_normal((H, d, w.hidden)) / np.sqrt(d)
        W2 = rng.standard_normal((H, w.hidden, d)) / np.sqrt(w.hidden)
        out["W1"] = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(W1, (B, H, d, w.hidden)), dtype=np.float32))
        out["W2"] = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(W2, (B, H, w.hidden, d)), dtype=np.float32))
        out["S1"] = None
        out["S2"] = None
    else:
        if w.m0_std > 0:
            M0 = rng.standard_normal((H, d, d)) * w.m0_std
            out["M0"] = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(M0, (B, H, d, d)), dtype=np.float32))
        else:
            out["M0"] = None
        out["S0"] = None
    return out


def make_cotangents(w: Workload, seed: int | None = None, states: bool = True, chunks=None) -> dict:
    """Draw derivatives of an outer loss with respect to the memory's outputs.

    ``dz`` [B,H,T,d] ~ N(0,1) float32; with ``states``, ``dM_T, dS_T``
    [B,H,d,d] ~ N(0,1) float32 (else None).  ``chunks=(c0, c1)`` keeps dz only
    on the tokens of chunks c0 .. c1-1 (chunk size w.b) and zeroes the rest.
    Seed: ``numpy.random.default_rng(2000 + id)``.
    """
    rng = np.random.default_rng(2000 + w.id if seed is None else seed)
    B, H, T, d = w.B, w.H, w.T, w.d
    dz = _normal(rng, (B, H, T, d)).astype(np.float32)
    if chunks is not None:
        c0, c1 = chunks
        keep = np.zeros(T, dtype=bool)
        keep[c0 * w.b:min(c1 * w.b, T)] = True
        dz[:, :, ~keep, :] = 0.0
    out = {"dz": torch.from_numpy(dz), "dM_T": None, "dS_T": None}
    if states:
        out["dM_T"] = torch.from_numpy(rng.standard_normal((B, H, d, d)).astype(np.float32))
        out["dS_T"] = torch.from_numpy(rng.standard_normal((B, H, d, d)).astype(np.float32))
    return out


def to_numpy64(t):
    """A CPU tensor (any float dtype) as a float64 numpy array; None stays None."""
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def varlen_lengths(total, seed=3001, mean=1024):
    """Seeded document lengths for a packed batch: lognormal (sigma 1) around `mean`,
    clipped to [1, 8192], the last one trimmed so that they sum to `total`."""
    rng = np.random.default_rng(seed)
    out, acc = [], 0
    while acc < total:
        n = int(np.clip(rng.lognormal(np.log(mean) - 0.5, 1.0), 1, 8192))
        n = min(n, total - acc)
        out.append(n)
        acc += n
    return out


def set_chunk_gates(w, inp):
    """Replace the per-token gates of `inp` by one gate triple per (batch, head,
    chunk), drawn from the same Titans distributions (seed 4003)."""
    nc = (w.T + w.b - 1) // w.b
    rng = np.random.default_rng(4003)
    sig = lambda x: 1.0 / (1.0 + np.exp(-x))  # noqa: E731
    gsh = (w.B, w.H, nc)
    inp["theta"] = torch.from_numpy((0.1 * sig(rng.standard_normal(gsh))).astype(np.float32))
    inp["eta"] = torch.from_numpy(sig(rng.normal(2.0, np.sqrt(0.5), gsh)).astype(np.float32))
    inp["alpha"] = torch.from_numpy((0.05 * sig(rng.normal(-1.0, 1.0, gsh))).astype(np.float32))


def deep_layer_shapes(d: int, hidden: int, depth: int):
    """(fan_in, fan_out) of each layer of a depth-L deep memory: d -> hidden,
    (depth - 2) x hidden -> hidden, hidden -> d."""
    return [(d, hidden)] + [(hidden, hidden)] * (depth - 2) + [(hidden, d)]


def make_deep_layers(w: Workload, depth: int, seed: int = 5) -> list:
    """Initial layers of a depth-L deep memory for workload ``w``: each layer
    N(0, 1 / fan_in) float32, drawn per head and shared by the batch
    ([B, H, fan_in, fan_out] CPU tensors).  Seed: ``default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    out = []
    for (fi, fo) in deep_layer_shapes(w.d, w.hidden, depth):
        x = rng.standard_normal((w.H, fi, fo)) / np.sqrt(fi)
        out.append(torch.from_numpy(np.ascontiguousarray(np.broadcast_to(x, (w.B, w.H, fi, fo)), dtype=np.float32)))
    return out
