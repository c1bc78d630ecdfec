"""Shared helpers for parity tests: run the HIP path and the oracle on the same inputs."""

from __future__ import annotations

import numpy as np
import torch

from oracle import linear_forward
from test_neural_memory_amd import memory as tm
from test_neural_memory_amd.workloads import to_numpy64

# Tolerances on max|x_gpu - x_ref| / rms(x_ref), per output tensor.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(x - ref)))
    return err / rms if rms > 0 else err


def bf16_half_ulp(x):
    """Half a bf16 ulp at each |x| (the most that rounding a float to bf16 moves it)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, np.finfo(np.float64).tiny)))
    return np.where(a > 0, np.exp2(e - 8), 0.0)


def rel_err_bf16_out(x, ref):
    """``rel_err`` of an output stored in bf16, not counting the rounding of
    the output itself: each element's error is first reduced by half a bf16
    ulp of the reference value (never below zero).  The bound then applies to
    the computation; the storage format adds at most that half ulp."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.maximum(np.abs(x - ref) - bf16_half_ulp(ref), 0.0)))
    return err / rms if rms > 0 else err


def to_dev(inp, device="cuda"):
    return {k: (None if v is None else v.to(device)) for k, v in inp.items()}


def run_gpu(inp, b, raw=False, **kw):
    """Linear memory on the GPU; returns float64 numpy (z, M_T, S_T), or the
    device tensors themselves with ``raw``.  z is bf16 for bf16 inputs unless
    ``z_dtype=torch.float32`` is passed."""
    dev = to_dev(inp)
    z, M, S = tm.forward(dev["q"], dev["k"], dev["v"], dev["theta"], dev["eta"], dev["alpha"],
                         dev.get("M0"), dev.get("S0"), b=b, **kw)
    torch.cuda.synchronize()
    if raw:
        return z, M, S
    return to_numpy64(z.cpu()), to_numpy64(M.cpu()), to_numpy64(S.cpu())


def run_oracle(inp, b, heads=None, rows=None):
    """Oracle on (batch, head) pairs ``heads`` and value rows ``rows`` (None = all).

    Value rows of a linear memory are independent, so a subset of rows is the
    oracle's exact answer for those rows.  Returns z [nh, T, nr], M_T, S_T [nh, nr, d].
    """
    B, H, T, d = inp["q"].shape
    if heads is None:
        heads = [(i, j) for i in range(B) for j in range(H)]
    bi = np.array([h[0] for h in heads])
    hi = np.array([h[1] for h in heads])
    rows = np.arange(d) if rows is None else np.asarray(rows)
    g = {k: to_numpy64(v) for k, v in inp.items()}
    q, k = g["q"][bi, hi], g["k"][bi, hi]
    v = g["v"][bi, hi][..., rows]
    th, et, al = g["theta"][bi, hi], g["eta"][bi, hi], g["alpha"][bi, hi]
    M0 = None if g.get("M0") is None else g["M0"][bi, hi][:, rows, :]
    S0 = None if g.get("S0") is None else g["S0"][bi, hi][:, rows, :]
    return linear_forward(q, k, v, th, et, al, M0, S0, b=b)


def select(x, heads, rows, state=False):
    bi = np.array([h[0] for h in heads])
    hi = np.array([h[1] for h in heads])
    y = x[bi, hi]
    return y[:, rows, :] if state else y[..., rows]
