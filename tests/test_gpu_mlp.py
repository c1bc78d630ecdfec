"""GPU parity of the HIP deep (2-layer MLP) memory against the float64 oracle.

Every comparison is element by element on the same seeded inputs, per output
tensor (z, W1_T, W2_T, S1_T, S2_T), as max|gpu - oracle| / rms(oracle) <= 2e-2
(bf16 inputs, fp16 MFMA operands, float32 accumulation and weights).
"""

import numpy as np
import pytest
import torch

from oracle import mlp_forward
from tests._parity import TOL, rel_err, to_dev
from test_neural_memory_amd import memory as tm
from test_neural_memory_amd._lib import TTTError
from test_neural_memory_amd.workloads import WORKLOADS, make_inputs, to_numpy64

pytestmark = pytest.mark.gpu
TOL_MLP = TOL["bf16"]
NAMES = ("z", "W1_T", "W2_T", "S1_T", "S2_T")


def _say(msg):
    print(msg, flush=True)


def run_gpu(inp, b, **kw):
    dev = to_dev(inp)
    outs = tm.ttt_mem_mlp_forward_bf16(dev["q"], dev["k"], dev["v"], dev["theta"], dev["eta"], dev["alpha"],
                                       dev["W1"], dev["W2"], dev.get("S1"), dev.get("S2"), b=b, **kw)
    torch.cuda.synchronize()
    return [to_numpy64(x.cpu()) for x in outs]


def run_oracle(inp, b, heads=None):
    B, H = inp["q"].shape[:2]
    if heads is None:
        heads = [(i, j) for i in range(B) for j in range(H)]
    bi = np.array([h[0] for h in heads])
    hi = np.array([h[1] for h in heads])
    g = {k: (None if v is None else to_numpy64(v)[bi, hi]) for k, v in inp.items()}
    return mlp_forward(g["q"], g["k"], g["v"], g["theta"], g["eta"], g["alpha"], g["W1"], g["W2"],
                       g.get("S1"), g.get("S2"), b=b)


def _check(inp, b, heads=None, tol=TOL_MLP, ref=None, **kw):
    got = run_gpu(inp, b, **kw)
    ref = run_oracle(inp, b, heads) if ref is None else ref
    if heads is None:
        got = [x.reshape((-1,) + x.shape[2:]) for x in got]   # (batch, head) pairs in row-major order
    else:
        bi = np.array([h[0] for h in heads])
        hi = np.array([h[1] for h in heads])
        got = [x[bi, hi] for x in got]
    errs = [rel_err(x, r) for x, r in zip(got, ref)]
    _say("  errors " + " ".join(f"{n}={e:.3e}" for n, e in zip(NAMES, errs)) + f" (tol {tol})")
    assert max(errs) <= tol, errs
    return errs


def _small(**kw):
    return WORKLOADS[5].replace(**kw)


def _with_momenta(inp, seed=3, scale=0.02):
    rng = np.random.default_rng(seed)
    S1 = rng.standard_normal(tuple(inp["W1"].shape)) * scale
    S2 = rng.standard_normal(tuple(inp["W2"].shape)) * scale
    inp = dict(inp)
    inp["S1"] = torch.from_numpy(S1.astype(np.float32))
    inp["S2"] = torch.from_numpy(S2.astype(np.float32))
    return inp


CASES = [
    # (label, overrides): several chunks and ragged final chunks
    ("deep-small", dict(B=2, H=2, T=200)),
    ("deep-ragged-b5", dict(B=1, H=2, T=203, b=5)),
    ("deep-b1", dict(B=1, H=1, T=37, b=1)),
    ("deep-b13", dict(B=1, H=3, T=131, b=13)),
    ("deep-T1", dict(B=2, H=1, T=1)),
    ("deep-odd-bh", dict(B=3, H=3, T=50)),
]


@pytest.mark.parametrize("label,kw", CASES, ids=[c[0] for c in CASES])
def test_small_cases(label, kw):
    w = _small(**kw)
    _say(f"case {label} {w}")
    _check(make_inputs(w), w.b)


def test_initial_momenta():
    w = _small(B=1, H=2, T=150)
    _say(f"case initial momenta {w}")
    _check(_with_momenta(make_inputs(w)), w.b)


def test_titans_gates():
    w = _small(B=1, H=2, T=160, gates="titans")
    _say(f"case titans gates {w}")
    _check(make_inputs(w), w.b)


@pytest.mark.parametrize("gates", ["eta0", "alpha1", "theta0"])
def test_degenerate_gates(gates):
    w = _small(B=1, H=2, T=70)
    inp = make_inputs(w)
    if gates == "eta0":
        inp["eta"].zero_()
    elif gates == "alpha1":
        inp["alpha"][..., 17] = 1.0
        inp["alpha"][..., 40] = 1.0
    else:
        inp["theta"].zero_()
    _say(f"case degenerate {gates}")
    _check(_with_momenta(inp), w.b)


def test_theta0_is_plain_read():
    # theta = eta = alpha = 0: the weights never change and z_t = f(q_t).
    w = _small(B=1, H=1, T=40)
    inp = make_inputs(w)
    for g in ("theta", "eta", "alpha"):
        inp[g].zero_()
    z, W1, W2, S1, S2 = run_gpu(inp, w.b)
    g = {k: (None if v is None else to_numpy64(v)) for k, v in inp.items()}
    h = g["q"] @ g["W1"]
    f = g["q"] + (h / (1 + np.exp(-h))) @ g["W2"]
    _say(f"  plain read error {rel_err(z, f):.3e}")
    assert rel_err(z, f) <= TOL_MLP
    assert np.array_equal(W1, g["W1"]) and np.array_equal(W2, g["W2"])
    assert not S1.any() and not S2.any()


def test_full_size_sampled():
    # The deep-memory workload at full size; the oracle checks two sequences,
    # for bf16 z and for float32 z; over the whole output the bf16 z is the
    # float32 z rounded to nearest even.
    w = WORKLOADS[5]
    _say(f"case full size {w}")
    inp = make_inputs(w)
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    ref = run_oracle(inp, w.b, heads)
    _check(inp, w.b, heads=heads, ref=ref)
    _check(inp, w.b, heads=heads, ref=ref, z_dtype=torch.float32)
    dev = to_dev(inp)
    args = (dev["q"], dev["k"], dev["v"], dev["theta"], dev["eta"], dev["alpha"], dev["W1"], dev["W2"])
    zb = tm.ttt_mem_mlp_forward_bf16(*args, b=w.b)[0]
    zf = tm.ttt_mem_mlp_forward_bf16(*args, b=w.b, z_dtype=torch.float32)[0]
    torch.cuda.synchronize()
    assert zb.dtype == torch.bfloat16 and torch.equal(zb, zf.to(torch.bfloat16))


def test_empty_sequence_copies_weights():
    w = _small(B=1, H=2, T=0)
    inp = _with_momenta(make_inputs(w))
    z, W1, W2, S1, S2 = run_gpu(inp, w.b)
    assert z.size == 0
    for x, name in ((W1, "W1"), (W2, "W2"), (S1, "S1"), (S2, "S2")):
        assert np.array_equal(x, to_numpy64(inp[name]))


def test_empty_batch():
    w = _small(B=0, H=2, T=16)
    z, W1, W2, S1, S2 = run_gpu(make_inputs(w), w.b)
    assert z.size == 0 and W1.size == 0


def test_resume_bit_identical():
    # Splitting at a chunk boundary and carrying (W1, W2, S1, S2) reproduces one call exactly.
    w = _small(B=1, H=2, T=96)
    inp = to_dev(make_inputs(w))
    args = (inp["q"], inp["k"], inp["v"], inp["theta"], inp["eta"], inp["alpha"])
    full = tm.ttt_mem_mlp_forward_bf16(*args, inp["W1"], inp["W2"], b=w.b)
    cut = 48
    part = [a[..., :cut, :].contiguous() if a.dim() == 4 else a[..., :cut].contiguous() for a in args]
    rest = [a[..., cut:, :].contiguous() if a.dim() == 4 else a[..., cut:].contiguous() for a in args]
    z1, W1, W2, S1, S2 = tm.ttt_mem_mlp_forward_bf16(*part, inp["W1"], inp["W2"], b=w.b)
    z2, W1b, W2b, S1b, S2b = tm.ttt_mem_mlp_forward_bf16(*rest, W1, W2, S1, S2, b=w.b)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([z1, z2], dim=2), full[0])
    for a, b_ in zip((W1b, W2b, S1b, S2b), full[1:]):
        assert torch.equal(a, b_)


def test_in_place_carry_and_no_outputs():
    w = _small(B=1, H=2, T=64)
    inp = to_dev(_with_momenta(make_inputs(w)))
    args = (inp["q"], inp["k"], inp["v"], inp["theta"], inp["eta"], inp["alpha"])
    ref = tm.ttt_mem_mlp_forward_bf16(*args, inp["W1"], inp["W2"], inp["S1"], inp["S2"], b=w.b)
    W1, W2, S1, S2 = (inp[k].clone() for k in ("W1", "W2", "S1", "S2"))
    z = torch.empty_like(ref[0])
    tm.ttt_mem_mlp_forward_bf16(*args, W1, W2, S1, S2, b=w.b, out=(z, W1, W2, S1, S2))
    z_only = torch.empty_like(ref[0])
    tm.ttt_mem_mlp_forward_bf16(*args, inp["W1"], inp["W2"], inp["S1"], inp["S2"], b=w.b,
                                out=(z_only, None, None, None, None))
    torch.cuda.synchronize()
    assert torch.equal(z, ref[0]) and torch.equal(z_only, ref[0])
    for a, b_ in zip((W1, W2, S1, S2), ref[1:]):
        assert torch.equal(a, b_)


def test_deterministic():
    w = _small(B=2, H=2, T=100)
    a = run_gpu(make_inputs(w), w.b)
    b = run_gpu(make_inputs(w), w.b)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_argument_errors():
    w = _small(B=1, H=1, T=32)
    inp = to_dev(make_inputs(w))
    args = (inp["q"], inp["k"], inp["v"], inp["theta"], inp["eta"], inp["alpha"], inp["W1"], inp["W2"])
    with pytest.raises(TTTError) as e:
        tm.ttt_mem_mlp_forward_bf16(*args, b=17)
    assert e.value.status == -2
    with pytest.raises(TTTError) as e:
        tm.ttt_mem_mlp_forward_bf16(*args, b=0)
    assert e.value.status == -1
    w2 = _small(B=1, H=1, T=32, d=32, hidden=128)
    inp2 = to_dev(make_inputs(w2))
    with pytest.raises(TTTError) as e:
        tm.ttt_mem_mlp_forward_bf16(inp2["q"], inp2["k"], inp2["v"], inp2["theta"], inp2["eta"], inp2["alpha"],
                                    inp2["W1"], inp2["W2"], b=16)
    assert e.value.status == -2
