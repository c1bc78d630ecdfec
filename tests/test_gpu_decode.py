"""GPU parity of the token-by-token (primal) linear memory against the float64 oracle.

The primal form is the chunked recurrence with chunks of one token, so the
oracle is ``linear_forward(..., b=1)``.  The kernel computes in float32 on both
entry points (bf16 inputs widen exactly), so both are held to the float32
bound: max|gpu - oracle| / rms(oracle) <= 1e-4 per output (z, M_T, S_T).
"""

import numpy as np
import pytest
import torch

from tests._parity import TOL, rel_err, run_oracle, to_dev
from test_neural_memory_amd import memory as tm
from test_neural_memory_amd._lib import TTTError
from test_neural_memory_amd.workloads import WORKLOADS, make_inputs, to_numpy64

pytestmark = pytest.mark.gpu
TOL_DEC = TOL["f32"]


def _say(msg):
    print(msg, flush=True)


def _with_state(inp, seed=11, scale=0.05):
    """Nonzero carried state: what a decode call receives after a prefill."""
    B, H, T, d = inp["q"].shape
    rng = np.random.default_rng(seed)
    inp = dict(inp)
    inp["M0"] = torch.from_numpy((rng.standard_normal((B, H, d, d)) * scale).astype(np.float32))
    inp["S0"] = torch.from_numpy((rng.standard_normal((B, H, d, d)) * scale * 0.1).astype(np.float32))
    return inp


def _run(inp, **kw):
    dev = to_dev(inp)
    z, M, S = tm.decode(dev["q"], dev["k"], dev["v"], dev["theta"], dev["eta"], dev["alpha"],
                        dev.get("M0"), dev.get("S0"), **kw)
    torch.cuda.synchronize()
    return to_numpy64(z.cpu()), to_numpy64(M.cpu()), to_numpy64(S.cpu())


def _check(inp, tol=TOL_DEC):
    z, M, S = _run(inp)
    zo, Mo, So = run_oracle(inp, 1)
    errs = (rel_err(z.reshape(zo.shape), zo), rel_err(M.reshape(Mo.shape), Mo), rel_err(S.reshape(So.shape), So))
    _say(f"  errors z={errs[0]:.3e} M_T={errs[1]:.3e} S_T={errs[2]:.3e} (tol {tol})")
    assert max(errs) <= tol, errs


CASES = [
    # (label, workload id, overrides): every head size, one token and short runs
    ("d16-T1", 1, dict(B=2, H=3, T=1)),
    ("d16-T37", 1, dict(B=1, H=2, T=37)),
    ("d64-T1", 2, dict(B=2, H=3, T=1)),
    ("d64-T20", 2, dict(B=1, H=2, T=20)),
    ("d32-T9", 3, dict(B=1, H=3, T=9, d=32)),
    ("d128-T1", 3, dict(B=2, H=4, T=1)),
    ("d128-T33", 3, dict(B=1, H=2, T=33)),
]


@pytest.mark.parametrize("label,wid,kw", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_parity(label, wid, kw, dtype):
    w = WORKLOADS[wid].replace(dtype=dtype, **kw)
    _say(f"case {label} {dtype} {w}")
    _check(_with_state(make_inputs(w)))


def test_decode_zero_state_titans_gates():
    w = WORKLOADS[3].replace(B=1, H=2, T=16)
    _say(f"case zero state {w}")
    _check(make_inputs(w))


@pytest.mark.parametrize("gates", ["eta0", "alpha1", "theta0"])
def test_decode_degenerate_gates(gates):
    w = WORKLOADS[3].replace(B=1, H=2, T=12, dtype="f32")
    inp = _with_state(make_inputs(w))
    if gates == "eta0":
        inp["eta"].zero_()
    elif gates == "alpha1":
        inp["alpha"][..., 5] = 1.0
    else:
        inp["theta"].zero_()
    _say(f"case degenerate {gates}")
    _check(inp)


def test_decode_full_size_one_token():
    # The decode workload at full size: every (batch, head), every row, one token.
    w = WORKLOADS[3].replace(T=1)
    _say(f"case full size decode {w}")
    _check(_with_state(make_inputs(w)))


def test_streaming_in_place_matches_one_call():
    # T calls of one token with the state carried in place == one call of T tokens, bit for bit.
    w = WORKLOADS[3].replace(B=1, H=3, T=10)
    inp = to_dev(_with_state(make_inputs(w)))
    args = (inp["q"], inp["k"], inp["v"], inp["theta"], inp["eta"], inp["alpha"])
    z_all, M_all, S_all = tm.decode(*args, inp["M0"], inp["S0"])
    M, S = inp["M0"].clone(), inp["S0"].clone()
    zs = []
    for t in range(w.T):
        one = [a[..., t:t + 1, :].contiguous() if a.dim() == 4 else a[..., t:t + 1].contiguous() for a in args]
        z = torch.empty_like(one[0], dtype=torch.float32)
        tm.decode(*one, M, S, out=(z, M, S))
        zs.append(z)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(zs, dim=2), z_all)
    assert torch.equal(M, M_all) and torch.equal(S, S_all)


def test_decode_matches_forward_b1_f32():
    # The primal kernel and the chunked kernel with b = 1 compute the same recurrence.
    w = WORKLOADS[3].replace(B=1, H=2, T=24, dtype="f32")
    inp = to_dev(_with_state(make_inputs(w)))
    args = (inp["q"], inp["k"], inp["v"], inp["theta"], inp["eta"], inp["alpha"], inp["M0"], inp["S0"])
    zd, Md, Sd = tm.decode(*args)
    zf, Mf, Sf = tm.forward(*args, b=1)
    torch.cuda.synchronize()
    for a, b_ in ((zd, zf), (Md, Mf), (Sd, Sf)):
        assert rel_err(to_numpy64(a.cpu()), to_numpy64(b_.cpu())) <= TOL_DEC


def test_decode_empty_and_null():
    w = WORKLOADS[3].replace(B=1, H=2, T=0, dtype="f32")
    inp = to_dev(_with_state(make_inputs(w)))
    args = (inp["q"], inp["k"], inp["v"], inp["theta"], inp["eta"], inp["alpha"])
    z, M, S = tm.decode(*args, inp["M0"], inp["S0"])
    torch.cuda.synchronize()
    assert z.numel() == 0 and torch.equal(M, inp["M0"]) and torch.equal(S, inp["S0"])
    z, M, S = tm.decode(*args)   # NULL initial state: zeros
    torch.cuda.synchronize()
    assert not M.any() and not S.any()
    w0 = WORKLOADS[3].replace(B=0, H=2, T=4, dtype="f32")
    e = to_dev(make_inputs(w0))
    z, M, S = tm.decode(e["q"], e["k"], e["v"], e["theta"], e["eta"], e["alpha"])
    assert z.numel() == 0


def test_decode_outputs_optional():
    w = WORKLOADS[3].replace(B=1, H=2, T=5, dtype="f32")
    inp = to_dev(_with_state(make_inputs(w)))
    args = (inp["q"], inp["k"], inp["v"], inp["theta"], inp["eta"], inp["alpha"], inp["M0"], inp["S0"])
    ref = tm.decode(*args)
    z = torch.empty_like(ref[0])
    tm.decode(*args, out=(z, None, None))
    torch.cuda.synchronize()
    assert torch.equal(z, ref[0])


def test_decode_argument_errors():
    w = WORKLOADS[3].replace(B=1, H=1, T=4, dtype="f32", d=48)
    inp = to_dev(make_inputs(w))
    with pytest.raises(TTTError) as e:
        tm.decode(inp["q"], inp["k"], inp["v"], inp["theta"], inp["eta"], inp["alpha"])
    assert e.value.status == -2
    w = WORKLOADS[3].replace(B=1, H=1, T=4, dtype="f32", d=16)
    inp = to_dev(make_inputs(w))
    with pytest.raises(TTTError) as e:   # z aliasing q
        tm.decode(inp["q"], inp["k"], inp["v"], inp["theta"], inp["eta"], inp["alpha"],
                  out=(inp["q"], None, None))
    assert e.value.status == -1


def test_decode_graph_replays_match_eager():
    # The bench times decode steps replayed from a HIP graph (state carried in
    # place).  Each replay continues the state; every replay must equal the
    # same steps run eagerly, with eager work and synchronisation in between.
    w = WORKLOADS[3].replace(B=1, H=4, T=3)
    inp = to_dev(_with_state(make_inputs(w)))
    toks = [tuple(inp[x][:, :, t:t + 1, :].contiguous() if inp[x].dim() == 4 else inp[x][:, :, t:t + 1].contiguous()
                  for x in ("q", "k", "v", "theta", "eta", "alpha")) for t in range(w.T)]
    M, S = inp["M0"].clone(), inp["S0"].clone()
    z = torch.empty(w.B, w.H, 1, w.d, dtype=torch.float32, device="cuda")
    tm.decode(*toks[0], M.clone(), S.clone())   # load the library before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t in range(w.T):
            tm.decode(*toks[t], M, S, out=(z, M, S))
    # Capture launches nothing: reset the carried state before the first replay.
    M.copy_(inp["M0"])
    S.copy_(inp["S0"])
    Me, Se = inp["M0"].clone(), inp["S0"].clone()
    ze = torch.empty_like(z)
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for t in range(w.T):
            tm.decode(*toks[t], Me, Se, out=(ze, Me, Se))
        torch.cuda.synchronize()
        _say(f"  replay {rep}: max|dz| {float((z - ze).abs().max()):.3e}")
        assert torch.equal(z, ze) and torch.equal(M, Me) and torch.equal(S, Se)
