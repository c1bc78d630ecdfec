"""GPU parity of the linear memory over packed variable-length documents.

Every document starts from its own state and is chunked on its own, so the
oracle runs ``linear_forward`` on each (document, head) separately.  Bounds as
for the dense forward: max|gpu - oracle| / rms(oracle) <= 1e-4 (float32) and
<= 2e-2 (bf16 inputs), per output (z, M_T, S_T).
"""

import numpy as np
import pytest
import torch

from oracle import linear_forward
from tests._parity import TOL, rel_err
from test_neural_memory_amd import memory as tm
from test_neural_memory_amd._lib import TTTError
from test_neural_memory_amd.workloads import WORKLOADS, make_inputs, to_numpy64

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _packed(wid, H, lengths, dtype, d=None, tail=0, states=True, seed=21):
    """Packed inputs [H, T, d] for documents of the given lengths (plus `tail` unused tokens)."""
    T = int(sum(lengths)) + tail
    kw = dict(B=1, H=H, T=max(T, 1), dtype=dtype)
    if d is not None:
        kw["d"] = d
    w = WORKLOADS[wid].replace(**kw)
    inp = make_inputs(w)
    g = {k: v[0, :, :T].contiguous() for k, v in inp.items() if v is not None and k in ("q", "k", "v")}
    g.update({k: inp[k][0, :, :T].contiguous() for k in ("theta", "eta", "alpha")})
    N = len(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    if states:
        rng = np.random.default_rng(seed)
        g["M0"] = torch.from_numpy((rng.standard_normal((N, H, w.d, w.d)) * 0.05).astype(np.float32))
        g["S0"] = torch.from_numpy((rng.standard_normal((N, H, w.d, w.d)) * 0.005).astype(np.float32))
    return w, g, torch.from_numpy(cu)


def _run(g, cu, b, out=None):
    dev = {k: v.cuda() for k, v in g.items()}
    res = tm.forward_varlen(dev["q"], dev["k"], dev["v"], dev["theta"], dev["eta"], dev["alpha"], cu.cuda(),
                            dev.get("M0"), dev.get("S0"), b=b, out=out)
    torch.cuda.synchronize()
    return res


def _check(g, cu, b, tol):
    z, M, S = (to_numpy64(x.cpu()) for x in _run(g, cu, b))
    n64 = {k: to_numpy64(v) for k, v in g.items()}
    H = n64["q"].shape[0]
    errs = [0.0, 0.0, 0.0]
    zr, Mr, Sr, zg, Mg, Sg = [], [], [], [], [], []
    for s in range(len(cu) - 1):
        t0, t1 = int(cu[s]), int(cu[s + 1])
        for h in range(H):
            sl = (h, slice(t0, t1))
            M0 = n64["M0"][s, h] if "M0" in n64 else None
            S0 = n64["S0"][s, h] if "S0" in n64 else None
            zo, Mo, So = linear_forward(n64["q"][sl], n64["k"][sl], n64["v"][sl], n64["theta"][sl], n64["eta"][sl],
                                        n64["alpha"][sl], M0, S0, b=b)
            zr.append(zo.reshape(-1)); Mr.append(Mo.reshape(-1)); Sr.append(So.reshape(-1))
            zg.append(z[sl].reshape(-1)); Mg.append(M[s, h].reshape(-1)); Sg.append(S[s, h].reshape(-1))
    errs = [rel_err(np.concatenate(a), np.concatenate(r)) for a, r in ((zg, zr), (Mg, Mr), (Sg, Sr))]
    _say(f"  errors z={errs[0]:.3e} M_T={errs[1]:.3e} S_T={errs[2]:.3e} (tol {tol})")
    assert max(errs) <= tol, errs


CASES = [
    # (label, workload id, H, document lengths, b, d): lengths below, at and above b, ragged tails
    ("titans-mixed", 3, 2, [130, 1, 64, 0, 257, 33], 64, None),
    ("titans-short-docs", 3, 3, [5, 17, 63, 2, 40], 64, None),
    ("titans-d64-b16", 3, 2, [50, 16, 7, 100], 16, 64),
    ("ttt-b16", 2, 2, [31, 90, 16, 3], 16, None),
    ("tiny-d16", 1, 2, [9, 1, 24, 8], 8, None),
    # 100 documents: the in-kernel longest-first ranking uses both of its 64-lane groups.
    # 150 and 600 documents: the order comes from the ranking pass before the launch
    # (lengths 0 .. 40, so empty documents and many ties).
    ("hundred-docs", 3, 1, [int(x) for x in np.random.default_rng(6).integers(0, 41, 100)], 16, 32),
    ("many-docs", 3, 1, [int(x) for x in np.random.default_rng(5).integers(0, 41, 150)], 16, 32),
    ("600-docs", 3, 2, [int(x) for x in np.random.default_rng(7).integers(0, 41, 600)], 16, 32),
    # bf16 at d >= 64 runs persistent workgroups that walk a table of documents:
    # 600 documents dealt in boustrophedon order; one 8000-token document among
    # 400 short ones (longest-processing-time head, then the lanes below the
    # average); 700 documents, past the in-LDS ranking's limit at d = 64, b = 16
    # (one workgroup per document, ordered by the pass before the launch).
    ("600-docs-d64", 3, 2, [int(x) for x in np.random.default_rng(8).integers(0, 41, 600)], 16, 64),
    ("skewed-d128", 3, 4, [int(x) for x in np.random.default_rng(9).integers(20, 61, 150)] + [8000]
     + [int(x) for x in np.random.default_rng(10).integers(0, 61, 250)], 64, None),
    ("700-docs-d64", 3, 1, [int(x) for x in np.random.default_rng(11).integers(0, 11, 700)], 16, 64),
]


@pytest.mark.parametrize("label,wid,H,lengths,b,d", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_varlen_parity(label, wid, H, lengths, b, d, dtype):
    w, g, cu = _packed(wid, H, lengths, dtype, d=d)
    _say(f"case {label} {dtype} H={H} N={len(lengths)} lengths={lengths[:8]} b={b} d={w.d}")
    _check(g, cu, b, TOL[dtype])


def test_varlen_zero_states():
    w, g, cu = _packed(3, 2, [70, 129, 12], "bf16", states=False)
    _say("case zero initial states")
    _check(g, cu, 64, TOL["bf16"])


def test_varlen_equals_dense_bitwise():
    # N documents of equal length packed == the dense forward with B = N, bit for bit.
    w = WORKLOADS[3].replace(B=3, H=2, T=150)
    inp = make_inputs(w)
    dense = {k: v.cuda() for k, v in inp.items() if v is not None}
    zd, Md, Sd = tm.forward(dense["q"], dense["k"], dense["v"], dense["theta"], dense["eta"], dense["alpha"], b=64,
                            z_dtype=torch.float32)
    pack = {k: v.transpose(0, 1).reshape(w.H, w.B * w.T, *v.shape[3:]).contiguous() for k, v in dense.items()}
    cu = torch.arange(0, (w.B + 1) * w.T, w.T, dtype=torch.int32, device="cuda")
    zp, Mp, Sp = tm.forward_varlen(pack["q"], pack["k"], pack["v"], pack["theta"], pack["eta"], pack["alpha"], cu,
                                   b=64)
    torch.cuda.synchronize()
    assert torch.equal(zp.reshape(w.H, w.B, w.T, w.d).transpose(0, 1), zd)
    assert torch.equal(Mp, Md) and torch.equal(Sp, Sd)


def test_varlen_unused_tail_and_empty_docs():
    # Tokens after the last document are neither read into any state nor written.
    w, g, cu = _packed(3, 2, [0, 40, 0], "f32", tail=9)
    dev = {k: v.cuda() for k, v in g.items()}
    H, T, d = dev["q"].shape
    z = torch.full((H, T, d), float("nan"), device="cuda")
    M = torch.empty(3, H, d, d, device="cuda")
    S = torch.empty_like(M)
    tm.forward_varlen(dev["q"], dev["k"], dev["v"], dev["theta"], dev["eta"], dev["alpha"], cu.cuda(),
                      dev["M0"], dev["S0"], b=64, out=(z, M, S))
    torch.cuda.synchronize()
    assert torch.isnan(z[:, 40:]).all() and not torch.isnan(z[:, :40]).any()
    for s in (0, 2):   # empty documents copy their initial state
        assert torch.equal(M[s], dev["M0"][s]) and torch.equal(S[s], dev["S0"][s])
    _check(g, cu, 64, TOL["f32"])


def test_varlen_argument_errors():
    w, g, cu = _packed(3, 1, [10, 6], "f32")
    dev = {k: v.cuda() for k, v in g.items()}
    args = (dev["q"], dev["k"], dev["v"], dev["theta"], dev["eta"], dev["alpha"])
    with pytest.raises(TTTError) as e:
        tm.forward_varlen(*args, cu.cuda(), b=65)
    assert e.value.status == -2
    with pytest.raises(TTTError) as e:
        tm.forward_varlen(*args, cu.cuda(), b=0)
    assert e.value.status == -1
    with pytest.raises(ValueError):
        tm.forward_varlen(*args, cu, b=16)   # offsets must be on the device


def test_varlen_full_size_sampled():
    # The packed workload in the launch configuration of the bench: 32768
    # tokens per head in 31 documents of seeded lognormal lengths, H=16,
    # d=128, b=64, bf16.  Checked on documents 0 and 1 and the longest, on
    # heads 0 and 15, every row of z and both final states.
    from test_neural_memory_amd.workloads import varlen_lengths
    w = WORKLOADS[3].replace(B=1, T=4 * 8192)
    L = varlen_lengths(w.T)
    inp = make_inputs(w)
    dev = {k: v[0].cuda() for k, v in inp.items() if v is not None}
    cu = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    _say(f"case full-size packed forward: {len(L)} documents, T={w.T}")
    z, M, S = tm.forward_varlen(dev["q"], dev["k"], dev["v"], dev["theta"], dev["eta"], dev["alpha"],
                                torch.from_numpy(cu).cuda(), b=w.b)
    torch.cuda.synchronize()
    for h in (0, w.H - 1):
        n = {k: to_numpy64(v[0, h]) for k, v in inp.items() if v is not None}
        for s in (0, 1, int(np.argmax(L))):
            t0, t1 = int(cu[s]), int(cu[s + 1])
            zo, Mo, So = linear_forward(n["q"][t0:t1], n["k"][t0:t1], n["v"][t0:t1], n["theta"][t0:t1],
                                        n["eta"][t0:t1], n["alpha"][t0:t1], None, None, b=w.b)
            errs = [rel_err(to_numpy64(z[h, t0:t1].cpu()), zo), rel_err(to_numpy64(M[s, h].cpu()), Mo),
                    rel_err(to_numpy64(S[s, h].cpu()), So)]
            _say(f"  head {h} document {s} ({t1 - t0} tokens): z={errs[0]:.2e} M_T={errs[1]:.2e} S_T={errs[2]:.2e}")
            assert max(errs) <= TOL["bf16"], errs
