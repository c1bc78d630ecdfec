"""GPU parity of training over packed variable-length documents.

Every document is its own sequence with its own initial state, so the oracle
is ``linear_backward`` run on each (document, head) separately.  Bounds as for
the dense backward: max|gpu - oracle| / rms(oracle) <= 1e-4 (float32) and
<= 2e-2 (bf16 inputs), per gradient over all documents.
"""

import numpy as np
import pytest
import torch

from oracle import linear_backward
from tests._parity import TOL, rel_err
from test_neural_memory_amd import memory as tm
from test_neural_memory_amd._lib import TTTError
from test_neural_memory_amd.workloads import WORKLOADS, make_inputs, to_numpy64

pytestmark = pytest.mark.gpu
NAMES = ("dq", "dk", "dv", "dtheta", "deta", "dalpha", "dM0", "dS0")


def _say(msg):
    print(msg, flush=True)


def _packed(wid, H, lengths, dtype, d=None, tail=0, seed=41):
    """Packed inputs [H, T, d], gates [H, T], per-document states and cotangents."""
    T = int(sum(lengths)) + tail
    kw = dict(B=1, H=H, T=max(T, 1), dtype=dtype)
    if d is not None:
        kw["d"] = d
    w = WORKLOADS[wid].replace(**kw)
    inp = make_inputs(w)
    g = {k: inp[k][0, :, :T].contiguous() for k in ("q", "k", "v", "theta", "eta", "alpha")}
    N = len(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    rng = np.random.default_rng(seed)
    g["M0"] = torch.from_numpy((rng.standard_normal((N, H, w.d, w.d)) * 0.05).astype(np.float32))
    g["S0"] = torch.from_numpy((rng.standard_normal((N, H, w.d, w.d)) * 0.005).astype(np.float32))
    cot = {"dz": torch.from_numpy(rng.standard_normal((H, T, w.d)).astype(np.float32)),
           "dM_T": torch.from_numpy((rng.standard_normal((N, H, w.d, w.d)) * 0.1).astype(np.float32)),
           "dS_T": torch.from_numpy((rng.standard_normal((N, H, w.d, w.d)) * 0.1).astype(np.float32))}
    return w, g, cot, torch.from_numpy(cu)


def _gpu(g, cot, cu, b, out=None):
    dev = {k: v.cuda() for k, v in g.items()}
    cd = {k: v.cuda() for k, v in cot.items()}
    cud = cu.cuda()
    args = (dev["q"], dev["k"], dev["v"], dev["theta"], dev["eta"], dev["alpha"])
    ckpt = tm.new_ckpt_varlen(dev["q"], cud, b)
    z, M, S, ckpt = tm.forward_varlen(*args, cud, dev["M0"], dev["S0"], b=b, ckpt=ckpt)
    grads = tm.backward_varlen(*args, cud, ckpt, cd["dz"], cd["dM_T"], cd["dS_T"], b=b, out=out)
    torch.cuda.synchronize()
    return grads


def _check(g, cot, cu, b, tol):
    grads = [to_numpy64(x.cpu()) for x in _gpu(g, cot, cu, b)]
    n = {k: to_numpy64(v) for k, v in g.items()}
    c = {k: to_numpy64(v) for k, v in cot.items()}
    H = n["q"].shape[0]
    gpu_parts = [[] for _ in NAMES]
    ref_parts = [[] for _ in NAMES]
    for s in range(len(cu) - 1):
        t0, t1 = int(cu[s]), int(cu[s + 1])
        for h in range(H):
            sl = (h, slice(t0, t1))
            ref = linear_backward(n["q"][sl], n["k"][sl], n["v"][sl], n["theta"][sl], n["eta"][sl],
                                  n["alpha"][sl], c["dz"][sl], c["dM_T"][s, h], c["dS_T"][s, h],
                                  n["M0"][s, h], n["S0"][s, h], b=b)
            got = [grads[i][sl] for i in range(6)] + [grads[6][s, h], grads[7][s, h]]
            for i in range(8):
                gpu_parts[i].append(np.asarray(got[i]).reshape(-1))
                ref_parts[i].append(np.asarray(ref[i]).reshape(-1))
    errs = {nm: rel_err(np.concatenate(gp), np.concatenate(rp)) for nm, gp, rp in zip(NAMES, gpu_parts, ref_parts)}
    _say("  errors " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()) + f" (tol {tol})")
    assert max(errs.values()) <= tol, errs


CASES = [
    # (label, workload id, H, document lengths, b, d): lengths below, at and above b, empty documents
    ("titans-mixed", 3, 2, [130, 1, 64, 0, 200, 33], 64, None),
    ("titans-d64-b16", 3, 2, [50, 16, 7, 100], 16, 64),
    ("ttt-b16", 2, 2, [31, 90, 16, 3], 16, None),
    ("tiny-d16", 1, 2, [9, 1, 24, 8], 8, None),
    # 150 documents: the gradient kernel's document search takes three 64-lane
    # steps, and above 128 documents the carry walk takes its order from the
    # ranking pass before the launch (600: ten steps, many ties and empty ones).
    # 100 documents: the in-kernel longest-first ranking uses both of its 64-lane groups.
    ("hundred-docs", 3, 1, [int(x) for x in np.random.default_rng(6).integers(0, 41, 100)], 16, 32),
    ("many-docs", 3, 1, [int(x) for x in np.random.default_rng(5).integers(0, 41, 150)], 16, 32),
    ("600-docs", 3, 1, [int(x) for x in np.random.default_rng(7).integers(0, 41, 600)], 16, 32),
    # bf16 at d = 64: the forward with checkpoints and the carry walk run the
    # persistent document walks (checkpoint slots from the in-kernel chunk
    # prefix, 300 documents, empty ones among them).
    ("300-docs-d64", 3, 1, [int(x) for x in np.random.default_rng(12).integers(0, 41, 300)], 16, 64),
    # One long document among short ones at d = 128: the persistent carry walk's
    # longest-processing-time head (and the forward's) take the long one alone.
    ("skewed-d128", 3, 2, [int(x) for x in np.random.default_rng(13).integers(5, 41, 40)] + [1500]
     + [int(x) for x in np.random.default_rng(14).integers(0, 41, 60)], 64, None),
]


@pytest.mark.parametrize("label,wid,H,lengths,b,d", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_varlen_backward_parity(label, wid, H, lengths, b, d, dtype):
    w, g, cot, cu = _packed(wid, H, lengths, dtype, d=d)
    _say(f"case {label} {dtype} H={H} N={len(lengths)} lengths={lengths[:8]} b={b} d={w.d}")
    _check(g, cot, cu, b, TOL[dtype])


def test_varlen_backward_equals_dense_bitwise():
    # N equal-length documents packed == the dense training step with B = N, bit for bit.
    w = WORKLOADS[3].replace(B=3, H=2, T=150)
    inp = make_inputs(w)
    rng = np.random.default_rng(7)
    dense = {k: v.cuda() for k, v in inp.items() if v is not None}
    dz = torch.from_numpy(rng.standard_normal((w.B, w.H, w.T, w.d)).astype(np.float32)).cuda()
    dMT = torch.from_numpy((rng.standard_normal((w.B, w.H, w.d, w.d)) * 0.1).astype(np.float32)).cuda()
    dST = torch.from_numpy((rng.standard_normal((w.B, w.H, w.d, w.d)) * 0.1).astype(np.float32)).cuda()
    args = (dense["q"], dense["k"], dense["v"], dense["theta"], dense["eta"], dense["alpha"])
    _, _, _, ckpt = tm.forward_train(*args, b=64)
    gd = tm.backward(*args, ckpt, dz, dMT, dST, b=64)
    pack = {k: v.transpose(0, 1).reshape(w.H, w.B * w.T, *v.shape[3:]).contiguous() for k, v in dense.items()}
    dzp = dz.transpose(0, 1).reshape(w.H, w.B * w.T, w.d).contiguous()
    cu = torch.arange(0, (w.B + 1) * w.T, w.T, dtype=torch.int32, device="cuda")
    pargs = (pack["q"], pack["k"], pack["v"], pack["theta"], pack["eta"], pack["alpha"])
    ckp = tm.new_ckpt_varlen(pack["q"], cu, 64)
    tm.forward_varlen(*pargs, cu, b=64, ckpt=ckp)
    gp = tm.backward_varlen(*pargs, cu, ckp, dzp, dMT, dST, b=64)
    torch.cuda.synchronize()
    for i in range(3):
        assert torch.equal(gp[i].reshape(w.H, w.B, w.T, w.d).transpose(0, 1), gd[i]), NAMES[i]
    for i in range(3, 6):
        assert torch.equal(gp[i].reshape(w.H, w.B, w.T).transpose(0, 1), gd[i]), NAMES[i]
    assert torch.equal(gp[6], gd[6]) and torch.equal(gp[7], gd[7])


def test_varlen_backward_unused_tail_and_empty_docs():
    # Gradients of tokens outside every document are not written; an empty
    # document passes its state cotangents straight through.
    w, g, cot, cu = _packed(3, 2, [0, 40, 0], "f32", tail=9)
    H, T, d = g["q"].shape
    out = [torch.full((H, T, d), float("nan"), device="cuda") for _ in range(3)] + \
          [torch.full((H, T), float("nan"), device="cuda") for _ in range(3)] + \
          [torch.empty(3, H, d, d, device="cuda") for _ in range(2)]
    _gpu(g, cot, cu, 64, out=out)
    for t in out[:3]:
        assert torch.isnan(t[:, 40:]).all() and not torch.isnan(t[:, :40]).any()
    for t in out[3:6]:
        assert torch.isnan(t[:, 40:]).all() and not torch.isnan(t[:, :40]).any()
    for s in (0, 2):
        assert torch.equal(out[6][s].cpu(), cot["dM_T"][s])
        assert torch.equal(out[7][s].cpu(), cot["dS_T"][s])
    _check(g, cot, cu, 64, TOL["f32"])


def test_varlen_backward_argument_errors():
    w, g, cot, cu = _packed(3, 1, [10, 6], "f32")
    dev = {k: v.cuda() for k, v in g.items()}
    args = (dev["q"], dev["k"], dev["v"], dev["theta"], dev["eta"], dev["alpha"])
    ck = tm.new_ckpt_varlen(dev["q"], cu, 16)
    with pytest.raises(ValueError):   # wrong checkpoint shape
        tm.backward_varlen(*args, cu.cuda(), ck[:, :1], cot["dz"].cuda(), b=16)
    with pytest.raises(TTTError) as e:
        tm.backward_varlen(*args, cu.cuda(), tm.new_ckpt_varlen(dev["q"], cu, 65), cot["dz"].cuda(), b=65)
    assert e.value.status == -2


def test_varlen_training_overlapping_offsets_stay_in_slots():
    # Offsets that are not non-decreasing make documents overlap, so their
    # chunks can outnumber the ceil(T/b) + N slots of a head.  The values are
    # then undefined, but every checkpoint and work-buffer write stays within
    # the caller's slots: a canary head placed behind both buffers is untouched.
    w, g, cot, _ = _packed(3, 2, [100, 100], "bf16", d=64)
    dev = {k: v.cuda() for k, v in g.items() if k not in ("M0", "S0")}
    args = (dev["q"], dev["k"], dev["v"], dev["theta"], dev["eta"], dev["alpha"])
    cu = torch.tensor([0, 200, 0, 200, 200], dtype=torch.int32, device="cuda")
    H = dev["q"].shape[0]
    shape = tm.new_ckpt_varlen(dev["q"], cu, 16).shape
    ck_big = torch.full((H + 1,) + tuple(shape[1:]), 7.0, dtype=torch.float16, device="cuda")
    need = tm.backward_work_bytes(dev["q"], 16, cu)
    wk_big = torch.full((need + 4096,), 7, dtype=torch.uint8, device="cuda")
    _say(f"case overlapping offsets {cu.tolist()} b=16 slots={shape[1]}")
    tm.forward_varlen(*args, cu, b=16, ckpt=ck_big[:H])
    tm.backward_varlen(*args, cu, ck_big[:H], cot["dz"].cuda(), b=16, work=wk_big[:need])
    torch.cuda.synchronize()
    assert (ck_big[H] == 7.0).all() and (wk_big[need:] == 7).all()


def test_varlen_training_full_size_sampled():
    # Training over the packed workload in the launch configuration of the
    # bench (32768 tokens per head in 31 documents of seeded lognormal
    # lengths, H=16, d=128, b=64, bf16, seeded N(0,1) dz).  Every gradient of
    # documents 0 and 1 and of the longest one, on heads 0 and 15, against the
    # oracle's backward of each document alone.
    from test_neural_memory_amd.workloads import make_cotangents, varlen_lengths
    w = WORKLOADS[3].replace(B=1, T=4 * 8192)
    L = varlen_lengths(w.T)
    inp = make_inputs(w)
    dev = {k: v[0].cuda() for k, v in inp.items() if v is not None}
    dz = make_cotangents(w, states=False)["dz"][0]
    cu = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    cud = torch.from_numpy(cu).cuda()
    args = (dev["q"], dev["k"], dev["v"], dev["theta"], dev["eta"], dev["alpha"])
    _say(f"case full-size packed training: {len(L)} documents, T={w.T}")
    ckpt = tm.new_ckpt_varlen(dev["q"], cud, w.b)
    tm.forward_varlen(*args, cud, b=w.b, ckpt=ckpt)
    g = tm.backward_varlen(*args, cud, ckpt, dz.cuda(), b=w.b)
    torch.cuda.synchronize()
    for h in (0, w.H - 1):
        n = {k: to_numpy64(v[0, h]) for k, v in inp.items() if v is not None}
        dzn = to_numpy64(dz[h])
        for s in (0, 1, int(np.argmax(L))):
            t0, t1 = int(cu[s]), int(cu[s + 1])
            ref = linear_backward(n["q"][t0:t1], n["k"][t0:t1], n["v"][t0:t1], n["theta"][t0:t1],
                                  n["eta"][t0:t1], n["alpha"][t0:t1], dzn[t0:t1], None, None, None, None, b=w.b)
            got = [to_numpy64(x[h, t0:t1].cpu()) for x in g[:6]] + [to_numpy64(g[6][s, h].cpu()),
                                                                      to_numpy64(g[7][s, h].cpu())]
            errs = {nm: rel_err(x, r) for nm, x, r in zip(NAMES, got, ref)}
            _say(f"  head {h} document {s} ({t1 - t0} tokens): max error {max(errs.values()):.2e}")
            assert max(errs.values()) <= TOL["bf16"], errs
