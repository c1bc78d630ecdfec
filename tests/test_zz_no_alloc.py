"""The deep-memory entry point that allocates nothing (its exchange workspace
is a file-scope device array), called through the C ABI and checked against
the allocating entry point on two calls in a row, the second smaller."""

import ctypes

import numpy as np
import pytest
import torch

from oracle import mlp_forward
from tests._parity import TOL, rel_err, rel_err_bf16_out, to_dev
from test_neural_memory_amd import _lib
from test_neural_memory_amd import memory as tm
from test_neural_memory_amd.workloads import WORKLOADS, make_inputs, to_numpy64

pytestmark = pytest.mark.gpu


def _noalloc(dev, w):
    lib = _lib.load()
    B, H, T, d = dev["q"].shape
    hid = dev["W1"].shape[-1]
    z = torch.empty((B, H, T, d), dtype=torch.bfloat16, device="cuda")
    outs = [torch.empty_like(dev["W1"]), torch.empty_like(dev["W2"]), torch.empty_like(dev["W1"]),
            torch.empty_like(dev["W2"])]
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.ttt_mem_mlp_forward_bf16_noalloc(p(dev["q"]), p(dev["k"]), p(dev["v"]), p(dev["theta"]), p(dev["eta"]),
                                              p(dev["alpha"]), p(dev["W1"]), p(dev["W2"]), None, None, p(z),
                                              *[p(o) for o in outs], B, H, T, d, hid, w.b, stream)
    assert st == 0, st
    return (z, *outs)


@pytest.mark.parametrize("first,second", [(dict(B=4, H=8, T=100), dict(B=1, H=3, T=40))])
def test_noalloc_matches_allocating_entry_point_twice(first, second):
    for kw in (first, second):
        w = WORKLOADS[5].replace(**kw)
        print(f"case no-alloc deep memory {w}", flush=True)
        inp = make_inputs(w)
        dev = to_dev(inp)
        got = _noalloc(dev, w)
        ref = tm.ttt_mem_mlp_forward_bf16(dev["q"], dev["k"], dev["v"], dev["theta"], dev["eta"], dev["alpha"],
                                          dev["W1"], dev["W2"], b=w.b)
        torch.cuda.synchronize()
        # The same kernel computes every sequence the same way whatever group runs it.
        for a, b_ in zip(got, ref):
            assert torch.equal(a, b_)
        # And against the oracle on the last sequence (bound as for the deep memory).
        g = {k: (None if v is None else to_numpy64(v)[-1, -1]) for k, v in inp.items()}
        zo, W1o, W2o, S1o, S2o = mlp_forward(g["q"], g["k"], g["v"], g["theta"], g["eta"], g["alpha"], g["W1"],
                                             g["W2"], b=w.b)
        errs = [rel_err_bf16_out(to_numpy64(got[0].cpu())[-1, -1], zo)]
        errs += [rel_err(to_numpy64(x.cpu())[-1, -1], r) for x, r in zip(got[1:], (W1o, W2o, S1o, S2o))]
        print("  errors", [f"{e:.2e}" for e in errs], flush=True)
        assert max(errs) <= TOL["bf16"]


def test_noalloc_binding_requires_outputs_and_matches():
    w = WORKLOADS[5].replace(B=1, H=2, T=70)
    dev = to_dev(make_inputs(w))
    args = (dev["q"], dev["k"], dev["v"], dev["theta"], dev["eta"], dev["alpha"], dev["W1"], dev["W2"])
    with pytest.raises(ValueError):
        tm.ttt_mem_mlp_forward_bf16_noalloc(*args, b=w.b, out=None)
    ref = tm.ttt_mem_mlp_forward_bf16(*args, b=w.b)
    out = tuple(torch.full_like(t, float("nan")) for t in ref)
    got = tm.ttt_mem_mlp_forward_bf16_noalloc(*args, b=w.b, out=out)
    torch.cuda.synchronize()
    for a, b_ in zip(got, ref):
        assert torch.equal(a, b_)
