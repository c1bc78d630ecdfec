"""Pins of the float64 deep-memory oracle of any depth (``deep_forward``).

"论文速览 | Titans" section 3.9 defines the deep memory as L linear maps with a
nonlinearity between them, and section 8.5 compares depths 1 to 4; the pages
print no values for it.  So the oracle is pinned by:
* its explicit backprop (``deep_chunk_grads``) against torch.autograd (a
  library routine) and against central finite differences, at depths 2-4;
* the generic chunked TTT loop of ``tests/test_oracle_mlp.py`` (gradients from
  torch.autograd; its linear instance reproduces the linear oracle, itself
  pinned by the pages' worked examples), at depths 2-4 with momentum and
  forgetting;
* the depth-2 instance against ``mlp_forward``;
* the plain read when nothing is written (theta = eta = alpha = 0), and the
  bit-identical resume at a chunk boundary.
"""

import numpy as np
import pytest
import torch

from oracle import deep_chunk_grads, deep_forward, mlp_forward
from tests.test_oracle_mlp import _generic_ttt


def _weights(rng, L, d, hid):
    dims = [d] + [hid] * (L - 1) + [d]
    return [rng.standard_normal((dims[i], dims[i + 1])) / np.sqrt(dims[i]) for i in range(L)]


def _inputs(rng, T, d):
    q = rng.standard_normal((T, d))
    k = rng.standard_normal((T, d))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, d))
    return q, k, v


def _torch_deep(u, *Ws):
    x = u
    for W in Ws[:-1]:
        x = torch.nn.functional.silu(x @ W)
    return u + x @ Ws[-1]


@pytest.mark.parametrize("L", [2, 3, 4])
def test_explicit_backprop_matches_autograd(L):
    rng = np.random.default_rng(40 + L)
    for _ in range(4):
        Ws = _weights(rng, L, 5, 7)
        k, v = rng.standard_normal(5), rng.standard_normal(5)
        G = deep_chunk_grads(k, v, Ws)
        tw = [torch.tensor(W, requires_grad=True) for W in Ws]
        loss = 0.5 * ((_torch_deep(torch.tensor(k), *tw) - torch.tensor(v)) ** 2).sum()
        g = torch.autograd.grad(loss, tw)
        assert len(G) == L
        for a, b_ in zip(G, g):
            np.testing.assert_allclose(a, b_.numpy(), atol=1e-13)


def test_explicit_backprop_matches_finite_differences_depth3():
    rng = np.random.default_rng(50)
    Ws = _weights(rng, 3, 3, 4)
    k, v = rng.standard_normal(3), rng.standard_normal(3)

    def loss(Wl):
        x = k
        for W in Wl[:-1]:
            h = x @ W
            x = h / (1 + np.exp(-h))
        return 0.5 * np.sum((k + x @ Wl[-1] - v) ** 2)

    G = deep_chunk_grads(k, v, Ws)
    eps = 1e-6
    for li, W in enumerate(Ws):
        num = np.zeros_like(W)
        for idx in np.ndindex(W.shape):
            Wp = [w.copy() for w in Ws]
            Wm = [w.copy() for w in Ws]
            Wp[li][idx] += eps
            Wm[li][idx] -= eps
            num[idx] = (loss(Wp) - loss(Wm)) / (2 * eps)
        np.testing.assert_allclose(G[li], num, atol=1e-8)


def _gates(rng, T):
    return rng.uniform(0.02, 0.3, T), rng.uniform(0.5, 0.95, T), rng.uniform(0.0, 0.1, T)


@pytest.mark.parametrize("L", [2, 3, 4])
@pytest.mark.parametrize("b", [1, 3, 5])
def test_generic_loop_reproduces_deep_oracle(L, b):
    rng = np.random.default_rng(60 + 10 * L + b)
    T, d, hid = 11, 4, 6
    q, k, v = _inputs(rng, T, d)
    Ws = _weights(rng, L, d, hid)
    th, et, al = _gates(rng, T)
    z, Ws_T, Ss_T = deep_forward(q, k, v, th, et, al, Ws, b=b)
    zg, Wg, Sg = _generic_ttt(_torch_deep, Ws, q, k, v, th, et, al, b)
    np.testing.assert_allclose(z, zg, atol=1e-12)
    for a, b_ in zip(Ws_T + Ss_T, Wg + Sg):
        np.testing.assert_allclose(a, b_, atol=1e-12)


@pytest.mark.parametrize("b", [1, 4, 16])
def test_depth_two_equals_mlp_oracle(b):
    rng = np.random.default_rng(70 + b)
    T, d, hid = 20, 5, 8
    q, k, v = _inputs(rng, T, d)
    W1, W2 = _weights(rng, 2, d, hid)
    S1 = rng.standard_normal(W1.shape) * 0.01
    S2 = rng.standard_normal(W2.shape) * 0.01
    th, et, al = _gates(rng, T)
    z, (W1d, W2d), (S1d, S2d) = deep_forward(q, k, v, th, et, al, [W1, W2], [S1, S2], b=b)
    zm, W1m, W2m, S1m, S2m = mlp_forward(q, k, v, th, et, al, W1, W2, S1, S2, b=b)
    np.testing.assert_allclose(z, zm, atol=1e-13)
    for a, b_ in ((W1d, W1m), (W2d, W2m), (S1d, S1m), (S2d, S2m)):
        np.testing.assert_allclose(a, b_, atol=1e-13)


@pytest.mark.parametrize("L", [3, 4])
def test_no_write_is_plain_read(L):
    rng = np.random.default_rng(80 + L)
    T, d, hid = 9, 4, 6
    q, k, v = _inputs(rng, T, d)
    Ws = _weights(rng, L, d, hid)
    zero = np.zeros(T)
    z, Ws_T, Ss_T = deep_forward(q, k, v, zero, zero, zero, Ws, b=4)
    x = q
    for W in Ws[:-1]:
        h = x @ W
        x = h / (1 + np.exp(-h))
    np.testing.assert_allclose(z, q + x @ Ws[-1], atol=1e-14)
    for W, W_T, S_T in zip(Ws, Ws_T, Ss_T):
        assert np.array_equal(W, W_T) and not S_T.any()


def test_resume_at_chunk_boundary_and_batch_independence():
    rng = np.random.default_rng(90)
    T, d, hid, L, b = 12, 4, 6, 3, 4
    q = np.stack([_inputs(rng, T, d)[0] for _ in range(2)])
    k = np.stack([_inputs(rng, T, d)[1] for _ in range(2)])
    v = rng.standard_normal((2, T, d))
    Ws = _weights(rng, L, d, hid)
    th, et, al = (np.stack([g, g[::-1]]) for g in _gates(rng, T))
    full = deep_forward(q, k, v, th, et, al, Ws, b=b)
    a = deep_forward(q[:, :8], k[:, :8], v[:, :8], th[:, :8], et[:, :8], al[:, :8], Ws, b=b)
    c = deep_forward(q[:, 8:], k[:, 8:], v[:, 8:], th[:, 8:], et[:, 8:], al[:, 8:], a[1], a[2], b=b)
    assert np.array_equal(np.concatenate([a[0], c[0]], axis=1), full[0])
    for x, y in zip(c[1] + c[2], full[1] + full[2]):
        assert np.array_equal(x, y)
    one = deep_forward(q[1], k[1], v[1], th[1], et[1], al[1], Ws, b=b)
    np.testing.assert_allclose(one[0], full[0][1], atol=1e-14)


def test_chunking_changes_the_result():
    # One result per chunk size (the chunk-start gradients differ from online ones).
    rng = np.random.default_rng(91)
    T, d, hid = 8, 4, 6
    q, k, v = _inputs(rng, T, d)
    Ws = _weights(rng, 3, d, hid)
    th, et, al = _gates(rng, T)
    z1 = deep_forward(q, k, v, th, et, al, Ws, b=1)[0]
    z4 = deep_forward(q, k, v, th, et, al, Ws, b=4)[0]
    np.testing.assert_allclose(z1[0], z4[0], atol=1e-15)      # the first token sees the same state
    assert np.max(np.abs(z1 - z4)) > 1e-6


def test_bf16_output_allowance_is_half_an_ulp():
    # The parity helper that discounts the bf16 rounding of a stored output
    # subtracts exactly half an ulp: RNE-rounded values score 0, anything a
    # full ulp off does not.
    import torch
    from tests._parity import bf16_half_ulp, rel_err_bf16_out
    rng = np.random.default_rng(3)
    x = rng.standard_normal(10000) * 3.0
    xb = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert rel_err_bf16_out(xb, x) == 0.0
    assert np.all(np.abs(xb - x) <= bf16_half_ulp(x))
    off = xb + 2 * bf16_half_ulp(x) * np.sign(x)
    assert rel_err_bf16_out(off, x) > 0.0
    assert bf16_half_ulp(np.array([1.0, 1.5, 2.0, 0.0])).tolist() == [2.0 ** -8, 2.0 ** -8, 2.0 ** -7, 0.0]
