"""Pins of the float64 deep-memory (2-layer MLP) oracle.

The pages print no MLP values, so the deep-memory oracle is pinned by:
* its explicit backprop against torch.autograd (a library routine) and against
  central finite differences ("5.1.1 · TTT layers 与 fast weights" recommends
  finite-difference checks);
* a generic TTT loop in this file whose gradient comes from torch.autograd:
  with a linear inner model it must reproduce the linear oracle (itself pinned
  by the pages' worked examples), and with the MLP it must reproduce the MLP
  oracle -- so the chunked schedule with momentum and forgetting is checked
  independently of the hand-written backprop.
"""

import numpy as np
import pytest
import torch

from oracle import linear_forward, mlp_chunk_grads, mlp_forward


def _inputs(rng, T=11, d=4, hid=6, lead=()):
    q = rng.standard_normal(lead + (T, d))
    k = rng.standard_normal(lead + (T, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal(lead + (T, d))
    W1 = rng.standard_normal((d, hid)) / np.sqrt(d)
    W2 = rng.standard_normal((hid, d)) / np.sqrt(hid)
    return q, k, v, W1, W2


def _torch_f(u, W1, W2):
    return u + torch.nn.functional.silu(u @ W1) @ W2


@pytest.mark.parametrize("loss_on", ["full", "mlp"])
def test_explicit_backprop_matches_autograd(loss_on):
    rng = np.random.default_rng(20)
    for _ in range(5):
        _, k, v, W1, W2 = _inputs(rng, T=1, d=5, hid=9)
        k, v = k[0], v[0]
        G1, G2 = mlp_chunk_grads(k, v, W1, W2, loss_on)
        t1 = torch.tensor(W1, requires_grad=True)
        t2 = torch.tensor(W2, requires_grad=True)
        kt, vt = torch.tensor(k), torch.tensor(v)
        out = _torch_f(kt, t1, t2) if loss_on == "full" else torch.nn.functional.silu(kt @ t1) @ t2
        loss = 0.5 * ((out - vt) ** 2).sum()
        g1, g2 = torch.autograd.grad(loss, (t1, t2))
        np.testing.assert_allclose(G1, g1.numpy(), atol=1e-14)
        np.testing.assert_allclose(G2, g2.numpy(), atol=1e-14)


def test_explicit_backprop_matches_finite_differences():
    rng = np.random.default_rng(21)
    _, k, v, W1, W2 = _inputs(rng, T=1, d=3, hid=5)
    k, v = k[0], v[0]

    def loss(W1_, W2_):
        h = k @ W1_
        out = k + (h / (1 + np.exp(-h))) @ W2_
        return 0.5 * np.sum((out - v) ** 2)

    G1, G2 = mlp_chunk_grads(k, v, W1, W2)
    eps = 1e-6
    for W, G, which in ((W1, G1, 0), (W2, G2, 1)):
        num = np.zeros_like(W)
        for idx in np.ndindex(W.shape):
            Wp, Wm = W.copy(), W.copy()
            Wp[idx] += eps
            Wm[idx] -= eps
            lp = loss(Wp, W2) if which == 0 else loss(W1, Wp)
            lm = loss(Wm, W2) if which == 0 else loss(W1, Wm)
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(G, num, atol=1e-8)


def _generic_ttt(f, params0, q, k, v, theta, eta, alpha, b):
    """Chunked TTT with momentum and forgetting for any inner model ``f(u, *params)``.

    The gradient of 1/2||f(k_t) - v_t||^2 at the chunk-start parameters comes
    from torch.autograd; every parameter tensor gets its own momentum.
    """
    T = q.shape[0]
    P = [torch.tensor(p, dtype=torch.float64) for p in params0]
    S = [torch.zeros_like(p) for p in P]
    zs = []
    for c0 in range(0, T, b):
        Pc = [p.clone() for p in P]
        for t in range(c0, min(c0 + b, T)):
            Pv = [p.clone().requires_grad_(True) for p in Pc]
            kt, vt = torch.tensor(k[t]), torch.tensor(v[t])
            loss = 0.5 * ((f(kt, *Pv) - vt) ** 2).sum()
            grads = torch.autograd.grad(loss, Pv)
            S = [eta[t] * s - theta[t] * g for s, g in zip(S, grads)]
            P = [(1 - alpha[t]) * p + s for p, s in zip(P, S)]
            zs.append(f(torch.tensor(q[t]), *P).detach().numpy())
    return np.stack(zs), [p.numpy() for p in P], [s.numpy() for s in S]


def _gates(rng, T):
    return rng.uniform(0.02, 0.3, T), rng.uniform(0.5, 0.95, T), rng.uniform(0.0, 0.1, T)


@pytest.mark.parametrize("b", [1, 3, 4])
def test_generic_loop_reproduces_linear_oracle(b):
    # Anchors the generic loop: with f(u) = M u it must equal the linear oracle.
    rng = np.random.default_rng(22)
    q, k, v, _, _ = _inputs(rng, T=10, d=4)
    th, et, al = _gates(rng, 10)
    M0 = rng.standard_normal((4, 4))
    z, M, S = linear_forward(q, k, v, th, et, al, M0, None, b=b)
    zg, (Mg,), (Sg,) = _generic_ttt(lambda u, M_: M_ @ u, [M0], q, k, v, th, et, al, b)
    np.testing.assert_allclose(z, zg, atol=1e-12)
    np.testing.assert_allclose(M, Mg, atol=1e-12)
    np.testing.assert_allclose(S, Sg, atol=1e-12)


@pytest.mark.parametrize("b", [1, 3, 4, 16])
def test_generic_loop_reproduces_mlp_oracle(b):
    rng = np.random.default_rng(23)
    T = 13
    q, k, v, W1, W2 = _inputs(rng, T=T, d=4, hid=8)
    th, et, al = _gates(rng, T)
    z, W1_T, W2_T, S1_T, S2_T = mlp_forward(q, k, v, th, et, al, W1, W2, b=b)
    zg, (W1g, W2g), (S1g, S2g) = _generic_ttt(_torch_f, [W1, W2], q, k, v, th, et, al, b)
    np.testing.assert_allclose(z, zg, atol=1e-12)
    for a_, b_ in ((W1_T, W1g), (W2_T, W2g), (S1_T, S1g), (S2_T, S2g)):
        np.testing.assert_allclose(a_, b_, atol=1e-12)


def test_mlp_resume_and_batch_independence():
    rng = np.random.default_rng(24)
    T = 12
    q, k, v, W1, W2 = _inputs(rng, T=T, d=4, hid=8, lead=(2,))
    th, et, al = (np.stack([g, g[::-1]]) for g in _gates(rng, T))
    full = mlp_forward(q, k, v, th, et, al, W1, W2, b=4)
    a = mlp_forward(q[:, :8], k[:, :8], v[:, :8], th[:, :8], et[:, :8], al[:, :8], W1, W2, b=4)
    bb = mlp_forward(q[:, 8:], k[:, 8:], v[:, 8:], th[:, 8:], et[:, 8:], al[:, 8:],
                     a[1], a[2], a[3], a[4], b=4)
    assert np.array_equal(np.concatenate([a[0], bb[0]], axis=1), full[0])
    for x, y in zip(bb[1:], full[1:]):
        assert np.array_equal(x, y)
    one = mlp_forward(q[1], k[1], v[1], th[1], et[1], al[1], W1, W2, b=4)
    np.testing.assert_allclose(one[0], full[0][1], atol=1e-14)
