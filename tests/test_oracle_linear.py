"""Pins of the float64 linear-memory oracle against what the pages and mathematics fix.

Nothing here compares the oracle with itself: each test checks it against a
printed worked example (``tests/golden``), a closed form, a library gradient
(torch.autograd), or an invariant of the recurrence.
"""

import glob
import json
import os

import numpy as np
import pytest
import torch

from oracle import linear_forward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _arr(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _run_case(inp):
    return linear_forward(
        _arr(inp["q"]), _arr(inp["k"]), _arr(inp["v"]),
        _arr(inp["theta"]), _arr(inp["eta"]), _arr(inp["alpha"]),
        _arr(inp["M0"]), _arr(inp["S0"]), b=inp["b"], grad=inp.get("grad", "l2"))


def _golden_cases():
    out = []
    for path in sorted(glob.glob(os.path.join(GOLDEN, "p*.json"))):
        with open(path) as f:
            fx = json.load(f)
        cases = fx.get("cases", [{"inputs": fx.get("inputs"), "expected": fx.get("expected")}])
        for i, c in enumerate(cases):
            out.append(pytest.param(c, id=f"{os.path.basename(path)}[{i}]"))
    return out


@pytest.mark.parametrize("case", _golden_cases())
def test_worked_examples(case):
    z, M, S = _run_case(case["inputs"])
    exp = case["expected"]
    if "z" in exp:
        np.testing.assert_allclose(z, _arr(exp["z"]), atol=1e-12, rtol=0)
    if "z_last" in exp:
        np.testing.assert_allclose(z[-1], _arr(exp["z_last"]), atol=1e-12, rtol=0)
    if "M_T" in exp:
        np.testing.assert_allclose(M, _arr(exp["M_T"]), atol=1e-12, rtol=0)
    if "S_T" in exp:
        np.testing.assert_allclose(S, _arr(exp["S_T"]), atol=1e-12, rtol=0)


def test_every_golden_file_is_cited():
    files = sorted(glob.glob(os.path.join(GOLDEN, "*.json")))
    assert len(files) >= 8
    for path in files:
        with open(path) as f:
            fx = json.load(f)
        assert fx.get("citation"), path
        assert "section" in fx["citation"] or "eq" in fx["citation"], path


def _rand(rng, T=24, dk=5, dv=3, lead=()):
    q = rng.standard_normal(lead + (T, dk))
    k = rng.standard_normal(lead + (T, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal(lead + (T, dv))
    return q, k, v


def test_b1_no_momentum_is_the_delta_rule():
    # DeltaNet's erase-then-write form S_t = S_{t-1}(I - beta k k^T) + beta v k^T
    # ("5.1.1 · TTT layers 与 fast weights", eq. (5)), beta = theta under the 1/2 loss.
    rng = np.random.default_rng(1)
    q, k, v = _rand(rng, T=30, dk=6, dv=4)
    theta = rng.uniform(0.1, 0.9, 30)
    M0 = rng.standard_normal((4, 6)) * 0.3
    z, M, S = linear_forward(q, k, v, theta, np.zeros(30), np.zeros(30), M0, None, b=1)
    W = M0.copy()
    for t in range(30):
        W = W @ (np.eye(6) - theta[t] * np.outer(k[t], k[t])) + theta[t] * np.outer(v[t], k[t])
        np.testing.assert_allclose(z[t], W @ q[t], atol=1e-12)
    np.testing.assert_allclose(M, W, atol=1e-12)


@pytest.mark.parametrize("b", [1, 3, 7, 40])
def test_additive_gradient_gives_linear_attention(b):
    # Unnormalised linear attention M_t = M_{t-1} + v_t k_t^T, read z_t = M_t q_t
    # ("论文速览 | Titans" section 2.3).  In matrix form the reads are
    # Z = Q M0^T + tril(Q K^T) V (causal, diagonal included).
    rng = np.random.default_rng(2)
    q, k, v = _rand(rng, T=29, dk=5, dv=3)
    M0 = rng.standard_normal((3, 5))
    ones, zeros = np.ones(29), np.zeros(29)
    z, M, _ = linear_forward(q, k, v, ones, zeros, zeros, M0, None, b=b, grad="neg_vk")
    Z = q @ M0.T + np.tril(q @ k.T) @ v
    np.testing.assert_allclose(z, Z, atol=1e-12)
    np.testing.assert_allclose(M, M0 + v.T @ k, atol=1e-12)


def test_one_chunk_from_zero_is_weighted_linear_attention():
    # M0 = 0, no momentum/forgetting, b >= T: every gradient is taken at zero,
    # so M_T = sum_j theta_j v_j k_j^T ("5.1.1 ..." section 1.1, b = 2 example).
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, T=16, dk=4, dv=4)
    theta = rng.uniform(0.01, 0.2, 16)
    z, M, _ = linear_forward(q, k, v, theta, np.zeros(16), np.zeros(16), None, None, b=16)
    np.testing.assert_allclose(M, (v * theta[:, None]).T @ k, atol=1e-12)


@pytest.mark.parametrize("b", [1, 4, 5, 64])
def test_each_chunk_is_one_batch_gradient_step(b):
    # With no momentum or forgetting, the state after each chunk is one step of
    # batch gradient descent on sum_{j in chunk} theta_j * 1/2||M k_j - v_j||^2
    # taken at the chunk-start state.  The gradient comes from torch.autograd.
    rng = np.random.default_rng(4)
    T = 23
    q, k, v = _rand(rng, T=T, dk=5, dv=3)
    theta = rng.uniform(0.05, 0.5, T)
    M0 = rng.standard_normal((3, 5)) * 0.5
    _, M_T, _ = linear_forward(q, k, v, theta, np.zeros(T), np.zeros(T), M0, None, b=b)
    M = torch.tensor(M0, dtype=torch.float64)
    kt, vt, tt = (torch.tensor(x, dtype=torch.float64) for x in (k, v, theta))
    for c0 in range(0, T, b):
        Mv = M.clone().requires_grad_(True)
        sl = slice(c0, min(c0 + b, T))
        loss = (tt[sl] * 0.5 * ((kt[sl] @ Mv.T - vt[sl]) ** 2).sum(-1)).sum()
        (g,) = torch.autograd.grad(loss, Mv)
        M = (M - g).detach()
    np.testing.assert_allclose(M_T, M.numpy(), atol=1e-12)


def test_one_step_loss_contraction_is_exact():
    # b=1, no momentum: e_new = (1 - theta ||k||^2) e_old, so
    # l(M_t; x_t) / l(M_{t-1}; x_t) = (1 - theta||k||^2)^2 < 1 for 0 < theta||k||^2 < 2
    # ("Continual Learning..." section 3.3; "5.1.1 ..." eqs. (11)-(12)).
    rng = np.random.default_rng(5)
    T = 12
    q, k, v = _rand(rng, T=T, dk=4, dv=3)
    k *= rng.uniform(0.5, 1.5, (T, 1))            # non-unit keys
    theta = rng.uniform(0.05, 1.9, T) / (k ** 2).sum(-1)
    M_prev = rng.standard_normal((3, 4))
    S_prev = None
    for t in range(T):
        _, M_new, S_prev = linear_forward(q[t:t + 1], k[t:t + 1], v[t:t + 1], theta[t:t + 1],
                                          np.zeros(1), np.zeros(1), M_prev, S_prev, b=1)
        l_old = 0.5 * np.sum((M_prev @ k[t] - v[t]) ** 2)
        l_new = 0.5 * np.sum((M_new @ k[t] - v[t]) ** 2)
        ratio = (1 - theta[t] * k[t] @ k[t]) ** 2
        np.testing.assert_allclose(l_new, ratio * l_old, rtol=1e-11)
        assert l_new < l_old
        M_prev = M_new


@pytest.mark.parametrize("b", [1, 6])
def test_constant_gate_momentum_expansion(b):
    # With constant gates, U_t = -theta (g_t + mu g_{t-1} + mu^2 g_{t-2} + ...)
    # ("Continual Learning..." section 5.1).  grad='neg_vk' makes g_j = -v_j k_j^T
    # independent of the state, so the expansion is closed-form for any b.
    rng = np.random.default_rng(6)
    T, mu, th = 17, 0.7, 0.3
    q, k, v = _rand(rng, T=T, dk=4, dv=2)
    M0 = rng.standard_normal((2, 4))
    z, M, S = linear_forward(q, k, v, np.full(T, th), np.full(T, mu), np.zeros(T),
                             M0, None, b=b, grad="neg_vk")
    g = [-np.outer(v[j], k[j]) for j in range(T)]
    S_t = [-th * sum(mu ** (t - j) * g[j] for j in range(t + 1)) for t in range(T)]
    np.testing.assert_allclose(S, S_t[-1], atol=1e-12)
    # No forgetting: M_t = M_0 + sum_{s<=t} S_s.
    np.testing.assert_allclose(M, M0 + sum(S_t), atol=1e-12)
    for t in range(T):
        np.testing.assert_allclose(z[t], (M0 + sum(S_t[:t + 1])) @ q[t], atol=1e-12)


def test_weight_decay_unrolling():
    # "论文速览 | Titans" section 4.3: without momentum,
    # M_t = beta_t M_0 - sum_i (beta_t / beta_i) theta_i grad_i,
    # beta_t = prod_{j<=t} (1 - alpha_j).  One chunk (b >= T) puts every gradient
    # at M_0: grad_i = (M_0 k_i - v_i) k_i^T.
    rng = np.random.default_rng(7)
    T = 20
    q, k, v = _rand(rng, T=T, dk=5, dv=3)
    theta = rng.uniform(0.01, 0.3, T)
    alpha = rng.uniform(0.0, 0.3, T)
    M0 = rng.standard_normal((3, 5))
    z, M, _ = linear_forward(q, k, v, theta, np.zeros(T), alpha, M0, None, b=T)
    beta = np.cumprod(1 - alpha)
    grads = [np.outer(M0 @ k[i] - v[i], k[i]) for i in range(T)]
    for t in range(T):
        Mt = beta[t] * M0 - sum(beta[t] / beta[i] * theta[i] * grads[i] for i in range(t + 1))
        np.testing.assert_allclose(z[t], Mt @ q[t], atol=1e-12)
    np.testing.assert_allclose(M, Mt, atol=1e-12)


def _gates(rng, T):
    theta = rng.uniform(0.01, 0.3, T)
    eta = rng.uniform(0.5, 0.95, T)
    alpha = rng.uniform(0.0, 0.2, T)
    return theta, eta, alpha


@pytest.mark.parametrize("b,split", [(4, 8), (5, 15), (1, 7), (16, 16)])
def test_resume_at_chunk_boundary_is_bit_identical(b, split):
    # Checkpoints belong on chunk boundaries ("5.1.1 ..." section on state
    # lifecycle): carrying (M, S) across a split at a multiple of b reproduces
    # the uninterrupted run exactly.
    rng = np.random.default_rng(8)
    T = 37
    q, k, v = _rand(rng, T=T)
    th, et, al = _gates(rng, T)
    M0 = rng.standard_normal((3, 5))
    S0 = rng.standard_normal((3, 5)) * 0.1
    z, M, S = linear_forward(q, k, v, th, et, al, M0, S0, b=b)
    z1, M1, S1 = linear_forward(q[:split], k[:split], v[:split], th[:split], et[:split], al[:split], M0, S0, b=b)
    z2, M2, S2 = linear_forward(q[split:], k[split:], v[split:], th[split:], et[split:], al[split:], M1, S1, b=b)
    assert np.array_equal(np.concatenate([z1, z2]), z)
    assert np.array_equal(M2, M) and np.array_equal(S2, S)


def test_value_rows_are_independent_and_permute():
    # Row i of M only ever meets v[:, i]; slicing or permuting value coordinates
    # slices or permutes z, M, S the same way.
    rng = np.random.default_rng(9)
    T = 19
    q, k, v = _rand(rng, T=T, dk=6, dv=5)
    th, et, al = _gates(rng, T)
    M0 = rng.standard_normal((5, 6))
    S0 = rng.standard_normal((5, 6)) * 0.1
    z, M, S = linear_forward(q, k, v, th, et, al, M0, S0, b=4)
    perm = np.array([3, 0, 4, 1, 2])
    zp, Mp, Sp = linear_forward(q, k, v[:, perm], th, et, al, M0[perm], S0[perm], b=4)
    np.testing.assert_allclose(zp, z[:, perm], atol=1e-13)
    np.testing.assert_allclose(Mp, M[perm], atol=1e-13)
    rows = np.array([1, 4])
    zr, Mr, Sr = linear_forward(q, k, v[:, rows], th, et, al, M0[rows], S0[rows], b=4)
    np.testing.assert_allclose(zr, z[:, rows], atol=1e-13)
    np.testing.assert_allclose(Sr, S[rows], atol=1e-13)


def test_leading_dims_are_independent_sequences():
    rng = np.random.default_rng(10)
    T = 13
    q, k, v = _rand(rng, T=T, lead=(2, 3))
    th, et, al = (np.stack([np.stack([g for g in _gates(rng, T)]) for _ in range(6)]).reshape(2, 3, 3, T)[:, :, i]
                  for i in range(3))
    M0 = rng.standard_normal((2, 3, 3, 5))
    z, M, S = linear_forward(q, k, v, th, et, al, M0, None, b=5)
    for i in range(2):
        for j in range(3):
            zi, Mi, Si = linear_forward(q[i, j], k[i, j], v[i, j], th[i, j], et[i, j], al[i, j], M0[i, j], None, b=5)
            np.testing.assert_allclose(z[i, j], zi, atol=1e-14)
            np.testing.assert_allclose(M[i, j], Mi, atol=1e-14)


def _segprod(x, lo, hi):
    """prod_{l=lo..hi} x_l, empty product = 1 (brute force)."""
    return float(np.prod(x[lo:hi + 1])) if hi >= lo else 1.0


@pytest.mark.parametrize("b,T,zero_eta", [(4, 16, False), (5, 13, False), (1, 6, False),
                                          (8, 8, True), (6, 20, True), (64, 50, False)])
def test_chunk_closed_form_matches_loop(b, T, zero_eta):
    # Brute force on tiny inputs ("5.1.1 ..." recommends comparing token-wise and
    # dual forms in double precision on small blocks).  Within a chunk, with
    # gradients u_j = e_j k_j^T at the chunk-start state (M0, S0):
    #   S_i = E_i S0 - sum_{j<=i} theta_j P_ij u_j,   P_ij = prod_{l=j+1..i} eta_l
    #   M_i = A_i M0 + c_i S0 - sum_{j<=i} theta_j gamma_ij u_j
    # with A_i = prod_{l<=i} a_l, E_i = prod_{l<=i} eta_l, c_i = sum_m (prod_{l=m+1..i} a_l) E_m,
    # gamma_ij = sum_{m=j..i} (prod_{l=m+1..i} a_l) P_mj, a = 1 - alpha.
    rng = np.random.default_rng(11 + b + T)
    q, k, v = _rand(rng, T=T, dk=4, dv=3)
    th, et, al = _gates(rng, T)
    if zero_eta:
        et[:] = 0.0
    M0 = rng.standard_normal((3, 4))
    S0 = rng.standard_normal((3, 4)) * 0.2
    z, M_T, S_T = linear_forward(q, k, v, th, et, al, M0, S0, b=b)
    a = 1 - al
    M, S = M0.copy(), S0.copy()
    zz = np.zeros_like(z)
    for c0 in range(0, T, b):
        idx = list(range(c0, min(c0 + b, T)))
        u = {j: np.outer(M @ k[j] - v[j], k[j]) for j in idx}
        for i in idx:
            A_i = _segprod(a, c0, i)
            E_i = _segprod(et, c0, i)
            c_i = sum(_segprod(a, m + 1, i) * _segprod(et, c0, m) for m in range(c0, i + 1))
            gam = {j: sum(_segprod(a, m + 1, i) * _segprod(et, j + 1, m) for m in range(j, i + 1)) for j in idx if j <= i}
            Mi = A_i * M + c_i * S - sum(th[j] * gam[j] * u[j] for j in gam)
            zz[i] = Mi @ q[i]
            if i == idx[-1]:
                Si = E_i * S - sum(th[j] * _segprod(et, j + 1, i) * u[j] for j in gam)
                M_next, S_next = Mi, Si
        M, S = M_next, S_next
    np.testing.assert_allclose(z, zz, atol=1e-12)
    np.testing.assert_allclose(M_T, M, atol=1e-12)
    np.testing.assert_allclose(S_T, S, atol=1e-12)


def test_bad_arguments_raise():
    q = np.zeros((4, 2))
    with pytest.raises(ValueError):
        linear_forward(q, q, q, np.zeros(4), np.zeros(4), np.zeros(4), b=0)
    with pytest.raises(ValueError):
        linear_forward(q, q, q, np.zeros(4), np.zeros(4), np.zeros(4), grad="nope")
