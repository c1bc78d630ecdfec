"""Pins of the float64 backward oracle (``linear_backward``).

The gradient is checked against central finite differences of the forward
oracle (itself pinned by the worked examples and closed forms of
``test_oracle_linear.py``), against the pages' scalar outer-gradient examples
(``tests/golden/*outer_gradient*.json``), and against the closed-form
gradients of weighted linear attention, which the recurrence reduces to with
zero momentum and forgetting, zero initial state and one chunk.
"""

import glob
import json
import os

import numpy as np
import pytest

from oracle import linear_backward, linear_forward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NAMES = ("dq", "dk", "dv", "dtheta", "deta", "dalpha", "dM0", "dS0")


def _arr(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _inputs(rng, lead=(2,), T=7, dk=4, dv=3, gates="titans"):
    q = rng.standard_normal(lead + (T, dk))
    k = rng.standard_normal(lead + (T, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal(lead + (T, dv))
    if gates == "titans":
        theta = rng.uniform(0.05, 0.6, lead + (T,))
        eta = rng.uniform(0.3, 0.95, lead + (T,))
        alpha = rng.uniform(0.0, 0.3, lead + (T,))
    else:
        theta = rng.uniform(0.05, 0.6, lead + (T,))
        eta = np.zeros(lead + (T,))
        alpha = np.zeros(lead + (T,))
    M0 = rng.standard_normal(lead + (dv, dk)) * 0.3
    S0 = rng.standard_normal(lead + (dv, dk)) * 0.1
    return dict(q=q, k=k, v=v, theta=theta, eta=eta, alpha=alpha, M0=M0, S0=S0)


def _objective(x, dz, dM, dS, b):
    z, M, S = linear_forward(x["q"], x["k"], x["v"], x["theta"], x["eta"], x["alpha"], x["M0"], x["S0"], b=b)
    return np.sum(z * dz) + np.sum(M * dM) + np.sum(S * dS)


@pytest.mark.parametrize("b", [1, 3, 7, 10])
def test_matches_central_differences(b):
    rng = np.random.default_rng(100 + b)
    x = _inputs(rng)
    lead, T, dv, dk = (2,), 7, 3, 4
    dz = rng.standard_normal(lead + (T, dv))
    dM = rng.standard_normal(lead + (dv, dk))
    dS = rng.standard_normal(lead + (dv, dk))
    grads = linear_backward(x["q"], x["k"], x["v"], x["theta"], x["eta"], x["alpha"], dz, dM, dS,
                            x["M0"], x["S0"], b=b)
    eps = 1e-6
    for name, key in zip(NAMES, ("q", "k", "v", "theta", "eta", "alpha", "M0", "S0")):
        g = grads[NAMES.index(name)]
        fd = np.zeros_like(x[key])
        for idx in np.ndindex(x[key].shape):
            xp = {kk: vv.copy() for kk, vv in x.items()}
            xm = {kk: vv.copy() for kk, vv in x.items()}
            xp[key][idx] += eps
            xm[key][idx] -= eps
            fd[idx] = (_objective(xp, dz, dM, dS, b) - _objective(xm, dz, dM, dS, b)) / (2 * eps)
        scale = max(np.abs(fd).max(), 1.0)
        np.testing.assert_allclose(g, fd, atol=2e-7 * scale, rtol=0, err_msg=f"{name} b={b}")


def _golden():
    out = []
    for path in sorted(glob.glob(os.path.join(GOLDEN, "*outer_gradient*.json"))):
        with open(path) as f:
            fx = json.load(f)
        for i, c in enumerate(fx["cases"]):
            out.append(pytest.param(c, id=f"{os.path.basename(path)}[{i}]"))
    return out


@pytest.mark.parametrize("case", _golden())
def test_worked_outer_gradients(case):
    x = {k: _arr(v) for k, v in case["inputs"].items() if k != "b"}
    b = case["inputs"]["b"]
    z, M, S = linear_forward(x["q"], x["k"], x["v"], x["theta"], x["eta"], x["alpha"], x["M0"], x["S0"], b=b)
    g = dict(zip(NAMES, linear_backward(x["q"], x["k"], x["v"], x["theta"], x["eta"], x["alpha"], x["dz"],
                                        x["dM_T"], x["dS_T"], x["M0"], x["S0"], b=b)))
    exp = case["expected"]
    if "z" in exp:
        np.testing.assert_allclose(z, _arr(exp["z"]), atol=1e-12, rtol=0)
    if "M_T" in exp:
        np.testing.assert_allclose(M, _arr(exp["M_T"]), atol=1e-12, rtol=0)
    for name in NAMES:
        if name in exp:
            np.testing.assert_allclose(g[name], _arr(exp[name]), atol=1e-12, rtol=0, err_msg=name)


def test_golden_outer_gradients_present():
    assert len(_golden()) >= 3


def test_linear_attention_closed_form():
    # eta = alpha = 0, zero initial state, one chunk (b >= T): every gradient is
    # taken at M = 0, so M_t = sum_{j<=t} theta_j v_j k_j^T and
    # z_t = sum_{j<=t} theta_j (k_j . q_t) v_j: weighted linear attention
    # ("5.1.1 · TTT layers 与 fast weights", section 1.1: batch GD over the
    # whole sequence is linear attention).  Its gradients are textbook; the
    # gate gradients at zero gates follow from dM_s/dalpha_t = -M_{t-1} and
    # dS_t/deta_t = S_{t-1} = theta_{t-1} v_{t-1} k_{t-1}^T (no propagation
    # through S when eta = 0).
    rng = np.random.default_rng(7)
    T, dk, dv = 9, 4, 3
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    theta = rng.uniform(0.1, 0.9, T)
    zero = np.zeros(T)
    dz = rng.standard_normal((T, dv))
    dM = rng.standard_normal((dv, dk))
    dS = rng.standard_normal((dv, dk))
    g = dict(zip(NAMES, linear_backward(q, k, v, theta, zero, zero, dz, dM, dS, None, None, b=T)))

    A = np.tril(q @ k.T)                # A[t, j] = q_t . k_j for j <= t
    VD = dz @ v.T                       # VD[t, j] = dz_t . v_j
    dq = (np.tril(VD) * theta[None, :]) @ k
    dk_ = theta[:, None] * (np.tril(VD).T @ q) + theta[:, None] * (v @ dM)
    dv_ = theta[:, None] * (A.T @ dz) + theta[:, None] * (k @ dM.T)
    dth = np.sum(np.tril(A * VD), axis=0) + np.einsum("ti,ij,tj->t", v, dM, k)
    # With eta = 0 the final momentum is the last write alone, S_T = theta_{T-1} v_{T-1} k_{T-1}^T.
    dk_[-1] += theta[-1] * (v[-1] @ dS)
    dv_[-1] += theta[-1] * (dS @ k[-1])
    dth[-1] += v[-1] @ dS @ k[-1]
    # M_t before token t: sum_{j<t} theta_j v_j k_j^T.
    Mprev = np.cumsum(theta[:, None, None] * v[:, :, None] * k[:, None, :], axis=0)
    Mprev = np.concatenate([np.zeros((1, dv, dk)), Mprev[:-1]])
    dal = np.array([-sum(dz[s] @ Mprev[t] @ q[s] for s in range(t, T)) - np.sum(dM * Mprev[t]) for t in range(T)])
    Sprev = np.concatenate([np.zeros((1, dv, dk)), theta[:-1, None, None] * v[:-1, :, None] * k[:-1, None, :]])
    det = np.array([sum(dz[s] @ Sprev[t] @ q[s] for s in range(t, T)) + np.sum(dM * Sprev[t])
                    + (np.sum(dS * Sprev[t]) if t == T - 1 else 0.0) for t in range(T)])
    for name, ref in (("dq", dq), ("dk", dk_), ("dv", dv_), ("dtheta", dth), ("dalpha", dal), ("deta", det)):
        np.testing.assert_allclose(g[name], ref, atol=1e-12, rtol=1e-12, err_msg=name)


def test_chunk_start_collects_gradient_paths():
    # One chunk (b = T), zero momentum and forgetting, dz on the last token
    # only.  z_{T-1} = M0 q - sum_j theta_j (M0 k_j - v_j)(k_j . q): the
    # chunk-start memory reaches the read directly and through every residual
    # of the chunk, so dM0 = dz (q - sum_j theta_j (k_j . q) k_j)^T.  Dropping
    # the residual paths (a detached chunk-start state) fails this.
    rng = np.random.default_rng(8)
    T, dk, dv = 5, 3, 2
    q, k, v = rng.standard_normal((T, dk)), rng.standard_normal((T, dk)), rng.standard_normal((T, dv))
    theta = rng.uniform(0.1, 0.5, T)
    zero = np.zeros(T)
    dz = np.zeros((T, dv))
    dz[-1] = rng.standard_normal(dv)
    M0 = rng.standard_normal((dv, dk))
    g = dict(zip(NAMES, linear_backward(q, k, v, theta, zero, zero, dz, None, None, M0, None, b=T)))
    # z_{T-1} = M0 q - sum_j theta_j (M0 k_j - v_j) (k_j . q)  =>  dM0 = dz (q - sum_j theta_j (k_j . q) k_j)^T
    qT = q[-1]
    ref = np.outer(dz[-1], qT - sum(theta[j] * (k[j] @ qT) * k[j] for j in range(T)))
    np.testing.assert_allclose(g["dM0"], ref, atol=1e-12, rtol=0)
