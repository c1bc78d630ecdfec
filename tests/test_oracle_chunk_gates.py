"""Pins of the chunk-shared-gate oracle ("论文速览 | Titans", section 4.6).

With gates shared by a chunk's tokens the recurrence inside a chunk is
linear and time-invariant, which gives closed forms that the per-token loop
must reproduce; the gate gradients are checked by central differences.
"""

import numpy as np
import pytest

from oracle import linear_backward_chunk_gates, linear_forward_chunk_gates


def test_time_invariant_chunk_closed_form():
    # One chunk (b >= T), zero initial state, constant a = 1 - alpha, eta,
    # theta: every gradient is taken at M = 0, so S_t = theta sum_{j<=t}
    # eta^(t-j) v_j k_j^T and M_t = theta sum_{j<=t} gamma(t-j) v_j k_j^T with
    # the geometric sum gamma(m) = (a^(m+1) - eta^(m+1)) / (a - eta).
    rng = np.random.default_rng(3)
    T, dk, dv = 11, 4, 3
    q, k, v = rng.standard_normal((T, dk)), rng.standard_normal((T, dk)), rng.standard_normal((T, dv))
    th, et, al = 0.3, 0.7, 0.1
    a = 1 - al
    z, M, S = linear_forward_chunk_gates(q, k, v, [th], [et], [al], None, None, b=16)
    gam = lambda m: (a ** (m + 1) - et ** (m + 1)) / (a - et)  # noqa: E731
    for t in range(T):
        Mt = th * sum(gam(t - j) * np.outer(v[j], k[j]) for j in range(t + 1))
        np.testing.assert_allclose(z[t], Mt @ q[t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(M, th * sum(gam(T - 1 - j) * np.outer(v[j], k[j]) for j in range(T)), atol=1e-12)
    np.testing.assert_allclose(S, th * sum(et ** (T - 1 - j) * np.outer(v[j], k[j]) for j in range(T)), atol=1e-12)


def test_chunk_entries_apply_to_their_chunks_only():
    # Changing the gates of the last chunk leaves every read of earlier chunks unchanged.
    rng = np.random.default_rng(4)
    T, d, b = 10, 3, 4
    q, k, v = (rng.standard_normal((T, d)) for _ in range(3))
    th, et, al = rng.uniform(0.1, 0.5, 3), rng.uniform(0.5, 0.9, 3), rng.uniform(0, 0.2, 3)
    z1 = linear_forward_chunk_gates(q, k, v, th, et, al, b=b)[0]
    th2 = th.copy()
    th2[-1] += 0.3
    z2 = linear_forward_chunk_gates(q, k, v, th2, et, al, b=b)[0]
    np.testing.assert_array_equal(z1[:8], z2[:8])
    assert np.abs(z1[8:] - z2[8:]).max() > 1e-3


@pytest.mark.parametrize("b", [3, 4, 9])
def test_chunk_gate_gradients_match_central_differences(b):
    rng = np.random.default_rng(20 + b)
    T, dk, dv = 9, 3, 2
    nc = (T + b - 1) // b
    q, k, v = rng.standard_normal((T, dk)), rng.standard_normal((T, dk)), rng.standard_normal((T, dv))
    gates = {"theta": rng.uniform(0.1, 0.5, nc), "eta": rng.uniform(0.4, 0.9, nc), "alpha": rng.uniform(0, 0.3, nc)}
    M0, S0 = rng.standard_normal((dv, dk)) * 0.3, rng.standard_normal((dv, dk)) * 0.1
    dz, dM, dS = rng.standard_normal((T, dv)), rng.standard_normal((dv, dk)), rng.standard_normal((dv, dk))

    def obj(g):
        z, M, S = linear_forward_chunk_gates(q, k, v, g["theta"], g["eta"], g["alpha"], M0, S0, b=b)
        return np.sum(z * dz) + np.sum(M * dM) + np.sum(S * dS)

    grads = linear_backward_chunk_gates(q, k, v, gates["theta"], gates["eta"], gates["alpha"], dz, dM, dS, M0, S0,
                                        b=b)
    eps = 1e-6
    for i, name in ((3, "theta"), (4, "eta"), (5, "alpha")):
        fd = np.zeros(nc)
        for c in range(nc):
            gp = {kk: vv.copy() for kk, vv in gates.items()}
            gm = {kk: vv.copy() for kk, vv in gates.items()}
            gp[name][c] += eps
            gm[name][c] -= eps
            fd[c] = (obj(gp) - obj(gm)) / (2 * eps)
        np.testing.assert_allclose(grads[i], fd, atol=2e-7 * max(1.0, np.abs(fd).max()), rtol=0, err_msg=name)
