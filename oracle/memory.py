"""Per-token float64 loops for the chunked TTT / Titans memory (test infrastructure only).

Notation (column vectors): the linear memory is a matrix ``M`` of shape
``[dv, dk]`` read as ``z = M q``; ``M[i, j]`` carries key coordinate ``j`` into
value coordinate ``i``.  Gates per token: ``theta`` (inner learning rate),
``eta`` (momentum decay), ``alpha`` (forgetting).  All arrays may carry any
number of leading batch dimensions (batch, head, ...); the loops below run over
tokens only and treat every leading index independently, as independent
sequences do on the pages.

Sources (page title, then section / equation):

* "Continual Learning: From Attention to Neural Memory", sections 3.2-3.3: the
  loss ``1/2 ||k W - v||^2`` and its gradient as an outer product of key and
  error (row-vector form there; ``W`` there is ``M`` transposed here).
* same page, section 4.2: a TTT step ``W_t = W_{t-1} - lr * grad``, the read
  ``z_t = f(q_t; W_t)`` after the write, one same-shaped gradient per tensor.
* same page, section 4.7: mini-batch TTT -- gradients of a chunk share the
  chunk-start state; a token's read still sees only its own prefix of writes.
* same page, section 5.2 and "论文速览 | Titans" sections 3.4 and 3.7: momentum
  ``S_t = eta_t S_{t-1} - theta_t grad`` and forgetting
  ``M_t = (1 - alpha_t) M_{t-1} + S_t``, the gradient evaluated at the old
  memory.
* "论文速览 | Titans" section 4.2: the chunk-start reference state
  ``t' = t - mod(t, b)``, read here as "the state after the last token of the
  previous chunk" (0-based tokens), which is what the worked examples require.
* "5.1.1 · TTT layers 与 fast weights" section 1.1, eq. (6): mini-batch GD as the
  third choice of descent direction, gradients relative to the end of the
  previous mini-batch.
"""

from __future__ import annotations

import numpy as np

__all__ = ["linear_forward", "linear_backward", "linear_forward_chunk_gates", "linear_backward_chunk_gates",
           "mlp_forward", "silu", "silu_grad", "mlp_chunk_grads", "deep_forward", "deep_chunk_grads"]


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _matvec(A, x):
    """``A @ x`` for stacks: A [..., m, n], x [..., n] -> [..., m]."""
    return np.matmul(A, x[..., :, None])[..., :, 0]


def _outer(a, b):
    """Outer product for stacks: a [..., m], b [..., n] -> [..., m, n]."""
    return a[..., :, None] * b[..., None, :]


def linear_forward(q, k, v, theta, eta, alpha, M0=None, S0=None, b=1, grad="l2"):
    """Linear memory, chunk-start gradients, per-token momentum and forgetting.

    Arguments: ``q, k`` ``[..., T, dk]``; ``v`` ``[..., T, dv]``; ``theta, eta,
    alpha`` ``[..., T]``; ``M0, S0`` ``[..., dv, dk]`` or None for zeros;
    ``b`` the chunk (mini-batch) size, ``b >= 1``; the last chunk may be short.

    ``grad="l2"`` uses the gradient of ``1/2 ||M k - v||^2`` at the chunk-start
    memory, ``(M_c k - v) k^T`` ("Continual Learning..." section 3.3).
    ``grad="neg_vk"`` replaces it by ``-v k^T``, which turns the update into
    the additive write of unnormalised linear attention ("Continual
    Learning..." section 3.1; "论文速览 | Titans" section 2.3); it exists only
    so that tests can pin the schedule against closed forms.

    Returns ``z [..., T, dv], M_T [..., dv, dk], S_T [..., dv, dk]`` (float64).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    theta, eta, alpha = _f64(theta), _f64(eta), _f64(alpha)
    if b < 1:
        raise ValueError("chunk size b must be >= 1")
    if grad not in ("l2", "neg_vk"):
        raise ValueError("grad must be 'l2' or 'neg_vk'")
    lead, T, dk = q.shape[:-2], q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    M = np.zeros(lead + (dv, dk)) if M0 is None else np.array(np.broadcast_to(_f64(M0), lead + (dv, dk)))
    S = np.zeros(lead + (dv, dk)) if S0 is None else np.array(np.broadcast_to(_f64(S0), lead + (dv, dk)))
    z = np.zeros(lead + (T, dv))

    for c0 in range(0, T, b):
        # Chunk-start memory: the state after every write of the previous chunks.
        M_c = M.copy()
        for t in range(c0, min(c0 + b, T)):
            k_t, v_t = k[..., t, :], v[..., t, :]
            if grad == "l2":
                err = _matvec(M_c, k_t) - v_t          # prediction minus target
                G = _outer(err, k_t)                   # d/dM of 1/2||M k - v||^2
            else:
                G = -_outer(v_t, k_t)
            th = theta[..., t][..., None, None]
            et = eta[..., t][..., None, None]
            al = alpha[..., t][..., None, None]
            S = et * S - th * G                        # momentum ("surprise")
            M = (1.0 - al) * M + S                     # forget, then add momentum
            z[..., t, :] = _matvec(M, q[..., t, :])    # read after this token's write
    return z, M, S


def linear_backward(q, k, v, theta, eta, alpha, dz, dM_T=None, dS_T=None, M0=None, S0=None, b=1):
    """Reverse-mode gradient of ``linear_forward`` (``grad="l2"``), token by token.

    The outer loss is any function of the outputs; ``dz [..., T, dv]``,
    ``dM_T, dS_T [..., dv, dk]`` (None for zero) are its derivatives with respect
    to ``z``, ``M_T`` and ``S_T``.  Returns the derivatives with respect to every
    input: ``dq, dk, dv, dtheta, deta, dalpha, dM0, dS0``.

    The inner update is ordinary arithmetic, so its outer gradient is the chain
    rule applied backward through the sequence of state transitions ("Continual
    Learning: From Attention to Neural Memory", section 4.5: backpropagation
    through time over the unrolled writes, no gradient path detached;
    "5.1.1 · TTT layers 与 fast weights", section 1.1, eqs. (15)-(16): the
    outer gradient of a key runs through the inner gradient it produced).
    Each gradient of a chunk was taken at the chunk-start memory, so that
    memory collects the key/value paths of the whole chunk before the walk
    moves on to the previous chunk.

    The forward states are recomputed and kept for every token (plain and
    memory-hungry: small inputs only).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    theta, eta, alpha, dz = _f64(theta), _f64(eta), _f64(alpha), _f64(dz)
    if b < 1:
        raise ValueError("chunk size b must be >= 1")
    lead, T, dk_ = q.shape[:-2], q.shape[-2], q.shape[-1]
    dv_ = v.shape[-1]
    shape = lead + (dv_, dk_)
    M = np.zeros(shape) if M0 is None else np.array(np.broadcast_to(_f64(M0), shape))
    S = np.zeros(shape) if S0 is None else np.array(np.broadcast_to(_f64(S0), shape))

    # Forward, keeping what the reverse walk needs: the state before and after
    # each token, and each chunk's start memory and residuals.
    M_prev, S_prev, M_new = [], [], []
    M_start, err = [], []
    for c0 in range(0, T, b):
        M_c = M.copy()
        for t in range(c0, min(c0 + b, T)):
            e = _matvec(M_c, k[..., t, :]) - v[..., t, :]
            th = theta[..., t][..., None, None]
            et = eta[..., t][..., None, None]
            al = alpha[..., t][..., None, None]
            M_prev.append(M)
            S_prev.append(S)
            M_start.append(M_c)
            err.append(e)
            S = et * S - th * _outer(e, k[..., t, :])
            M = (1.0 - al) * M + S
            M_new.append(M)

    gq, gk, gv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    gth, get, gal = np.zeros_like(theta), np.zeros_like(eta), np.zeros_like(alpha)
    gM = np.zeros(shape) if dM_T is None else np.array(np.broadcast_to(_f64(dM_T), shape))
    gS = np.zeros(shape) if dS_T is None else np.array(np.broadcast_to(_f64(dS_T), shape))
    starts = list(range(0, T, b))
    for c0 in reversed(starts):
        gMc = np.zeros(shape)                  # collects every path through M_c
        for t in reversed(range(c0, min(c0 + b, T))):
            q_t, k_t, dz_t = q[..., t, :], k[..., t, :], dz[..., t, :]
            e, M_c = err[t], M_start[t]
            th = theta[..., t][..., None, None]
            et = eta[..., t][..., None, None]
            al = alpha[..., t][..., None, None]
            # z_t = M_t q_t
            gM = gM + _outer(dz_t, q_t)
            gq[..., t, :] = _matvec(np.swapaxes(M_new[t], -1, -2), dz_t)
            # M_t = (1 - alpha_t) M_{t-1} + S_t
            gS = gS + gM
            gal[..., t] = -np.sum(gM * M_prev[t], axis=(-1, -2))
            gM = (1.0 - al) * gM
            # S_t = eta_t S_{t-1} - theta_t e_t k_t^T
            G = _outer(e, k_t)
            get[..., t] = np.sum(gS * S_prev[t], axis=(-1, -2))
            gth[..., t] = -np.sum(gS * G, axis=(-1, -2))
            gG = -th * gS
            gS = et * gS
            # G = e k^T with e = M_c k - v
            ge = _matvec(gG, k_t)
            gk[..., t, :] = _matvec(np.swapaxes(gG, -1, -2), e) + _matvec(np.swapaxes(M_c, -1, -2), ge)
            gv[..., t, :] = -ge
            gMc = gMc + _outer(ge, k_t)
        gM = gM + gMc                          # M_c is the state entering the chunk
    return gq, gk, gv, gth, get, gal, gM, gS


def _expand_chunk_gates(g, T, b):
    """[..., NC] per-chunk values -> [..., T]: every token of chunk c takes entry c."""
    g = _f64(g)
    return np.repeat(g, b, axis=-1)[..., :T]


def linear_forward_chunk_gates(q, k, v, theta, eta, alpha, M0=None, S0=None, b=1):
    """``linear_forward`` with gates shared by the tokens of each chunk.

    "论文速览 | Titans" section 4.6: a faster variant in which alpha, theta and
    eta do not depend on the token but are shared within a chunk.  ``theta,
    eta, alpha`` are ``[..., ceil(T/b)]``; token t of chunk c = t // b uses
    entry c.  The iteration itself is unchanged.
    """
    T = np.shape(q)[-2]
    return linear_forward(q, k, v, _expand_chunk_gates(theta, T, b), _expand_chunk_gates(eta, T, b),
                          _expand_chunk_gates(alpha, T, b), M0, S0, b=b)


def linear_backward_chunk_gates(q, k, v, theta, eta, alpha, dz, dM_T=None, dS_T=None, M0=None, S0=None, b=1):
    """Gradient of ``linear_forward_chunk_gates``: a gate shared by a chunk's
    tokens collects the sum of their per-token gradients (chain rule through
    the broadcast)."""
    T = np.shape(q)[-2]
    g = linear_backward(q, k, v, _expand_chunk_gates(theta, T, b), _expand_chunk_gates(eta, T, b),
                        _expand_chunk_gates(alpha, T, b), dz, dM_T, dS_T, M0, S0, b=b)
    nc = (T + b - 1) // b

    def per_chunk(x):
        pad = nc * b - T
        x = np.concatenate([x, np.zeros(x.shape[:-1] + (pad,))], axis=-1) if pad else x
        return x.reshape(x.shape[:-1] + (nc, b)).sum(axis=-1)

    return g[0], g[1], g[2], per_chunk(g[3]), per_chunk(g[4]), per_chunk(g[5]), g[6], g[7]


def silu(x):
    """SiLU(x) = x * sigmoid(x)."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def silu_grad(x):
    """d/dx SiLU(x) = s (1 + x (1 - s)) with s = sigmoid(x)."""
    x = np.asarray(x, dtype=np.float64)
    s = 1.0 / (1.0 + np.exp(-x))
    return s * (1.0 + x * (1.0 - s))


def _mlp_apply(u, W1, W2):
    """Deep memory read, row-vector form: ``f(u) = u + SiLU(u W1) W2``."""
    h = np.matmul(u[..., None, :], W1)[..., 0, :]
    return u + np.matmul(silu(h)[..., None, :], W2)[..., 0, :]


def mlp_chunk_grads(k, v, W1, W2, loss_on="full"):
    """Gradients of ``1/2 ||f(k) - v||^2`` w.r.t. ``W1 [.., dk, hid]`` and ``W2 [.., hid, dv]``.

    Explicit backprop through ``f(u) = u + SiLU(u W1) W2`` (row vectors), for one
    key/value pair per leading index (``k [..., dk]``, ``v [..., dv]``).  With
    ``loss_on="mlp"`` the residual ``u`` is left out of the loss target (the
    other reading of the deep-memory description); the read is unchanged.

    Chain rule, step by step: ``h = k W1``; ``a = SiLU(h)``; ``r = k + a W2 - v``;
    ``dL/dW2 = a^T r``; ``dL/da = r W2^T``; ``dL/dh = dL/da * SiLU'(h)``;
    ``dL/dW1 = k^T dL/dh``.
    """
    h = np.matmul(k[..., None, :], W1)[..., 0, :]
    a = silu(h)
    y = np.matmul(a[..., None, :], W2)[..., 0, :]
    if loss_on == "full":
        r = k + y - v
    elif loss_on == "mlp":
        r = y - v
    else:
        raise ValueError("loss_on must be 'full' or 'mlp'")
    dW2 = _outer(a, r)
    da = np.matmul(r[..., None, :], np.swapaxes(W2, -1, -2))[..., 0, :]
    dh = da * silu_grad(h)
    dW1 = _outer(k, dh)
    return dW1, dW2


def mlp_forward(q, k, v, theta, eta, alpha, W1_0, W2_0, S1_0=None, S2_0=None, b=1, loss_on="full"):
    """Deep (2-layer MLP) memory with the same chunked schedule as ``linear_forward``.

    ``f(u) = u + SiLU(u W1) W2`` in row-vector form ("论文速览 | Titans" section
    3.9: a memory of at least two layers; "Nested Learning ... part 11/14"
    eq. (89): a residual MLP block without biases).  Both tensors get their own
    momentum and use the same per-token ``theta, eta, alpha`` ("Continual
    Learning..." section 4.2: one same-shaped gradient per tensor; section 5.1:
    the update history has the same structure as the weights).

    Shapes: ``q, k, v [..., T, d]``; ``W1_0, S1_0 [..., d, hid]``;
    ``W2_0, S2_0 [..., hid, d]``.  Returns ``z, W1_T, W2_T, S1_T, S2_T``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    theta, eta, alpha = _f64(theta), _f64(eta), _f64(alpha)
    if b < 1:
        raise ValueError("chunk size b must be >= 1")
    lead, T, d = q.shape[:-2], q.shape[-2], q.shape[-1]
    W1_0, W2_0 = _f64(W1_0), _f64(W2_0)
    hid = W1_0.shape[-1]
    W1 = np.array(np.broadcast_to(W1_0, lead + (d, hid)))
    W2 = np.array(np.broadcast_to(W2_0, lead + (hid, d)))
    S1 = np.zeros_like(W1) if S1_0 is None else np.array(np.broadcast_to(_f64(S1_0), W1.shape))
    S2 = np.zeros_like(W2) if S2_0 is None else np.array(np.broadcast_to(_f64(S2_0), W2.shape))
    z = np.zeros(lead + (T, d))

    for c0 in range(0, T, b):
        W1_c, W2_c = W1.copy(), W2.copy()          # chunk-start weights
        for t in range(c0, min(c0 + b, T)):
            G1, G2 = mlp_chunk_grads(k[..., t, :], v[..., t, :], W1_c, W2_c, loss_on)
            th = theta[..., t][..., None, None]
            et = eta[..., t][..., None, None]
            al = alpha[..., t][..., None, None]
            S1 = et * S1 - th * G1
            S2 = et * S2 - th * G2
            W1 = (1.0 - al) * W1 + S1
            W2 = (1.0 - al) * W2 + S2
            z[..., t, :] = _mlp_apply(q[..., t, :], W1, W2)
    return z, W1, W2, S1, S2


def _deep_apply(u, Ws):
    """Deep memory read with L = len(Ws) >= 2 layers, row-vector form:
    ``f(u) = u + SiLU(...SiLU(SiLU(u W_1) W_2)...) W_L``."""
    x = u
    for W in Ws[:-1]:
        x = silu(np.matmul(x[..., None, :], W)[..., 0, :])
    return u + np.matmul(x[..., None, :], Ws[-1])[..., 0, :]


def deep_chunk_grads(k, v, Ws):
    """Gradients of ``1/2 ||f(k) - v||^2`` w.r.t. every layer of the L-layer memory.

    Explicit backprop through ``f(u) = u + SiLU(...SiLU(u W_1)...) W_L`` for one
    key/value pair per leading index.  Forward: ``x_0 = k``, ``h_l = x_{l-1} W_l``
    and ``x_l = SiLU(h_l)`` for l < L, ``r = k + x_{L-1} W_L - v``.  Backward:
    ``delta_L = r``, ``dL/dW_L = x_{L-1}^T r``, and for l = L-1 .. 1
    ``delta_l = (delta_{l+1} W_{l+1}^T) * SiLU'(h_l)``, ``dL/dW_l = x_{l-1}^T delta_l``.
    """
    L = len(Ws)
    xs, hs = [k], []
    for W in Ws[:-1]:
        h = np.matmul(xs[-1][..., None, :], W)[..., 0, :]
        hs.append(h)
        xs.append(silu(h))
    r = k + np.matmul(xs[-1][..., None, :], Ws[-1])[..., 0, :] - v
    grads = [None] * L
    delta = r
    grads[L - 1] = _outer(xs[L - 1], delta)
    for l in range(L - 2, -1, -1):
        back = np.matmul(delta[..., None, :], np.swapaxes(Ws[l + 1], -1, -2))[..., 0, :]
        delta = back * silu_grad(hs[l])
        grads[l] = _outer(xs[l], delta)
    return grads


def deep_forward(q, k, v, theta, eta, alpha, Ws0, Ss0=None, b=1):
    """Deep memory of depth L = len(Ws0) >= 2 with the chunked schedule of ``linear_forward``.

    "论文速览 | Titans" section 3.9: a deep memory is a stack of L linear maps
    with a nonlinearity between them; section 8.5 compares depths 1 to 4.
    Here, in row-vector form with the residual and no biases of the 2-layer
    memory (``mlp_forward``): ``f(u) = u + SiLU(...SiLU(u W_1)...) W_L`` with
    ``W_1 [d, hid]``, ``W_l [hid, hid]`` for 1 < l < L, ``W_L [hid, d]``.
    Every layer has its own momentum; all use the token's ``theta, eta, alpha``;
    every gradient of a chunk is taken at the chunk-start weights and the read
    ``z_t = f(q_t)`` uses the weights after token t's own write.

    ``Ws0``, ``Ss0``: lists of L arrays (leading dimensions broadcast);
    ``Ss0=None`` means zero momenta.  Returns ``(z, Ws_T, Ss_T)``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    theta, eta, alpha = _f64(theta), _f64(eta), _f64(alpha)
    if b < 1:
        raise ValueError("chunk size b must be >= 1")
    if len(Ws0) < 2:
        raise ValueError("a deep memory has at least two layers")
    lead, T, d = q.shape[:-2], q.shape[-2], q.shape[-1]
    Ws = [np.array(np.broadcast_to(_f64(W), lead + np.shape(W)[-2:])) for W in Ws0]
    if Ss0 is None:
        Ss = [np.zeros_like(W) for W in Ws]
    else:
        Ss = [np.zeros_like(W) if S is None else np.array(np.broadcast_to(_f64(S), W.shape))
              for S, W in zip(Ss0, Ws)]
    z = np.zeros(lead + (T, d))
    for c0 in range(0, T, b):
        Wc = [W.copy() for W in Ws]                 # chunk-start weights
        for t in range(c0, min(c0 + b, T)):
            Gs = deep_chunk_grads(k[..., t, :], v[..., t, :], Wc)
            th = theta[..., t][..., None, None]
            et = eta[..., t][..., None, None]
            al = alpha[..., t][..., None, None]
            Ss = [et * S - th * G for S, G in zip(Ss, Gs)]
            Ws = [(1.0 - al) * W + S for W, S in zip(Ws, Ss)]
            z[..., t, :] = _deep_apply(q[..., t, :], Ws)
    return z, Ws, Ss
