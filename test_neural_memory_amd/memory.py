"""Thin torch binding of libttt_mem: argument marshalling only.

Every function here validates tensor placement and layout, allocates the
outputs with torch (device memory), and calls the C ABI of the same name on
torch's current HIP stream.  All arithmetic happens in the HIP kernels.
"""

from __future__ import annotations

import torch

from . import _lib


def _ptr(t):
    return None if t is None else t.data_ptr()


def _as_dev(t, name, dtype, shape, device):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.contiguous()


def _forward(name, in_dtype, q, k, v, theta, eta, alpha, M0, S0, b, out, with_b=True, extra=None,
             gate_len=None, pass_extra=False, z_dtype=torch.float32):
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    B, H, T, d = q.shape
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be HIP device tensors (torch 'cuda' device)")
    q = _as_dev(q, "q", in_dtype, (B, H, T, d), dev)
    k = _as_dev(k, "k", in_dtype, (B, H, T, d), dev)
    v = _as_dev(v, "v", in_dtype, (B, H, T, d), dev)
    gl = T if gate_len is None else gate_len
    theta = _as_dev(theta, "theta", torch.float32, (B, H, gl), dev)
    eta = _as_dev(eta, "eta", torch.float32, (B, H, gl), dev)
    alpha = _as_dev(alpha, "alpha", torch.float32, (B, H, gl), dev)
    M0 = _as_dev(M0, "M0", torch.float32, (B, H, d, d), dev)
    S0 = _as_dev(S0, "S0", torch.float32, (B, H, d, d), dev)
    if out is None:
        z = torch.empty((B, H, T, d), dtype=z_dtype, device=dev)
        M_T = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
        S_T = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    else:
        z, M_T, S_T = out
        for t, nm, shp, dt in ((z, "z", (B, H, T, d), z_dtype), (M_T, "M_T", (B, H, d, d), torch.float32),
                               (S_T, "S_T", (B, H, d, d), torch.float32)):
            if t is not None and (not t.is_contiguous() or t.dtype != dt
                                  or tuple(t.shape) != shp or t.device != dev):
                raise ValueError(f"out tensor {nm} must be contiguous {dt} {shp} on {dev}")
    lib = _lib.load()
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        sizes = (B, H, T, d, int(b)) if with_b else (B, H, T, d)
        ptrs = [_ptr(q), _ptr(k), _ptr(v), _ptr(theta), _ptr(eta), _ptr(alpha), _ptr(M0), _ptr(S0),
                _ptr(z), _ptr(M_T), _ptr(S_T)]
        if extra is not None or pass_extra:
            ptrs.append(_ptr(extra))
        status = getattr(lib, name)(*ptrs, *sizes, stream)
    _lib.check(name, status)
    return z, M_T, S_T


def ttt_mem_forward_f32(q, k, v, theta, eta, alpha, M0=None, S0=None, *, b, out=None):
    """float32 linear memory; returns ``(z, M_T, S_T)`` (see include/ttt_mem.h)."""
    return _forward("ttt_mem_forward_f32", torch.float32, q, k, v, theta, eta, alpha, M0, S0, b, out)


def ttt_mem_forward_bf16(q, k, v, theta, eta, alpha, M0=None, S0=None, *, b, out=None):
    """bf16-input linear memory: bf16 z, float32 state; returns ``(z, M_T, S_T)``."""
    return _forward("ttt_mem_forward_bf16", torch.bfloat16, q, k, v, theta, eta, alpha, M0, S0, b, out,
                    z_dtype=torch.bfloat16)


def ttt_mem_forward_bf16_zf32(q, k, v, theta, eta, alpha, M0=None, S0=None, *, b, out=None):
    """bf16-input linear memory with float32 z (and state); returns ``(z, M_T, S_T)``."""
    return _forward("ttt_mem_forward_bf16_zf32", torch.bfloat16, q, k, v, theta, eta, alpha, M0, S0, b, out)


def forward(q, k, v, theta, eta, alpha, M0=None, S0=None, *, b, out=None, z_dtype=None):
    """Dispatch on the input dtype (float32 or bfloat16).

    z has the input dtype unless ``z_dtype=torch.float32`` asks for float32 z
    from bf16 inputs.
    """
    if q.dtype == torch.float32:
        if z_dtype not in (None, torch.float32):
            raise TypeError("float32 inputs give float32 z")
        return ttt_mem_forward_f32(q, k, v, theta, eta, alpha, M0, S0, b=b, out=out)
    if q.dtype == torch.bfloat16:
        if z_dtype in (None, torch.bfloat16):
            return ttt_mem_forward_bf16(q, k, v, theta, eta, alpha, M0, S0, b=b, out=out)
        if z_dtype == torch.float32:
            return ttt_mem_forward_bf16_zf32(q, k, v, theta, eta, alpha, M0, S0, b=b, out=out)
        raise TypeError(f"unsupported z dtype {z_dtype}")
    raise TypeError(f"unsupported input dtype {q.dtype}")


def _nch(T, b):
    return (T + b - 1) // b


def ckpt_dtype(in_dtype):
    """Element type of the checkpoints (and of the backward's work buffer):
    float32 for float32 inputs, fp16 for bf16 inputs (the precision every use
    of the states rounds them to on that path)."""
    return torch.float32 if in_dtype == torch.float32 else torch.float16


def new_ckpt(q, b):
    """An uninitialised checkpoint tensor for the inputs ``q [B, H, T, d]`` and chunk size b."""
    B, H, T, d = q.shape
    return torch.empty((B, H, _nch(T, int(b)), 2, d, d), dtype=ckpt_dtype(q.dtype), device=q.device)


def forward_train(q, k, v, theta, eta, alpha, M0=None, S0=None, *, b, out=None, ckpt=None):
    """Forward that also saves the state entering every chunk for ``backward``.

    Returns ``(z, M_T, S_T, ckpt)`` with ``ckpt [B, H, ceil(T/b), 2, d, d]``
    (``ckpt[..., c, 0]`` = M and ``[..., c, 1]`` = S before chunk c), float32
    for float32 inputs and fp16 for bf16 inputs.
    """
    if q.dtype == torch.float32:
        name = "ttt_mem_forward_ckpt_f32"
    elif q.dtype == torch.bfloat16:
        name = "ttt_mem_forward_ckpt_bf16"
    else:
        raise TypeError(f"unsupported input dtype {q.dtype}")
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    B, H, T, d = q.shape
    shape = (B, H, _nch(T, int(b)), 2, d, d)
    cdt = ckpt_dtype(q.dtype)
    if ckpt is None:
        ckpt = torch.empty(shape, dtype=cdt, device=q.device)
    elif (not ckpt.is_contiguous() or ckpt.dtype != cdt or tuple(ckpt.shape) != shape
          or ckpt.device != q.device):
        raise ValueError(f"ckpt must be contiguous {cdt} {shape} on {q.device}")
    z, M_T, S_T = _forward(name, q.dtype, q, k, v, theta, eta, alpha, M0, S0, b, out, extra=ckpt)
    return z, M_T, S_T, ckpt


def forward_chunk_gates(q, k, v, theta, eta, alpha, M0=None, S0=None, *, b, out=None, ckpt=None):
    """Linear memory with gates shared by the tokens of each chunk.

    ``theta, eta, alpha`` are ``[B, H, ceil(T/b)]``: every token of chunk c uses
    entry c.  Returns ``(z, M_T, S_T)``, or ``(z, M_T, S_T, ckpt)`` when a
    ``ckpt`` tensor (``[B, H, ceil(T/b), 2, d, d]`` of ``ckpt_dtype(q.dtype)``,
    as from ``new_ckpt``) is given to keep the chunk-start states for
    ``backward(..., chunk_gates=True)``.
    """
    if q.dtype == torch.float32:
        name = "ttt_mem_forward_cg_f32"
    elif q.dtype == torch.bfloat16:
        name = "ttt_mem_forward_cg_bf16"
    else:
        raise TypeError(f"unsupported input dtype {q.dtype}")
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    B, H, T, d = q.shape
    nc = _nch(T, int(b))
    if ckpt is not None:
        shape = (B, H, nc, 2, d, d)
        cdt = ckpt_dtype(q.dtype)
        if (not ckpt.is_contiguous() or ckpt.dtype != cdt or tuple(ckpt.shape) != shape
                or ckpt.device != q.device):
            raise ValueError(f"ckpt must be contiguous {cdt} {shape} on {q.device}")
    res = _forward(name, q.dtype, q, k, v, theta, eta, alpha, M0, S0, b, out, extra=ckpt, gate_len=nc,
                   pass_extra=True)
    return res if ckpt is None else res + (ckpt,)


def backward(q, k, v, theta, eta, alpha, ckpt, dz, dM_T=None, dS_T=None, *, b, work=None, out=None,
             want_state_grads=True, chunk_gates=False):
    """Gradients of the linear memory from ``forward_train``'s checkpoints.

    ``ckpt`` is ``forward_train``'s (float32, or fp16 for bf16 inputs).
    ``dz [B, H, T, d]``, ``dM_T, dS_T [B, H, d, d]`` (float32; None = zero) are
    the derivatives of the outer loss with respect to ``z, M_T, S_T``.
    Returns ``(dq, dk, dv, dtheta, deta, dalpha, dM0, dS0)``, all float32
    (``dM0, dS0`` are None when ``want_state_grads`` is False).  ``work`` may
    pass a contiguous scratch tensor of at least ``backward_work_bytes(q, b)``
    bytes; ``out`` preallocated outputs in the same order.
    """
    suffix = "_cg" if chunk_gates else ""
    if q.dtype == torch.float32:
        name = f"ttt_mem_backward{suffix}_f32"
    elif q.dtype == torch.bfloat16:
        name = f"ttt_mem_backward{suffix}_bf16"
    else:
        raise TypeError(f"unsupported input dtype {q.dtype}")
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    B, H, T, d = q.shape
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be HIP device tensors (torch 'cuda' device)")
    b = int(b)
    in_dtype = q.dtype
    q = _as_dev(q, "q", in_dtype, (B, H, T, d), dev)
    k = _as_dev(k, "k", in_dtype, (B, H, T, d), dev)
    v = _as_dev(v, "v", in_dtype, (B, H, T, d), dev)
    gl = _nch(T, b) if chunk_gates else T
    theta = _as_dev(theta, "theta", torch.float32, (B, H, gl), dev)
    eta = _as_dev(eta, "eta", torch.float32, (B, H, gl), dev)
    alpha = _as_dev(alpha, "alpha", torch.float32, (B, H, gl), dev)
    ck_shape = (B, H, _nch(T, b), 2, d, d)
    cdt = ckpt_dtype(in_dtype)
    ckpt = _as_dev(ckpt, "ckpt", cdt, ck_shape, dev)
    dz = _as_dev(dz, "dz", torch.float32, (B, H, T, d), dev)
    dM_T = _as_dev(dM_T, "dM_T", torch.float32, (B, H, d, d), dev)
    dS_T = _as_dev(dS_T, "dS_T", torch.float32, (B, H, d, d), dev)
    work = _work_buffer(work, backward_work_bytes(q, b), dev)
    shapes = [(B, H, T, d)] * 3 + [(B, H, gl)] * 3 + [(B, H, d, d)] * 2
    if out is None:
        out = [torch.empty(s_, dtype=torch.float32, device=dev) for s_ in shapes]
        if not want_state_grads:
            out[6] = out[7] = None
    else:
        out = list(out)
        for i, (t, shp) in enumerate(zip(out, shapes)):
            if t is not None and (not t.is_contiguous() or t.dtype != torch.float32
                                  or tuple(t.shape) != shp or t.device != dev):
                raise ValueError(f"out tensor {i} must be contiguous float32 {shp} on {dev}")
    lib = _lib.load()
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        status = getattr(lib, name)(
            _ptr(q), _ptr(k), _ptr(v), _ptr(theta), _ptr(eta), _ptr(alpha), _ptr(ckpt), _ptr(dz),
            _ptr(dM_T), _ptr(dS_T), *[_ptr(t) for t in out], _ptr(work), B, H, T, d, b, stream)
    _lib.check(name, status)
    return tuple(out)


def backward_work_bytes(q, b, cu_seqlens=None):
    """Bytes of the backward's work buffer for inputs like ``q`` (``[B, H, T, d]``,
    or ``[H, T, d]`` with ``cu_seqlens`` for packed documents) and chunk size ``b``."""
    lib = _lib.load()
    bf = q.dtype == torch.bfloat16
    if cu_seqlens is None:
        B, H, T, d = q.shape
        fn = lib.ttt_mem_backward_work_bytes_bf16 if bf else lib.ttt_mem_ckpt_bytes
        return int(fn(B, H, T, d, int(b)))
    H, T, d = q.shape
    N = cu_seqlens.numel() - 1
    fn = lib.ttt_mem_backward_work_bytes_varlen_bf16 if bf else lib.ttt_mem_ckpt_bytes_varlen
    return int(fn(N, H, T, d, int(b)))


def _work_buffer(work, nbytes, dev):
    if work is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if not work.is_contiguous() or work.device != dev or work.numel() * work.element_size() < nbytes:
        raise ValueError(f"work must be a contiguous tensor of at least {nbytes} bytes on {dev}")
    return work


class LinearMemoryFunction(torch.autograd.Function):
    """``(z, M_T, S_T) = memory(q, k, v, theta, eta, alpha, M0, S0)`` with a HIP backward.

    Forward saves the chunk-start states; backward calls ``backward``.  Gradients
    of bf16 inputs are returned in bf16 (computed in float32).
    """

    @staticmethod
    def forward(ctx, q, k, v, theta, eta, alpha, M0, S0, b):
        z, M_T, S_T, ckpt = forward_train(q, k, v, theta, eta, alpha, M0, S0, b=b)
        ctx.save_for_backward(q, k, v, theta, eta, alpha, ckpt)
        ctx.b = b
        ctx.has_state = (M0 is not None, S0 is not None)
        return z, M_T, S_T

    @staticmethod
    def backward(ctx, dz, dM_T, dS_T):
        q, k, v, theta, eta, alpha, ckpt = ctx.saved_tensors
        B, H, T, d = q.shape
        if dz is None:
            dz = torch.zeros((B, H, T, d), dtype=torch.float32, device=q.device)
        g = backward(q, k, v, theta, eta, alpha, ckpt, dz.float().contiguous(),
                     None if dM_T is None else dM_T.float().contiguous(),
                     None if dS_T is None else dS_T.float().contiguous(), b=ctx.b)
        dq, dk, dv = (x.to(q.dtype) for x in g[:3])
        dM0 = g[6] if ctx.has_state[0] else None
        dS0 = g[7] if ctx.has_state[1] else None
        return dq, dk, dv, g[3], g[4], g[5], dM0, dS0, None


def linear_memory(q, k, v, theta, eta, alpha, M0=None, S0=None, *, b):
    """Differentiable linear memory: ``(z, M_T, S_T)``, gradients through the HIP backward."""
    return LinearMemoryFunction.apply(q, k, v, theta, eta, alpha, M0, S0, b)


def varlen_slots(N, T, b):
    """Chunk slots per head of the packed-document checkpoints: ceil(T/b) + N."""
    return _nch(T, int(b)) + N


def new_ckpt_varlen(q, cu_seqlens, b):
    """An uninitialised checkpoint tensor ``[H, slots, 2, d, d]`` for packed documents."""
    H, T, d = q.shape
    N = cu_seqlens.numel() - 1
    return torch.empty((H, varlen_slots(N, T, b), 2, d, d), dtype=ckpt_dtype(q.dtype), device=q.device)


def forward_varlen(q, k, v, theta, eta, alpha, cu_seqlens, M0=None, S0=None, *, b, out=None, ckpt=None):
    """Linear memory over packed variable-length documents; returns ``(z, M_T, S_T)``.

    ``q, k, v`` are ``[H, T, d]`` (float32 or bfloat16), the gates ``[H, T]``,
    ``cu_seqlens`` an int32 device tensor ``[N + 1]`` of document offsets, and
    the states ``[N, H, d, d]``: each document starts from its own state.  With
    ``ckpt`` (``new_ckpt_varlen``), the chunk-start states of every document are
    kept for ``backward_varlen`` and ``(z, M_T, S_T, ckpt)`` is returned.
    """
    if q.dim() != 3:
        raise ValueError("q must be [H, T, d]")
    H, T, d = q.shape
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be HIP device tensors (torch 'cuda' device)")
    tail = "_ckpt" if ckpt is not None else ""
    if q.dtype == torch.float32:
        name = f"ttt_mem_forward_varlen{tail}_f32"
    elif q.dtype == torch.bfloat16:
        name = f"ttt_mem_forward_varlen{tail}_bf16"
    else:
        raise TypeError(f"unsupported input dtype {q.dtype}")
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D tensor of N + 1 offsets")
    N = cu_seqlens.numel() - 1
    cu = _as_dev(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    q = _as_dev(q, "q", q.dtype, (H, T, d), dev)
    k = _as_dev(k, "k", q.dtype, (H, T, d), dev)
    v = _as_dev(v, "v", q.dtype, (H, T, d), dev)
    theta = _as_dev(theta, "theta", torch.float32, (H, T), dev)
    eta = _as_dev(eta, "eta", torch.float32, (H, T), dev)
    alpha = _as_dev(alpha, "alpha", torch.float32, (H, T), dev)
    M0 = _as_dev(M0, "M0", torch.float32, (N, H, d, d), dev)
    S0 = _as_dev(S0, "S0", torch.float32, (N, H, d, d), dev)
    shapes = ((H, T, d), (N, H, d, d), (N, H, d, d))
    if out is None:
        out = tuple(torch.empty(s_, dtype=torch.float32, device=dev) for s_ in shapes)
    else:
        for t, nm, shp in zip(out, ("z", "M_T", "S_T"), shapes):
            if t is not None and (not t.is_contiguous() or t.dtype != torch.float32
                                  or tuple(t.shape) != shp or t.device != dev):
                raise ValueError(f"out tensor {nm} must be contiguous float32 {shp} on {dev}")
    z, M_T, S_T = out
    extra = []
    if ckpt is not None:
        ckpt = _as_dev(ckpt, "ckpt", ckpt_dtype(q.dtype), (H, varlen_slots(N, T, b), 2, d, d), dev)
        extra = [_ptr(ckpt)]
    lib = _lib.load()
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        status = getattr(lib, name)(
            _ptr(q), _ptr(k), _ptr(v), _ptr(theta), _ptr(eta), _ptr(alpha), _ptr(M0), _ptr(S0),
            _ptr(z), _ptr(M_T), _ptr(S_T), *extra, _ptr(cu), N, H, T, d, int(b), stream)
    _lib.check(name, status)
    return (z, M_T, S_T) if ckpt is None else (z, M_T, S_T, ckpt)


def backward_varlen(q, k, v, theta, eta, alpha, cu_seqlens, ckpt, dz, dM_T=None, dS_T=None, *, b, work=None,
                    out=None):
    """Gradients over packed documents from ``forward_varlen(..., ckpt=...)``.

    ``dz [H, T, d]``, ``dM_T, dS_T [N, H, d, d]`` (float32; None = zero).
    Returns ``(dq, dk, dv, dtheta, deta, dalpha, dM0, dS0)``, float32, with
    ``dq, dk, dv [H, T, d]``, the gate gradients ``[H, T]`` and ``dM0, dS0
    [N, H, d, d]``.  Tokens outside every document are not written.
    """
    if q.dim() != 3:
        raise ValueError("q must be [H, T, d]")
    H, T, d = q.shape
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be HIP device tensors (torch 'cuda' device)")
    if q.dtype == torch.float32:
        name = "ttt_mem_backward_varlen_f32"
    elif q.dtype == torch.bfloat16:
        name = "ttt_mem_backward_varlen_bf16"
    else:
        raise TypeError(f"unsupported input dtype {q.dtype}")
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D tensor of N + 1 offsets")
    N = cu_seqlens.numel() - 1
    b = int(b)
    in_dtype = q.dtype
    cu = _as_dev(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    q = _as_dev(q, "q", in_dtype, (H, T, d), dev)
    k = _as_dev(k, "k", in_dtype, (H, T, d), dev)
    v = _as_dev(v, "v", in_dtype, (H, T, d), dev)
    theta = _as_dev(theta, "theta", torch.float32, (H, T), dev)
    eta = _as_dev(eta, "eta", torch.float32, (H, T), dev)
    alpha = _as_dev(alpha, "alpha", torch.float32, (H, T), dev)
    ck_shape = (H, varlen_slots(N, T, b), 2, d, d)
    cdt = ckpt_dtype(in_dtype)
    ckpt = _as_dev(ckpt, "ckpt", cdt, ck_shape, dev)
    dz = _as_dev(dz, "dz", torch.float32, (H, T, d), dev)
    dM_T = _as_dev(dM_T, "dM_T", torch.float32, (N, H, d, d), dev)
    dS_T = _as_dev(dS_T, "dS_T", torch.float32, (N, H, d, d), dev)
    work = _work_buffer(work, backward_work_bytes(q, b, cu), dev)
    shapes = [(H, T, d)] * 3 + [(H, T)] * 3 + [(N, H, d, d)] * 2
    if out is None:
        out = [torch.empty(s_, dtype=torch.float32, device=dev) for s_ in shapes]
    else:
        out = list(out)
        for i, (t, shp) in enumerate(zip(out, shapes)):
            if t is not None and (not t.is_contiguous() or t.dtype != torch.float32
                                  or tuple(t.shape) != shp or t.device != dev):
                raise ValueError(f"out tensor {i} must be contiguous float32 {shp} on {dev}")
    lib = _lib.load()
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        status = getattr(lib, name)(
            _ptr(q), _ptr(k), _ptr(v), _ptr(theta), _ptr(eta), _ptr(alpha), _ptr(ckpt), _ptr(dz),
            _ptr(dM_T), _ptr(dS_T), *[_ptr(t) for t in out], _ptr(work), _ptr(cu), N, H, T, d, b, stream)
    _lib.check(name, status)
    return tuple(out)


def ttt_mem_decode_f32(q, k, v, theta, eta, alpha, M0=None, S0=None, *, out=None):
    """float32 token-by-token (primal) linear memory; returns ``(z, M_T, S_T)``.

    Pass ``out=(z, M0, S0)`` to carry the state in place between calls.
    """
    return _forward("ttt_mem_decode_f32", torch.float32, q, k, v, theta, eta, alpha, M0, S0, 1, out, with_b=False)


def ttt_mem_decode_bf16(q, k, v, theta, eta, alpha, M0=None, S0=None, *, out=None):
    """bf16-input token-by-token (primal) linear memory (float32 arithmetic, state and z)."""
    return _forward("ttt_mem_decode_bf16", torch.bfloat16, q, k, v, theta, eta, alpha, M0, S0, 1, out, with_b=False)


def decode(q, k, v, theta, eta, alpha, M0=None, S0=None, *, out=None):
    """Dispatch the token-by-token form on the input dtype (float32 or bfloat16)."""
    if q.dtype == torch.float32:
        return ttt_mem_decode_f32(q, k, v, theta, eta, alpha, M0, S0, out=out)
    if q.dtype == torch.bfloat16:
        return ttt_mem_decode_bf16(q, k, v, theta, eta, alpha, M0, S0, out=out)
    raise TypeError(f"unsupported input dtype {q.dtype}")


def ttt_mem_mlp_forward_bf16(q, k, v, theta, eta, alpha, W1_0, W2_0, S1_0=None, S2_0=None, *, b, out=None,
                             z_dtype=torch.bfloat16):
    """bf16-input deep (2-layer MLP) memory; returns ``(z, W1_T, W2_T, S1_T, S2_T)``.

    ``W1_0, S1_0`` are ``[B, H, d, hidden]`` and ``W2_0, S2_0`` ``[B, H, hidden, d]``
    float32; z is bf16 (``z_dtype=torch.float32`` for float32 z); ``out`` may
    pass preallocated ``(z, W1_T, W2_T, S1_T, S2_T)``.
    """
    if z_dtype == torch.bfloat16:
        name = "ttt_mem_mlp_forward_bf16"
    elif z_dtype == torch.float32:
        name = "ttt_mem_mlp_forward_bf16_zf32"
    else:
        raise TypeError(f"unsupported z dtype {z_dtype}")
    return _mlp_forward(name, z_dtype, q, k, v, theta, eta, alpha, W1_0, W2_0, S1_0, S2_0, b, out)


def ttt_mem_mlp_forward_bf16_noalloc(q, k, v, theta, eta, alpha, W1_0, W2_0, S1_0=None, S2_0=None, *, b, out):
    """As :func:`ttt_mem_mlp_forward_bf16` (bf16 z), with the library allocating
    no device memory: ``out`` (preallocated ``(z, W1_T, W2_T, S1_T, S2_T)``) is
    required and the exchange workspace is the library's fixed per-GPU array, so
    calls that overlap in time on one GPU race.  At most 8 sequences run at a time.
    """
    if out is None or any(t is None for t in out):
        raise ValueError("the no-allocation entry point needs every output preallocated")
    return _mlp_forward("ttt_mem_mlp_forward_bf16_noalloc", torch.bfloat16, q, k, v, theta, eta, alpha, W1_0, W2_0,
                        S1_0, S2_0, b, out)


def _mlp_forward(name, z_dtype, q, k, v, theta, eta, alpha, W1_0, W2_0, S1_0, S2_0, b, out):
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    B, H, T, d = q.shape
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be HIP device tensors (torch 'cuda' device)")
    if W1_0 is None or W2_0 is None:
        raise ValueError("W1_0 and W2_0 are required")
    hid = W1_0.shape[-1]
    q = _as_dev(q, "q", torch.bfloat16, (B, H, T, d), dev)
    k = _as_dev(k, "k", torch.bfloat16, (B, H, T, d), dev)
    v = _as_dev(v, "v", torch.bfloat16, (B, H, T, d), dev)
    theta = _as_dev(theta, "theta", torch.float32, (B, H, T), dev)
    eta = _as_dev(eta, "eta", torch.float32, (B, H, T), dev)
    alpha = _as_dev(alpha, "alpha", torch.float32, (B, H, T), dev)
    W1_0 = _as_dev(W1_0, "W1_0", torch.float32, (B, H, d, hid), dev)
    W2_0 = _as_dev(W2_0, "W2_0", torch.float32, (B, H, hid, d), dev)
    S1_0 = _as_dev(S1_0, "S1_0", torch.float32, (B, H, d, hid), dev)
    S2_0 = _as_dev(S2_0, "S2_0", torch.float32, (B, H, hid, d), dev)
    shapes = ((B, H, T, d), (B, H, d, hid), (B, H, hid, d), (B, H, d, hid), (B, H, hid, d))
    dts = (z_dtype,) + (torch.float32,) * 4
    if out is None:
        out = tuple(torch.empty(s, dtype=dt, device=dev) for s, dt in zip(shapes, dts))
    else:
        for t, nm, shp, dt in zip(out, ("z", "W1_T", "W2_T", "S1_T", "S2_T"), shapes, dts):
            if t is not None and (not t.is_contiguous() or t.dtype != dt
                                  or tuple(t.shape) != shp or t.device != dev):
                raise ValueError(f"out tensor {nm} must be contiguous {dt} {shp} on {dev}")
    z, W1_T, W2_T, S1_T, S2_T = out
    lib = _lib.load()
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        status = getattr(lib, name)(
            _ptr(q), _ptr(k), _ptr(v), _ptr(theta), _ptr(eta), _ptr(alpha), _ptr(W1_0), _ptr(W2_0),
            _ptr(S1_0), _ptr(S2_0), _ptr(z), _ptr(W1_T), _ptr(W2_T), _ptr(S1_T), _ptr(S2_T),
            B, H, T, d, int(hid), int(b), stream)
    _lib.check(name, status)
    return z, W1_T, W2_T, S1_T, S2_T


def deep_param_count(d, hidden, depth):
    """Floats per (batch, head) of the packed deep-memory parameters."""
    return int(_lib.load().ttt_mem_deep_param_count(int(d), int(hidden), int(depth)))


def deep_layer_shapes(d, hidden, depth):
    """Shapes of the layers of a deep memory: [d, hid], [hid, hid] * (depth - 2), [hid, d]."""
    return [(d, hidden)] + [(hidden, hidden)] * (depth - 2) + [(hidden, d)]


def deep_pack(layers):
    """[B, H, *shape_l] float32 layers -> one contiguous [B, H, P] tensor (layer-major per sequence)."""
    B, H = layers[0].shape[:2]
    return torch.cat([x.reshape(B, H, -1) for x in layers], dim=-1).contiguous()


def deep_unpack(packed, d, hidden, depth):
    """The inverse of ``deep_pack``: views of the layers of a [B, H, P] tensor."""
    B, H = packed.shape[:2]
    out, off = [], 0
    for shp in deep_layer_shapes(d, hidden, depth):
        n = shp[0] * shp[1]
        out.append(packed[..., off:off + n].reshape(B, H, *shp))
        off += n
    return out


def new_deep_work(B, H, d, hidden, depth, device):
    """A workspace for ``deep_forward`` (uninitialised; the launch clears what it needs)."""
    n = int(_lib.load().ttt_mem_deep_work_bytes(int(B), int(H), int(d), int(hidden), int(depth)))
    if n == 0:
        raise ValueError("unsupported deep-memory sizes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def deep_forward(q, k, v, theta, eta, alpha, W0, S0=None, *, hidden, depth, b, work=None, out=None):
    """bf16-input deep memory of depth 2-4 with packed parameters.

    ``W0, S0`` are ``[B, H, P]`` float32 (``deep_pack``), P =
    ``deep_param_count(d, hidden, depth)``.  Returns
    ``(z, W_T, S_T)`` with bf16 z.  ``work`` (``new_deep_work``) is the
    exchange workspace; if None, the call takes one from the stream-ordered
    allocator.  ``out`` may pass ``(z, W_T, S_T)``.
    """
    name = "ttt_mem_deep_forward_bf16"
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    B, H, T, d = q.shape
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be HIP device tensors (torch 'cuda' device)")
    if W0 is None:
        raise ValueError("W0 is required")
    P = deep_param_count(d, hidden, depth)
    q = _as_dev(q, "q", torch.bfloat16, (B, H, T, d), dev)
    k = _as_dev(k, "k", torch.bfloat16, (B, H, T, d), dev)
    v = _as_dev(v, "v", torch.bfloat16, (B, H, T, d), dev)
    theta = _as_dev(theta, "theta", torch.float32, (B, H, T), dev)
    eta = _as_dev(eta, "eta", torch.float32, (B, H, T), dev)
    alpha = _as_dev(alpha, "alpha", torch.float32, (B, H, T), dev)
    W0 = _as_dev(W0, "W0", torch.float32, (B, H, P), dev)
    S0 = _as_dev(S0, "S0", torch.float32, (B, H, P), dev)
    if out is None:
        z = torch.empty((B, H, T, d), dtype=torch.bfloat16, device=dev)
        W_T = torch.empty((B, H, P), dtype=torch.float32, device=dev)
        S_T = torch.empty((B, H, P), dtype=torch.float32, device=dev)
    else:
        z, W_T, S_T = out
        for t, nm, shp, dt in ((z, "z", (B, H, T, d), torch.bfloat16), (W_T, "W_T", (B, H, P), torch.float32),
                               (S_T, "S_T", (B, H, P), torch.float32)):
            if t is not None and (not t.is_contiguous() or t.dtype != dt or tuple(t.shape) != shp or t.device != dev):
                raise ValueError(f"out tensor {nm} must be contiguous {dt} {shp} on {dev}")
    nbytes = 0
    if work is not None:
        if work.device != dev or not work.is_contiguous():
            raise ValueError("work must be a contiguous tensor on the inputs' device")
        nbytes = work.numel() * work.element_size()
    lib = _lib.load()
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        status = lib.ttt_mem_deep_forward_bf16(
            _ptr(q), _ptr(k), _ptr(v), _ptr(theta), _ptr(eta), _ptr(alpha), _ptr(W0), _ptr(S0),
            _ptr(z), _ptr(W_T), _ptr(S_T), B, H, T, d, int(hidden), int(depth),
            int(b), _ptr(work), nbytes, stream)
    _lib.check(name, status)
    return z, W_T, S_T


def deep_status(work):
    """Synchronize torch's current stream and check the deep-memory status in ``work``."""
    lib = _lib.load()
    stream = torch.cuda.current_stream(work.device).cuda_stream
    with torch.cuda.device(work.device):
        _lib.check("ttt_mem_deep_status", lib.ttt_mem_deep_status(_ptr(work), stream))
