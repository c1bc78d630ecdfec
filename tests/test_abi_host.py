"""Host-only checks of the C ABI (no GPU needed, no kernel launched)."""

import ctypes

import pytest

from test_neural_memory_amd import _lib


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_library_exports_every_declared_symbol(lib):
    names = _lib.header_symbols()
    assert {"ttt_mem_forward_f32", "ttt_mem_forward_bf16", "ttt_mem_forward_bf16_zf32", "ttt_mem_mlp_forward_bf16",
            "ttt_mem_mlp_forward_bf16_zf32", "ttt_mem_mlp_forward_bf16_noalloc", "ttt_mem_status_string",
            "ttt_mem_abi_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings(lib):
    assert lib.ttt_mem_abi_version() == (3 << 16) | 0
    assert lib.ttt_mem_abi_version() >> 16 == _lib.ABI_MAJOR
    assert lib.ttt_mem_status_string(0) == b"ok"
    for s in (-1, -2, -3, 12345):
        assert lib.ttt_mem_status_string(s)


def _call(lib, name, ptrs=None, B=1, H=1, T=8, d=16, b=4):
    p = [None] * 11 if ptrs is None else ptrs
    return getattr(lib, name)(*p, B, H, T, d, b, None)


@pytest.mark.parametrize("name", ["ttt_mem_forward_f32", "ttt_mem_forward_bf16", "ttt_mem_forward_bf16_zf32"])
def test_rejections_happen_before_any_launch(lib, name):
    # NULL required pointers, bad sizes: every one returns before touching HIP.
    assert _call(lib, name) == -1                    # NULL q, k, v, ...
    assert _call(lib, name, d=48) == -2              # unsupported head dim
    assert _call(lib, name, b=0) == -1
    assert _call(lib, name, b=65) == -2
    assert _call(lib, name, T=-1) == -1
    assert _call(lib, name, B=-2) == -1
    fake = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(11)]
    fake[0] = ctypes.c_void_p(0x1002)               # misaligned q
    assert _call(lib, name, ptrs=fake) == -1
    fake = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(11)]
    fake[8] = fake[0]                                # z aliases q
    assert _call(lib, name, ptrs=fake) == -1


@pytest.mark.parametrize("name", ["ttt_mem_forward_f32", "ttt_mem_forward_bf16", "ttt_mem_forward_bf16_zf32"])
def test_empty_batch_returns_ok_without_pointers(lib, name):
    assert _call(lib, name, B=0) == 0
    assert _call(lib, name, H=0) == 0


def test_mlp_rejections_happen_before_any_launch(lib):
    for name in ("ttt_mem_mlp_forward_bf16", "ttt_mem_mlp_forward_bf16_zf32", "ttt_mem_mlp_forward_bf16_noalloc"):
        def call(B=1, H=1, T=8, d=64, hid=256, b=4):
            return getattr(lib, name)(*([None] * 15), B, H, T, d, hid, b, None)
        assert call() == -1                 # NULL weights
        assert call(d=32) == -2
        assert call(hid=128) == -2
        assert call(b=17) == -2
        assert call(B=0) == 0


def test_ckpt_bytes(lib):
    # [B, H, ceil(T/b), M | S, d, d] float32.
    assert lib.ttt_mem_ckpt_bytes(2, 3, 130, 64, 64) == 2 * 3 * 3 * 2 * 64 * 64 * 4
    assert lib.ttt_mem_ckpt_bytes(1, 1, 0, 16, 8) == 0
    assert lib.ttt_mem_ckpt_bytes(-1, 1, 8, 16, 8) == 0
    assert lib.ttt_mem_ckpt_bytes_bf16(2, 3, 130, 64, 64) == 2 * 3 * 3 * 2 * 64 * 64 * 2


@pytest.mark.parametrize("name", ["ttt_mem_forward_ckpt_f32", "ttt_mem_forward_ckpt_bf16"])
def test_training_forward_requires_ckpt(lib, name):
    assert getattr(lib, name)(*([None] * 12), 1, 1, 8, 16, 4, None) == -1


@pytest.mark.parametrize("name", ["ttt_mem_backward_f32", "ttt_mem_backward_bf16", "ttt_mem_backward_cg_f32",
                                  "ttt_mem_backward_cg_bf16"])
def test_backward_rejections_happen_before_any_launch(lib, name):
    def call(B=1, H=1, T=8, d=16, b=4):
        return getattr(lib, name)(*([None] * 19), B, H, T, d, b, None)
    assert call() == -1                      # NULL required pointers
    assert call(d=48) == -2                  # unsupported head dim
    assert call(b=0) == -1
    assert call(b=65) == -2
    assert call(T=-1) == -1
    assert call(B=0) == 0                    # nothing to do: no pointer is touched


def test_backward_work_bytes(lib):
    # bf16 backward: the fp16 cotangent slots, then 16 floats per sequence (per
    # document and head for packed documents) at the next 256-byte boundary.
    ck = lib.ttt_mem_ckpt_bytes_bf16(2, 3, 130, 64, 64)
    assert lib.ttt_mem_backward_work_bytes_bf16(2, 3, 130, 64, 64) == (ck + 255) // 256 * 256 + 2 * 3 * 16 * 4
    ck = lib.ttt_mem_ckpt_bytes_bf16(1, 1, 5, 16, 4)
    assert lib.ttt_mem_backward_work_bytes_bf16(1, 1, 5, 16, 4) == (ck + 255) // 256 * 256 + 16 * 4
    ck = lib.ttt_mem_ckpt_bytes_varlen_bf16(3, 2, 100, 16, 8)
    assert lib.ttt_mem_backward_work_bytes_varlen_bf16(3, 2, 100, 16, 8) == (ck + 255) // 256 * 256 + 3 * 2 * 16 * 4
    assert lib.ttt_mem_backward_work_bytes_bf16(-1, 1, 8, 16, 8) == 0
    assert lib.ttt_mem_backward_work_bytes_varlen_bf16(1, 1, 8, 16, 0) == 0


def test_ckpt_bytes_varlen(lib):
    # [H, ceil(T/b) + N, M | S, d, d]: every document adds at most one partial chunk.
    assert lib.ttt_mem_ckpt_bytes_varlen(3, 2, 100, 16, 8) == 2 * (13 + 3) * 2 * 16 * 16 * 4
    assert lib.ttt_mem_ckpt_bytes_varlen_bf16(3, 2, 100, 16, 8) == 2 * (13 + 3) * 2 * 16 * 16 * 2
    assert lib.ttt_mem_ckpt_bytes_varlen(-1, 2, 100, 16, 8) == 0


@pytest.mark.parametrize("name", ["ttt_mem_forward_varlen_ckpt_f32", "ttt_mem_forward_varlen_ckpt_bf16"])
def test_varlen_training_forward_requires_ckpt(lib, name):
    # q k v theta eta alpha M0 S0 z M_T S_T ckpt cu; N H T d b; stream
    assert getattr(lib, name)(*([None] * 13), 2, 1, 8, 16, 4, None) == -1


@pytest.mark.parametrize("name", ["ttt_mem_backward_varlen_f32", "ttt_mem_backward_varlen_bf16"])
def test_varlen_backward_requires_offsets(lib, name):
    # 19 arrays, then cu_seqlens (NULL); N H T d b; stream
    assert getattr(lib, name)(*([None] * 20), 2, 1, 8, 16, 4, None) == -1


@pytest.mark.parametrize("name", ["ttt_mem_backward_varlen_f32", "ttt_mem_backward_varlen_bf16"])
def test_varlen_backward_large_document_count_is_checked_not_refused(lib, name):
    # 100000 documents of a 4M-token packed row on 32 heads: the gradient grid
    # is H * (ceil(T/b) + N) workgroups, well inside int, so the size check
    # passes and the NULL arrays are what is rejected (no array is touched:
    # the offsets pointer is a never-read stand-in).
    fake_cu = ctypes.c_void_p(1 << 20)
    assert getattr(lib, name)(*([None] * 19), fake_cu, 100000, 32, 1 << 22, 128, 64, None) == -1


def test_deep_sizes(lib):
    d, h = 64, 256
    assert lib.ttt_mem_deep_param_count(d, h, 2) == 2 * d * h
    assert lib.ttt_mem_deep_param_count(d, h, 4) == 2 * d * h + 2 * h * h
    assert lib.ttt_mem_deep_param_count(d, h, 1) == 0
    assert lib.ttt_mem_deep_work_bytes(4, 8, d, h, 2) > 0
    # Deeper memories also keep their hidden-to-hidden momenta in the workspace.
    assert lib.ttt_mem_deep_work_bytes(4, 8, d, h, 4) > lib.ttt_mem_deep_work_bytes(4, 8, d, h, 3) > 0
    assert lib.ttt_mem_deep_work_bytes(4, 8, d, h, 5) == 0
    assert lib.ttt_mem_deep_work_bytes(4, 8, 32, h, 2) == 0      # unsupported width


def test_deep_rejections_happen_before_any_launch(lib):
    # q k v theta eta alpha W0 S0 z W_T S_T; B H T d hidden depth b; work, work_bytes, stream
    def call(B=1, H=1, T=8, d=64, hid=256, depth=2, b=4):
        return lib.ttt_mem_deep_forward_bf16(*([None] * 11), B, H, T, d, hid, depth, b, None, 0, None)
    assert call() == -1                 # NULL W0
    assert call(depth=5) == -2
    assert call(d=32) == -1             # no parameters to size either way: NULL W0 first
    assert call(B=0) == -1
    assert lib.ttt_mem_deep_status(None, None) == -1
