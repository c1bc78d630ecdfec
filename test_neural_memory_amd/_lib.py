"""ctypes loader for libttt_mem.so (the HIP library built by ``build.py``).

Loading fails loudly: there is no fallback implementation anywhere in this
package.  If the library is missing, build it with
``python -m test_neural_memory_amd.build``.
"""

from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libttt_mem.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "ttt_mem.h")

_lib = None
ABI_MAJOR = 3

_P = ctypes.c_void_p
_I = ctypes.c_int
_SIGNATURES = {
    # name: (restype, argtypes) -- mirrors include/ttt_mem.h
    "ttt_mem_forward_f32": (_I, [_P] * 11 + [_I] * 5 + [_P]),
    "ttt_mem_forward_bf16": (_I, [_P] * 11 + [_I] * 5 + [_P]),
    "ttt_mem_forward_bf16_zf32": (_I, [_P] * 11 + [_I] * 5 + [_P]),
    "ttt_mem_mlp_forward_bf16": (_I, [_P] * 15 + [_I] * 6 + [_P]),
    "ttt_mem_mlp_forward_bf16_zf32": (_I, [_P] * 15 + [_I] * 6 + [_P]),
    "ttt_mem_mlp_forward_bf16_noalloc": (_I, [_P] * 15 + [_I] * 6 + [_P]),
    "ttt_mem_deep_param_count": (ctypes.c_size_t, [_I] * 3),
    "ttt_mem_deep_work_bytes": (ctypes.c_size_t, [_I] * 5),
    "ttt_mem_deep_forward_bf16": (_I, [_P] * 11 + [_I] * 7 + [_P, ctypes.c_size_t, _P]),
    "ttt_mem_deep_status": (_I, [_P, _P]),
    "ttt_mem_forward_varlen_f32": (_I, [_P] * 12 + [_I] * 5 + [_P]),
    "ttt_mem_forward_varlen_bf16": (_I, [_P] * 12 + [_I] * 5 + [_P]),
    "ttt_mem_decode_f32": (_I, [_P] * 11 + [_I] * 4 + [_P]),
    "ttt_mem_decode_bf16": (_I, [_P] * 11 + [_I] * 4 + [_P]),
    "ttt_mem_forward_ckpt_f32": (_I, [_P] * 12 + [_I] * 5 + [_P]),
    "ttt_mem_forward_ckpt_bf16": (_I, [_P] * 12 + [_I] * 5 + [_P]),
    "ttt_mem_ckpt_bytes": (ctypes.c_size_t, [_I] * 5),
    "ttt_mem_ckpt_bytes_bf16": (ctypes.c_size_t, [_I] * 5),
    "ttt_mem_backward_work_bytes_bf16": (ctypes.c_size_t, [_I] * 5),
    "ttt_mem_backward_f32": (_I, [_P] * 19 + [_I] * 5 + [_P]),
    "ttt_mem_backward_bf16": (_I, [_P] * 19 + [_I] * 5 + [_P]),
    "ttt_mem_forward_cg_f32": (_I, [_P] * 12 + [_I] * 5 + [_P]),
    "ttt_mem_forward_cg_bf16": (_I, [_P] * 12 + [_I] * 5 + [_P]),
    "ttt_mem_backward_cg_f32": (_I, [_P] * 19 + [_I] * 5 + [_P]),
    "ttt_mem_backward_cg_bf16": (_I, [_P] * 19 + [_I] * 5 + [_P]),
    "ttt_mem_ckpt_bytes_varlen": (ctypes.c_size_t, [_I] * 5),
    "ttt_mem_ckpt_bytes_varlen_bf16": (ctypes.c_size_t, [_I] * 5),
    "ttt_mem_backward_work_bytes_varlen_bf16": (ctypes.c_size_t, [_I] * 5),
    "ttt_mem_forward_varlen_ckpt_f32": (_I, [_P] * 13 + [_I] * 5 + [_P]),
    "ttt_mem_forward_varlen_ckpt_bf16": (_I, [_P] * 13 + [_I] * 5 + [_P]),
    "ttt_mem_backward_varlen_f32": (_I, [_P] * 20 + [_I] * 5 + [_P]),
    "ttt_mem_backward_varlen_bf16": (_I, [_P] * 20 + [_I] * 5 + [_P]),
    "ttt_mem_status_string": (ctypes.c_char_p, [_I]),
    "ttt_mem_abi_version": (_I, []),
}


class TTTError(RuntimeError):
    """A libttt_mem call returned a non-zero status."""

    def __init__(self, name: str, status: int, message: str):
        super().__init__(f"{name} failed with status {status}: {message}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load (once) and return the HIP library with typed entry points."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} not found: the HIP library has not been built "
            "(run `python -m test_neural_memory_amd.build`)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    abi = lib.ttt_mem_abi_version()
    if abi >> 16 != ABI_MAJOR:
        raise RuntimeError(f"libttt_mem ABI major version {abi >> 16}, expected {ABI_MAJOR}")
    _lib = lib
    return lib


def header_symbols(path: str = HEADER) -> list[str]:
    """Names of the functions that include/ttt_mem.h declares."""
    with open(path) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return sorted(set(re.findall(r"\b(ttt_mem_\w+)\s*\(", text)))


def check(name: str, status: int) -> None:
    if status != 0:
        msg = load().ttt_mem_status_string(status).decode()
        raise TTTError(name, status, msg)
