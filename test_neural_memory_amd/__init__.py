"""MI355X-native chunked test-time-training memory (TTT / Titans neural memory).

The compute lives in ``libttt_mem.so`` (HIP for gfx950, C ABI in
``include/ttt_mem.h``); this package holds its build script, a thin torch
binding and the seeded synthetic workloads used by the tests and the bench.
"""

from .memory import (LinearMemoryFunction, backward, backward_varlen, backward_work_bytes, decode, deep_forward, deep_pack, deep_status,
                     deep_unpack, forward, forward_chunk_gates, new_deep_work,
                     forward_train, forward_varlen, linear_memory, new_ckpt_varlen,
                     ttt_mem_decode_bf16, ttt_mem_decode_f32, ttt_mem_forward_bf16, ttt_mem_forward_bf16_zf32,
                     ttt_mem_forward_f32,
                     ttt_mem_mlp_forward_bf16, ttt_mem_mlp_forward_bf16_noalloc)

__all__ = ["LinearMemoryFunction", "backward", "backward_varlen", "backward_work_bytes", "decode", "deep_forward", "deep_pack", "deep_status",
           "deep_unpack", "forward", "forward_chunk_gates", "new_deep_work",
           "forward_train", "forward_varlen", "linear_memory", "new_ckpt_varlen",
           "ttt_mem_decode_bf16", "ttt_mem_decode_f32", "ttt_mem_forward_bf16", "ttt_mem_forward_bf16_zf32",
           "ttt_mem_forward_f32",
           "ttt_mem_mlp_forward_bf16", "ttt_mem_mlp_forward_bf16_noalloc"]
