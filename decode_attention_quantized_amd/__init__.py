"""kvq: sparse-V decode attention over a block-quantized KV cache on MI355X.

The computation runs in ``libkvq.so`` (HIP kernels for gfx950 behind a C ABI,
``include/kvq.h``); this package is its Python binding plus a small helper that
allocates device buffers with torch.
"""
from .binding import (EXPORTS, FMT, KVQ_FP8_B128, KVQ_LUT3, KVQ_Q4_0, KVQ_Q8_0, KVQ_Q_BF16, KVQ_Q_F32, KVQ_SKIP_KEYS,
                      KVQ_SKIP_RUNNING, KvqError, kvq_append, kvq_append_kv, kvq_decode_attn, kvq_key_norms,
                      kvq_key_norms_device, kvq_lut3_levels, kvq_pack, kvq_phase_count, kvq_row_bytes, kvq_stats,
                      kvq_stream_read, kvq_strerror, kvq_unpack, kvq_workspace_bytes, lib, make_cache, make_launch)
from .runtime import DecodeAttention, PackedCache

__all__ = [
    "EXPORTS", "FMT", "KVQ_Q8_0", "KVQ_Q4_0", "KVQ_LUT3", "KVQ_FP8_B128", "KVQ_Q_F32", "KVQ_Q_BF16", "KVQ_SKIP_RUNNING", "KVQ_SKIP_KEYS",
    "KvqError", "kvq_append", "kvq_append_kv", "kvq_decode_attn", "kvq_key_norms", "kvq_key_norms_device", "kvq_lut3_levels", "kvq_pack", "kvq_phase_count", "kvq_row_bytes", "kvq_stats",
    "kvq_stream_read", "kvq_strerror", "kvq_unpack", "kvq_workspace_bytes", "lib", "make_cache", "make_launch",
    "DecodeAttention", "PackedCache",
]
