"""The C ABI library (CPU only, no compute): it loads, exports every function
include/kvq.h declares, and rejects bad arguments with the documented codes
before touching a device."""
import ctypes
import os
import re

import pytest

import decode_attention_quantized_amd as kvq
from decode_attention_quantized_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kvq_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert "kvq_decode_attn" in names and "kvq_pack" in names and "kvq_stats" in names
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/kvq.h but not exported"
    assert set(names) == set(B.EXPORTS), "binding and header disagree"


def test_strerror_covers_codes():
    for code in range(0, -9, -1):
        assert kvq.kvq_strerror(code) != "unknown error"
    assert kvq.kvq_strerror(-99) == "unknown error"


def _cache(batch=1, heads=1, dim=128, cap=1024):
    # fake but aligned device addresses: validation must fail before any use
    return B.kvq_cache(0x10000, 0x20000, batch, heads, dim, cap)


def _call(q=0x30000, k=None, v="same", fmt=B.KVQ_Q4_0, ctx=100, tau=1e-6, out=0x40000, launch=None):
    L = B.lib()
    k = _cache() if k is None else k
    v = _cache() if v == "same" else v
    launch = B.kvq_launch(4, 0, 0.0, 0, 0x50000, 1 << 30, None, None, 0, 0, None) if launch is None else launch
    return L.kvq_decode_attn(q, ctypes.byref(k), ctypes.byref(v) if v is not None else None, fmt, ctx,
                             ctypes.c_float(tau), out, ctypes.byref(launch))


def test_decode_argument_validation_without_gpu():
    assert _call(q=None) == -1                                   # ARG
    assert _call(out=None) == -1
    assert _call(tau=float("nan")) == -3                         # RANGE
    assert _call(tau=-0.1) == -3
    assert _call(tau=1.0) == -3
    assert _call(ctx=0) == -3
    assert _call(ctx=1025) == -3
    assert _call(fmt=7) == -1
    bad = B.kvq_launch(3, 0, 0.0, 0, 0x50000, 1 << 30, None, None, 0, 0, None)   # 3 % 1 ok, use heads=2
    assert _call(k=_cache(heads=2), v=_cache(heads=2), launch=bad) == -1        # q_heads % kv heads
    badflags = B.kvq_launch(4, 0, 0.0, 0, 0x50000, 1 << 30, None, None, 0, 16, None)
    assert _call(launch=badflags) == -1
    assert _call(k=_cache(dim=64), v=_cache(dim=64)) == -7       # UNSUPPORTED head dim
    g16 = B.kvq_launch(16, 0, 0.0, 0, 0x50000, 1 << 30, None, None, 0, 0, None)
    assert _call(launch=g16) == -7                               # group size 16 not built


def test_workspace_query_validation():
    L = B.lib()
    b = ctypes.c_int64()
    launch = B.kvq_launch(4, 0, 0.0, 0, None, 0, None, None, 0, 0, None)
    assert L.kvq_workspace_bytes(B.KVQ_Q4_0, ctypes.byref(_cache()), ctypes.byref(launch), 0, ctypes.byref(b)) == -3
    assert L.kvq_workspace_bytes(B.KVQ_Q4_0, ctypes.byref(_cache()), ctypes.byref(launch), 10, None) == -1


def test_append_argument_validation_without_gpu():
    L = B.lib()
    src, dst, c, s = 0x10000, 0x20000, 0x30000, 0x40000   # fake aligned addresses: never dereferenced
    assert L.kvq_append(9, src, 4, 128, dst, c, s, 16, None, None) == -1          # bad fmt
    assert L.kvq_append(B.KVQ_Q4_0, src, 4, 100, dst, c, s, 16, None, None) == -7  # dim % 32
    assert L.kvq_append(B.KVQ_LUT3, src, 4, 64, dst, c, s, 16, None, None) == -7   # lut3 is 128 wide
    assert L.kvq_append(B.KVQ_Q8_0, src, -1, 128, dst, c, s, 16, None, None) == -1
    assert L.kvq_append(B.KVQ_Q8_0, src, 4, 128, dst, c, s, -1, None, None) == -1
    assert L.kvq_append(B.KVQ_Q8_0, src, 0, 128, dst, c, s, 16, None, None) == 0   # nothing to do
    assert L.kvq_append(B.KVQ_Q8_0, None, 4, 128, dst, c, s, 16, None, None) == -1
    assert L.kvq_append(B.KVQ_Q8_0, src, 4, 128, dst, None, s, 16, None, None) == -1
    assert L.kvq_append(B.KVQ_Q8_0, src, 4, 128, dst, c, None, 16, None, None) == -1
    assert L.kvq_append(B.KVQ_Q8_0, src + 2, 4, 128, dst, c, s, 16, None, None) == -2   # ALIGN
    assert L.kvq_append(B.KVQ_Q8_0, src, 4, 128, dst + 4, c, s, 16, None, None) == -2
    assert L.kvq_append(B.KVQ_Q8_0, src, 4, 128, dst, c + 8, s, 16, None, None) == -2
    assert L.kvq_append(B.KVQ_Q8_0, src, 4, 128, dst, c, s + 8, 16, None, None) == -2
    assert L.kvq_append(B.KVQ_Q8_0, src, 17, 128, None, c, s, 16, None, None) == -3    # RANGE: n > cache rows


def test_append_kv_argument_validation_without_gpu():
    L = B.lib()
    k, v, dst = 0x10000, 0x18000, 0x20000
    kc, ks, vc, vs = 0x30000, 0x40000, 0x50000, 0x60000
    assert L.kvq_append_kv(9, k, v, 4, 128, dst, kc, ks, vc, vs, 16, None, None) == -1
    assert L.kvq_append_kv(B.KVQ_Q4_0, k, None, 4, 128, dst, kc, ks, vc, vs, 16, None, None) == -1
    assert L.kvq_append_kv(B.KVQ_Q4_0, k, v, 4, 128, dst, kc, ks, None, vs, 16, None, None) == -1
    assert L.kvq_append_kv(B.KVQ_Q4_0, k, v, 4, 128, dst, kc, ks, vc, vs + 4, 16, None, None) == -2
    assert L.kvq_append_kv(B.KVQ_Q4_0, k, v + 2, 4, 128, dst, kc, ks, vc, vs, 16, None, None) == -2
    assert L.kvq_append_kv(B.KVQ_Q4_0, k, v, 0, 128, dst, kc, ks, vc, vs, 16, None, None) == 0


def test_stream_read_argument_validation_without_gpu():
    L = B.lib()
    src, sink = 0x10000, 0x20000                           # fake aligned addresses: never dereferenced
    assert L.kvq_stream_read(None, 1024, 4, 1024, sink, None) == -1
    assert L.kvq_stream_read(src, 1024, 4, 1024, None, None) == -1
    assert L.kvq_stream_read(src, 0, 4, 1024, sink, None) == -1
    assert L.kvq_stream_read(src, 1000, 4, 1024, sink, None) == -1     # not a multiple of 16
    assert L.kvq_stream_read(src, 1024, 0, 1024, sink, None) == -1
    assert L.kvq_stream_read(src, 1024, (1 << 20) + 1, 1024, sink, None) == -1
    assert L.kvq_stream_read(src, 1024, 4, 128, sink, None) == -1      # workgroup size not built
    assert L.kvq_stream_read(0x10008, 1024, 4, 1024, sink, None) == -2  # ALIGN
