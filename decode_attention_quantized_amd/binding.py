"""ctypes binding of ``libkvq.so`` with the C ABI's names (argument marshalling
only: every step of the computation runs in the library's kernels).

Device buffers are torch tensors on a ROCm device (``tensor.data_ptr()`` is a
device pointer); host buffers are numpy arrays. If the library is missing the
first call raises; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")

KVQ_Q8_0, KVQ_Q4_0, KVQ_LUT3, KVQ_FP8_B128, KVQ_LUT3_WHT = 0, 1, 2, 3, 4
KVQ_Q_F32, KVQ_Q_BF16 = 0, 1
KVQ_LAUNCH_COOPERATIVE = 1
KVQ_SKIP_RUNNING = 2
KVQ_TEST_WITHHOLD = 4
KVQ_SKIP_KEYS = 8
FMT = {"q8_0": KVQ_Q8_0, "q4_0": KVQ_Q4_0, "lut3": KVQ_LUT3, "fp8_b128": KVQ_FP8_B128, "lut3_wht": KVQ_LUT3_WHT}

ERRORS = {0: "OK", -1: "ARG", -2: "ALIGN", -3: "RANGE", -4: "NONFINITE", -5: "WORKSPACE",
          -6: "LAUNCH", -7: "UNSUPPORTED", -8: "DEVICE"}


class KvqError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        self.name = ERRORS.get(code, str(code))
        super().__init__(f"{where}: {self.name} ({code}) {kvq_strerror(code) if code in ERRORS else ''}")


class kvq_cache(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("batch", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("dim", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("block_norms", ctypes.c_void_p)]


class kvq_launch(ctypes.Structure):
    _fields_ = [("q_heads", ctypes.c_int32), ("q_dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("v_dim", ctypes.c_int32), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
                ("stream", ctypes.c_void_p), ("mask_out", ctypes.c_void_p), ("splits", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("phase_times", ctypes.c_void_p), ("key_skip_out", ctypes.c_void_p)]


class kvq_stats_t(ctypes.Structure):
    _fields_ = [("positions", ctypes.c_int64), ("pairs", ctypes.c_int64), ("kept_pairs", ctypes.c_int64),
                ("rows_fetched", ctypes.c_int64), ("k_bytes", ctypes.c_int64), ("v_bytes", ctypes.c_int64),
                ("v_bytes_dense", ctypes.c_int64), ("status", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("q_heads", ctypes.c_int32), ("live_tiles", ctypes.c_int64),
                ("launches", ctypes.c_int32), ("reserved", ctypes.c_int32), ("key_rows_skipped", ctypes.c_int64)]


EXPORTS = ["kvq_row_bytes", "kvq_pack", "kvq_unpack", "kvq_lut3_levels", "kvq_append", "kvq_append_kv",
           "kvq_workspace_bytes", "kvq_decode_attn", "kvq_decode_attn_noalloc", "kvq_stats", "kvq_phase_count",
           "kvq_strerror", "kvq_stream_read", "kvq_key_norms", "kvq_key_norms_device"]

_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree library once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with "
                              "`python -m decode_attention_quantized_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        L.kvq_row_bytes.argtypes = [i32, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.kvq_pack.argtypes = [i32, vp, i64, i32, vp, vp]
        L.kvq_unpack.argtypes = [i32, vp, vp, i64, i32, vp]
        L.kvq_lut3_levels.argtypes = [vp]
        L.kvq_append.argtypes = [i32, vp, i64, i32, vp, vp, vp, i64, vp, vp]
        L.kvq_append_kv.argtypes = [i32, vp, vp, i64, i32, vp, vp, vp, vp, vp, i64, vp, vp]
        L.kvq_workspace_bytes.argtypes = [i32, ctypes.POINTER(kvq_cache), ctypes.POINTER(kvq_launch), i32,
                                          ctypes.POINTER(i64)]
        L.kvq_decode_attn.argtypes = [vp, ctypes.POINTER(kvq_cache), ctypes.POINTER(kvq_cache), i32, i32,
                                      ctypes.c_float, vp, ctypes.POINTER(kvq_launch)]
        L.kvq_decode_attn_noalloc.argtypes = [vp, ctypes.POINTER(kvq_cache), ctypes.POINTER(kvq_cache), i32, i32,
                                              ctypes.c_float, vp, ctypes.POINTER(kvq_launch)]
        L.kvq_stats.argtypes = [ctypes.POINTER(kvq_launch), ctypes.POINTER(kvq_stats_t), vp]
        L.kvq_phase_count.argtypes = [ctypes.POINTER(kvq_launch), ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.kvq_strerror.argtypes = [i32]
        L.kvq_stream_read.argtypes = [vp, i64, i32, i32, vp, vp]
        L.kvq_key_norms.argtypes = [i32, vp, vp, i64, i32, i32, vp]
        L.kvq_key_norms_device.argtypes = [i32, vp, vp, i64, i32, i32, vp, i64, vp, vp, vp]
        L.kvq_strerror.restype = ctypes.c_char_p
        for name in EXPORTS:
            if name != "kvq_strerror":
                getattr(L, name).restype = i32
        _lib = L
    return _lib


def _check(rc: int, where: str):
    if rc != 0:
        raise KvqError(rc, where)


def _fmt(fmt) -> int:
    return FMT[fmt] if isinstance(fmt, str) else int(fmt)


def kvq_strerror(code: int) -> str:
    return lib().kvq_strerror(int(code)).decode()


def kvq_row_bytes(fmt, dim: int):
    cb, sb = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().kvq_row_bytes(_fmt(fmt), int(dim), ctypes.byref(cb), ctypes.byref(sb)), "kvq_row_bytes")
    return cb.value, sb.value


def kvq_pack(fmt, src: np.ndarray):
    """float32 [..., dim] host rows -> (codes uint8 [..., cb], scales uint8 [..., sb])."""
    src = np.ascontiguousarray(src, dtype=np.float32)
    dim = src.shape[-1]
    cb, sb = kvq_row_bytes(fmt, dim)
    n = src.size // dim
    codes = np.empty(src.shape[:-1] + (cb,), np.uint8)
    scales = np.empty(src.shape[:-1] + (sb,), np.uint8)
    _check(lib().kvq_pack(_fmt(fmt), src.ctypes.data, n, dim, codes.ctypes.data, scales.ctypes.data), "kvq_pack")
    return codes, scales


def kvq_unpack(fmt, codes: np.ndarray, scales: np.ndarray, dim: int):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    n = codes.size // codes.shape[-1]
    dst = np.empty(codes.shape[:-1] + (dim,), np.float32)
    _check(lib().kvq_unpack(_fmt(fmt), codes.ctypes.data, scales.ctypes.data, n, dim, dst.ctypes.data),
           "kvq_unpack")
    return dst


def kvq_lut3_levels():
    out = np.zeros(4, np.uint16)
    _check(lib().kvq_lut3_levels(out.ctypes.data), "kvq_lut3_levels")
    return out


def kvq_append(fmt, src, dst_rows, codes, scales, status=None, stream=None):
    """Pack device float32 rows ``src`` [n, dim] into the device planes ``codes`` /
    ``scales`` (tensors whose leading dimensions hold ``cache_rows`` rows) at the
    plane rows ``dst_rows`` (device int64 [n], or None for rows 0..n-1).
    ``status``: optional device int32 tensor that receives the skipped-row bits."""
    dim = int(src.shape[-1])
    n = src.numel() // dim if dim else 0
    cb, sb = kvq_row_bytes(fmt, dim)
    cache_rows = codes.numel() // cb
    if scales.numel() // sb != cache_rows:
        raise KvqError(-1, "kvq_append: code and scale planes hold different row counts")
    if dst_rows is not None and dst_rows.numel() != n:
        raise KvqError(-1, "kvq_append: one destination row per source row")
    _check(lib().kvq_append(_fmt(fmt), src.data_ptr(), n, dim, None if dst_rows is None else dst_rows.data_ptr(),
                            codes.data_ptr(), scales.data_ptr(), cache_rows,
                            None if status is None else status.data_ptr(), stream), "kvq_append")


def kvq_append_kv(fmt, k_src, v_src, dst_rows, k_codes, k_scales, v_codes, v_scales, status=None, stream=None):
    """kvq_append for a key and a value cache in one launch (same rows, same
    destination rows, same format and width)."""
    dim = int(k_src.shape[-1])
    n = k_src.numel() // dim if dim else 0
    if v_src.shape != k_src.shape:
        raise KvqError(-1, "kvq_append_kv: key and value rows differ in shape")
    cb, sb = kvq_row_bytes(fmt, dim)
    cache_rows = k_codes.numel() // cb
    for p, b in ((k_scales, sb), (v_codes, cb), (v_scales, sb)):
        if p.numel() // b != cache_rows:
            raise KvqError(-1, "kvq_append_kv: planes hold different row counts")
    if dst_rows is not None and dst_rows.numel() != n:
        raise KvqError(-1, "kvq_append_kv: one destination row per source row")
    _check(lib().kvq_append_kv(_fmt(fmt), k_src.data_ptr(), v_src.data_ptr(), n, dim,
                               None if dst_rows is None else dst_rows.data_ptr(), k_codes.data_ptr(),
                               k_scales.data_ptr(), v_codes.data_ptr(), v_scales.data_ptr(), cache_rows,
                               None if status is None else status.data_ptr(), stream), "kvq_append_kv")


def make_cache(codes, scales, dim: int, block_norms=None) -> kvq_cache:
    """kvq_cache for device tensors shaped [batch][heads][capacity][bytes]
    (block_norms: optional device float32 [batch][heads][ceil(capacity/64)])."""
    B, H, cap = codes.shape[:3]
    return kvq_cache(codes.data_ptr(), scales.data_ptr(), B, H, dim, cap,
                     None if block_norms is None else block_norms.data_ptr())


def kvq_key_norms(fmt, codes: np.ndarray, scales: np.ndarray, dim: int) -> np.ndarray:
    """Host block summaries of host planes [batch][heads][capacity][bytes]:
    float32 [batch][heads][ceil(capacity/64)]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    B, H, cap = codes.shape[:3]
    out = np.zeros((B, H, (cap + 63) // 64), np.float32)
    _check(lib().kvq_key_norms(_fmt(fmt), codes.ctypes.data, scales.ctypes.data, B * H, cap, dim, out.ctypes.data),
           "kvq_key_norms")
    return out


def kvq_key_norms_device(fmt, codes, scales, dim: int, norms, blocks=None, status=None, stream=None):
    """Device block summaries of device planes [batch][heads][capacity][bytes]
    into the device float32 tensor ``norms`` [batch][heads][ceil(capacity/64)]:
    every block, or the flat block ids of the device int64 tensor ``blocks``."""
    B, H, cap = codes.shape[:3]
    if norms.numel() != B * H * ((cap + 63) // 64):
        raise KvqError(-1, "kvq_key_norms_device: norms must hold one value per block")
    st = stream.cuda_stream if stream is not None else None
    _check(lib().kvq_key_norms_device(_fmt(fmt), codes.data_ptr(), scales.data_ptr(), B * H, cap, dim,
                                      None if blocks is None else blocks.data_ptr(),
                                      0 if blocks is None else blocks.numel(), norms.data_ptr(),
                                      None if status is None else status.data_ptr(), st), "kvq_key_norms_device")


def make_launch(q_heads: int, *, q_dtype=KVQ_Q_F32, softmax_scale=0.0, v_dim=0, workspace=None,
                stream=None, mask_out=None, splits=0, phase_times=None, flags=0, key_skip_out=None) -> kvq_launch:
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = stream.cuda_stream if stream is not None else None
    mo = mask_out.data_ptr() if mask_out is not None else None
    pt = phase_times.data_ptr() if phase_times is not None else None
    ko = key_skip_out.data_ptr() if key_skip_out is not None else None
    return kvq_launch(q_heads, q_dtype, float(softmax_scale), v_dim, ws_ptr, ws_bytes, st, mo, splits, flags, pt, ko)


def kvq_workspace_bytes(fmt, kcache: kvq_cache, launch: kvq_launch, ctx_len: int) -> int:
    b = ctypes.c_int64()
    _check(lib().kvq_workspace_bytes(_fmt(fmt), ctypes.byref(kcache), ctypes.byref(launch), int(ctx_len),
                                     ctypes.byref(b)), "kvq_workspace_bytes")
    return b.value


def kvq_decode_attn(q, kcache: kvq_cache, vcache, fmt, ctx_len: int, threshold: float, out,
                    launch: kvq_launch):
    """Enqueue one decode-attention call (q, out: device tensors)."""
    vptr = ctypes.byref(vcache) if vcache is not None else None
    _check(lib().kvq_decode_attn(q.data_ptr(), ctypes.byref(kcache), vptr, _fmt(fmt), int(ctx_len),
                                 float(threshold), out.data_ptr(), ctypes.byref(launch)), "kvq_decode_attn")


def kvq_decode_attn_noalloc(q, kcache: kvq_cache, vcache, fmt, ctx_len: int, threshold: float, out,
                            launch: kvq_launch):
    """kvq_decode_attn on the library's own fixed device array instead of
    launch.workspace (allocates nothing)."""
    vptr = ctypes.byref(vcache) if vcache is not None else None
    _check(lib().kvq_decode_attn_noalloc(q.data_ptr(), ctypes.byref(kcache), vptr, _fmt(fmt), int(ctx_len),
                                         float(threshold), out.data_ptr(), ctypes.byref(launch)),
           "kvq_decode_attn_noalloc")


def kvq_stats(launch: kvq_launch, kept_mass: bool = True):
    """Synchronize and return the last call's statistics as a dict."""
    s = kvq_stats_t()
    km = None
    ptr = None
    rc0 = 0
    if kept_mass:
        # size from a first header read
        rc0 = lib().kvq_stats(ctypes.byref(launch), ctypes.byref(s), None)
        km = np.zeros(max(1, s.batch * s.q_heads), np.float32)
        ptr = km.ctypes.data
    rc = lib().kvq_stats(ctypes.byref(launch), ctypes.byref(s), ptr)
    d = {f: getattr(s, f) for f, _ in kvq_stats_t._fields_}
    if kept_mass:
        d["kept_mass"] = km[: s.batch * s.q_heads].reshape(s.batch, s.q_heads)
    d["rc"] = rc if rc else rc0
    return d


def kvq_stream_read(src, grid: int, sink, stream=None, nbytes: int | None = None, threads: int = 1024):
    """Streaming-read reference: read ``nbytes`` (default: all) bytes of the
    device tensor ``src`` with ``grid`` workgroups of ``threads`` threads on
    ``stream`` (a torch.cuda.Stream, or None for the default stream); each
    workgroup XORs the 32-bit words it read into ``sink[g]`` (device int32
    tensor of at least ``grid`` elements)."""
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    if sink.numel() < grid:
        raise KvqError(-1, "kvq_stream_read: sink holds fewer words than the grid")
    st = stream.cuda_stream if stream is not None else None
    _check(lib().kvq_stream_read(src.data_ptr(), n, int(grid), int(threads), sink.data_ptr(), st),
           "kvq_stream_read")


def kvq_phase_count(launch: kvq_launch):
    """(workgroups, stamps per workgroup) of the last call on this workspace."""
    nwg, ns = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().kvq_phase_count(ctypes.byref(launch), ctypes.byref(nwg), ctypes.byref(ns)), "kvq_phase_count")
    return nwg.value, ns.value
