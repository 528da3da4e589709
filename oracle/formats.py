"""Bit-exact KV-cache encodings, written out step by step in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[SV] "Почему это работает для любой квантизации" names the cache formats the
skip rule was validated on: q8_0 (8 bit), q4_0 (4 bit, plain scaling) and turbo3
(a LUT codebook with a per-vector norm). "14 попыток, которые провалились" says
turbo3's dequant is a LUT read plus index extraction, sign application and a
multiply by the norm. [MLA] gives the fp8 latent with BlockWise1x128 scaling.
The pages fix no byte layout and no rounding rule; the readings taken here are
listed in the design notes and restated per function below.

A packed cache is two byte planes, both in row order [batch][head][position]:
a *code plane* with a fixed number of bytes per row and a *scale plane* with a
fixed number of bytes per row. All multi-byte values are little-endian.

Arithmetic: inputs are float32, widened exactly to float64. Every narrowing
(to fp16, fp32 or e4m3) is a single round-to-nearest-even of the float64 value.
Half-way cases of integer code rounding are decided exactly (the fractional
part of a float64 is computed exactly).
"""
from __future__ import annotations

import math

import numpy as np

from . import lloyd_max

Q8_0 = "q8_0"
Q4_0 = "q4_0"
LUT3 = "lut3"
FP8 = "fp8_b128"
LUT3_WHT = "lut3_wht"
FORMATS = (Q8_0, Q4_0, LUT3, FP8, LUT3_WHT)

BLOCK = 32          # q8_0 / q4_0 block length
FP8_GROUP = 128     # fp8 scale group length (the last group may be shorter)
E4M3_MAX = 448.0


class NonFinite(ValueError):
    pass


def row_bytes(fmt: str, dim: int) -> tuple[int, int]:
    """(code bytes, scale bytes) of one row of ``dim`` elements."""
    if fmt == Q8_0:
        _need(dim % BLOCK == 0, "q8_0 needs dim % 32 == 0")
        return dim, 2 * (dim // BLOCK)
    if fmt == Q4_0:
        _need(dim % BLOCK == 0, "q4_0 needs dim % 32 == 0")
        return dim // 2, 2 * (dim // BLOCK)
    if fmt in (LUT3, LUT3_WHT):
        _need(dim == 128, "lut3 rows are 128 wide")
        return 48, 2
    if fmt == FP8:
        return dim, 4 * (-(-dim // FP8_GROUP))
    raise ValueError(fmt)


def _need(c, msg):
    if not c:
        raise ValueError(msg)


def _check_finite(x64):
    if not np.all(np.isfinite(x64)):
        raise NonFinite("non-finite input")


def _f16(x64):
    """float64 -> float16, one round-to-nearest-even (overflow gives inf)."""
    with np.errstate(over="ignore"):
        return np.asarray(x64, dtype=np.float64).astype(np.float16)


def _round_half_away(t):
    """Nearest integer, halves away from zero; exact for any float64."""
    a = np.abs(t)
    f = np.floor(a)
    r = f + ((a - f) >= 0.5)
    return np.copysign(r, t)


def _round_half_up(t):
    """Nearest integer, halves towards +infinity (i.e. floor(t + 1/2)); exact."""
    f = np.floor(t)
    return f + ((t - f) >= 0.5)


# --------------------------------------------------------------------------- q8_0
def pack_q8_0(x: np.ndarray):
    """q8_0: per block of 32, d = fp16(max|x| / 127); code = round(x / d), halves
    away from zero, clamped to [-127, 127]; a zero scale gives zero codes.

    Row = D int8 codes in element order, then D/32 fp16 scales (block order).
    """
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    _check_finite(x64)
    R, D = x64.shape
    row_bytes(Q8_0, D)
    xb = x64.reshape(R, D // BLOCK, BLOCK)
    amax = np.max(np.abs(xb), axis=2)
    d16 = _f16(amax / 127.0)
    if np.isinf(d16).any():
        raise OverflowError("q8_0 scale overflows fp16")
    d = d16.astype(np.float64)[..., None]
    t = np.divide(xb, d, out=np.zeros_like(xb), where=(d != 0))
    q = np.clip(_round_half_away(t), -127, 127).astype(np.int8)
    codes = q.reshape(R, D).view(np.uint8).copy()
    scales = d16.astype("<f2").view(np.uint8).reshape(R, -1).copy()
    return codes, scales


def unpack_q8_0(codes, scales, dim):
    R = codes.shape[0]
    q = codes.view(np.int8).astype(np.float64).reshape(R, dim // BLOCK, BLOCK)
    d = scales.view("<f2").astype(np.float64).reshape(R, dim // BLOCK, 1)
    return (q * d).reshape(R, dim)


# --------------------------------------------------------------------------- q4_0
def pack_q4_0(x: np.ndarray):
    """q4_0: per block of 32, m = the element of largest magnitude (first on
    ties, sign kept), d = fp16(m / -8); code c = clamp(8 + round(x / d), 0, 15)
    with halves rounded up (c = floor(x/d + 8.5)); a zero scale gives c = 8.
    Value = (c - 8) * d.

    Row = D/2 bytes (block b at bytes 16b..16b+15; byte j of a block holds
    element 2j in its low nibble and 2j+1 in its high nibble), then D/32 fp16
    scales.
    """
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    _check_finite(x64)
    R, D = x64.shape
    row_bytes(Q4_0, D)
    xb = x64.reshape(R, D // BLOCK, BLOCK)
    idx = np.argmax(np.abs(xb), axis=2)
    m = np.take_along_axis(xb, idx[..., None], axis=2)[..., 0]
    d16 = _f16(m / -8.0)
    if np.isinf(d16).any():
        raise OverflowError("q4_0 scale overflows fp16")
    d = d16.astype(np.float64)[..., None]
    t = np.divide(xb, d, out=np.zeros_like(xb), where=(d != 0))
    c = np.clip(8 + _round_half_up(t), 0, 15).astype(np.uint8)
    packed = c[..., 0::2] | (c[..., 1::2] << 4)
    codes = packed.reshape(R, D // 2).copy()
    scales = d16.astype("<f2").view(np.uint8).reshape(R, -1).copy()
    return codes, scales


def unpack_q4_0(codes, scales, dim):
    R = codes.shape[0]
    b = codes.reshape(R, dim // BLOCK, BLOCK // 2)
    c = np.empty((R, dim // BLOCK, BLOCK), dtype=np.float64)
    c[..., 0::2] = (b & 0x0F)
    c[..., 1::2] = (b >> 4)
    d = scales.view("<f2").astype(np.float64).reshape(R, dim // BLOCK, 1)
    return ((c - 8.0) * d).reshape(R, dim)


# --------------------------------------------------------------------------- LUT3
def lut3_table():
    """(M, thresholds): the four fp16 magnitudes (as float64) and the three
    decision points halfway between adjacent magnitudes."""
    M = lloyd_max.lut3_magnitudes_f16().astype(np.float64)
    thr = (M[:-1] + M[1:]) / 2.0
    return M, thr


def pack_lut3(x: np.ndarray):
    """LUT3 of float32 rows (see _pack_lut3_f64)."""
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    _check_finite(x64)
    return _pack_lut3_f64(x64)


def _pack_lut3_f64(x64: np.ndarray):
    """LUT3: a 128-wide row becomes 128 three-bit codes (top bit = sign, low two
    bits = magnitude index into M) and one fp16 scalar nu.

    Steps (float64): ss = sum of x_i^2 in element order; norm = sqrt(ss);
    r = sqrt(128) / norm; t_i = x_i * r; sign_i = (x_i < 0); magnitude index =
    number of decision points strictly below |t_i| (exact ties go to the smaller
    magnitude); nu = fp16(norm * sqrt(128) / sqrt(sum_i M[m_i]^2)), which keeps
    the decoded row's norm equal to the input's up to the fp16 rounding of nu.
    A zero row gives zero codes and nu = 0. Value = nu * (-1)^sign * M[m] / sqrt(128).

    Row = 48 B: the 128 codes as one little-endian 384-bit string, element i at
    bits 3i..3i+2 (code = sign << 2 | magnitude index); scale plane = nu.
    """
    R, D = x64.shape
    row_bytes(LUT3, D)
    M, thr = lut3_table()
    ss = np.zeros(R, dtype=np.float64)
    for i in range(D):                       # sequential sum in element order
        ss = ss + x64[:, i] * x64[:, i]
    norm = np.sqrt(ss)
    nz = norm > 0
    r = np.zeros(R, dtype=np.float64)
    r[nz] = math.sqrt(128.0) / norm[nz]
    t = x64 * r[:, None]
    a = np.abs(t)
    mag = ((a > thr[0]).astype(np.uint8) + (a > thr[1]) + (a > thr[2])).astype(np.uint8)
    sign = (x64 < 0).astype(np.uint8)
    mag[~nz] = 0
    sign[~nz] = 0
    lsq = np.zeros(R, dtype=np.float64)
    for i in range(D):
        lsq = lsq + M[mag[:, i]] * M[mag[:, i]]
    nu64 = np.zeros(R, dtype=np.float64)
    nu64[nz] = (norm[nz] * math.sqrt(128.0)) / np.sqrt(lsq[nz])
    nu16 = _f16(nu64)
    if np.isinf(nu16).any():
        raise OverflowError("lut3 norm overflows fp16")
    code = (sign << 2) | mag                                     # [R][128], 3 bits each
    # bit 3i+k of the row is bit k of code i: unpack to bits, then pack 8 per byte
    bits = ((code[:, :, None] >> np.arange(3, dtype=np.uint8)) & 1).reshape(R, 384)
    codes = np.packbits(bits, axis=1, bitorder="little")
    scales = nu16.astype("<f2").view(np.uint8).reshape(R, 2).copy()
    return codes, scales


def lut3_fields(codes):
    """Split a LUT3 code plane into per-element (magnitude index, sign bit)."""
    R = codes.shape[0]
    bits = np.unpackbits(codes[:, :48], axis=1, bitorder="little").reshape(R, 128, 3)
    code = bits[..., 0] | (bits[..., 1] << 1) | (bits[..., 2] << 2)
    return (code & 3).astype(np.uint8), (code >> 2).astype(np.uint8)


def unpack_lut3(codes, scales, dim=128):
    M, _ = lut3_table()
    mag, sign = lut3_fields(codes)
    nu = scales.view("<f2").astype(np.float64).reshape(-1, 1)
    val = np.where(sign == 1, -M[mag], M[mag])
    return (nu * val) / math.sqrt(128.0)


# --------------------------------------------------------------------------- LUT3 with a Walsh-Hadamard rotation
# [SV] "Почему это работает для любой квантизации": turbo3 rotates the row with
# a Walsh-Hadamard transform before its codebook quantization (the page names
# it as the reason turbo3's dequantization is the most expensive). Reading
# taken here: the orthonormal transform y = H x / sqrt(128) with H the 128x128
# Sylvester Hadamard matrix (H[i][j] = (-1)^popcount(i & j)), applied in
# float64 as the butterfly network below, then LUT3 of y. The transform is its
# own inverse, so a decoded row is H LUT3^-1(codes) / sqrt(128).

WHT_SCALE = float("0.08838834764831844055010554526310613")   # the float64 nearest 1/sqrt(128)


def fwht(x64: np.ndarray) -> np.ndarray:
    """H x along the last axis (length 128), as butterflies in a fixed order:
    for h = 1, 2, 4, ..., 64 and every pair (j, j + h) with j mod 2h < h,
    (a, b) -> (a + b, a - b), each a single float64 addition."""
    y = np.array(x64, dtype=np.float64, copy=True)
    n = y.shape[-1]
    h = 1
    while h < n:
        v = y.reshape(y.shape[:-1] + (n // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        h *= 2
    return y


def wht_rotate(x64: np.ndarray) -> np.ndarray:
    """y = H x / sqrt(128): the butterflies, then one multiply by WHT_SCALE."""
    return fwht(x64) * WHT_SCALE


def pack_lut3_wht(x: np.ndarray):
    """LUT3 of the rotated float32 rows (the rotated row stays float64)."""
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    _check_finite(x64)
    _need(x64.shape[1] == 128, "lut3 rows are 128 wide")
    return _pack_lut3_f64(wht_rotate(x64))


def unpack_lut3_wht(codes, scales, dim=128):
    return wht_rotate(unpack_lut3(codes, scales, dim))


# --------------------------------------------------------------------------- e4m3
def e4m3_value(code: int) -> float:
    """Value of an OCP FP8 E4M3 (e4m3fn) byte; 0x7F and 0xFF are NaN."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0xF and m == 7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3_MAG = np.array([e4m3_value(c) for c in range(0x7F)], dtype=np.float64)   # codes 0..0x7E


def e4m3_encode(t):
    """Round float64 values in [-448, 448] to the nearest e4m3 code, ties to the
    even code (the code with a zero mantissa LSB); the sign bit is the input's."""
    t = np.asarray(t, dtype=np.float64)
    a = np.abs(t)
    if np.any(a > E4M3_MAX):
        raise ValueError("e4m3 input out of range")
    hi = np.searchsorted(_E4M3_MAG, a, side="left")          # first magnitude >= a
    hi = np.minimum(hi, len(_E4M3_MAG) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _E4M3_MAG[lo]
    dhi = _E4M3_MAG[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _E4M3_MAG[hi], hi, code)
    return (code | (np.signbit(t).astype(np.int64) << 7)).astype(np.uint8)


def e4m3_decode(codes):
    table = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


# --------------------------------------------------------------------------- FP8-B128
def fp8_groups(dim):
    return [(g0, min(g0 + FP8_GROUP, dim)) for g0 in range(0, dim, FP8_GROUP)]


def pack_fp8(x: np.ndarray):
    """FP8-B128: per group of 128 elements along the row (the last group may be
    shorter, e.g. the 64-wide rope tail of a 576-wide latent), s = fp32(max|x| /
    448); code = e4m3(clamp(x / s, -448, 448)) with round-to-nearest-even; a zero
    scale gives zero codes. Value = e4m3 value * s.

    Row = D e4m3 bytes in element order; scale plane = one fp32 per group.
    """
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    _check_finite(x64)
    R, D = x64.shape
    groups = fp8_groups(D)
    codes = np.zeros((R, D), dtype=np.uint8)
    sc = np.zeros((R, len(groups)), dtype=np.float32)
    for gi, (a0, a1) in enumerate(groups):
        xg = x64[:, a0:a1]
        amax = np.max(np.abs(xg), axis=1)
        s32 = (amax / E4M3_MAX).astype(np.float32)
        s = s32.astype(np.float64)[:, None]
        t = np.divide(xg, s, out=np.zeros_like(xg), where=(s != 0))
        t = np.clip(t, -E4M3_MAX, E4M3_MAX)
        codes[:, a0:a1] = e4m3_encode(t)
        sc[:, gi] = s32
    scales = sc.astype("<f4").view(np.uint8).reshape(R, -1).copy()
    return codes, scales


def unpack_fp8(codes, scales, dim):
    R = codes.shape[0]
    vals = e4m3_decode(codes[:, :dim])
    s = scales.view("<f4").astype(np.float64).reshape(R, -1)
    out = np.empty((R, dim), dtype=np.float64)
    for gi, (a0, a1) in enumerate(fp8_groups(dim)):
        out[:, a0:a1] = vals[:, a0:a1] * s[:, gi:gi + 1]
    return out


# --------------------------------------------------------------------------- dispatch
def pack(fmt: str, x: np.ndarray):
    """Pack float32 rows [R][D] -> (codes uint8 [R][cb], scales uint8 [R][sb])."""
    x = np.asarray(x)
    shape = x.shape
    x2 = x.reshape(-1, shape[-1])
    fn = {Q8_0: pack_q8_0, Q4_0: pack_q4_0, LUT3: pack_lut3, FP8: pack_fp8, LUT3_WHT: pack_lut3_wht}[fmt]
    c, s = fn(x2)
    return c.reshape(shape[:-1] + (c.shape[-1],)), s.reshape(shape[:-1] + (s.shape[-1],))


def unpack(fmt: str, codes, scales, dim: int):
    """Decode packed rows to float64 [..][dim]."""
    lead = codes.shape[:-1]
    c2 = np.ascontiguousarray(codes).reshape(-1, codes.shape[-1])
    s2 = np.ascontiguousarray(scales).reshape(-1, scales.shape[-1])
    fn = {Q8_0: unpack_q8_0, Q4_0: unpack_q4_0, LUT3: unpack_lut3, FP8: unpack_fp8, LUT3_WHT: unpack_lut3_wht}[fmt]
    return fn(c2, s2, dim).reshape(lead + (dim,))
