"""Brute-force reference for tiny contexts: an independent byte parser plus
50-digit mpmath arithmetic (test infrastructure only).

It reads the packed planes byte by byte with plain Python integers (no numpy
views, no shared helpers with ``formats``) and evaluates the same definition as
``attend`` (normalized softmax weight, keep iff p >= tau, no renormalization)
in high precision. Agreement with ``attend`` to float64 rounding pins the
oracle's decoding and its softmax against a second, differently written
implementation.
"""
from __future__ import annotations

import mpmath

mpmath.mp.dps = 50

_M_BITS = (0x33D8, 0x3A0C, 0x3D60, 0x404E)   # the LUT3 magnitudes (fp16 bit patterns)


def _half(bits: int):
    s = -1 if bits >> 15 else 1
    e = (bits >> 10) & 0x1F
    m = bits & 0x3FF
    if e == 0:
        return s * mpmath.mpf(m) * mpmath.mpf(2) ** -24
    if e == 31:
        raise ValueError("inf/nan scale")
    return s * (1 + mpmath.mpf(m) / 1024) * mpmath.mpf(2) ** (e - 15)


def _single(b4) -> mpmath.mpf:
    bits = b4[0] | (b4[1] << 8) | (b4[2] << 16) | (b4[3] << 24)
    s = -1 if bits >> 31 else 1
    e = (bits >> 23) & 0xFF
    m = bits & 0x7FFFFF
    if e == 0:
        return s * mpmath.mpf(m) * mpmath.mpf(2) ** -149
    return s * (1 + mpmath.mpf(m) / 2 ** 23) * mpmath.mpf(2) ** (e - 127)


def _e4m3(byte: int):
    s = -1 if byte & 0x80 else 1
    e = (byte >> 3) & 0xF
    m = byte & 7
    if e == 15 and m == 7:
        raise ValueError("nan code")
    if e == 0:
        return s * mpmath.mpf(m) / 512
    return s * (1 + mpmath.mpf(m) / 8) * mpmath.mpf(2) ** (e - 7)


def decode_row(fmt: str, code_bytes, scale_bytes, dim: int):
    cb = [int(x) for x in code_bytes]
    sb = [int(x) for x in scale_bytes]
    out = []
    if fmt == "q8_0":
        for i in range(dim):
            c = cb[i] - 256 if cb[i] >= 128 else cb[i]
            blk = i // 32
            out.append(c * _half(sb[2 * blk] | (sb[2 * blk + 1] << 8)))
    elif fmt == "q4_0":
        for i in range(dim):
            blk, j = divmod(i, 32)
            byte = cb[blk * 16 + j // 2]
            c = (byte >> 4) if (j & 1) else (byte & 15)
            out.append((c - 8) * _half(sb[2 * blk] | (sb[2 * blk + 1] << 8)))
    elif fmt == "lut3":
        nu = _half(sb[0] | (sb[1] << 8))
        row = 0
        for k, byte in enumerate(cb[:48]):
            row |= byte << (8 * k)                 # the row as one 384-bit integer
        for i in range(dim):
            code = (row >> (3 * i)) & 7
            val = _half(_M_BITS[code & 3])
            out.append(nu * (-val if code >> 2 else val) / mpmath.sqrt(128))
    elif fmt == "fp8_b128":
        for i in range(dim):
            gi = i // 128
            out.append(_e4m3(cb[i]) * _single(sb[4 * gi:4 * gi + 4]))
    else:
        raise ValueError(fmt)
    return out


def attend_one(q_row, k_rows, v_rows, sigma, tau):
    """One (sequence, head): lists of packed (codes, scales) rows already decoded
    by ``decode_row``. Returns (p list, keep list, out list) as mpmath numbers."""
    sig = mpmath.mpf(float(sigma))
    qv = [mpmath.mpf(float(x)) for x in q_row]
    s = [sig * mpmath.fsum(a * b for a, b in zip(qv, k)) for k in k_rows]
    m = max(s)
    e = [mpmath.exp(x - m) for x in s]
    den = mpmath.fsum(e)
    p = [x / den for x in e]
    t = mpmath.mpf(float(tau))
    keep = [x >= t for x in p]
    dv = len(v_rows[0])
    out = [mpmath.fsum(p[i] * v_rows[i][d] for i in range(len(p)) if keep[i]) for d in range(dv)]
    return p, keep, out
