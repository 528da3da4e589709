"""Pins for the oracle's encodings (CPU only).

Each test checks the oracle against something other than itself: a hand-worked
block, a textbook table, a library rounding routine, an exhaustive search, or
an invariant a wrong implementation would break (a dropped term, a wrong sign,
a transposed nibble, a wrong rounding direction).
"""
import math

import numpy as np
import pytest
import torch

from conftest import golden_path
from oracle import formats as F
from oracle import lloyd_max
from oracle import mp as MP


def _lines(name):
    return [l for l in open(golden_path(name)).read().splitlines() if l.strip() and not l.startswith("#")]


# ----------------------------------------------------------------- fp16 rounding
def _all_f16():
    bits = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    ok = np.isfinite(vals) & (bits < 0x8000)
    return bits[ok], vals[ok]


def test_f16_rounding_is_nearest_even_by_exhaustive_search():
    bits, vals = _all_f16()                # non-negative finite fp16, increasing
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.uniform(0, 70000, 20000),
        np.exp(rng.uniform(-20, 11, 20000)),
        (vals[:-1] + vals[1:]) / 2.0,     # exact ties
    ])
    got = F._f16(x)
    # brute force: nearest finite fp16, ties to even mantissa, beyond max+half-ulp -> inf
    hi = np.searchsorted(vals, x)
    hi = np.minimum(hi, len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = x - vals[lo], vals[hi] - x
    pick = np.where(dhi < dlo, hi, np.where(dlo < dhi, lo, np.where(bits[hi] % 2 == 0, hi, lo)))
    want = vals[pick].copy()
    want[x >= 65520.0] = np.inf
    assert np.array_equal(got.astype(np.float64), want)


# ----------------------------------------------------------------- q8_0
def test_q8_0_hand_worked_block():
    l = _lines("q8_0_block.txt")
    x = np.array([float(v) for v in l[0].split()], np.float32)[None]
    want = np.array([int(v) for v in l[1].split()], np.int8)
    c, s = F.pack_q8_0(x)
    assert np.array_equal(c.view(np.int8)[0], want)
    assert s.view("<u2")[0, 0] == int(l[2], 16)


def _rand_rows(rng, R, D, scale_spread=True):
    x = rng.standard_normal((R, D)).astype(np.float32)
    if scale_spread:
        x *= np.exp(rng.uniform(-6, 6, (R, 1))).astype(np.float32)
    return x


@pytest.mark.parametrize("fmt", [F.Q8_0, F.Q4_0])
def test_block_formats_roundtrip_idempotent(fmt):
    rng = np.random.default_rng(11)
    x = _rand_rows(rng, 40000, 128)
    c, s = F.pack(fmt, x)
    xr = F.unpack(fmt, c, s, 128)
    # decode is exact in fp32 (integer code times fp16 scale)
    assert np.array_equal(xr.astype(np.float32).astype(np.float64), xr)
    c2, s2 = F.pack(fmt, xr.astype(np.float32))
    assert np.array_equal(c, c2) and np.array_equal(s, s2)


def test_q8_0_error_bound_and_extreme_element():
    rng = np.random.default_rng(12)
    x = _rand_rows(rng, 20000, 128)
    c, s = F.pack_q8_0(x)
    xr = F.unpack_q8_0(c, s, 128).reshape(-1, 4, 32)
    d = s.view("<f2").astype(np.float64).reshape(-1, 4, 1)
    xb = x.astype(np.float64).reshape(-1, 4, 32)
    # rounding to the nearest code: error at most half a step (plus the tiny
    # excess from fp16-rounding the scale, which can clip the extreme element)
    err = np.abs(xr - xb)
    assert np.all(err <= 0.5 * d * (1 + 1e-12) + np.abs(xb) * 2.0 ** -10)
    # the extreme element lands on +-127
    q = c.view(np.int8).reshape(-1, 4, 32)
    idx = np.argmax(np.abs(xb), axis=2)
    assert np.all(np.abs(np.take_along_axis(q, idx[..., None], 2)) == 127)


def test_q8_0_zero_nonfinite_overflow():
    z = np.zeros((1, 64), np.float32)
    c, s = F.pack_q8_0(z)
    assert not c.any() and not s.any()
    bad = np.zeros((1, 32), np.float32)
    bad[0, 3] = np.nan
    with pytest.raises(F.NonFinite):
        F.pack_q8_0(bad)
    big = np.full((1, 32), 3e38, np.float32)
    with pytest.raises(OverflowError):
        F.pack_q8_0(big)


# ----------------------------------------------------------------- q4_0
def test_q4_0_hand_worked_block():
    l = _lines("q4_0_block.txt")
    x = np.array([float(v) for v in l[0].split()], np.float32)[None]
    want = np.array([int(v) for v in l[1].split()])
    c, s = F.pack_q4_0(x)
    got = np.empty(32, int)
    got[0::2] = c[0] & 15
    got[1::2] = c[0] >> 4
    assert np.array_equal(got, want)
    assert s.view("<u2")[0, 0] == int(l[2], 16)
    assert [int(b) for b in c[0, :4]] == [int(v, 16) for v in l[3].split()]


def test_q4_0_positive_extreme_flips_scale_sign():
    x = np.zeros((1, 32), np.float32)
    x[0, 5] = 8.0
    x[0, 6] = -3.0
    c, s = F.pack_q4_0(x)
    assert s.view("<f2")[0, 0] == -1.0
    xr = F.unpack_q4_0(c, s, 32)
    assert xr[0, 5] == 8.0 and xr[0, 6] == -3.0 and xr[0, 0] == 0.0


def test_q4_0_error_bound():
    rng = np.random.default_rng(13)
    x = _rand_rows(rng, 20000, 128)
    c, s = F.pack_q4_0(x)
    xr = F.unpack_q4_0(c, s, 128).reshape(-1, 4, 32)
    d = np.abs(s.view("<f2").astype(np.float64)).reshape(-1, 4, 1)
    xb = x.astype(np.float64).reshape(-1, 4, 32)
    t = np.divide(xb, -np.sign(s.view("<f2").astype(np.float64)).reshape(-1, 4, 1) * d,
                  out=np.zeros_like(xb), where=d != 0)
    inside = t > -7.5           # not clipped at code 15 (t measured against d = m/-8)
    err = np.abs(xr - xb)
    assert np.all(err[inside] <= (0.5 * d * (1 + 1e-12) + np.abs(xb) * 2.0 ** -10)[inside])


# ----------------------------------------------------------------- LUT3
def test_lloyd_max_matches_max_1960_table():
    l = {r.split()[0]: [float(v) for v in r.split()[1:]] for r in _lines("lloyd_max_gauss8.txt")}
    y, t, mse = lloyd_max.levels(4)
    tol = l["tolerance"][0]
    assert np.allclose(y, l["levels"], atol=tol)
    assert np.allclose(t, l["thresholds"], atol=tol)
    assert abs(mse - l["mse"][0]) < 1e-4
    # centroid and midpoint conditions hold at the fixed point
    from oracle.lloyd_max import _phi, _Phi
    edges = [0.0] + list(t) + [math.inf]
    for k in range(4):
        cm = (_phi(edges[k]) - _phi(edges[k + 1])) / (_Phi(edges[k + 1]) - _Phi(edges[k]))
        assert abs(cm - y[k]) < 1e-12


def test_lut3_levels_fp16_bits_and_mp_table_agree():
    bits = lloyd_max.lut3_magnitudes_f16().view(np.uint16)
    assert [int(b) for b in bits] == list(MP._M_BITS)
    # each level sits well away from an fp16 rounding tie
    y, _, _ = lloyd_max.levels(4)
    for v in y:
        ulp = 2.0 ** (math.floor(math.log2(v)) - 10)
        frac = (v / ulp) % 1.0
        assert abs(frac - 0.5) > 0.1      # so any accurate derivation rounds the same way


def test_lut3_nearest_level_norm_and_idempotence():
    rng = np.random.default_rng(14)
    x = _rand_rows(rng, 20000, 128)
    c, s = F.pack_lut3(x)
    mag, sign = F.lut3_fields(c)
    M, _ = F.lut3_table()
    x64 = x.astype(np.float64)
    norm = np.sqrt((x64 * x64).sum(1))
    t = np.abs(x64 * (math.sqrt(128.0) / norm)[:, None])
    best = np.argmin(np.abs(t[..., None] - M[None, None, :]), axis=2)
    assert np.array_equal(mag, best)
    assert np.array_equal(sign.astype(bool), x64 < 0)
    xr = F.unpack_lut3(c, s)
    nr = np.sqrt((xr * xr).sum(1))
    assert np.all(np.abs(nr / norm - 1) <= 2.0 ** -11 * 1.01)
    c2, s2 = F.pack_lut3(xr.astype(np.float32))
    assert np.array_equal(c, c2) and np.array_equal(s, s2)


def test_lut3_bit_layout_single_elements():
    for i in [0, 1, 2, 3, 5, 10, 21, 63, 64, 85, 127]:
        x = np.full((1, 128), 1e-3, np.float32)
        x[0, i] = -10.0
        c, s = F.pack_lut3(x)
        row = int.from_bytes(c[0].tobytes(), "little")
        # the large negative element is code 0b111 (sign + top magnitude) at bits 3i..3i+2;
        # every other (small positive) element is code 0
        assert (row >> (3 * i)) & 7 == 7
        assert row & ~(7 << (3 * i)) == 0
    z = np.zeros((1, 128), np.float32)
    c, s = F.pack_lut3(z)
    assert not c.any() and not s.any()


# ----------------------------------------------------------------- e4m3 / FP8-B128
def test_e4m3_table_against_ocp_spec_and_torch():
    for line in _lines("e4m3_ocp.txt"):
        code, val = line.split()
        got = F.e4m3_value(int(code, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = F.e4m3_decode(np.arange(256))
    same = (codes == mine) | (np.isnan(codes) & np.isnan(mine))
    assert same.all()


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(15)
    v = np.concatenate([rng.uniform(-448, 448, 50000), rng.standard_normal(50000) * 0.01,
                        np.array([F.e4m3_value(c) for c in range(0x7F)]) * 1.0,
                        (F._E4M3_MAG[:-1] + F._E4M3_MAG[1:]) / 2.0])          # exact ties
    v32 = v.astype(np.float32).astype(np.float64)       # values torch sees exactly
    want = torch.from_numpy(v32.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(v32)
    assert np.array_equal(got, want)


def test_fp8_b128_groups_roundtrip_and_extremes():
    rng = np.random.default_rng(16)
    x = _rand_rows(rng, 4000, 576)
    c, s = F.pack_fp8(x)
    assert c.shape == (4000, 576) and s.shape == (4000, 20)
    sc = s.view("<f4").astype(np.float64)
    for gi, (a0, a1) in enumerate(F.fp8_groups(576)):
        amax = np.abs(x[:, a0:a1].astype(np.float64)).max(1)
        assert np.array_equal(sc[:, gi], (amax / 448.0).astype(np.float32).astype(np.float64))
        # the extreme element of each group codes to +-448 (0x7E / 0xFE)
        idx = np.argmax(np.abs(x[:, a0:a1]), axis=1)
        assert np.all((c[np.arange(4000), a0 + idx] & 0x7F) == 0x7E)
    assert [g for g in F.fp8_groups(576)] == [(0, 128), (128, 256), (256, 384), (384, 512), (512, 576)]
    xr = F.unpack_fp8(c, s, 576)
    c2, s2 = F.pack_fp8(xr.astype(np.float32))
    assert np.array_equal(c, c2) and np.array_equal(s, s2)
    # relative error of each element at most half an e4m3 step of its group
    rel = np.abs(xr - x) / np.repeat(sc, [128, 128, 128, 128, 64], axis=1)
    assert np.all(rel <= 32.0 / 2 + 1e-9)          # coarsest step is 32 (values in [256, 448])


# ----------------------------------------------------------------- second parser
@pytest.mark.parametrize("fmt,dim", [(F.Q8_0, 128), (F.Q4_0, 128), (F.LUT3, 128), (F.FP8, 576)])
def test_unpack_agrees_with_independent_byte_parser(fmt, dim):
    rng = np.random.default_rng(17)
    x = _rand_rows(rng, 6, dim)
    c, s = F.pack(fmt, x)
    ours = F.unpack(fmt, c, s, dim)
    for r in range(6):
        ref = MP.decode_row(fmt, c[r], s[r], dim)
        assert np.array_equal(ours[r], np.array([float(v) for v in ref])) or \
            np.allclose(ours[r], np.array([float(v) for v in ref]), rtol=2e-16, atol=0)


def test_row_bytes_table():
    assert F.row_bytes(F.Q8_0, 128) == (128, 8)
    assert F.row_bytes(F.Q4_0, 128) == (64, 8)
    assert F.row_bytes(F.LUT3, 128) == (48, 2)
    assert F.row_bytes(F.FP8, 576) == (576, 20)
