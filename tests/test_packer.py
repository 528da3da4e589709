"""The library's C++ packer against the oracle's packer (CPU only): bit-exact
bytes on random rows and on edge rows, and the documented error codes."""
import zlib

import numpy as np
import pytest

import decode_attention_quantized_amd as kvq
from oracle import formats as F

FMTS = [("q8_0", 128), ("q4_0", 128), ("lut3", 128), ("fp8_b128", 576), ("q8_0", 64), ("q4_0", 256), ("lut3_wht", 128),
        ("fp8_b128", 128), ("fp8_b128", 200)]


def _random_rows(rng, n, dim):
    x = rng.standard_normal((n, dim)).astype(np.float32)
    x *= np.exp(rng.uniform(-9, 6, (n, 1))).astype(np.float32)       # scales across many binades
    return x


def _edge_rows(dim):
    rows = []
    rows.append(np.zeros(dim))                                  # zero row
    z = np.zeros(dim); z[::2] = -0.0; rows.append(z)             # signed zeros
    t = np.zeros(dim); t[0] = 127.0; t[1:] = np.arange(1, dim) % 32 - 15.5; rows.append(t)   # .5 ties
    h = np.zeros(dim); h[0] = -8.0; h[1:] = (np.arange(1, dim) % 17) - 8.5; rows.append(h)
    rows.append(np.full(dim, 1e-30))                             # subnormal fp16 scales / zero scales
    rows.append(np.full(dim, 3e-7))
    rows.append(np.full(dim, 60000.0 * 100))                     # large q8_0 scale
    rows.append(np.linspace(-448, 448, dim))
    rows.append(np.tile([1.0, -1.0], dim // 2))
    one = np.zeros(dim); one[dim // 3] = 5.0; rows.append(one)   # a single non-zero
    return np.array(rows, dtype=np.float32)


@pytest.mark.parametrize("fmt,dim", FMTS)
def test_packer_bit_exact_against_oracle(fmt, dim):
    if fmt == "lut3" and dim != 128:
        pytest.skip("lut3 rows are 128 wide")
    rng = np.random.default_rng(zlib.crc32(f"{fmt}/{dim}".encode()))
    edges = []
    for r in _edge_rows(dim):                     # drop edge rows whose scale overflows fp16 here
        try:
            F.pack(fmt, r[None])
            edges.append(r)
        except OverflowError:
            pass
    x = np.concatenate([_random_rows(rng, 30000, dim), np.array(edges, dtype=np.float32)])
    c, s = kvq.kvq_pack(fmt, x)
    co, so = F.pack(fmt, x)
    assert np.array_equal(c, co), f"{fmt}: {np.sum(np.any(c != co, axis=1))} rows differ in codes"
    assert np.array_equal(s, so), f"{fmt}: {np.sum(np.any(s != so, axis=1))} rows differ in scales"
    # the library's decoder gives the exact decoded values rounded once to float32
    u = kvq.kvq_unpack(fmt, c, s, dim)
    assert np.array_equal(u, F.unpack(fmt, co, so, dim).astype(np.float32))


def test_packer_shapes_and_row_bytes():
    for fmt, dim in FMTS:
        if fmt == "lut3" and dim != 128:
            continue
        assert kvq.kvq_row_bytes(fmt, dim) == F.row_bytes(fmt, dim)
    x = np.zeros((2, 3, 128), np.float32)
    c, s = kvq.kvq_pack("q4_0", x)
    assert c.shape == (2, 3, 64) and s.shape == (2, 3, 8)


def test_packer_errors():
    bad = np.zeros((4, 128), np.float32)
    bad[2, 5] = np.nan
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_pack("q8_0", bad)
    assert e.value.name == "NONFINITE"
    bad[2, 5] = np.inf
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_pack("lut3", bad)
    assert e.value.name == "NONFINITE"
    big = np.full((1, 128), 3e38, np.float32)
    for fmt in ("q8_0", "q4_0"):
        with pytest.raises(kvq.KvqError) as e:
            kvq.kvq_pack(fmt, big)
        assert e.value.name == "RANGE"
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_pack("lut3", np.zeros((1, 64), np.float32))
    assert e.value.name == "UNSUPPORTED"
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_row_bytes(9, 128)
    assert e.value.name == "ARG"


def test_lut3_levels_match_oracle_derivation():
    from oracle import lloyd_max
    assert np.array_equal(kvq.kvq_lut3_levels(), lloyd_max.lut3_magnitudes_f16().view(np.uint16))
