"""Pins of the oracle's Walsh-Hadamard-rotated LUT3 format (CPU only):
the butterfly network against scipy's Hadamard matrix, orthonormality, a
closed-form one-hot case, idempotence of pack/unpack, and the reconstruction
error on rows with outlier channels."""
import math

import numpy as np
import scipy.linalg

from oracle import formats as F


def test_fwht_matches_hadamard_matrix():
    H = scipy.linalg.hadamard(128).astype(np.float64)
    rng = np.random.default_rng(1)
    xi = rng.integers(-1000, 1000, (20, 128)).astype(np.float64)
    assert np.array_equal(F.fwht(xi), xi @ H.T)                # integer sums are exact either way
    x = rng.standard_normal((20, 128))
    assert np.allclose(F.fwht(x), x @ H.T, rtol=0, atol=1e-12)


def test_rotation_is_orthonormal_and_self_inverse():
    x = np.random.default_rng(2).standard_normal((50, 128)) * 3
    y = F.wht_rotate(x)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    assert np.allclose(F.wht_rotate(y), x, rtol=0, atol=1e-13)


def test_hadamard_row_packs_to_one_code():
    # x = row k of H (entries +-1): H x / sqrt(128) = sqrt(128) e_k, so after the
    # rotation element k has |t| = sqrt(128) (magnitude index 3, positive) and
    # every other element is 0 (index 0, sign bit 0)
    H = scipy.linalg.hadamard(128).astype(np.float32)
    for k in (0, 5, 127):
        codes, scales = F.pack(F.LUT3_WHT, H[k:k + 1])
        mag, sign = F.lut3_fields(codes)
        want = np.zeros(128, np.uint8)
        want[k] = 3
        assert np.array_equal(mag[0], want) and not sign.any()
        M, _ = F.lut3_table()
        nu = math.sqrt(128.0) * math.sqrt(128.0) / math.sqrt(M[3] ** 2 + 127 * M[0] ** 2)
        assert scales.view("<f2")[0, 0] == np.float16(nu)


def test_pack_unpack_pack_is_stable():
    x = np.random.default_rng(3).standard_normal((2000, 128)).astype(np.float32)
    c, s = F.pack(F.LUT3_WHT, x)
    u = F.unpack(F.LUT3_WHT, c, s, 128).astype(np.float32)
    c2, s2 = F.pack(F.LUT3_WHT, u)
    assert np.array_equal(c2, c) and np.array_equal(s2, s)


def test_rotation_lowers_error_on_outlier_channels():
    # rows with a few large channels (the case the rotation is for): the rotated
    # codebook spreads them over all elements before quantizing
    rng = np.random.default_rng(4)
    x = rng.standard_normal((4000, 128)).astype(np.float32)
    x[:, [3, 40, 99]] *= 12.0
    def err(fmt):
        c, s = F.pack(fmt, x)
        return float(np.mean((F.unpack(fmt, c, s, 128) - x) ** 2) / np.mean(x.astype(np.float64) ** 2))
    plain, rotated = err(F.LUT3), err(F.LUT3_WHT)
    assert rotated < 0.1 * plain, (plain, rotated)          # 0.030 against 0.362 here
    # on i.i.d. normal rows the two are equally good
    x = rng.standard_normal((4000, 128)).astype(np.float32)
    assert abs(err(F.LUT3_WHT) / err(F.LUT3) - 1) < 0.05
