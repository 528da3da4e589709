"""Pins of the K-side skipping analysis (CPU only): both score bounds hold on
random blocks, each is exact in the case it is built for, and leaving out
the blocks they mark changes the attention output by no more than the
dropped weight allows."""
import numpy as np

from oracle import kskip as K


def _scores_max(q, k, sigma, block):
    s = sigma * (q @ k.T)
    nb = -(-k.shape[0] // block)
    return np.stack([s[:, j * block:(j + 1) * block].max(axis=1) for j in range(nb)], axis=1)


def test_bounds_hold_on_random_blocks():
    rng = np.random.default_rng(1)
    for n, block in ((1000, 64), (257, 16), (64, 64)):
        q = rng.standard_normal((8, 96))
        k = rng.standard_normal((n, 96)) * rng.uniform(0.2, 3.0, (n, 1)) + rng.standard_normal(96)
        exact = _scores_max(q, k, 0.1, block)
        for kind in ("norm", "centroid"):
            ub = K.block_bounds(q, k, 0.1, block, kind)
            assert np.all(ub >= exact - 1e-12), kind


def test_bounds_are_tight_where_built_to_be():
    rng = np.random.default_rng(2)
    c = rng.standard_normal(64)
    q = rng.standard_normal((3, 64))
    # a block of identical rows: radius 0, the centroid bound is the score itself
    k = np.tile(c, (32, 1))
    assert np.allclose(K.block_bounds(q, k, 0.5, 32, "centroid")[:, 0], 0.5 * q @ c, rtol=0, atol=1e-12)
    # a query parallel to the longest row: Cauchy-Schwarz holds with equality
    k = rng.standard_normal((32, 64))
    i = np.argmax(np.linalg.norm(k, axis=1))
    qp = 2.5 * k[i][None, :]
    assert np.isclose(K.block_bounds(qp, k, 0.5, 32, "norm")[0, 0], 0.5 * qp[0] @ k[i], rtol=1e-12)


def test_dropping_marked_blocks_keeps_the_result():
    # keys: background rows plus a few rows aligned with the queries, strong
    # enough that blocks of background can be proven negligible
    rng = np.random.default_rng(3)
    n, D, block = 4096, 128, 64
    q = rng.standard_normal((4, D))
    k = rng.standard_normal((n, D)) * 0.5
    hot = rng.choice(n, 6, replace=False)
    k[hot] += 80.0 * q.mean(axis=0) / np.linalg.norm(q.mean(axis=0))
    v = rng.standard_normal((n, D))
    sigma = 1 / np.sqrt(D)
    for kind in ("norm", "centroid"):
        drop = K.droppable_blocks(q, k, sigma, block, kind)
        assert drop.any() and not drop.all(), kind
        keep_rows = np.repeat(~drop, block)[:n]
        s = sigma * (q @ k.T)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        full = (p / p.sum(axis=1, keepdims=True)) @ v
        ps = p * keep_rows
        part = (ps / ps.sum(axis=1, keepdims=True)) @ v
        dropped_mass = (p * ~keep_rows).sum(axis=1) / p.sum(axis=1)
        assert dropped_mass.max() <= 1e-7 * drop.sum()
        # the rows left out move the output by at most twice their mass times max|v|
        assert np.abs(part - full).max() <= 2 * dropped_mass.max() * np.abs(v).max() + 1e-15


def test_iid_keys_leave_nothing_to_drop():
    # the long-context shape: i.i.d. keys and a few positions 20 logits up;
    # no block of background keys can be bounded that far below the LSE
    rng = np.random.default_rng(4)
    n, D = 8192, 128
    q = rng.standard_normal((8, D))
    k = rng.standard_normal((n, D))
    sigma = 1 / np.sqrt(D)
    hot = rng.choice(n, 8, replace=False)
    k[hot] += (20.0 / sigma) * q.mean(axis=0) / (np.linalg.norm(q.mean(axis=0)) ** 2)
    assert K.dropped_fraction(q, k[None], sigma, 64, "norm") == 0.0
    assert K.dropped_fraction(q, k[None], sigma, 64, "centroid") == 0.0
