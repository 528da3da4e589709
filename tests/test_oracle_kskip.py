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


# ---------------------------------------------------------------- block summaries and the kernel's rule

def test_block_max_norms_exact_and_rounded_up():
    rows = np.zeros((70, 128))
    rows[0, :2] = (3.0, 4.0)                     # norm 5: exact in float32
    rows[5, :] = 1.0                             # norm sqrt(128): rounded up
    rows[66, 7] = -2.0                           # second block: norm 2
    r = K.block_max_norms(rows, 64)
    assert r.dtype == np.float32 and r.shape == (2,)
    s = np.sqrt(128.0)
    assert float(r[0]) >= s and float(np.nextafter(r[0], np.float32(0))) < s
    assert float(r[1]) == 2.0
    assert float(K.block_max_norms(rows[:1], 64)[0]) == 5.0


def test_cache_block_norms_bound_every_row():
    from oracle import formats as F
    rng = np.random.default_rng(7)
    for fmt in ("q8_0", "q4_0", "lut3", "lut3_wht", "fp8_b128"):
        dim = 576 if fmt == "fp8_b128" else 128
        x = (rng.standard_normal((2, 3, 150, dim)) * rng.uniform(0.1, 5.0, (2, 3, 150, 1))).astype(np.float32)
        c, s = F.pack(fmt, x)
        summ = K.cache_block_norms(fmt, c, s, dim)
        assert summ.shape == (2, 3, 3)
        rows = F.unpack(fmt, c, s, dim)
        norms = np.linalg.norm(rows, axis=-1)
        for k in range(3):
            m = norms[:, :, 64 * k:64 * k + 64].max(axis=-1)
            assert np.all(summ[:, :, k].astype(np.float64) >= m), fmt
            assert np.all(summ[:, :, k].astype(np.float64) <= m * (1 + 2.0 ** -22)), fmt


def _kskip_case(rng, n=1024, G=4, D=128, hot=(100, 700), zero_blocks=(3, 12), medium_blocks=(6,)):
    """q8_0 keys over n positions, every query of norm sqrt(D) (so
    sigma * ||q|| = 1 with sigma = 1/sqrt(D)): background rows of norm about
    0.6 * (sqrt(D) + 2.5) ~ 8.3, rows of some blocks exactly zero, rows of
    norm 16 in `medium_blocks`, and at each hot position p, rows p .. p+G-1
    of norm 3 sqrt(D) ~ 33.9 along the queries of heads 0 .. G-1 (scores
    ~ 33.9, so L ~ 34 for every head and the candidates are the hot blocks:
    16 < 33.9 / 2)."""
    from oracle import formats as F
    q = rng.standard_normal((1, G, D))
    q = (q * np.sqrt(D) / np.linalg.norm(q, axis=-1, keepdims=True)).astype(np.float32)
    k = (rng.standard_normal((1, 1, n, D)) * 0.6).astype(np.float32)
    for z in zero_blocks:
        k[0, 0, 64 * z:64 * z + 64] = 0.0
    for m in medium_blocks:
        r = rng.standard_normal((64, D))
        k[0, 0, 64 * m:64 * m + 64] = 16.0 * r / np.linalg.norm(r, axis=1, keepdims=True)
    for p in hot:
        for h in range(G):
            k[0, 0, p + h] = 3.0 * np.sqrt(D) * q[0, h] / np.linalg.norm(q[0, h])
    v = rng.standard_normal((1, 1, n, D)).astype(np.float32)
    kc, ks = F.pack("q8_0", k)
    vc, vs = F.pack("q8_0", v)
    return q, kc, ks, vc, vs


def test_kskip_without_dropping_is_the_exact_rule():
    from oracle import attend as A
    rng = np.random.default_rng(8)
    q, kc, ks, vc, vs = _kskip_case(rng)
    summ = K.cache_block_norms("q8_0", kc, ks, 128)
    kw = dict(fmt="q8_0", dim=128, v_dim=128, ctx_len=1000, sigma=1 / np.sqrt(128), threshold=1e-6)
    r, drop, _ = K.attend_kskip(q, kc, ks, vc, vs, summ, eps=0.0, **kw)
    ref = A.attend(q, kc, ks, vc, vs, **kw)
    assert not drop.any()
    assert np.array_equal(r.out64, ref.out64) and np.array_equal(r.mask, ref.mask)
    assert np.array_equal(r.kept_mass, ref.kept_mass)


def test_kskip_drops_exactly_the_constructed_blocks():
    """With L ~ 34 (hot scores) and log(1e-7 / 64) ~ -20.3, a block is dropped
    when its bound sigma ||q|| R = R is below ~ 13.7: the zero blocks (R = 0)
    and the background (R ~ 8.3) are, the medium block (R = 16) is not, and
    the hot blocks are the candidates."""
    rng = np.random.default_rng(9)
    q, kc, ks, vc, vs = _kskip_case(rng)
    summ = K.cache_block_norms("q8_0", kc, ks, 128)
    kw = dict(fmt="q8_0", dim=128, v_dim=128, ctx_len=1024, sigma=1 / np.sqrt(128), threshold=1e-6)
    r, drop, margin = K.attend_kskip(q, kc, ks, vc, vs, summ, **kw)
    want = np.ones(16, bool)
    want[[1, 10, 6]] = False
    assert np.array_equal(drop[0, 0], want)
    assert np.abs(margin[0, 0, [b for b in range(16) if b not in (1, 10)]]).min() > 1.0   # clear decisions
    # the dropped rows' exact weights are below the bound and move the output
    # by no more than their mass allows
    from oracle import attend as A
    ref = A.attend(q, kc, ks, vc, vs, **kw)
    pos = np.repeat(want, 64)
    per_block = ref.p[0][:, pos].reshape(4, -1, 64).sum(axis=2)
    assert per_block.max() <= 1e-7
    assert np.abs(r.out64 - ref.out64).max() <= 2 * per_block.sum(axis=1).max() * ref.vmax.max() + 1e-15


def test_kskip_dropped_weight_is_bounded_and_within_the_exact_lse_analysis():
    """On the tiny workload: the blocks the lower-bound rule drops are a
    subset of those the exact-LSE analysis allows, every dropped block's exact
    weight is at most 1e-7 for every head, and the result stays within the
    dropped weight of the exact rule (masks equal)."""
    import synth
    from oracle import attend as A
    from oracle import formats as F
    w = synth.workload("tiny")
    inp = synth.generate(w)
    kc, ks = F.pack(w.fmt, inp.k)
    vc, vs = F.pack(w.fmt, inp.v)
    summ = K.cache_block_norms(w.fmt, kc, ks, w.dim)
    kw = dict(fmt=w.fmt, dim=w.dim, v_dim=w.v_dim, ctx_len=w.ctx, sigma=w.sigma, threshold=w.threshold)
    r, drop, _ = K.attend_kskip(inp.q, kc, ks, vc, vs, summ, **kw)
    ref = A.attend(inp.q, kc, ks, vc, vs, **kw)
    kh = A.dequant_cache(w.fmt, kc, ks, w.dim, w.ctx)[0]
    exact = K.droppable_blocks(inp.q[0].astype(np.float64), kh[0], float(np.float32(w.sigma)), 64, "norm")
    assert drop[0, 0].sum() == 9 and np.all(exact[drop[0, 0]])      # 9 of 16 blocks (0.5625)
    pos = np.repeat(drop[0, 0], 64)
    per_block = ref.p[0][:, pos].reshape(ref.p.shape[1], -1, 64).sum(axis=2)
    assert per_block.max() <= 1e-7
    assert np.array_equal(r.mask, ref.mask)
    assert np.abs(r.out64 - ref.out64).max() <= 2 * per_block.sum(axis=1).max() * ref.vmax.max() + 1e-15


def test_kskip_candidates_follow_the_half_rule():
    """Candidates are the blocks with R >= max R / 2 and are never dropped,
    whatever their bound (here a summary that makes every bound tiny)."""
    rng = np.random.default_rng(10)
    q, kc, ks, vc, vs = _kskip_case(rng, zero_blocks=(), medium_blocks=())
    summ = np.full((1, 1, 16), 1e-3, np.float32)
    summ[0, 0, [1, 10]] = 8.0                                # the hot blocks: L ~ 34
    summ[0, 0, 5] = 4.0                                      # 8 / 2 exactly: a candidate
    summ[0, 0, 7] = np.nextafter(np.float32(4.0), np.float32(0))   # just below: not a candidate
    kw = dict(fmt="q8_0", dim=128, v_dim=128, ctx_len=1024, sigma=1 / np.sqrt(128), threshold=1e-6)
    _, drop, _ = K.attend_kskip(q, kc, ks, vc, vs, summ, **kw)
    assert not drop[0, 0, [1, 10, 5]].any()
    assert drop[0, 0, 7] and drop[0, 0].sum() == 13
