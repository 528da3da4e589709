"""GPU parity for the MLA shape: H heads over one 576-wide fp8 latent per
sequence, values = the first 512 dims, bf16 queries."""
import numpy as np
import pytest

import synth
from gpu_helpers import compare, oracle_for, run_gpu, say
from oracle import attend as A
from oracle import formats as F

pytestmark = pytest.mark.gpu


def _case(threshold=None, **kw):
    w = synth.resized(synth.workload("mla"), **kw)
    return synth.generate(w), (w.threshold if threshold is None else threshold)


@pytest.mark.parametrize("threshold", [1e-6, 0.0])
def test_mla_small(threshold):
    say("case mla batch 2, 128 heads, ctx 4096 tau", threshold)
    inp, tau = _case(threshold, batch=2, ctx=4096, hot=8)
    g = run_gpu(inp, tau, q_bf16=True)
    r, po = oracle_for(inp, tau)
    compare(inp, tau, g, r, po)


@pytest.mark.parametrize("heads", [32, 64])
@pytest.mark.parametrize("threshold", [None, 0.0])
def test_mla_head_counts(heads, threshold):
    """32 heads (no dense output kernel: row ranges of the per-block kernel
    at threshold 0) and 64 heads (one 64-head set per sequence)."""
    say("case mla heads", heads, "threshold", "of the workload" if threshold is None else threshold)
    inp, tau = _case(threshold, batch=1, q_heads=heads, ctx=3000, hot=6)
    g = run_gpu(inp, tau, q_bf16=True)
    r, po = oracle_for(inp, tau)
    compare(inp, tau, g, r, po)


@pytest.mark.parametrize("ctx", [1, 100, 3001])
@pytest.mark.parametrize("threshold", [None, 0.0])
def test_mla_ragged(ctx, threshold):
    say("case mla ragged ctx", ctx, "threshold", "of the workload" if threshold is None else threshold)
    inp, tau = _case(threshold, batch=1, ctx=ctx, hot=min(4, ctx))
    g = run_gpu(inp, tau, q_bf16=True)
    r, po = oracle_for(inp, tau)
    compare(inp, tau, g, r, po)


@pytest.mark.parametrize("heads", [32, 128])
def test_mla_scattered_weights(heads):
    """No planted rows and latent rows of standard deviation 2: the scaled
    logits spread over about 25 nats, so weights fall on both sides of 1e-6
    throughout the context (many live tiles, many heads keeping different
    positions, weights near the threshold)."""
    say("case mla scattered weights, heads", heads)
    inp, tau = _case(batch=2, q_heads=heads, ctx=5000, hot=0, key_std=2.0, seed=21)
    g = run_gpu(inp, tau, q_bf16=True)
    r, po = oracle_for(inp, tau)
    frac = r.kept_pairs / r.mask.size
    say(f"  kept fraction {frac:.4f}")
    assert 0.01 < frac < 0.9
    compare(inp, tau, g, r, po)


def test_mla_dense_row_ranges():
    """Threshold 0 at ctx 20000: every row is kept, so each output block is
    summed by three workgroups over unequal row ranges and the last one to
    finish adds the partials; repeated calls must give the same bits (the
    range counters reset themselves)."""
    say("case mla dense row ranges: batch 2, 128 heads, ctx 20000, tau 0, 3 calls")
    inp, tau = _case(0.0, batch=2, ctx=20000, hot=8)
    g = run_gpu(inp, tau, q_bf16=True, repeat=3)
    for o in g["outs"][1:]:
        assert np.array_equal(o, g["outs"][0])
    r, po = oracle_for(inp, tau)
    compare(inp, tau, g, r, po)
    assert g["stats"]["rows_fetched"] == 2 * 20000


def test_mla_every_fp8_code():
    say("case mla latent rows covering every non-NaN e4m3 code")
    inp, tau = _case(batch=1, ctx=256, hot=0, threshold=0.0)
    vals = np.array([F.e4m3_value(c) for c in range(256) if (c & 0x7F) != 0x7F], np.float32)   # 254 values
    rows = inp.k[0, 0]
    # each 128-group gets +448 (so its scale is exactly 1) and then code values in order
    for r in range(3):
        for g0, g1 in F.fp8_groups(576):
            seg = np.resize(np.roll(vals, 37 * r + g0), g1 - g0).astype(np.float32)
            seg[0] = 448.0
            rows[r, g0:g1] = seg
    codes, _ = F.pack(F.FP8, rows[:3])
    assert len(set(codes.ravel().tolist())) == 254
    g = run_gpu(inp, tau, q_bf16=True)
    r, po = oracle_for(inp, tau)
    compare(inp, tau, g, r, po)


@pytest.mark.parametrize("threshold", [None, 0.0])
def test_mla_full_size(threshold):
    """Full workload (batch 8, 128 heads, ctx 65536) on the GPU, with the
    workload's threshold and with every row kept (the dense output kernel,
    as timed); the oracle recomputes every sequence, one at a time, and each
    is compared in full: packed planes, per-head keep bits outside the band,
    output, kept mass."""
    say("case mla full size: batch 8, 128 heads, ctx 65536, every sequence, threshold",
        "1e-6" if threshold is None else threshold)
    inp, tau = _case(threshold)
    g = run_gpu(inp, tau, q_bf16=True)
    kept = rows = nband = 0
    for b in range(inp.w.batch):
        sub = synth.Inputs(synth.resized(inp.w, batch=1), inp.q[b:b + 1], inp.k[b:b + 1], None,
                           [inp.hot[b]])
        r, po = oracle_for(sub, tau)
        assert np.array_equal(g["planes"]["kc"][b:b + 1], po["kc"])
        assert np.array_equal(g["planes"]["ks"][b:b + 1], po["ks"])
        gb = dict(g, out=g["out"][b:b + 1], mask=g["mask"][b:b + 1],
                  planes={"kc": None, "ks": None, "vc": None, "vs": None})
        say("  sequence", b)
        compare(sub, tau, gb, r, {"kc": None, "ks": None, "vc": None, "vs": None}, check_stats=False)
        assert np.allclose(g["stats"]["kept_mass"][b], r.kept_mass[0], atol=1e-5)
        kept += r.kept_pairs
        rows += r.rows_fetched
        nband += int(A.band(r.p, tau).sum())
        del r
    st = g["stats"]
    assert st["status"] == 0
    assert abs(st["kept_pairs"] - kept) <= nband and abs(st["rows_fetched"] - rows) <= nband, (st, kept, rows)
    if tau > 0:
        # every sequence keeps exactly its 96 planted rows (the boost puts them far above the rest)
        assert st["rows_fetched"] == 8 * 96, st
    else:
        assert st["rows_fetched"] == 8 * 65536, st
        assert np.allclose(g["stats"]["kept_mass"], 1.0, atol=1e-5)


def _identical_rows(ctx, heads=128, seed=12):
    inp, _ = _case(0.0, batch=1, q_heads=heads, ctx=ctx, hot=0, seed=seed)
    inp.k[:] = inp.k[:, :, :1, :]                   # every position holds the same latent row
    return inp


@pytest.mark.parametrize("ctx", [4097, 32768])
def test_mla_identical_rows_all_skipped(ctx):
    """Every weight is 1/n; a threshold 1% above it skips every position:
    the output is exactly zero and no row is read. (Tiles may still be
    re-scored: the live-tile test takes the largest score of a group of four
    heads, and other heads of the group score these rows higher.)"""
    say("case mla identical rows, all skipped: ctx", ctx)
    inp = _identical_rows(ctx)
    tau = float(np.float32(1.01 / ctx))
    g = run_gpu(inp, tau, q_bf16=True)
    r, po = oracle_for(inp, tau)
    assert r.kept_pairs == 0 and r.rows_fetched == 0
    compare(inp, tau, g, r, po)
    assert np.all(g["out"] == 0.0), "output must be exactly zero when every position is skipped"
    assert g["stats"]["rows_fetched"] == 0 and g["stats"]["kept_pairs"] == 0, g["stats"]
    assert g["stats"]["live_tiles"] <= (ctx + 31) // 32, g["stats"]
    assert not g["mask"].any()


@pytest.mark.parametrize("ctx", [4097, 32768])
def test_mla_identical_rows_all_kept(ctx):
    """A threshold 1% below 1/n keeps every position: out = mean of the
    dequantized value parts of the rows."""
    say("case mla identical rows, all kept: ctx", ctx)
    inp = _identical_rows(ctx)
    tau = float(np.float32(0.99 / ctx))
    g = run_gpu(inp, tau, q_bf16=True)
    r, po = oracle_for(inp, tau)
    H = inp.w.q_heads
    assert r.kept_pairs == H * ctx
    compare(inp, tau, g, r, po)
    assert g["mask"].all()
    assert g["stats"]["rows_fetched"] == ctx and g["stats"]["kept_pairs"] == H * ctx, g["stats"]


@pytest.mark.parametrize("threshold", [1e-40, 1e-39])
def test_mla_threshold_below_smallest_normal(threshold):
    """Latent rows of standard deviation 16 spread the scaled logits over
    more than a hundred nats, so the threshold falls among subnormal float32
    weights; the keep test and the weights stay exact there."""
    say("case mla subnormal threshold", threshold)
    inp, tau = _case(threshold, batch=1, q_heads=32, ctx=8192, hot=0, key_std=16.0, seed=13)
    g = run_gpu(inp, tau, q_bf16=True)
    r, po = oracle_for(inp, tau)
    assert 0 < r.kept_pairs < inp.w.q_heads * inp.w.ctx, r.kept_pairs
    assert (r.p[r.mask] < 1.17549435e-38).any(), "some kept weights must be subnormal"
    compare(inp, tau, g, r, po)
