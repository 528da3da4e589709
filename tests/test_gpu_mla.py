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
    compare(inp, tau, g, r, po, mask=False)


@pytest.mark.parametrize("heads", [32, 64])
@pytest.mark.parametrize("threshold", [None, 0.0])
def test_mla_head_counts(heads, threshold):
    """32 heads (no dense output kernel: row ranges of the per-block kernel
    at threshold 0) and 64 heads (one 64-head set per sequence)."""
    say("case mla heads", heads, "threshold", "of the workload" if threshold is None else threshold)
    inp, tau = _case(threshold, batch=1, q_heads=heads, ctx=3000, hot=6)
    g = run_gpu(inp, tau, q_bf16=True)
    r, po = oracle_for(inp, tau)
    compare(inp, tau, g, r, po, mask=False)


@pytest.mark.parametrize("ctx", [1, 100, 3001])
@pytest.mark.parametrize("threshold", [None, 0.0])
def test_mla_ragged(ctx, threshold):
    say("case mla ragged ctx", ctx, "threshold", "of the workload" if threshold is None else threshold)
    inp, tau = _case(threshold, batch=1, ctx=ctx, hot=min(4, ctx))
    g = run_gpu(inp, tau, q_bf16=True)
    r, po = oracle_for(inp, tau)
    compare(inp, tau, g, r, po, mask=False)


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
    compare(inp, tau, g, r, po, mask=False)
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
    compare(inp, tau, g, r, po, mask=False)


@pytest.mark.parametrize("threshold", [None, 0.0])
def test_mla_full_size_sampled(threshold):
    """Full workload (batch 8, 128 heads, ctx 65536) on the GPU, with the
    workload's threshold and with every row kept (the dense output kernel,
    as timed); the oracle recomputes sequences 0 and 7 one by one."""
    say("case mla full size: batch 8, 128 heads, ctx 65536 (oracle on sequences 0 and 7), threshold",
        "1e-6" if threshold is None else threshold)
    inp, tau = _case(threshold)
    g = run_gpu(inp, tau, q_bf16=True)
    for b in (0, 7):
        sub = synth.Inputs(synth.resized(inp.w, batch=1), inp.q[b:b + 1], inp.k[b:b + 1], None,
                           [inp.hot[b]])
        r, po = oracle_for(sub, tau)
        assert np.array_equal(g["planes"]["kc"][b:b + 1], po["kc"])
        assert np.array_equal(g["planes"]["ks"][b:b + 1], po["ks"])
        gb = dict(g, out=g["out"][b:b + 1], planes={"kc": None, "ks": None, "vc": None, "vs": None})
        compare(sub, tau, gb, r, {"kc": None, "ks": None, "vc": None, "vs": None}, mask=False,
                check_stats=False)
        assert np.allclose(g["stats"]["kept_mass"][b], r.kept_mass[0], atol=1e-5)
    st = g["stats"]
    assert st["status"] == 0
    if tau > 0:
        # every sequence keeps exactly its 96 planted rows (the boost puts them far above the rest)
        assert st["rows_fetched"] == 8 * 96, st
    else:
        assert st["rows_fetched"] == 8 * 65536, st
        assert np.allclose(g["stats"]["kept_mass"], 1.0, atol=1e-5)
