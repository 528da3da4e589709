"""GPU parity on the method's own edge cases, through the C ABI:

- diffuse attention (no planted positions, unit-variance keys): every weight
  is small, so the value pass sums tens of thousands of tiny p * scale terms;
- identical keys: every weight is exactly 1/n, so a threshold 1% above 1/n
  skips every position (output exactly zero, no value row read) and one 1%
  below keeps every position (output = mean of the dequantized values);
- thresholds below the smallest normal float (the weights are compared in
  the subnormal range).

Each case prints its name before touching the GPU."""
import numpy as np
import pytest

import synth
from gpu_helpers import compare, oracle_for, run_gpu, say

pytestmark = pytest.mark.gpu

GROUPED = ["q8_0", "q4_0", "lut3", "lut3_wht"]


@pytest.mark.parametrize("threshold", [0.0, 1e-6])
@pytest.mark.parametrize("ctx", [32768, 65536])
@pytest.mark.parametrize("fmt", ["q4_0", "lut3"])
def test_diffuse_attention(fmt, ctx, threshold):
    """No hot positions, K and V ~ N(0,1): the value pass sums every (or most)
    rows with weights near 1/n, far below the fp16 normal range."""
    say("case diffuse", fmt, "ctx", ctx, "tau", threshold)
    w = synth.resized(synth.workload("long"), fmt=fmt, ctx=ctx, hot=0, seed=11)
    inp = synth.generate(w)
    g = run_gpu(inp, threshold)
    r, po = oracle_for(inp, threshold)
    compare(inp, threshold, g, r, po)


def _identical_keys(fmt, ctx, batch=1, q_heads=8, kv_heads=2, seed=12):
    w = synth.resized(synth.workload("long"), fmt=fmt, ctx=ctx, hot=0, batch=batch, q_heads=q_heads,
                      kv_heads=kv_heads, seed=seed)
    inp = synth.generate(w)
    inp.k[:] = inp.k[:, :, :1, :]                   # every position holds the same key row
    return inp


@pytest.mark.parametrize("ctx", [4097, 32768])
@pytest.mark.parametrize("fmt", GROUPED)
def test_identical_keys_all_skipped(fmt, ctx):
    """p = 1/n for every (head, position); a threshold 1% above it skips all."""
    say("case identical keys, all skipped:", fmt, "ctx", ctx)
    inp = _identical_keys(fmt, ctx)
    tau = float(np.float32(1.01 / ctx))
    g = run_gpu(inp, tau)
    r, po = oracle_for(inp, tau)
    assert r.kept_pairs == 0 and r.rows_fetched == 0
    compare(inp, tau, g, r, po)
    assert np.all(g["out"] == 0.0), "output must be exactly zero when every position is skipped"
    assert g["stats"]["rows_fetched"] == 0 and g["stats"]["kept_pairs"] == 0, g["stats"]
    assert not g["mask"].any()


@pytest.mark.parametrize("ctx", [4097, 32768])
@pytest.mark.parametrize("fmt", GROUPED)
def test_identical_keys_all_kept(fmt, ctx):
    """A threshold 1% below 1/n keeps every position: out = mean of v."""
    say("case identical keys, all kept:", fmt, "ctx", ctx)
    inp = _identical_keys(fmt, ctx)
    tau = float(np.float32(0.99 / ctx))
    g = run_gpu(inp, tau)
    r, po = oracle_for(inp, tau)
    w = inp.w
    assert r.kept_pairs == w.batch * w.q_heads * ctx
    compare(inp, tau, g, r, po)
    assert g["mask"].all()
    assert g["stats"]["rows_fetched"] == w.batch * w.kv_heads * ctx, g["stats"]
    assert g["stats"]["kept_pairs"] == w.batch * w.q_heads * ctx, g["stats"]


@pytest.mark.parametrize("threshold", [1e-40, 1e-39])
@pytest.mark.parametrize("fmt", GROUPED)
def test_threshold_below_smallest_normal(fmt, threshold):
    """Keys of standard deviation 16 spread the scaled logits over about 130
    nats, so weights reach far below 1e-40; the threshold then falls among
    subnormal float32 weights (about 6% of positions skipped)."""
    say("case subnormal threshold", threshold, fmt)
    w = synth.resized(synth.workload("long"), fmt=fmt, ctx=8192, hot=0, key_std=16.0, seed=13)
    inp = synth.generate(w)
    g = run_gpu(inp, threshold)
    r, po = oracle_for(inp, threshold)
    assert 0 < r.kept_pairs < w.batch * w.q_heads * w.ctx, r.kept_pairs
    compare(inp, threshold, g, r, po)
