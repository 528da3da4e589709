"""GPU parity: the fused HIP path against the oracle for grouped-query caches
(q8_0, q4_0). Every case prints its name before touching the GPU."""
import numpy as np
import pytest

import synth
from gpu_helpers import MAX_ABS, MAX_REL_L2, compare, oracle_for, run_gpu, say

pytestmark = pytest.mark.gpu


def _case(name, threshold=None, **kw):
    w = synth.resized(synth.workload(name), **kw) if kw else synth.workload(name)
    return synth.generate(w), (w.threshold if threshold is None else threshold)


@pytest.mark.parametrize("threshold", [1e-6, 0.0])
def test_tiny_q8_0(threshold):
    say("case tiny q8_0 tau", threshold)
    inp, tau = _case("tiny", threshold)
    g = run_gpu(inp, tau)
    r, po = oracle_for(inp, tau)
    compare(inp, tau, g, r, po)


@pytest.mark.parametrize("threshold", [1e-6, 0.0])
def test_long_q4_0_full_size(threshold):
    say("case long q4_0 ctx 32768 tau", threshold)
    inp, tau = _case("long", threshold)
    g = run_gpu(inp, tau)
    r, po = oracle_for(inp, tau)
    compare(inp, tau, g, r, po)
    if tau > 0:
        # only the planted rows are fetched: 32 per kv head
        assert g["stats"]["rows_fetched"] == 128


def test_long_q4_0_cooperative_launch():
    say("case long q4_0 ctx 32768, cooperative launch")
    inp, tau = _case("long")
    g = run_gpu(inp, tau, cooperative=True)
    r, po = oracle_for(inp, tau)
    compare(inp, tau, g, r, po)


def test_stress_scattered_mask():
    say("case stress q4_0 ctx 32768 (about 8% kept per head)")
    inp, tau = _case("stress")
    g = run_gpu(inp, tau)
    r, po = oracle_for(inp, tau)
    compare(inp, tau, g, r, po)


@pytest.mark.parametrize("threshold", [1e-6, 0.0])
@pytest.mark.parametrize("ctx", [1, 2, 63, 65, 1000, 4097])
def test_ragged_contexts(ctx, threshold):
    say("case ragged q4_0 ctx", ctx, "tau", threshold)
    inp, tau = _case("long", threshold, ctx=ctx, hot=min(4, ctx))
    g = run_gpu(inp, tau)
    r, po = oracle_for(inp, tau)
    compare(inp, tau, g, r, po)


def test_ctx_below_capacity():
    say("case q8_0 capacity 2048, ctx 1500")
    inp, tau = _case("tiny", ctx=2048)
    g = run_gpu(inp, tau, ctx_len=1500)
    r, po = oracle_for(inp, tau, ctx_len=1500)
    compare(inp, tau, g, r, po)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_group_sizes(G):
    say("case q8_0 group size", G)
    inp, tau = _case("long", fmt="q8_0", q_heads=2 * G, kv_heads=2, ctx=3000, hot=5)
    g = run_gpu(inp, tau)
    r, po = oracle_for(inp, tau)
    compare(inp, tau, g, r, po)


@pytest.mark.parametrize("fmt", ["q4_0", "lut3"])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_group_sizes_every_row_kept(fmt, G):
    """Threshold 0 keeps every row, so waves sum their value rows on the
    matrix cores (16-row batches, the last one partial) for every group size."""
    say("case", fmt, "group size", G, "tau 0")
    inp, tau = _case("long", 0.0, fmt=fmt, q_heads=2 * G, kv_heads=2, ctx=3001, hot=5)
    g = run_gpu(inp, tau)
    r, po = oracle_for(inp, tau)
    compare(inp, tau, g, r, po)


def test_batch_and_bf16_queries():
    say("case q4_0 batch 3, bf16 q")
    import torch
    inp, tau = _case("long", batch=3, ctx=5000, hot=6)
    g = run_gpu(inp, tau, q_bf16=True)
    qb = torch.from_numpy(inp.q).to(torch.bfloat16).float().numpy()
    r, po = oracle_for(inp, tau, q_override=qb)
    compare(inp, tau, g, r, po)


@pytest.mark.parametrize("splits", [4, 7, 64])
def test_split_count_does_not_change_result(splits):
    say("case q4_0 ctx 8192 splits", splits)
    inp, tau = _case("long", ctx=8192, hot=16)
    g = run_gpu(inp, tau, splits=splits)
    r, po = oracle_for(inp, tau)
    compare(inp, tau, g, r, po)


def test_split_too_large_for_lds_is_rejected():
    say("case one split over 8192 positions (scores exceed LDS) -> UNSUPPORTED, nothing launched")
    import decode_attention_quantized_amd as kvq
    inp, tau = _case("long", ctx=8192, hot=16)
    with pytest.raises(kvq.KvqError) as e:
        run_gpu(inp, tau, splits=1)
    assert e.value.name == "UNSUPPORTED"


def test_deterministic_repeats():
    say("case determinism stress ctx 16384, 3 calls")
    inp, tau = _case("stress", ctx=16384)
    g = run_gpu(inp, tau, repeat=3)
    for o in g["outs"][1:]:
        assert np.array_equal(o, g["outs"][0])
    for m in g["masks"][1:]:
        assert np.array_equal(m, g["masks"][0])


def test_sweep_lengths():
    for n in synth.SWEEP:
        say("case sweep ctx", n)
        inp, tau = _case(f"sweep_{n}")
        g = run_gpu(inp, tau)
        r, po = oracle_for(inp, tau)
        compare(inp, tau, g, r, po)


@pytest.mark.parametrize("name", ["lut3", "lut3_wht"])
@pytest.mark.parametrize("threshold", [1e-6, 0.0])
def test_lut3_small(threshold, name):
    say("case", name, "batch 2 ctx 3000 tau", threshold)
    inp, tau = _case(name, threshold, batch=2, ctx=3000)
    g = run_gpu(inp, tau)
    r, po = oracle_for(inp, tau)
    compare(inp, tau, g, r, po)


@pytest.mark.parametrize("name", ["lut3", "lut3_wht"])
@pytest.mark.parametrize("threshold", [1e-6, 0.0])
@pytest.mark.parametrize("ctx", [1, 77, 4100])
def test_lut3_ragged(ctx, threshold, name):
    say("case", name, "ragged ctx", ctx, "tau", threshold)
    inp, tau = _case(name, threshold, batch=1, ctx=ctx)
    g = run_gpu(inp, tau)
    r, po = oracle_for(inp, tau)
    compare(inp, tau, g, r, po)


@pytest.mark.parametrize("name", ["lut3", "lut3_wht"])
@pytest.mark.parametrize("threshold", [None, 0.0])
def test_lut3_full_size(name, threshold):
    say("case", name, "batch 8, 32/4 heads, ctx 32768, 8..64 hot per sequence, threshold",
        "of the workload" if threshold is None else threshold)
    inp, tau = _case(name, threshold)
    g = run_gpu(inp, tau)
    r, po = oracle_for(inp, tau)
    compare(inp, tau, g, r, po)


@pytest.mark.parametrize("threshold", [None, 0.0])
def test_lut3_batch_over_one_launch(threshold):
    """Batch 8 x 4 kv heads at ctx 40000: 8 splits of 5056 positions per
    group would not fit their scores in LDS, so the call runs as two
    launches of 16 groups with 16 splits each."""
    say("case lut3 batch 8, 32/4 heads, ctx 40000 (two launches), threshold",
        "of the workload" if threshold is None else threshold)
    inp, tau = _case("lut3", threshold, ctx=40000)
    g = run_gpu(inp, tau)
    assert g["stats"]["launches"] == 2 and g["stats"]["splits"] == 16, g["stats"]
    r, po = oracle_for(inp, tau)
    compare(inp, tau, g, r, po)


@pytest.mark.parametrize("threshold", [1e-6, 0.0])
def test_more_groups_than_compute_units(threshold):
    """72 sequences x 4 kv heads = 288 groups, more than one workgroup per
    compute unit allows in one launch: two launches of 144 groups."""
    say("case q4_0 batch 72, 32/4 heads, ctx 1000 (two launches), tau", threshold)
    inp, tau = _case("long", threshold, batch=72, ctx=1000, hot=4)
    g = run_gpu(inp, tau)
    assert g["stats"]["launches"] == 2, g["stats"]
    r, po = oracle_for(inp, tau)
    compare(inp, tau, g, r, po)


@pytest.mark.parametrize("name,heads,threshold", [("long", None, 1e-6), ("long", None, 0.0), ("mla", 32, 0.0),
                                                  ("mla", 128, 0.0), ("mla", 64, 1e-6)])
def test_one_workspace_for_shorter_contexts(name, heads, threshold):
    """A workspace sized for ctx_len serves every shorter call, although the
    rounding of positions per split makes the plan of ctx 4096 (64 splits of
    64 positions for the long shape) larger than the plan of 4097 (33 of
    128); the calls alternate so each finds the previous one's words in
    another layout (the latent range counters must not move)."""
    import torch

    import decode_attention_quantized_amd as kvq
    from decode_attention_quantized_amd.runtime import DecodeAttention, PackedCache
    kw = dict(ctx=4097)
    if name == "mla":
        kw.update(batch=2, q_heads=heads)
    w = synth.resized(synth.workload(name), **kw)
    inp = synth.generate(w)
    say("case one workspace:", name, "heads", w.q_heads, "threshold", threshold, "contexts 4097 4096 3000 4097 64")
    kc, ks = kvq.kvq_pack(w.fmt, inp.k)
    K = PackedCache.from_host(kc, ks, w.fmt, w.dim)
    V = None
    if inp.v is not None:
        vc, vs = kvq.kvq_pack(w.fmt, inp.v)
        V = PackedCache.from_host(vc, vs, w.fmt, w.v_dim)
    latent = V is None
    att = DecodeAttention(K, V, w.q_heads, ctx_len=w.ctx, softmax_scale=w.sigma,
                          q_dtype=kvq.KVQ_Q_BF16 if latent else kvq.KVQ_Q_F32, v_dim=w.v_dim if latent else 0)
    q = torch.from_numpy(inp.q).cuda()
    if latent:
        q = q.to(torch.bfloat16)
    splits = set()
    for n in (4097, 4096, 3000, 4097, 64):
        out = att(q, n, threshold).cpu().numpy()
        st = att.stats()
        assert st["status"] == 0, (n, st)
        splits.add(st["splits"])
        r, _ = oracle_for(inp, threshold, ctx_len=n)
        err = float(np.abs(out - r.out64).max())
        rel = float(np.linalg.norm(out - r.out64) / max(np.linalg.norm(r.out64), 1e-30))
        assert err <= MAX_ABS and rel <= MAX_REL_L2, (n, err, rel)
    assert len(splits) > 1, splits
