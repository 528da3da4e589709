"""GPU parity of key skipping (KVQ_SKIP_KEYS) against the oracle's rule
(oracle.kskip.attend_kskip): the dropped 64-position blocks (outside a small
margin band), masks, outputs and statistics; the device key-block summaries
against the host ones; a decode loop that appends rows on the GPU and
refreshes the summaries of the blocks it touched. Every case prints its name
before touching the GPU."""
import numpy as np
import pytest

import synth
from gpu_helpers import compare, say
from oracle import formats as F
from oracle import kskip as K

pytestmark = pytest.mark.gpu

# natural-log units: a block whose drop test is this close to its bound is
# decided by rounding (float32 scores and norms on the GPU, float64 here)
MARGIN_BAND = 1e-3


def _oracle(inp, tau, ctx_len=None):
    w = inp.w
    kc, ks = F.pack(w.fmt, inp.k)
    vc, vs = F.pack(w.fmt, inp.v)
    summ = K.cache_block_norms(w.fmt, kc, ks, w.dim)
    n = w.ctx if ctx_len is None else ctx_len
    r, drop, margin = K.attend_kskip(inp.q, kc, ks, vc, vs, summ, fmt=w.fmt, dim=w.dim, v_dim=w.v_dim, ctx_len=n,
                                     sigma=w.sigma, threshold=tau)
    return r, drop, margin, dict(kc=kc, ks=ks, vc=vc, vs=vs), summ


def _run(inp, tau, *, splits=0, ctx_len=None, device_norms=False):
    import torch

    import decode_attention_quantized_amd as kvq
    from decode_attention_quantized_amd.runtime import DecodeAttention, PackedCache, mask_words, unpack_mask
    w = inp.w
    n = w.ctx if ctx_len is None else ctx_len
    kc, ks = kvq.kvq_pack(w.fmt, inp.k)
    vc, vs = kvq.kvq_pack(w.fmt, inp.v)
    Kc = PackedCache.from_host(kc, ks, w.fmt, w.dim)
    Vc = PackedCache.from_host(vc, vs, w.fmt, w.dim)
    if device_norms:
        Kc.compute_norms()
    else:
        Kc.norms = torch.from_numpy(kvq.kvq_key_norms(w.fmt, kc, ks, w.dim)).cuda()
    att = DecodeAttention(Kc, Vc, w.q_heads, ctx_len=n, softmax_scale=w.sigma, splits=splits, skip_keys=True)
    q = torch.from_numpy(inp.q).cuda()
    mask = torch.full((w.batch, w.q_heads, mask_words(n)), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    skip = torch.full((w.batch, w.kv_heads, (n + 63) // 64), 7, dtype=torch.uint8, device="cuda")
    out = att(q, n, tau, mask_out=mask, key_skip_out=skip)
    torch.cuda.synchronize()
    st = att.stats()
    return dict(out=out.cpu().numpy(), mask=unpack_mask(mask.cpu().numpy().view(np.uint32), n), stats=st,
                planes=dict(kc=kc, ks=ks, vc=vc, vs=vs), splits=st["splits"], skip=skip.cpu().numpy(),
                norms=Kc.norms.cpu().numpy())


def _check(inp, tau, g, r, drop, margin, planes, summ, ctx_len=None):
    n = inp.w.ctx if ctx_len is None else ctx_len
    assert np.array_equal(g["norms"].view(np.uint32), summ.view(np.uint32)), "key-block summaries differ"
    assert set(np.unique(g["skip"]).tolist()) <= {0, 1}, "dropped-block map not written everywhere"
    got = g["skip"].astype(bool)
    sure = np.abs(margin) > MARGIN_BAND
    bad = (got != drop) & sure
    sizes = np.minimum(64, n - 64 * np.arange(drop.shape[-1]))
    want_rows = int((drop * sizes).sum())
    say(f"  dropped blocks {int(got.sum())} (oracle {int(drop.sum())}, band {int((~sure).sum())}), "
        f"key rows skipped {g['stats']['key_rows_skipped']} (oracle {want_rows})")
    assert not bad.any(), f"{int(bad.sum())} drop decisions differ outside the band"
    if sure.all():
        assert g["stats"]["key_rows_skipped"] == want_rows
    compare(inp, tau, g, r, planes)


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0", "lut3", "lut3_wht"])
@pytest.mark.parametrize("threshold", [1e-6, 0.0])
def test_tiny_shape(fmt, threshold):
    say("case key skipping, tiny shape", fmt, "tau", threshold)
    w = synth.resized(synth.workload("tiny"), fmt=fmt)
    inp = synth.generate(w)
    r, drop, margin, planes, summ = _oracle(inp, threshold)
    assert drop.any()
    g = _run(inp, threshold)
    _check(inp, threshold, g, r, drop, margin, planes, summ)


@pytest.mark.parametrize("splits", [0, 4])
def test_several_chunks_per_split(splits):
    """Batch 2, 16/2 heads (8 per group), ctx 8192 with 24 aligned hot keys
    per kv head; splits 4 puts 32 chunks in each split (listed passes of
    many tiles), the default plan 32 splits of 4 chunks."""
    say("case key skipping, batch 2, 16/2 heads, ctx 8192, splits", splits)
    w = synth.resized(synth.workload("tiny"), batch=2, q_heads=16, kv_heads=2, ctx=8192, hot=24)
    inp = synth.generate(w)
    r, drop, margin, planes, summ = _oracle(inp, w.threshold)
    assert drop.any()
    g = _run(inp, w.threshold, splits=splits)
    _check(inp, w.threshold, g, r, drop, margin, planes, summ)


def test_ragged_context_and_device_summaries():
    say("case key skipping, q4_0 tiny shape at ctx 1000 (capacity 1024), summaries from the device")
    w = synth.resized(synth.workload("tiny"), fmt="q4_0")
    inp = synth.generate(w)
    r, drop, margin, planes, summ = _oracle(inp, w.threshold, ctx_len=1000)
    g = _run(inp, w.threshold, ctx_len=1000, device_norms=True)
    _check(inp, w.threshold, g, r, drop, margin, planes, summ, ctx_len=1000)


def test_several_launches():
    """300 sequences of the tiny shape (one kv head each): 300 groups, more
    than one launch holds, so the call runs as two launches; key skipping
    per group is unchanged."""
    say("case key skipping over two launches: tiny shape, batch 300")
    w = synth.resized(synth.workload("tiny"), batch=300)
    inp = synth.generate(w)
    r, drop, margin, planes, summ = _oracle(inp, w.threshold)
    assert drop.any()
    g = _run(inp, w.threshold)
    assert g["stats"]["launches"] == 2, g["stats"]
    _check(inp, w.threshold, g, r, drop, margin, planes, summ)


def test_nothing_to_drop_on_the_long_shape():
    """i.i.d. keys with boosted hot positions: no block can be proven
    negligible, so the result is the exact rule's."""
    say("case key skipping, long q4_0 shape at ctx 8192 (nothing droppable)")
    w = synth.resized(synth.workload("long"), ctx=8192, hot=16)
    inp = synth.generate(w)
    r, drop, margin, planes, summ = _oracle(inp, w.threshold)
    assert not drop.any()
    g = _run(inp, w.threshold)
    assert g["stats"]["key_rows_skipped"] == 0
    _check(inp, w.threshold, g, r, drop, margin, planes, summ)


@pytest.mark.parametrize("fmt,dim", [("q8_0", 128), ("q4_0", 128), ("lut3", 128), ("lut3_wht", 128),
                                     ("fp8_b128", 576), ("q4_0", 64)])
def test_device_summaries_match_the_host(fmt, dim):
    import torch

    import decode_attention_quantized_amd as kvq
    say("case device key-block summaries", fmt, dim)
    rng = np.random.default_rng(dim)
    x = (rng.standard_normal((2, 2, 150, dim)) * rng.uniform(0.01, 20.0, (2, 2, 150, 1))).astype(np.float32)
    c, s = kvq.kvq_pack(fmt, x)
    host = kvq.kvq_key_norms(fmt, c, s, dim)
    cd, sd = torch.from_numpy(c).cuda(), torch.from_numpy(s).cuda()
    norms = torch.zeros(host.shape, dtype=torch.float32, device="cuda")
    kvq.kvq_key_norms_device(fmt, cd, sd, dim, norms)
    torch.cuda.synchronize()
    assert np.array_equal(norms.cpu().numpy().view(np.uint32), host.view(np.uint32))
    # a list of blocks: only those are written; an id out of range sets status bit 8
    part = torch.zeros(host.shape, dtype=torch.float32, device="cuda")
    ids = torch.tensor([1, 5, 11, 99], dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvq.kvq_key_norms_device(fmt, cd, sd, dim, part, blocks=ids, status=status)
    torch.cuda.synchronize()
    flat = part.cpu().numpy().reshape(-1)
    want = np.zeros_like(flat)
    want[[1, 5, 11]] = host.reshape(-1)[[1, 5, 11]]
    assert np.array_equal(flat.view(np.uint32), want.view(np.uint32))
    assert int(status.item()) == 8


def test_decode_loop_refreshes_touched_blocks():
    """Start from a cache holding 1000 positions, append four decode steps on
    the GPU (key and value rows of every kv head), refresh the summaries of
    the blocks those rows landed in, and attend with key skipping after each
    step; compare every step with the oracle over the grown context."""
    import torch

    import decode_attention_quantized_amd as kvq
    from decode_attention_quantized_amd.runtime import DecodeAttention, PackedCache, append_kv
    say("case key skipping in a decode loop: q8_0 tiny shape, ctx 1000 -> 1004, appends and refreshes on the GPU")
    w = synth.resized(synth.workload("tiny"), ctx=1024)
    inp = synth.generate(w)
    n0 = 1000
    k_host = inp.k.copy()
    k_host[:, :, n0:] = 0.0
    v_host = inp.v.copy()
    v_host[:, :, n0:] = 0.0
    kc, ks = kvq.kvq_pack(w.fmt, k_host)
    vc, vs = kvq.kvq_pack(w.fmt, v_host)
    Kc = PackedCache.from_host(kc, ks, w.fmt, w.dim)
    Vc = PackedCache.from_host(vc, vs, w.fmt, w.dim)
    Kc.compute_norms()
    att = DecodeAttention(Kc, Vc, w.q_heads, ctx_len=w.ctx, softmax_scale=w.sigma, skip_keys=True)
    q = torch.from_numpy(inp.q).cuda()
    nbc = (w.ctx + 63) // 64
    for step in range(4):
        pos = n0 + step
        rows_k = torch.from_numpy(np.ascontiguousarray(inp.k[:, :, pos])).cuda()
        rows_v = torch.from_numpy(np.ascontiguousarray(inp.v[:, :, pos])).cuda()
        append_kv(Kc, Vc, rows_k, rows_v, torch.full((w.batch,), pos, dtype=torch.int64, device="cuda"))
        ids = torch.tensor([(b * w.kv_heads + g) * nbc + pos // 64 for b in range(w.batch)
                            for g in range(w.kv_heads)], dtype=torch.int64, device="cuda")
        kvq.kvq_key_norms_device(w.fmt, Kc.codes, Kc.scales, w.dim, Kc.norms, blocks=ids)
        out = att(q, pos + 1, w.threshold)
        torch.cuda.synchronize()
        k_host[:, :, pos] = inp.k[:, :, pos]
        v_host[:, :, pos] = inp.v[:, :, pos]
        okc, oks = F.pack(w.fmt, k_host)
        ovc, ovs = F.pack(w.fmt, v_host)
        summ = K.cache_block_norms(w.fmt, okc, oks, w.dim)
        assert np.array_equal(Kc.norms.cpu().numpy().view(np.uint32), summ.view(np.uint32)), step
        r, drop, margin = K.attend_kskip(inp.q, okc, oks, ovc, ovs, summ, fmt=w.fmt, dim=w.dim, v_dim=w.v_dim,
                                         ctx_len=pos + 1, sigma=w.sigma, threshold=w.threshold)
        got = out.cpu().numpy()
        err = np.abs(got - r.out64).max()
        rel = np.linalg.norm(got - r.out64) / np.linalg.norm(r.out64)
        st = att.stats()
        sizes = np.minimum(64, pos + 1 - 64 * np.arange(drop.shape[-1]))
        say(f"  step {step}: ctx {pos + 1} max_abs {err:.2e} rel {rel:.2e} skipped {st['key_rows_skipped']}")
        assert st["status"] == 0 and err <= 2e-3 and rel <= 1e-3
        assert np.abs(margin).min() > MARGIN_BAND
        assert st["key_rows_skipped"] == int((drop * sizes).sum())


def test_rejected_combinations():
    import torch

    import decode_attention_quantized_amd as kvq
    from decode_attention_quantized_amd.runtime import DecodeAttention, PackedCache
    say("case key skipping: missing summaries -> ARG, with the single-pass rule -> UNSUPPORTED")
    w = synth.workload("tiny")
    inp = synth.generate(w)
    kc, ks = kvq.kvq_pack(w.fmt, inp.k)
    vc, vs = kvq.kvq_pack(w.fmt, inp.v)
    Kc = PackedCache.from_host(kc, ks, w.fmt, w.dim)
    Vc = PackedCache.from_host(vc, vs, w.fmt, w.dim)
    q = torch.from_numpy(inp.q).cuda()
    att = DecodeAttention(Kc, Vc, w.q_heads, ctx_len=w.ctx, softmax_scale=w.sigma, skip_keys=True)
    with pytest.raises(kvq.KvqError) as e:
        att(q, w.ctx, w.threshold)
    assert e.value.name == "ARG"
    Kc.compute_norms()
    att = DecodeAttention(Kc, Vc, w.q_heads, ctx_len=w.ctx, softmax_scale=w.sigma, skip_keys=True, running=True)
    with pytest.raises(kvq.KvqError) as e:
        att(q, w.ctx, w.threshold)
    assert e.value.name == "UNSUPPORTED"
