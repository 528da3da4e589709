"""The no-allocation entry point kvq_decode_attn_noalloc (for callers that
cannot allocate device memory), through the C ABI: its output equals that of
kvq_decode_attn with a caller workspace (same kernels, same plan), and both
meet the oracle bar; two calls in a row, the second on a smaller input, so
the fixed array is reused with another layout; and the latent shape, whose
plans need far more than the fixed array, is refused before any launch."""
import numpy as np
import pytest

import synth
from gpu_helpers import MAX_ABS, MAX_REL_L2, oracle_for, say

pytestmark = pytest.mark.gpu


def _inputs(name, **kw):
    import torch

    import decode_attention_quantized_amd as kvq
    from decode_attention_quantized_amd.runtime import PackedCache
    w = synth.resized(synth.workload(name), **kw)
    inp = synth.generate(w)
    kc, ks = kvq.kvq_pack(w.fmt, inp.k)
    vc, vs = kvq.kvq_pack(w.fmt, inp.v)
    K = PackedCache.from_host(kc, ks, w.fmt, w.dim)
    V = PackedCache.from_host(vc, vs, w.fmt, w.dim)
    q = torch.from_numpy(inp.q).cuda()
    return inp, K, V, q


def _both(inp, K, V, q, tau):
    import torch

    import decode_attention_quantized_amd as kvq
    from decode_attention_quantized_amd import binding as B
    from decode_attention_quantized_amd.runtime import DecodeAttention
    w = inp.w
    att = DecodeAttention(K, V, w.q_heads, ctx_len=w.ctx, softmax_scale=w.sigma)
    ref = att(q, w.ctx, tau)
    out = torch.full_like(ref, float("nan"))
    launch = B.make_launch(w.q_heads, softmax_scale=w.sigma)     # no workspace: the library's own array
    kvq.binding.kvq_decode_attn_noalloc(q, K.struct(), V.struct(), w.fmt, w.ctx, tau, out, launch)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), out.cpu().numpy()


@pytest.mark.parametrize("fmt", ["q4_0", "lut3"])
def test_noalloc_matches_workspace_call_twice(fmt):
    cases = [dict(batch=2, ctx=8192, hot=8), dict(batch=1, ctx=3000, hot=4)]   # the second is smaller
    for kw in cases:
        say("case no-alloc entry point:", fmt, kw)
        inp, K, V, q = _inputs("long", fmt=fmt, **kw)
        for tau in (1e-6, 0.0):
            ref, out = _both(inp, K, V, q, tau)
            assert np.array_equal(out, ref), "no-alloc output differs from the workspace call"
            r, _ = oracle_for(inp, tau)
            err = float(np.abs(out - r.out64).max())
            rel = float(np.linalg.norm(out - r.out64) / np.linalg.norm(r.out64))
            say(f"  tau {tau}: max_abs={err:.3e} rel_l2={rel:.3e}")
            assert err <= MAX_ABS and rel <= MAX_REL_L2


def test_noalloc_with_several_launches():
    """A call whose 288 groups need two launches runs on the fixed array
    too (each launch advances the epoch in it), then a one-launch call."""
    for kw in (dict(batch=72, ctx=1000, hot=4), dict(batch=1, ctx=2000, hot=4)):
        say("case no-alloc entry point:", kw)
        inp, K, V, q = _inputs("long", **kw)
        ref, out = _both(inp, K, V, q, 1e-6)
        assert np.array_equal(out, ref), "no-alloc output differs from the workspace call"
        r, _ = oracle_for(inp, 1e-6)
        assert float(np.abs(out - r.out64).max()) <= MAX_ABS


def test_noalloc_refuses_latent_plans():
    import torch

    import decode_attention_quantized_amd as kvq
    from decode_attention_quantized_amd import binding as B
    from decode_attention_quantized_amd.runtime import PackedCache
    say("case no-alloc entry point refuses the latent shape")
    w = synth.resized(synth.workload("mla"), batch=1, ctx=256, hot=2)
    inp = synth.generate(w)
    kc, ks = kvq.kvq_pack(w.fmt, inp.k)
    K = PackedCache.from_host(kc, ks, w.fmt, w.dim)
    q = torch.from_numpy(inp.q).cuda().to(torch.bfloat16)
    out = torch.zeros((1, w.q_heads, 512), dtype=torch.float32, device="cuda")
    launch = B.make_launch(w.q_heads, q_dtype=kvq.KVQ_Q_BF16, v_dim=512, softmax_scale=w.sigma)
    with pytest.raises(kvq.KvqError) as e:
        kvq.binding.kvq_decode_attn_noalloc(q, K.struct(), None, w.fmt, w.ctx, 1e-6, out, launch)
    assert e.value.name == "UNSUPPORTED"
    torch.cuda.synchronize()
    assert not out.any()
