"""The give-up path of the bounded waits, forced from the host: with the
KVQ_TEST_WITHHOLD launch flag, context split 0 of the first group (grouped
formats: sequence 0, kv head 0; latent: sequence 0) never publishes its split
statistics and every wait gives up after a few thousand polls. Every kernel
still ends normally; the call reports KVQ_ERR_DEVICE through kvq_stats, the
outputs that depended on the withheld statistics are NaN, and every other
output still matches the oracle. A fresh workspace then works again."""
import numpy as np
import pytest

import synth
from gpu_helpers import MAX_ABS, MAX_REL_L2, oracle_for, say

pytestmark = pytest.mark.gpu


def _run(inp, tau, withhold):
    import torch

    import decode_attention_quantized_amd as kvq
    from decode_attention_quantized_amd.runtime import DecodeAttention, PackedCache
    w = inp.w
    kc, ks = kvq.kvq_pack(w.fmt, inp.k)
    K = PackedCache.from_host(kc, ks, w.fmt, w.dim)
    V = None
    if inp.v is not None:
        vc, vs = kvq.kvq_pack(w.fmt, inp.v)
        V = PackedCache.from_host(vc, vs, w.fmt, w.v_dim)
    latent = V is None
    att = DecodeAttention(K, V, w.q_heads, ctx_len=w.ctx, softmax_scale=w.sigma,
                          q_dtype=kvq.KVQ_Q_BF16 if latent else kvq.KVQ_Q_F32, v_dim=w.v_dim if latent else 0,
                          test_withhold=withhold)
    q = torch.from_numpy(inp.q).cuda()
    if latent:
        q = q.to(torch.bfloat16)
    out = att(q, w.ctx, tau).cpu().numpy()
    return out, att.stats()


@pytest.mark.parametrize("name,kw,tau", [
    ("long", dict(ctx=5000, hot=6, batch=2), 1e-6),
    ("long", dict(ctx=5000, hot=6, batch=2), 0.0),
    ("lut3", dict(ctx=3000, batch=2), 1e-6),
    ("mla", dict(ctx=3000, batch=2, hot=4), 1e-6),
    ("mla", dict(ctx=3000, batch=2, hot=4), 0.0),
])
def test_withheld_statistics(name, kw, tau):
    w = synth.resized(synth.workload(name), **kw)
    inp = synth.generate(w)
    say("case withheld statistics:", name, kw, "tau", tau)
    out, st = _run(inp, tau, withhold=True)
    assert st["rc"] == -8 and st["status"] & 1, st           # KVQ_ERR_DEVICE, wait-timeout bit
    G = w.q_heads // w.kv_heads
    poisoned = np.zeros((w.batch, w.q_heads), dtype=bool)
    if w.latent:
        poisoned[0, :] = True                               # sequence 0
    else:
        poisoned[0, :G] = True                              # sequence 0, kv head 0
    assert np.isnan(out[poisoned]).all(), "outputs that used the withheld statistics must be NaN"
    assert np.isnan(st["kept_mass"][poisoned]).all()
    assert np.isfinite(out[~poisoned]).all()
    r, _ = oracle_for(inp, tau)
    ref = r.out64[~poisoned]
    got = out[~poisoned]
    err = float(np.abs(got - ref).max())
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    say(f"  other outputs: max_abs={err:.3e} rel_l2={rel:.3e}")
    assert err <= MAX_ABS and rel <= MAX_REL_L2
    # the GPU and the library are fine: a fresh workspace gives the exact result
    out2, st2 = _run(inp, tau, withhold=False)
    assert st2["rc"] == 0 and st2["status"] == 0, st2
    err2 = float(np.abs(out2 - r.out64).max())
    assert err2 <= MAX_ABS, err2
