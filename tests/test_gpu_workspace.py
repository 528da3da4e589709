"""kvq_workspace_bytes covers every shorter context: the size returned for a
context length is at least the size any shorter call needs (the split count
of a plan falls and rises as the context grows, through the rounding of
positions per split to whole 64-position chunks). Size queries only; no
kernel runs."""
import numpy as np
import pytest

from gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt,batch,kv_heads,q_heads,dim,v_dim,cap", [
    ("q4_0", 1, 4, 32, 128, 0, 70001),      # the long shape, one split per CU
    ("lut3", 8, 4, 32, 128, 0, 32768),      # the LUT3 batch at its largest one-launch context
    ("lut3", 8, 4, 32, 128, 0, 40000),      # ... and past it (two launches)
    ("q4_0", 72, 4, 32, 128, 0, 5000),      # more groups than compute units (several launches)
    ("q8_0", 1, 1, 4, 128, 0, 9000),
    ("fp8_b128", 8, 1, 128, 576, 512, 70001),
    ("fp8_b128", 1, 1, 32, 576, 512, 30000),
])
def test_workspace_size_covers_every_shorter_context(fmt, batch, kv_heads, q_heads, dim, v_dim, cap):
    import decode_attention_quantized_amd as kvq
    from decode_attention_quantized_amd import binding as B
    say("case workspace sizes", fmt, batch, kv_heads, q_heads, "capacity", cap)
    k = B.kvq_cache(0x10000, 0x20000, batch, kv_heads, dim, cap)   # sizes only: never dereferenced
    latent = fmt == "fp8_b128"
    launch = kvq.make_launch(q_heads, q_dtype=kvq.KVQ_Q_BF16 if latent else kvq.KVQ_Q_F32, v_dim=v_dim)
    f = B.FMT[fmt]
    top = kvq.kvq_workspace_bytes(f, k, launch, cap)
    rng = np.random.default_rng(cap)
    probes = sorted(n for n in set([1, 2, 63, 64, 65, 127, 128, 129, cap - 1, cap] + list(range(4032, 4224)) +
                                   rng.integers(1, cap + 1, 3000).tolist()) if n <= cap)
    worst = 0
    for n in probes:
        b = kvq.kvq_workspace_bytes(f, k, launch, int(n))
        worst = max(worst, b)
        assert b <= top, (n, b, top)
    say("  capacity size", top, "largest shorter", worst)
