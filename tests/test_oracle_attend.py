"""Pins for the oracle's attention and skip rule (CPU only)."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import attend as A
from oracle import formats as F
from oracle import mp as MP


def _small(name, **kw):
    return synth.generate(synth.resized(synth.workload(name), **kw))


def _sdpa_fp64(q, kh, vh, sigma):
    """torch scaled_dot_product_attention in float64 on the CPU, GQA expanded."""
    B, Hq, D = q.shape
    Hkv = kh.shape[1]
    G = Hq // Hkv
    K = torch.from_numpy(np.repeat(kh, G, axis=1))
    V = torch.from_numpy(np.repeat(vh, G, axis=1))
    Q = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=float(sigma))
    return o[:, :, 0, :].numpy()


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("long", dict(ctx=2048, hot=4)),
    ("lut3", dict(batch=2, ctx=1024)),
    ("mla", dict(batch=1, q_heads=16, ctx=512, hot=6)),
])
def test_threshold_zero_equals_library_softmax_attention(name, kw):
    inp = _small(name, **kw)
    w = inp.w
    r, pk = A.attend_inputs(inp, threshold=0.0)
    kh = A.dequant_cache(w.fmt, pk["kc"], pk["ks"], w.dim, w.ctx)
    vh = kh[..., :w.v_dim] if pk["vc"] is None else A.dequant_cache(w.fmt, pk["vc"], pk["vs"], w.v_dim, w.ctx)
    ref = _sdpa_fp64(inp.q, kh, vh, w.sigma)
    assert np.allclose(r.out64, ref, rtol=1e-12, atol=1e-13)
    assert r.mask.all() and r.kept_pairs == w.batch * w.q_heads * w.ctx


@pytest.mark.parametrize("name,kw", [("tiny", {}), ("stress", dict(ctx=4096)),
                                     ("lut3", dict(batch=2, ctx=2048))])
def test_skip_identity_and_bound(name, kw):
    inp = _small(name, **kw)
    r0, pk = A.attend_inputs(inp, threshold=0.0)
    rt, _ = A.attend_inputs(inp, packed=pk)
    w = inp.w
    vh = A.dequant_cache(w.fmt, pk["vc"], pk["vs"], w.v_dim, w.ctx)
    # out_0 - out_tau = sum over skipped positions of p_i v_i, exactly the dropped terms
    G = w.q_heads // w.kv_heads
    for b in range(w.batch):
        for h in range(w.q_heads):
            skip = ~rt.mask[b, h]
            dropped = (rt.p[b, h] * skip) @ vh[b, h // G]
            # (to float64 rounding of two n-term sums)
            tol = 64 * np.finfo(np.float64).eps * (np.abs(rt.p[b, h]) @ np.abs(vh[b, h // G]))
            assert np.all(np.abs(r0.out64[b, h] - rt.out64[b, h] - dropped) <= tol)
            bound = (1.0 - rt.kept_mass[b, h]) * rt.vmax[b, h // G]
            assert np.abs(r0.out64[b, h] - rt.out64[b, h]).max() <= bound * (1 + 1e-9) + 1e-15
    # the threshold is compared against normalized weights: every kept p >= tau, skipped < tau
    assert np.all(rt.p[rt.mask] >= np.float32(1e-6)) and np.all(rt.p[~rt.mask] < np.float32(1e-6))


def test_ctx_one_returns_first_value_row():
    inp = _small("long", ctx=64, hot=0)
    r, pk = A.attend_inputs(inp, ctx_len=1)
    vh = A.dequant_cache("q4_0", pk["vc"], pk["vs"], 128, 1)
    G = 8
    for h in range(32):
        assert np.array_equal(r.out64[0, h], vh[0, h // G, 0])
    assert r.kept_pairs == 32 and r.rows_fetched == 4


@pytest.mark.parametrize("fmt", [F.Q8_0, F.Q4_0, F.LUT3])
def test_identical_keys_give_uniform_weights_and_threshold_flip(fmt):
    rng = np.random.default_rng(3)
    n, D = 200, 128
    q = rng.standard_normal((1, 2, D)).astype(np.float32)
    krow = rng.standard_normal(D).astype(np.float32)
    k = np.broadcast_to(krow, (1, 1, n, D)).copy()
    v = rng.standard_normal((1, 1, n, D)).astype(np.float32)
    kc, ks = F.pack(fmt, k)
    vc, vs = F.pack(fmt, v)
    vh = A.dequant_cache(fmt, vc, vs, D, n)[0, 0]
    kw = dict(fmt=fmt, dim=D, v_dim=D, ctx_len=n, sigma=0.1)
    r = A.attend(q, kc, ks, vc, vs, threshold=(1 - 1e-2) / n, **kw)
    assert np.allclose(r.p, 1.0 / n, rtol=1e-13)
    assert np.allclose(r.out64[0, 0], vh.mean(0), rtol=1e-11, atol=1e-14)
    assert r.mask.all()
    r2 = A.attend(q, kc, ks, vc, vs, threshold=(1 + 1e-2) / n, **kw)
    assert not r2.mask.any() and not r2.out.any() and r2.rows_fetched == 0


def test_permutation_invariance():
    inp = _small("stress", ctx=1024)
    r, pk = A.attend_inputs(inp)
    perm = np.random.default_rng(5).permutation(1024)
    pk2 = {k: (v[:, :, perm] if v is not None else None) for k, v in pk.items()}
    r2, _ = A.attend_inputs(inp, packed=pk2)
    assert np.allclose(r.out64, r2.out64, rtol=1e-12, atol=1e-15)
    assert np.array_equal(r.mask[..., perm], r2.mask)


def test_scaling_values_by_power_of_two_scales_output_exactly():
    inp = _small("tiny")
    r, pk = A.attend_inputs(inp)
    v2 = inp.v * np.float32(8.0)
    vc2, vs2 = F.pack(F.Q8_0, v2)
    assert np.array_equal(vc2, pk["vc"])               # codes unchanged, scales x8
    r2 = A.attend(inp.q, pk["kc"], pk["ks"], vc2, vs2, fmt=F.Q8_0, dim=128, v_dim=128,
                  ctx_len=1024, sigma=inp.w.sigma, threshold=1e-6)
    assert np.array_equal(r2.out64, 8.0 * r.out64)


def test_gqa_head_mapping():
    # value rows of kv head g all equal 127*2^g (exact in q8_0): head h must read floor(h*Hkv/Hq)
    B, Hq, Hkv, n, D = 1, 12, 3, 40, 128
    rng = np.random.default_rng(9)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, n, D)).astype(np.float32)
    v = np.zeros((B, Hkv, n, D), np.float32)
    for g in range(Hkv):
        v[0, g] = 127.0 * 2.0 ** g
    kc, ks = F.pack(F.Q8_0, k)
    vc, vs = F.pack(F.Q8_0, v)
    r = A.attend(q, kc, ks, vc, vs, fmt=F.Q8_0, dim=D, v_dim=D, ctx_len=n, sigma=0.09, threshold=0.0)
    for h in range(Hq):
        assert np.allclose(r.out64[0, h], 127.0 * 2.0 ** ((h * Hkv) // Hq), rtol=1e-12)


@pytest.mark.parametrize("fmt,dim,vdim", [(F.Q8_0, 128, 128), (F.Q4_0, 128, 128),
                                          (F.LUT3, 128, 128), (F.FP8, 576, 512)])
def test_brute_force_mpmath_small_context(fmt, dim, vdim):
    rng = np.random.default_rng(21)
    n = 48
    q = rng.standard_normal((1, 2, dim)).astype(np.float32)
    k = (rng.standard_normal((1, 1, n, dim)) * 2.5).astype(np.float32)
    k[0, 0, 7] = q[0, 0] * 0.6                   # one dominant key so the mask is non-trivial
    kc, ks = F.pack(fmt, k)
    if fmt == F.FP8:
        vc = vs = None
    else:
        v = rng.standard_normal((1, 1, n, vdim)).astype(np.float32)
        vc, vs = F.pack(fmt, v)
    sigma, tau = float(np.float32(1 / math.sqrt(dim))), 1e-3
    r = A.attend(q, kc, ks, vc, vs, fmt=fmt, dim=dim, v_dim=vdim, ctx_len=n, sigma=sigma, threshold=tau)
    krows = [MP.decode_row(fmt, kc[0, 0, i], ks[0, 0, i], dim) for i in range(n)]
    vrows = [row[:vdim] for row in krows] if vc is None else \
        [MP.decode_row(fmt, vc[0, 0, i], vs[0, 0, i], vdim) for i in range(n)]
    for h in range(2):
        p, keep, out = MP.attend_one(q[0, h], krows, vrows, np.float32(sigma), np.float32(tau))
        assert np.allclose(r.p[0, h], [float(x) for x in p], rtol=1e-12, atol=1e-300)
        assert list(r.mask[0, h]) == keep
        assert np.allclose(r.out64[0, h], [float(x) for x in out], rtol=1e-12, atol=1e-14)
    assert 0 < r.kept_pairs < 2 * n


def test_workloads_match_the_pages_regime():
    # long: every KV head keeps exactly its planted positions (all +20 logits)
    inp = _small("long", ctx=8192, hot=16)
    r, _ = A.attend_inputs(inp)
    for g in range(4):
        assert set(np.nonzero(r.union[0, g])[0]) == set(inp.hot[0][g].tolist())
    # stress: more than 90% of weights fall below 1e-6 (the pages' claim at long context)
    inp = _small("stress", ctx=32768)
    r, _ = A.attend_inputs(inp)
    assert r.kept_pairs / r.mask.size < 0.10
    assert 1.0 - r.kept_mass.min() < 5e-3


def test_band_is_relative_to_the_float32_threshold():
    """The mask band (weights within 1e-3 relative of the threshold, measured
    on the float32 value the kernels receive) against constructed weights:
    just inside / just outside the relative band on both sides, the threshold
    itself, a band that an absolute 1e-3 or a factor of 1e-2 would get wrong,
    and no band at threshold 0."""
    for tau in (1e-6, 3e-5, 0.01, 0.25):
        t32 = float(np.float32(tau))
        p = np.array([t32, t32 * (1 + 0.999e-3), t32 * (1 - 0.999e-3), t32 * (1 + 1.001e-3), t32 * (1 - 1.001e-3),
                      t32 * 1.005, t32 * 0.995, t32 * 2, t32 / 2, 0.0, 1.0])
        want = np.array([True, True, True, False, False, False, False, False, False, False, False])
        assert np.array_equal(A.band(p, tau), want), tau
    # relative, not absolute: at tau = 0.01 an absolute band of 1e-3 would take
    # 0.0105, which is 5% away
    assert not A.band(np.array([0.0105, 0.0095]), 0.01).any()
    # the float64 threshold 1e-6 is not the float32 one the kernels use; the
    # band is taken around the float32 value
    t32 = float(np.float32(1e-6))
    assert t32 != 1e-6
    p = np.array([t32 * (1 + 0.9995e-3)])
    assert A.band(p, 1e-6).all()
    assert not A.band(np.array([0.5, 1e-6, 1e-30]), 0.0).any()
    # shape is kept (per (batch, head, position) weights)
    assert A.band(np.full((2, 3, 4), 1e-6), 1e-6).shape == (2, 3, 4)
