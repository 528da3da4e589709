"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
and compare it with the oracle on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np

import synth
from oracle import attend as A
from oracle import formats as F

MAX_ABS = 2e-3
MAX_REL_L2 = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_gpu(inp, threshold, *, ctx_len=None, splits=0, q_bf16=False, repeat=1, cooperative=False, running=False):
    """Pack with the library, run kvq_decode_attn on cuda:0. Returns dict."""
    import torch

    import decode_attention_quantized_amd as kvq
    from decode_attention_quantized_amd.runtime import DecodeAttention, PackedCache, mask_words, unpack_mask

    w = inp.w
    n = w.ctx if ctx_len is None else ctx_len
    kc, ks = kvq.kvq_pack(w.fmt, inp.k)
    K = PackedCache.from_host(kc, ks, w.fmt, w.dim)
    if inp.v is not None:
        vc, vs = kvq.kvq_pack(w.fmt, inp.v)
        V = PackedCache.from_host(vc, vs, w.fmt, w.v_dim)
    else:
        vc = vs = None
        V = None
    att = DecodeAttention(K, V, w.q_heads, ctx_len=n, softmax_scale=w.sigma, splits=splits,
                          q_dtype=kvq.KVQ_Q_BF16 if q_bf16 else kvq.KVQ_Q_F32,
                          v_dim=w.v_dim if V is None else 0, cooperative=cooperative, running=running)
    q = torch.from_numpy(inp.q).cuda()
    if q_bf16:
        q = q.to(torch.bfloat16)
    outs = []
    masks = []
    stats = None
    for _ in range(repeat):
        # filled with a pattern no result has in every word, so a word the
        # kernel leaves unwritten shows up as a mismatch
        mask = torch.full((w.batch, w.q_heads, mask_words(n)), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
        out = att(q, n, threshold, mask_out=mask)
        torch.cuda.synchronize()
        stats = att.stats()
        outs.append(out.cpu().numpy())
        mw = mask.cpu().numpy().view(np.uint32)
        if n % 32:                               # bits past the context in the last word are zero
            assert not (mw[..., -1] >> np.uint32(n % 32)).any(), "mask bits set past the context"
        masks.append(unpack_mask(mw, n))
    return dict(out=outs[0], outs=outs, mask=masks[0], masks=masks, stats=stats,
                planes=dict(kc=kc, ks=ks, vc=vc, vs=vs), splits=att.stats()["splits"])


def oracle_for(inp, threshold, *, ctx_len=None, q_override=None):
    w = inp.w
    kc, ks = F.pack(w.fmt, inp.k)
    if inp.v is not None:
        vc, vs = F.pack(w.fmt, inp.v)
    else:
        vc = vs = None
    q = inp.q if q_override is None else q_override
    n = w.ctx if ctx_len is None else ctx_len
    r = A.attend(q, kc, ks, vc, vs, fmt=w.fmt, dim=w.dim, v_dim=w.v_dim, ctx_len=n, sigma=w.sigma,
                 threshold=threshold)
    return r, dict(kc=kc, ks=ks, vc=vc, vs=vs)


def compare(inp, threshold, g, r, planes_o, *, check_stats=True, mask=True):
    """Assert the acceptance bar: bit-exact planes, masks outside the band,
    max abs <= 2e-3 and rel-L2 <= 1e-3, statistics equal up to band weights."""
    for key in ("kc", "ks", "vc", "vs"):
        if planes_o[key] is not None:
            assert np.array_equal(g["planes"][key], planes_o[key]), f"packed plane {key} differs"
    out, ref = g["out"], r.out64
    assert np.all(np.isfinite(out)), "non-finite output"
    err = np.abs(out - ref).max()
    nrm = np.linalg.norm(ref)
    rel = np.linalg.norm(out - ref) / nrm if nrm > 0 else np.linalg.norm(out)
    band = A.band(r.p, threshold)
    mism = ((g["mask"] != r.mask) & ~band) if mask else np.zeros_like(band)
    say(f"  max_abs={err:.3e} rel_l2={rel:.3e} kept={r.kept_pairs} rows={r.rows_fetched} "
        f"band={int(band.sum())} mask_mismatch={int(mism.sum())} splits={g['splits']}")
    assert not mism.any(), f"{int(mism.sum())} mask bits differ outside the band"
    assert err <= MAX_ABS, f"max abs error {err}"
    assert rel <= MAX_REL_L2, f"rel-L2 error {rel}"
    if check_stats:
        st = g["stats"]
        assert st["status"] == 0, st
        nb = int(band.sum())
        assert abs(st["kept_pairs"] - r.kept_pairs) <= nb, (st["kept_pairs"], r.kept_pairs)
        assert abs(st["rows_fetched"] - r.rows_fetched) <= nb, (st["rows_fetched"], r.rows_fetched)
        assert np.allclose(st["kept_mass"], r.kept_mass, rtol=0, atol=1e-5)
        if inp.v is not None:
            # grouped formats: the 64-position chunks holding a kept row
            want = live_chunks(r.union, 64)
            assert abs(st["live_tiles"] - want) <= nb, (st["live_tiles"], want)
        else:
            # latent: the re-scored 32-position tiles include every tile with a kept row
            lo, hi = live_chunks(r.union, 32), live_chunks(np.ones_like(r.union), 32)
            assert lo <= st["live_tiles"] <= hi + r.union.shape[0] * 2, (st["live_tiles"], lo, hi)
    return err, rel


def live_chunks(union, width):
    """Chunks of `width` positions (aligned to position 0) holding a row of the
    union mask, summed over [B][Hkv]."""
    B, H, n = union.shape
    pad = (-n) % width
    u = np.pad(union, ((0, 0), (0, 0), (0, pad)))
    return int(u.reshape(B, H, -1, width).any(axis=-1).sum())
