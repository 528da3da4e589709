"""GPU append packer (kvq_append) against the oracle's packer: bit-exact code
and scale planes for every format on random and edge rows, rows scattered
into a cache at given positions with every other row untouched, the skipped
rows a bad input reports, and a decode loop that appends each new token on
the GPU before attending over it."""
import zlib

import numpy as np
import pytest

import synth
from gpu_helpers import MAX_ABS, MAX_REL_L2, say
from oracle import attend as A
from oracle import formats as F

pytestmark = pytest.mark.gpu

FMTS = [("q8_0", 128), ("q4_0", 128), ("lut3", 128), ("fp8_b128", 576), ("q8_0", 64), ("q4_0", 256),
        ("fp8_b128", 200), ("q8_0", 96), ("q4_0", 320), ("q8_0", 1088), ("fp8_b128", 1500), ("fp8_b128", 384),
        ("lut3_wht", 128)]


def _rows(fmt, dim, n, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, dim)).astype(np.float32)
    x *= np.exp(rng.uniform(-9, 6, (n, 1))).astype(np.float32)        # many binades
    edges = [np.zeros(dim), np.full(dim, 1e-30), np.full(dim, 3e-7), np.linspace(-448, 448, dim),
             np.tile([1.0, -1.0], dim // 2 + 1)[:dim]]
    t = np.zeros(dim); t[0] = 127.0; t[1:] = np.arange(1, dim) % 32 - 15.5; edges.append(t)   # .5 ties
    h = np.zeros(dim); h[0] = -8.0; h[1:] = (np.arange(1, dim) % 17) - 8.5; edges.append(h)
    e = np.zeros(dim); e[3] = 5.0; e[dim - 1] = -5.0; edges.append(e)   # equal magnitudes: first index wins
    z = np.zeros(dim); z[::2] = -0.0; edges.append(z)
    keep = []
    for r in edges:
        try:
            F.pack(fmt, np.asarray(r, np.float32)[None])
            keep.append(r)
        except OverflowError:
            pass
    return np.concatenate([x, np.array(keep, np.float32)])


def _device_pack(fmt, x, dst=None, cache_rows=None, fill=0):
    import torch

    import decode_attention_quantized_amd as kvq
    dim = x.shape[-1]
    cb, sb = kvq.kvq_row_bytes(fmt, dim)
    n = len(x) if cache_rows is None else cache_rows
    codes = torch.full((n, cb), fill, dtype=torch.uint8, device="cuda")
    scales = torch.full((n, sb), fill, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    src = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    d = None if dst is None else torch.from_numpy(np.asarray(dst, np.int64)).cuda()
    kvq.kvq_append(fmt, src, d, codes, scales, status)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), int(status.item())


@pytest.mark.parametrize("fmt,dim", FMTS)
def test_append_bit_exact_against_oracle(fmt, dim):
    say("case append", fmt, dim)
    x = _rows(fmt, dim, 6000, zlib.crc32(f"append/{fmt}/{dim}".encode()))
    c, s, st = _device_pack(fmt, x)
    co, so = F.pack(fmt, x)
    assert st == 0
    assert np.array_equal(c, co), f"{np.sum(np.any(c != co, axis=1))} rows differ in codes"
    assert np.array_equal(s, so), f"{np.sum(np.any(s != so, axis=1))} rows differ in scales"


def test_append_every_fp8_code():
    say("case append fp8 rows covering every non-NaN e4m3 code")
    vals = np.array([F.e4m3_value(c) for c in range(256) if (c & 0x7F) != 0x7F], np.float32)
    rows = np.stack([np.resize(np.roll(vals, 37 * r), 576) for r in range(4)]).astype(np.float32)
    rows[:, ::128] = 448.0                      # scale exactly 1 in every group
    c, s, st = _device_pack("fp8_b128", rows)
    co, so = F.pack("fp8_b128", rows)
    assert st == 0 and np.array_equal(c, co) and np.array_equal(s, so)
    assert len(set(c.ravel().tolist())) == 254


@pytest.mark.parametrize("fmt,dim", [("q4_0", 128), ("lut3", 128), ("fp8_b128", 576), ("lut3_wht", 128)])
def test_append_scatter_leaves_other_rows(fmt, dim):
    say("case append scatter", fmt)
    rng = np.random.default_rng(7)
    x = rng.standard_normal((40, dim)).astype(np.float32)
    dst = rng.permutation(300)[:40]
    c, s, st = _device_pack(fmt, x, dst=dst, cache_rows=300, fill=0xA5)
    co, so = F.pack(fmt, x)
    assert st == 0
    assert np.array_equal(c[dst], co) and np.array_equal(s[dst], so)
    other = np.setdiff1d(np.arange(300), dst)
    assert np.all(c[other] == 0xA5) and np.all(s[other] == 0xA5)


def test_append_reports_and_skips_bad_rows():
    say("case append bad rows (NaN, inf, fp16 overflow, destination out of range)")
    dim = 128
    x = np.random.default_rng(3).standard_normal((6, dim)).astype(np.float32)
    x[1, 5] = np.nan
    x[2, 9] = np.inf
    x[3, 96:] = 1e9                             # the last block's q8_0 scale 1e9/127 overflows fp16:
                                                # the whole row is skipped, not just that block
    dst = np.array([0, 1, 2, 3, 10, 5])         # row 4 goes outside a 10-row cache
    c, s, st = _device_pack("q8_0", x, dst=dst, cache_rows=10, fill=0x5A)
    assert st == 1 | 2 | 4
    co, so = F.pack("q8_0", x[[0, 5]])
    assert np.array_equal(c[[0, 5]], co) and np.array_equal(s[[0, 5]], so)
    assert np.all(c[1:4] == 0x5A) and np.all(s[1:4] == 0x5A) and np.all(c[6:] == 0x5A)
    # the same for q4_0 (scale from the largest element) and a long q8_0 row (more than 8 chunks)
    x4 = x[[0, 3]].copy()
    x4[1, :] = 1.0
    x4[1, 40] = -1e6                            # q4_0 scale 1e6/8 overflows fp16
    c, s, st = _device_pack("q4_0", x4, cache_rows=2, fill=0x5A)
    assert st == 2 and np.array_equal(c[0], F.pack("q4_0", x4[:1])[0][0]) and np.all(c[1] == 0x5A)
    xl = np.random.default_rng(4).standard_normal((3, 1024)).astype(np.float32)
    xl[2, 1000] = 1e9
    c, s, st = _device_pack("q8_0", xl, fill=0x5A)
    co, so = F.pack("q8_0", xl[:2])
    assert st == 2 and np.array_equal(c[:2], co) and np.array_equal(s[:2], so) and np.all(c[2] == 0x5A)


@pytest.mark.parametrize("fmt,together", [("q4_0", True), ("lut3", False), ("q8_0", True)])
def test_decode_loop_with_device_append(fmt, together):
    """Three decode steps: each appends the new token's K and V rows on the GPU
    at position n, then attends over n + 1 positions; the oracle packs the same
    rows on the host and attends over the same prefix."""
    import torch

    import decode_attention_quantized_amd as kvq
    from decode_attention_quantized_amd.runtime import DecodeAttention, PackedCache, append_kv
    say("case decode loop with device append", fmt, "K and V in one launch" if together else "")
    w = synth.resized(synth.workload("long"), fmt=fmt, batch=2, ctx=2048, hot=8)
    inp = synth.generate(w)
    K = PackedCache.empty(fmt, w.batch, w.kv_heads, w.ctx, w.dim)
    V = PackedCache.empty(fmt, w.batch, w.kv_heads, w.ctx, w.v_dim)
    start = w.ctx - 3
    # prefill on the device: every row before the decode start in one call per cache
    bh = np.arange(w.batch * w.kv_heads, dtype=np.int64).reshape(w.batch, w.kv_heads, 1)
    dst = torch.from_numpy((bh * w.ctx + np.arange(start, dtype=np.int64)).reshape(-1)).cuda()
    for cache, rows in ((K, inp.k), (V, inp.v)):
        src = torch.from_numpy(np.ascontiguousarray(rows[:, :, :start]).reshape(-1, rows.shape[-1])).cuda()
        kvq.kvq_append(fmt, src, dst, cache.codes, cache.scales)
    att = DecodeAttention(K, V, w.q_heads, ctx_len=w.ctx, softmax_scale=w.sigma)
    q = torch.from_numpy(inp.q).cuda()
    kc, ks = F.pack(fmt, inp.k)
    vc, vs = F.pack(fmt, inp.v)
    for step in range(3):
        n = start + step
        p = torch.full((w.batch,), n, dtype=torch.int64, device="cuda")
        kr = torch.from_numpy(np.ascontiguousarray(inp.k[:, :, n])).cuda()
        vr = torch.from_numpy(np.ascontiguousarray(inp.v[:, :, n])).cuda()
        if together:
            append_kv(K, V, kr, vr, p)
        else:
            K.append(kr, p)
            V.append(vr, p)
        out = att(q, n + 1, w.threshold).cpu().numpy()
        assert np.array_equal(K.codes.cpu().numpy()[:, :, :n + 1], kc[:, :, :n + 1])
        assert np.array_equal(K.scales.cpu().numpy()[:, :, :n + 1], ks[:, :, :n + 1])
        assert np.array_equal(V.codes.cpu().numpy()[:, :, :n + 1], vc[:, :, :n + 1])
        assert np.array_equal(V.scales.cpu().numpy()[:, :, :n + 1], vs[:, :, :n + 1])
        r = A.attend(inp.q, kc, ks, vc, vs, fmt=fmt, dim=w.dim, v_dim=w.v_dim, ctx_len=n + 1, sigma=w.sigma,
                     threshold=w.threshold)
        err = float(np.abs(out - r.out64).max())
        rel = float(np.linalg.norm(out - r.out64) / np.linalg.norm(r.out64))
        assert err <= MAX_ABS and rel <= MAX_REL_L2, (step, err, rel)


def test_append_kv_status_and_both_planes():
    import torch

    import decode_attention_quantized_amd as kvq
    say("case append_kv: both caches, one bad value row")
    rng = np.random.default_rng(11)
    k = rng.standard_normal((5, 128)).astype(np.float32)
    v = rng.standard_normal((5, 128)).astype(np.float32)
    v[2, 7] = np.nan
    planes = [torch.full((8, n), 0x33, dtype=torch.uint8, device="cuda") for n in (64, 8, 64, 8)]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dst = torch.tensor([7, 0, 3, 5, 1], dtype=torch.int64, device="cuda")
    kvq.kvq_append_kv("q4_0", torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), dst, *planes, status)
    torch.cuda.synchronize()
    kc, ks, vc, vs = (p.cpu().numpy() for p in planes)
    kco, kso = F.pack("q4_0", k)
    vco, vso = F.pack("q4_0", v[[0, 1, 3, 4]])
    d = [7, 0, 3, 5, 1]
    assert int(status.item()) == 1
    assert np.array_equal(kc[d], kco) and np.array_equal(ks[d], kso)
    assert np.array_equal(vc[[7, 0, 5, 1]], vco) and np.array_equal(vs[[7, 0, 5, 1]], vso)
    assert np.all(vc[3] == 0x33) and np.all(vs[3] == 0x33)
