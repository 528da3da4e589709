"""Pins of the oracle's single-pass (running-statistics) skip rule, checked
against hand-worked cases, library softmax and the exact rule (CPU only)."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import attend as A
from oracle import formats as F


def test_hand_worked_case():
    # scores 0, 10, 0, 0 (natural log), one split of 4, threshold 1e-4
    S = np.array([[0.0, 10.0, 0.0, 0.0]])
    # blocks of one position: position 0 alone has running weight 1 (kept), position 1 has
    # 1 / (1 + e^-10) (kept), positions 2 and 3 have e^-10 / (1 + 2e^-10) = 4.54e-5 and
    # e^-10 / (1 + 3e^-10) = 4.54e-5 (skipped); the exact rule keeps only position 1
    p_run, keep = A.running_keep(S, 4, 1, 1e-4)
    assert keep.tolist() == [[True, True, False, False]]
    assert p_run[0, 0] == 1.0
    e = math.exp(-10.0)
    assert abs(p_run[0, 1] - 1.0 / (1.0 + e)) < 1e-15
    assert abs(p_run[0, 2] - e / (1.0 + 2.0 * e)) < 1e-18
    assert abs(p_run[0, 3] - e / (1.0 + 3.0 * e)) < 1e-18
    # blocks of two: position 0 is decided with position 1 already in the denominator
    p_run, keep = A.running_keep(S, 4, 2, 1e-4)
    assert keep.tolist() == [[False, True, False, False]]
    # two splits of two: position 2 starts a new split and is alone in its first block
    p_run, keep = A.running_keep(S, 2, 1, 1e-4)
    assert keep.tolist() == [[True, True, True, True]]
    assert p_run[0, 2] == 1.0 and abs(p_run[0, 3] - 0.5) < 1e-15


def test_prefix_softmax_against_torch():
    rng = np.random.default_rng(5)
    S = rng.standard_normal((3, 50)) * 4
    p_run, _ = A.running_keep(S, 50, 1, 1e-6)
    for i in range(50):
        ref = torch.softmax(torch.from_numpy(S[:, :i + 1]), dim=1)[:, i].numpy()
        assert np.allclose(p_run[:, i], ref, rtol=1e-13, atol=0)
    # blocks of 7: every position of a block sees the prefix through the block's end
    p_run, _ = A.running_keep(S, 50, 7, 1e-6)
    for b0 in range(0, 50, 7):
        b1 = min(b0 + 7, 50)
        ref = torch.softmax(torch.from_numpy(S[:, :b1]), dim=1)[:, b0:b1].numpy()
        assert np.allclose(p_run[:, b0:b1], ref, rtol=1e-13, atol=0)


@pytest.mark.parametrize("split,block", [(64, 16), (512, 64), (100, 64), (33, 5)])
def test_running_weight_bounds_the_exact_weight(split, block):
    rng = np.random.default_rng(split * 7 + block)
    S = rng.standard_normal((4, 700)) * 3
    S[:, rng.integers(0, 700, 5)] += 12
    p = torch.softmax(torch.from_numpy(S), dim=1).numpy()
    p_run, keep = A.running_keep(S, split, block, 1e-6)
    assert np.all(p_run >= p * (1 - 1e-12))
    assert np.all(keep[p >= 1e-6])                       # every exactly kept position is kept
    # the last block of a split sees the whole split: its weights are the split's softmax
    for s0 in range(0, 700, split):
        s1 = min(s0 + split, 700)
        last = s0 + ((s1 - 1 - s0) // block) * block
        ref = torch.softmax(torch.from_numpy(S[:, s0:s1]), dim=1)[:, last - s0:].numpy()
        assert np.allclose(p_run[:, last:s1], ref, rtol=1e-12, atol=0)


def test_one_split_one_block_is_the_exact_rule():
    w = synth.resized(synth.workload("long"), batch=1, ctx=300, hot=4)
    inp = synth.generate(w)
    kc, ks = F.pack(w.fmt, inp.k)
    vc, vs = F.pack(w.fmt, inp.v)
    kw = dict(fmt=w.fmt, dim=w.dim, v_dim=w.v_dim, ctx_len=300, sigma=w.sigma, threshold=w.threshold)
    r = A.attend(inp.q, kc, ks, vc, vs, **kw)
    rr, p_run = A.attend_running(inp.q, kc, ks, vc, vs, positions_per_split=300, block=300, **kw)
    assert np.array_equal(rr.mask, r.mask)
    assert np.allclose(p_run, r.p, rtol=1e-12, atol=0)
    assert np.array_equal(rr.out64, r.out64)
    # smaller splits keep a superset; the output differs only by the extra kept terms
    rs, _ = A.attend_running(inp.q, kc, ks, vc, vs, positions_per_split=64, block=64, **kw)
    assert np.all(rs.mask[r.mask]) and rs.kept_pairs >= r.kept_pairs
    extra = rs.mask & ~r.mask
    vh = A.dequant_cache(w.fmt, vc, vs, w.v_dim, 300)[0]
    heads_g = [(h * w.kv_heads) // w.q_heads for h in range(w.q_heads)]
    for h in range(w.q_heads):
        want = r.out64[0, h] + (r.p[0, h] * extra[0, h]) @ vh[heads_g[h]]
        assert np.allclose(rs.out64[0, h], want, rtol=0, atol=1e-12)
