"""Dequantize-then-attend in float64 with the sparse-V skip rule.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, for every sequence b and query head h (g = floor(h*Hkv/Hq)
is the KV head h reads, n = ctx_len, sigma = softmax scale, tau = threshold):

1. k_i = dequant(K[b,g,i]), v_i = dequant(V[b,g,i]) for i < n (float64). For a
   latent cache the values are the leading ``v_dim`` dims of the same rows.
2. s_i = sigma * <q[b,h], k_i>, with q widened exactly to float64.
3. p_i = exp(s_i - m) / sum_j exp(s_j - m), m = max_j s_j: the normalized
   softmax weight, the denominator taken over all n positions.
   [SV] "Решение — не ускорять, а пропускать": the softmax weights come from
   the keys before any value is touched. FAQ: every key must be dequantized to
   know which weights are negligible, so the denominator covers all positions.
4. keep_i <=> p_i >= tau; a position is skipped when its weight is below the
   threshold ([SV] same section: below 1e-6, V dequantization *and*
   accumulation are skipped entirely).
5. out[b,h] = sum over kept i of p_i * v_i, with no renormalization over the
   kept set (only the V work is skipped), rounded once to float32. If every
   position is skipped the output is zero.

Also returned: the mask per (b,h,i), the kept mass sum_keep p_i per (b,h), the
union row mask per (b,g) (a value row is needed when any head of the group
keeps it) and integer counts. [SV] FAQ states the skipped contribution is below
a millionth of the maximum; here the identity out_0 - out_tau = sum_skip p_i v_i
gives the bound |out_tau - out_0| <= (sum_skip p_i) * max|v|.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import formats as F


@dataclasses.dataclass
class Result:
    out: np.ndarray          # float32 [B][Hq][Dv]
    out64: np.ndarray        # float64 [B][Hq][Dv] (before the final rounding)
    p: np.ndarray            # float64 [B][Hq][n] normalized weights
    mask: np.ndarray         # bool [B][Hq][n]
    kept_mass: np.ndarray    # float64 [B][Hq]
    union: np.ndarray        # bool [B][Hkv][n]
    kept_pairs: int
    rows_fetched: int
    vmax: np.ndarray         # float64 [B][Hkv] max |v| over the first n rows


def dequant_cache(fmt, codes, scales, dim, n):
    """[B][H][cap][bytes] planes -> float64 [B][H][n][dim] for the first n rows."""
    return F.unpack(fmt, codes[:, :, :n], scales[:, :, :n], dim)


def attend(q, k_codes, k_scales, v_codes, v_scales, *, fmt, dim, v_dim, ctx_len,
           sigma, threshold) -> Result:
    """The definition above. ``v_codes is None`` selects a latent cache whose
    values are the first ``v_dim`` dims of the key rows."""
    q = np.asarray(q)
    B, Hq, D = q.shape
    assert D == dim
    Hkv = k_codes.shape[1]
    if Hq % Hkv:
        raise ValueError("q heads must be a multiple of kv heads")
    n = int(ctx_len)
    if n < 1 or n > k_codes.shape[2]:
        raise ValueError("ctx_len out of range")
    sig = float(np.float32(sigma))
    tau = float(np.float32(threshold))
    out64 = np.zeros((B, Hq, v_dim), dtype=np.float64)
    P = np.zeros((B, Hq, n), dtype=np.float64)
    mask = np.zeros((B, Hq, n), dtype=bool)
    kept = np.zeros((B, Hq), dtype=np.float64)
    union = np.zeros((B, Hkv, n), dtype=bool)
    vmax = np.zeros((B, Hkv), dtype=np.float64)
    for b in range(B):
        kh = dequant_cache(fmt, k_codes[b:b + 1], k_scales[b:b + 1], dim, n)[0]       # [Hkv][n][D]
        if v_codes is None:
            vh = kh[..., :v_dim]
        else:
            vh = dequant_cache(fmt, v_codes[b:b + 1], v_scales[b:b + 1], v_dim, n)[0]
        for g in range(Hkv):
            heads = [h for h in range(Hq) if (h * Hkv) // Hq == g]
            Q = q[b, heads].astype(np.float64)                  # [G][D]
            S = sig * (Q @ kh[g].T)                             # [G][n]
            m = S.max(axis=1, keepdims=True)
            E = np.exp(S - m)
            p = E / E.sum(axis=1, keepdims=True)
            keep = p >= tau
            out64[b, heads] = (p * keep) @ vh[g]
            P[b, heads] = p
            mask[b, heads] = keep
            kept[b, heads] = (p * keep).sum(axis=1)
            union[b, g] = keep.any(axis=0)
            vmax[b, g] = np.abs(vh[g]).max()
    return Result(out=out64.astype(np.float32), out64=out64, p=P, mask=mask, kept_mass=kept,
                  union=union, kept_pairs=int(mask.sum()), rows_fetched=int(union.sum()), vmax=vmax)


def running_keep(S, positions_per_split, block, tau):
    """The single-pass (in-loop) skip rule on a score matrix S [G][n] (float64,
    natural-log domain): the context is cut into splits of
    ``positions_per_split`` positions, each split is walked in blocks of
    ``block`` positions in position order, and position i is kept when its
    weight under the softmax of its split's positions up to the end of i's
    block reaches ``tau``:
        p_run_i = exp(s_i - m_r) / sum_{j in split, j <= end of block(i)} exp(s_j - m_r),
        m_r = max over the same positions.
    This is the weight a flash-attention loop sees when it decides at block i
    with its running max and sum ([SV] "Решение — не ускорять, а
    пропускать": the skip is decided from the weights inside the loop); since
    the running denominator only grows, p_run_i >= p_i for the final
    normalized weight, so the kept set contains the exact rule's.
    Returns (p_run [G][n], keep [G][n])."""
    S = np.asarray(S, dtype=np.float64)
    G, n = S.shape
    p_run = np.zeros_like(S)
    for s0 in range(0, n, positions_per_split):
        s1 = min(s0 + positions_per_split, n)
        for b0 in range(s0, s1, block):
            b1 = min(b0 + block, s1)
            pre = S[:, s0:b1]                                  # the split's prefix through this block
            m = pre.max(axis=1, keepdims=True)
            den = np.exp(pre - m).sum(axis=1, keepdims=True)
            p_run[:, b0:b1] = np.exp(S[:, b0:b1] - m) / den
    return p_run, p_run >= float(np.float32(tau))


def attend_running(q, k_codes, k_scales, v_codes, v_scales, *, fmt, dim, v_dim, ctx_len, sigma, threshold,
                   positions_per_split, block=64) -> tuple[Result, np.ndarray]:
    """``attend`` with the single-pass keep rule of ``running_keep``: out =
    sum over kept i of p_i * v_i with p_i the exact normalized weight (only the
    set of kept positions changes). Returns (result, p_run [B][Hq][n])."""
    q = np.asarray(q)
    B, Hq, D = q.shape
    assert D == dim
    Hkv = k_codes.shape[1]
    n = int(ctx_len)
    sig = float(np.float32(sigma))
    tau = float(np.float32(threshold))
    out64 = np.zeros((B, Hq, v_dim), dtype=np.float64)
    P = np.zeros((B, Hq, n), dtype=np.float64)
    PR = np.zeros((B, Hq, n), dtype=np.float64)
    mask = np.zeros((B, Hq, n), dtype=bool)
    kept = np.zeros((B, Hq), dtype=np.float64)
    union = np.zeros((B, Hkv, n), dtype=bool)
    vmax = np.zeros((B, Hkv), dtype=np.float64)
    for b in range(B):
        kh = dequant_cache(fmt, k_codes[b:b + 1], k_scales[b:b + 1], dim, n)[0]
        vh = dequant_cache(fmt, v_codes[b:b + 1], v_scales[b:b + 1], v_dim, n)[0]
        for g in range(Hkv):
            heads = [h for h in range(Hq) if (h * Hkv) // Hq == g]
            S = sig * (q[b, heads].astype(np.float64) @ kh[g].T)
            m = S.max(axis=1, keepdims=True)
            E = np.exp(S - m)
            p = E / E.sum(axis=1, keepdims=True)
            p_run, keep = running_keep(S, positions_per_split, block, tau)
            out64[b, heads] = (p * keep) @ vh[g]
            P[b, heads] = p
            PR[b, heads] = p_run
            mask[b, heads] = keep
            kept[b, heads] = (p * keep).sum(axis=1)
            union[b, g] = keep.any(axis=0)
            vmax[b, g] = np.abs(vh[g]).max()
    res = Result(out=out64.astype(np.float32), out64=out64, p=P, mask=mask, kept_mass=kept,
                 union=union, kept_pairs=int(mask.sum()), rows_fetched=int(union.sum()), vmax=vmax)
    return res, PR


def attend_inputs(inp, *, threshold=None, ctx_len=None, packed=None) -> tuple[Result, dict]:
    """Pack a ``synth.Inputs`` with the oracle's own packer and attend.

    Returns (result, packed planes dict)."""
    w = inp.w
    fmt = w.fmt
    if packed is None:
        kc, ks = F.pack(fmt, inp.k)
        if inp.v is not None:
            vc, vs = F.pack(fmt, inp.v)
        else:
            vc = vs = None
        packed = dict(kc=kc, ks=ks, vc=vc, vs=vs)
    tau = w.threshold if threshold is None else threshold
    n = w.ctx if ctx_len is None else ctx_len
    res = attend(inp.q, packed["kc"], packed["ks"], packed["vc"], packed["vs"], fmt=fmt, dim=w.dim,
                 v_dim=w.v_dim, ctx_len=n, sigma=w.sigma, threshold=tau)
    return res, packed


def band(p, threshold, rel=1e-3):
    """Weights within ``rel`` relative of the threshold (excluded from mask parity)."""
    tau = float(np.float32(threshold))
    if tau == 0.0:
        return np.zeros_like(p, dtype=bool)
    return np.abs(p / tau - 1.0) <= rel
