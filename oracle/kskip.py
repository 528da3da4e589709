"""K-side skipping: how many key rows a provable score bound could leave out.

TEST INFRASTRUCTURE ONLY (see the package docstring). This module answers,
on given inputs, the question the sparse-V page leaves as future work (how
many key rows a bound could leave out, with the exact LSE), and defines the
rule the grouped kernel applies under its K-skipping launch flag, where only
a lower bound of the LSE is known (``attend_kskip``).

[SV] FAQ, "Почему нельзя пропускать и K-деквантизацию?": the keys are needed
to know which weights are negligible, so every key is dequantized; the
author names as future work a first pass with approximate weights that
filters key positions. To keep the result exact, that first pass has to
*bound* the scores, not estimate them: a block of key rows may be left out
of the softmax only when its total weight is provably negligible.

Bounds of the scores s_i = sigma * <q, k_i> over a block of rows B, from
summaries of its dequantized keys:

* norm bound (Cauchy-Schwarz): s_i <= sigma * ||q|| * max_{i in B} ||k_i||;
* centroid bound: with c = mean of the block's rows and r = max ||k_i - c||,
  s_i = sigma * (<q, c> + <q, k_i - c>) <= sigma * (<q, c> + ||q|| * r).

A block can be dropped for a head when |B| * exp(bound - LSE) <= eps, LSE
being the log-sum-exp of all scores of that head. Dropping blocks whose
bounded weights add up to W leaves out at most W of the mass and scales
every remaining weight by a factor in [1, 1 / (1 - W)], so with eps of
1e-7 per block (and few dropped blocks' worth of W) the result is the
oracle's within float32 rounding. The exact LSE is used here; a real first
pass would only have a lower bound of it, so these fractions are the most
a bound of this kind can skip. Under grouped-query attention a key row is
dropped only when every head of its group drops its block.
"""
from __future__ import annotations

import numpy as np


def block_bounds(q: np.ndarray, k: np.ndarray, sigma: float, block: int, kind: str) -> np.ndarray:
    """Upper bounds of the scores of query rows q [G][D] over each block of
    `block` consecutive key rows of k [n][D] (float64, dequantized); returns
    [G][ceil(n / block)]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    n = k.shape[0]
    nb = -(-n // block)
    qn = np.linalg.norm(q, axis=1)                      # [G]
    out = np.empty((q.shape[0], nb))
    for j in range(nb):
        kb = k[j * block:(j + 1) * block]
        if kind == "norm":
            out[:, j] = sigma * qn * np.linalg.norm(kb, axis=1).max()
        elif kind == "centroid":
            c = kb.mean(axis=0)
            r = np.linalg.norm(kb - c, axis=1).max()
            out[:, j] = sigma * (q @ c + qn * r)
        else:
            raise ValueError(kind)
    return out


def droppable_blocks(q: np.ndarray, k: np.ndarray, sigma: float, block: int, kind: str,
                     eps: float = 1e-7) -> np.ndarray:
    """bool [nblocks]: blocks every head of q [G][D] may leave out (bounded
    total weight of the block at most eps for each head)."""
    s = sigma * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)      # [G][n] exact scores
    m = s.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(s - m).sum(axis=1, keepdims=True)))[:, 0]        # [G]
    ub = block_bounds(q, k, sigma, block, kind)
    n = k.shape[0]
    sizes = np.minimum(block, n - block * np.arange(ub.shape[1]))
    w = sizes[None, :] * np.exp(ub - lse[:, None])      # bounded total weight per (head, block)
    return (w <= eps).all(axis=0)


def dropped_fraction(q: np.ndarray, k_groups: np.ndarray, sigma: float, block: int = 64, kind: str = "centroid",
                     eps: float = 1e-7) -> float:
    """Fraction of key rows a bound of `kind` could drop, for one sequence:
    q [Hq][D], k_groups [Hkv][n][D] (dequantized); query head h reads KV
    group h * Hkv // Hq."""
    Hq, Hkv, n = q.shape[0], k_groups.shape[0], k_groups.shape[1]
    dropped = 0
    for g in range(Hkv):
        heads = [h for h in range(Hq) if (h * Hkv) // Hq == g]
        d = droppable_blocks(q[heads], k_groups[g], sigma, block, kind, eps)
        sizes = np.minimum(block, n - block * np.arange(d.size))
        dropped += int(sizes[d].sum())
    return dropped / (Hkv * n)


def block_max_norms(k_rows, block: int = 64) -> np.ndarray:
    """Per-block summaries of dequantized key rows k_rows [n][D] (float64):
    the largest row norm of each block of ``block`` consecutive rows, each
    norm taken as the square root of the sum of squares added in element
    order, in float64, and the block maximum rounded UP to float32 (so the
    stored value never understates a norm). Returns float32 [ceil(n / block)]."""
    k = np.asarray(k_rows, dtype=np.float64)
    n = k.shape[0]
    nb = -(-n // block)
    # np.cumsum adds in element order; its last column is the sequential sum
    norms = np.sqrt(np.cumsum(k * k, axis=1)[:, -1]) if n else np.zeros(0)
    out = np.zeros(nb, dtype=np.float32)
    for j in range(nb):
        r = float(norms[j * block:(j + 1) * block].max())
        f = np.float32(r)
        if float(f) < r:
            f = np.nextafter(f, np.float32(np.inf))
        out[j] = f
    return out


def cache_block_norms(fmt, codes, scales, dim, block: int = 64) -> np.ndarray:
    """Summaries of a whole packed cache [B][H][cap][bytes]: float32
    [B][H][ceil(cap / block)] (every row of the capacity, written or not)."""
    from . import formats as F
    B, H, cap = codes.shape[:3]
    out = np.zeros((B, H, -(-cap // block)), dtype=np.float32)
    for b in range(B):
        kh = F.unpack(fmt, codes[b:b + 1], scales[b:b + 1], dim)[0]
        for h in range(H):
            out[b, h] = block_max_norms(kh[h], block)
    return out


RHO = 0.5          # candidate blocks: largest key norm at least RHO times the context's largest


def attend_kskip(q, k_codes, k_scales, v_codes, v_scales, summary, *, fmt, dim, v_dim, ctx_len, sigma,
                 threshold, eps=1e-7, block=64):
    """Exact-rule attention after K-side skipping with the norm bound, as a
    kernel can do it before it knows the exact LSE ([SV] FAQ, "Почему нельзя
    пропускать и K-деквантизацию?": a first pass has to filter key positions;
    here it leaves out only positions whose weights a bound proves
    negligible).

    For each sequence b and kv group g (heads h of the group, n = ctx_len,
    blocks k of ``block`` positions, R_k = summary[b, g, k] the block's
    largest key norm, float32):
      1. the candidate blocks are those with R_k >= RHO * max_k R_k (the
         product taken in float32; RHO = 1/2 makes it exact): the blocks
         that may hold the largest scores;
      2. L_h = log sum exp of head h's exact scores over the candidate
         blocks' positions: a lower bound of the head's full LSE;
      3. a block that is not a candidate is dropped when for every head h
         |B_k| * exp(sigma * ||q_h|| * R_k - L_h) <= eps, |B_k| its positions
         inside the context (Cauchy-Schwarz bounds every score of the block
         by sigma * ||q_h|| * R_k, so its total weight is at most eps);
      4. the softmax, the keep rule p >= tau and the output of ``attend``
         are taken over the positions of the blocks that are not dropped
         (the normalized weights there are the exact ones times at most
         1 / (1 - W), W <= eps * dropped blocks the dropped weight).

    Returns (Result, dropped bool [B][Hkv][nblocks], margin float64
    [B][Hkv][nblocks]): margin = max over the group's heads of
    sigma * ||q_h|| * R_k - L_h - log(eps / |B_k|) (a block with margin <= 0
    is dropped, candidates excepted; near 0 the decision rests on rounding).
    """
    from . import attend as A
    q = np.asarray(q)
    B, Hq, D = q.shape
    assert D == dim
    Hkv = k_codes.shape[1]
    n = int(ctx_len)
    sig = float(np.float32(sigma))
    tau = float(np.float32(threshold))
    nb = -(-n // block)
    sizes = np.minimum(block, n - block * np.arange(nb)).astype(np.float64)
    out64 = np.zeros((B, Hq, v_dim), dtype=np.float64)
    Pm = np.zeros((B, Hq, n), dtype=np.float64)
    mask = np.zeros((B, Hq, n), dtype=bool)
    kept = np.zeros((B, Hq), dtype=np.float64)
    union = np.zeros((B, Hkv, n), dtype=bool)
    vmax = np.zeros((B, Hkv), dtype=np.float64)
    dropped = np.zeros((B, Hkv, nb), dtype=bool)
    margin = np.full((B, Hkv, nb), -np.inf)
    for b in range(B):
        kh = A.dequant_cache(fmt, k_codes[b:b + 1], k_scales[b:b + 1], dim, n)[0]
        vh = A.dequant_cache(fmt, v_codes[b:b + 1], v_scales[b:b + 1], v_dim, n)[0]
        for g in range(Hkv):
            heads = [h for h in range(Hq) if (h * Hkv) // Hq == g]
            Q = q[b, heads].astype(np.float64)
            S = sig * (Q @ kh[g].T)                      # [G][n]
            R32 = np.asarray(summary[b, g, :nb], dtype=np.float32)
            cand = R32 >= np.float32(RHO) * R32.max()
            R = R32.astype(np.float64)
            cpos = np.repeat(cand, block)[:n]
            Sc = S[:, cpos]
            mc = Sc.max(axis=1, keepdims=True)
            L = (mc + np.log(np.exp(Sc - mc).sum(axis=1, keepdims=True)))[:, 0]     # [G]
            ub = sig * np.linalg.norm(Q, axis=1)[:, None] * R[None, :]              # [G][nb]
            with np.errstate(divide="ignore"):                 # eps = 0: log 0 = -inf, nothing drops
                d = (ub - L[:, None] - np.log(eps / sizes)[None, :]).max(axis=0)    # [nb]
            drop = (d <= 0) & ~cand
            dropped[b, g] = drop
            margin[b, g] = d
            alive = ~np.repeat(drop, block)[:n]
            Sa = np.where(alive[None, :], S, -np.inf)
            m = Sa.max(axis=1, keepdims=True)
            E = np.exp(Sa - m)
            p = E / E.sum(axis=1, keepdims=True)
            keep = (p >= tau) & alive[None, :]
            out64[b, heads] = (p * keep) @ vh[g]
            Pm[b, heads] = p
            mask[b, heads] = keep
            kept[b, heads] = (p * keep).sum(axis=1)
            union[b, g] = keep.any(axis=0)
            vmax[b, g] = np.abs(vh[g]).max()
    res = A.Result(out=out64.astype(np.float32), out64=out64, p=Pm, mask=mask, kept_mass=kept, union=union,
                   kept_pairs=int(mask.sum()), rows_fetched=int(union.sum()), vmax=vmax)
    return res, dropped, margin


def _report():
    """Fractions of key rows the two bounds could drop on the synthetic
    workloads (first sequence of each): python -m oracle.kskip"""
    import synth
    from . import attend as A
    from . import formats as F
    for name in ("tiny", "long", "lut3", "stress", "mla"):
        w = synth.workload(name)
        w1 = synth.resized(w, batch=1)
        inp = synth.generate(w1)
        kc, ks = F.pack(w.fmt, inp.k)
        kh = A.dequant_cache(w.fmt, kc, ks, w.dim, w.ctx)[0]                  # [Hkv][n][D]
        q = inp.q[0].astype(np.float64)
        fr = {kind: dropped_fraction(q, kh, float(np.float32(w.sigma)), 64, kind) for kind in ("norm", "centroid")}
        print(f"{name:8s} fmt {w.fmt:9s} ctx {w.ctx:6d}  droppable key rows: norm bound {fr['norm']:.4f}, "
              f"centroid bound {fr['centroid']:.4f}", flush=True)


if __name__ == "__main__":
    _report()
