"""K-side skipping: how many key rows a provable score bound could leave out.

TEST INFRASTRUCTURE ONLY (see the package docstring); the kernels do not
skip keys. This module answers, on given inputs, the question the sparse-V
page leaves as future work.

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
