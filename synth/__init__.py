"""Seeded synthetic inputs for single-token decode attention over a quantized KV cache.

This module only draws and shapes fp32 inputs (queries, keys, values, planted
"hot" positions). It holds none of the method's arithmetic: no quantization,
no scores, no softmax. Both the CPU oracle and the GPU path take their inputs
from here, and each packs and attends on its own.

Workloads (sizes as named in the method's evaluation; the Russian-language news
page on sparse V dequantization, section "Результаты", measures decode at
contexts 4K-32K, and its "Что такое разреженность внимания?" paragraph says
attention at long context concentrates on a few dozen positions while more
than 90% of weights fall below 1e-6):

- ``tiny``      q8_0, batch 1, 4 query heads / 1 KV head, dim 128, ctx 1024,
                8 hot positions (hot j serves head j mod 4, key = 3*sqrt(128)*q/|q|).
- ``long``      q4_0, batch 1, 32/4 heads, dim 128, ctx 32768, 32 hot positions
                per KV head, each raising every head's scaled logit by exactly +20.
- ``sweep_<n>`` ``long`` at ctx n in {4096, ..., 65536}, 16*log2(n/1024) hot.
- ``lut3``      3-bit LUT codebook, batch 8, 32/4 heads, ctx 32768, sequence b
                has 8*(b+1) hot positions per KV head.
- ``lut3_wht``  ``lut3`` (same seed, so the same arrays) stored as the
                Walsh-Hadamard-rotated LUT3 format.
- ``mla``       128 query heads over one 576-wide latent (512 value dims + 64 rope),
                fp8 e4m3 blocks of 128, bf16 queries, ctx 65536, batch 8, 96 hot
                positions per sequence shared by all heads, softmax scale 1/sqrt(192)
                (the kernelindex page on FP8 MLA KV compression lists
                qk_nope_head_dim 128 + qk_rope_head_dim 64).
- ``stress``    ``long`` shape with keys drawn 4.5*N(0,1) and no hot positions, so
                about 8% of weights per head survive the 1e-6 threshold.

Every array is float32 (queries for ``mla`` are float32 values that are exactly
bfloat16). Draw order per seed: q, K, V, hot positions (sorted, per sequence and
KV head), then the boost.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

FMT_Q8_0 = "q8_0"
FMT_Q4_0 = "q4_0"
FMT_LUT3 = "lut3"
FMT_LUT3_WHT = "lut3_wht"
FMT_FP8 = "fp8_b128"

THRESHOLD = 1e-6
LOGIT_BOOST = 20.0


@dataclasses.dataclass
class Workload:
    name: str
    fmt: str
    batch: int
    q_heads: int
    kv_heads: int
    dim: int            # key dim (latent width for mla)
    v_dim: int          # value dim (leading dims of the latent for mla)
    ctx: int
    seed: int
    sigma: float        # softmax scale, an exact float32 value
    q_bf16: bool = False
    hot: object = None  # callable (b) -> hot count per kv head, or int
    key_std: float = 1.0
    threshold: float = THRESHOLD
    hot_mode: str = "boost"   # "boost": +20 on every head's logit; "align": key = 3*sqrt(D)*q/|q|

    @property
    def latent(self) -> bool:
        return self.fmt == FMT_FP8


def _f32(x: float) -> float:
    return float(np.float32(x))


def workload(name: str) -> Workload:
    """Return the named workload's shape and seed (no arrays are drawn)."""
    if name == "tiny":
        return Workload(name, FMT_Q8_0, 1, 4, 1, 128, 128, 1024, 0, _f32(1 / math.sqrt(128)), hot=8,
                        hot_mode="align")
    if name == "long":
        return Workload(name, FMT_Q4_0, 1, 32, 4, 128, 128, 32768, 1, _f32(1 / math.sqrt(128)), hot=32)
    if name.startswith("sweep_"):
        n = int(name.split("_")[1])
        hot = int(round(16 * math.log2(n / 1024)))
        return Workload(name, FMT_Q4_0, 1, 32, 4, 128, 128, n, 2, _f32(1 / math.sqrt(128)), hot=hot)
    if name == "lut3":
        return Workload(name, FMT_LUT3, 8, 32, 4, 128, 128, 32768, 4, _f32(1 / math.sqrt(128)),
                        hot=lambda b: 8 * (b + 1))
    if name == "lut3_wht":
        return Workload(name, FMT_LUT3_WHT, 8, 32, 4, 128, 128, 32768, 4, _f32(1 / math.sqrt(128)),
                        hot=lambda b: 8 * (b + 1))
    if name == "mla":
        return Workload(name, FMT_FP8, 8, 128, 1, 576, 512, 65536, 5, _f32(1 / math.sqrt(192)),
                        q_bf16=True, hot=96)
    if name == "stress":
        return Workload(name, FMT_Q4_0, 1, 32, 4, 128, 128, 32768, 3, _f32(1 / math.sqrt(128)),
                        hot=0, key_std=4.5)
    raise KeyError(name)


SWEEP = [4096, 8192, 16384, 32768, 65536]
ALL = ["tiny", "long"] + [f"sweep_{n}" for n in SWEEP] + ["lut3", "lut3_wht", "mla", "stress"]


def resized(w: Workload, *, batch=None, q_heads=None, kv_heads=None, ctx=None, hot=None,
            seed=None, fmt=None, dim=None, v_dim=None, key_std=None, hot_mode=None,
            threshold=None) -> Workload:
    """A smaller (or reshaped) copy of a workload for tests; same value recipe."""
    d = dataclasses.asdict(w)
    d["hot"] = w.hot
    for k, v in dict(batch=batch, q_heads=q_heads, kv_heads=kv_heads, ctx=ctx, hot=hot,
                     seed=seed, fmt=fmt, dim=dim, v_dim=v_dim, key_std=key_std,
                     hot_mode=hot_mode, threshold=threshold).items():
        if v is not None:
            d[k] = v
    if fmt is not None and fmt != FMT_FP8 and v_dim is None:
        d["v_dim"] = d["dim"]
    return Workload(**d)


def _hot_count(w: Workload, b: int) -> int:
    h = w.hot
    if callable(h):
        return int(h(b))
    return int(h or 0)


def _to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even); return as float32."""
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


@dataclasses.dataclass
class Inputs:
    w: Workload
    q: np.ndarray          # [B][Hq][D] float32
    k: np.ndarray          # [B][Hkv][ctx][D] float32
    v: np.ndarray | None   # [B][Hkv][ctx][Dv] float32 (None for a latent cache)
    hot: list              # hot[b][g] -> sorted int array of positions


def generate(w: Workload) -> Inputs:
    """Draw the workload's inputs (deterministic in ``w.seed``)."""
    rng = np.random.default_rng(w.seed)
    B, Hq, Hkv, D, n = w.batch, w.q_heads, w.kv_heads, w.dim, w.ctx
    q = rng.standard_normal((B, Hq, D), dtype=np.float32)
    if w.q_bf16:
        q = _to_bf16_values(q)
    k = rng.standard_normal((B, Hkv, n, D), dtype=np.float32)
    if w.key_std != 1.0:
        k *= np.float32(w.key_std)
    v = None
    if not w.latent:
        v = rng.standard_normal((B, Hkv, n, w.v_dim), dtype=np.float32)
    hot = []
    for b in range(B):
        row = []
        for g in range(Hkv):
            c = min(_hot_count(w, b), n)
            row.append(np.sort(rng.choice(n, size=c, replace=False)) if c else np.zeros(0, np.int64))
        hot.append(row)

    G = Hq // Hkv
    for b in range(B):
        for g in range(Hkv):
            pos = hot[b][g]
            if len(pos) == 0:
                continue
            Q = q[b, g * G:(g + 1) * G].astype(np.float64)          # G x D
            if w.hot_mode == "align":
                # hot j serves head j mod G: key = 3*sqrt(D) * q_h / |q_h|
                for j, i in enumerate(pos):
                    qh = Q[j % G]
                    k[b, g, i] = (3.0 * math.sqrt(D) * qh / np.linalg.norm(qh)).astype(np.float32)
            else:
                # least-norm vector u with sigma * Q u = +20 for every head of the group
                rhs = np.full(G, LOGIT_BOOST / w.sigma)
                u = Q.T @ np.linalg.solve(Q @ Q.T, rhs)
                k[b, g, pos] = (k[b, g, pos].astype(np.float64) + u).astype(np.float32)
    return Inputs(w, q, k, v, hot)
