"""Device-buffer plumbing around the C ABI (torch supplies memory and streams).

``PackedCache`` holds the two byte planes of a cache on the GPU;
``DecodeAttention`` owns a workspace and calls ``kvq_decode_attn``. Neither
computes anything itself.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B


class PackedCache:
    """Code and scale planes [batch][heads][capacity][bytes] on a GPU."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor, fmt, dim: int, norms: torch.Tensor | None = None):
        assert codes.dtype == torch.uint8 and scales.dtype == torch.uint8
        assert codes.is_cuda and scales.is_cuda and codes.is_contiguous() and scales.is_contiguous()
        self.codes, self.scales, self.fmt, self.dim = codes, scales, B._fmt(fmt), int(dim)
        self.norms = norms          # optional float32 [batch][heads][ceil(capacity/64)] key-block summaries

    @classmethod
    def from_host(cls, codes: np.ndarray, scales: np.ndarray, fmt, dim: int, device="cuda"):
        c = torch.from_numpy(np.ascontiguousarray(codes)).to(device)
        s = torch.from_numpy(np.ascontiguousarray(scales)).to(device)
        return cls(c, s, fmt, dim)

    @property
    def shape(self):
        return tuple(self.codes.shape[:3])

    def struct(self) -> B.kvq_cache:
        return B.make_cache(self.codes, self.scales, self.dim, self.norms)

    def clone(self) -> "PackedCache":
        return PackedCache(self.codes.clone(), self.scales.clone(), self.fmt, self.dim,
                           None if self.norms is None else self.norms.clone())

    def compute_norms(self, stream=None) -> torch.Tensor:
        """(Re)compute every key-block summary on the GPU (kvq_key_norms_device)."""
        Bn, H, cap = self.shape
        if self.norms is None:
            self.norms = torch.zeros((Bn, H, (cap + 63) // 64), dtype=torch.float32, device=self.codes.device)
        B.kvq_key_norms_device(self.fmt, self.codes, self.scales, self.dim, self.norms, stream=stream)
        return self.norms

    @classmethod
    def empty(cls, fmt, batch: int, heads: int, capacity: int, dim: int, device="cuda"):
        cb, sb = B.kvq_row_bytes(fmt, dim)
        c = torch.zeros((batch, heads, capacity, cb), dtype=torch.uint8, device=device)
        s = torch.zeros((batch, heads, capacity, sb), dtype=torch.uint8, device=device)
        return cls(c, s, fmt, dim)

    def append(self, rows: torch.Tensor, positions: torch.Tensor, status: torch.Tensor | None = None,
               stream=None):
        """Quantize one new row per (batch, head) on the GPU into position
        ``positions[b]`` of sequence b: ``rows`` is float32 [batch][heads][dim]
        on the device, ``positions`` int64 [batch] on the device."""
        Bn, H, cap = self.shape
        assert rows.shape == (Bn, H, self.dim) and rows.dtype == torch.float32 and rows.is_contiguous()
        bh = torch.arange(Bn * H, device=rows.device, dtype=torch.int64).view(Bn, H)
        dst = (bh * cap + positions.to(torch.int64).view(Bn, 1)).contiguous()
        B.kvq_append(self.fmt, rows, dst, self.codes, self.scales, status, stream)


def append_kv(k: PackedCache, v: PackedCache, k_rows: torch.Tensor, v_rows: torch.Tensor, positions: torch.Tensor,
              status: torch.Tensor | None = None, stream=None):
    """One decode step's appends in one launch: the new key and value rows
    (float32 [batch][heads][dim] on the device) go to position ``positions[b]``
    of sequence b in both caches (same format, shape and width)."""
    Bn, H, cap = k.shape
    assert v.shape == k.shape and v.dim == k.dim and v.fmt == k.fmt
    assert k_rows.shape == (Bn, H, k.dim) and v_rows.shape == k_rows.shape
    bh = torch.arange(Bn * H, device=k_rows.device, dtype=torch.int64).view(Bn, H)
    dst = (bh * cap + positions.to(torch.int64).view(Bn, 1)).contiguous()
    B.kvq_append_kv(k.fmt, k_rows.contiguous(), v_rows.contiguous(), dst, k.codes, k.scales, v.codes, v.scales,
                    status, stream)


class DecodeAttention:
    """One decode-attention configuration with its own workspace."""

    def __init__(self, k: PackedCache, v: PackedCache | None, q_heads: int, *, ctx_len: int,
                 q_dtype=B.KVQ_Q_F32, softmax_scale: float = 0.0, v_dim: int = 0, splits: int = 0,
                 stream=None, cooperative: bool = False, running: bool = False, test_withhold: bool = False,
                 skip_keys: bool = False):
        self.k, self.v = k, v
        self.q_heads = q_heads
        self.fmt = k.fmt
        self.v_dim = v_dim if v is None else v.dim
        self.stream = stream
        self.launch_proto = dict(q_dtype=q_dtype, softmax_scale=softmax_scale,
                                 v_dim=v_dim if v is None else 0, splits=splits,
                                 flags=(B.KVQ_LAUNCH_COOPERATIVE if cooperative else 0)
                                 | (B.KVQ_SKIP_RUNNING if running else 0)
                                 | (B.KVQ_TEST_WITHHOLD if test_withhold else 0)
                                 | (B.KVQ_SKIP_KEYS if skip_keys else 0))
        probe = B.make_launch(q_heads, **self.launch_proto)
        nbytes = B.kvq_workspace_bytes(self.fmt, k.struct(), probe, ctx_len)
        # zero-filled on the launch stream, so the fill is ordered before the
        # first call (the epoch, tags and range counters must start at 0)
        with torch.cuda.stream(stream) if stream is not None else torch.cuda.device(k.codes.device):
            self.workspace = torch.zeros(nbytes, dtype=torch.uint8, device=k.codes.device)
        self._ks = k.struct()
        self._vs = v.struct() if v is not None else None

    def launch(self, mask_out=None, phase_times=None, key_skip_out=None) -> B.kvq_launch:
        return B.make_launch(self.q_heads, workspace=self.workspace, stream=self.stream, mask_out=mask_out,
                             phase_times=phase_times, key_skip_out=key_skip_out, **self.launch_proto)

    def __call__(self, q: torch.Tensor, ctx_len: int, threshold: float, out: torch.Tensor | None = None,
                 mask_out: torch.Tensor | None = None, k: PackedCache | None = None,
                 v: PackedCache | None = None, phase_times: torch.Tensor | None = None,
                 key_skip_out: torch.Tensor | None = None) -> torch.Tensor:
        bsz = self.k.shape[0]
        if out is None:
            out = torch.empty((bsz, self.q_heads, self.v_dim), dtype=torch.float32, device=q.device)
        ks = self._ks if k is None else k.struct()
        vs = self._vs if v is None else v.struct()
        B.kvq_decode_attn(q, ks, vs, self.fmt, ctx_len, threshold, out,
                          self.launch(mask_out, phase_times, key_skip_out))
        return out

    def stats(self):
        return B.kvq_stats(self.launch())

    def phase_profile(self, q, ctx_len: int, threshold: float, **kw) -> np.ndarray:
        """Run one call with phase stamps; returns int64 [workgroups][stamps]
        device wall-clock ticks (100 MHz) relative to the earliest stamp."""
        buf = torch.zeros((1 << 16, 16), dtype=torch.int64, device=q.device)
        self(q, ctx_len, threshold, phase_times=buf, **kw)
        nwg, ns = B.kvq_phase_count(self.launch())
        t = buf[:nwg, :ns].cpu().numpy()
        return t - t[:, 0].min()


def mask_words(ctx_len: int) -> int:
    return (ctx_len + 31) // 32


def unpack_mask(words: np.ndarray, ctx_len: int) -> np.ndarray:
    """uint32 [..., W] keep bits -> bool [..., ctx_len]."""
    w = np.ascontiguousarray(words, dtype=np.uint32)
    bits = np.unpackbits(w.view(np.uint8), axis=-1, bitorder="little")
    return bits[..., :ctx_len].astype(bool)
