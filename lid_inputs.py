"""Seeded synthetic inputs for the lightning-indexer top-k.

This module only draws random numbers and builds visibility structure (causal
masks, per-query key ranges).  It holds none of the indexer's arithmetic, so
both the CPU oracle and the HIP path can be fed from it without sharing code.

Workloads (shapes from the DeepSeek-V4-Flash indexer as described in ggml-org
llama.cpp issue 25468, "Root cause" comment: 64 indexer heads, head size 128,
a top-512 selection, f16 indexer keys compressed 4x along the context):

  c1     tiny:  n_tok 4,    n_kv 256,     H 4,  D 32,  k_top 16,  f32, w~U(0,1)
  c2     decode: n_tok 1,   n_kv 32768,   H 64, D 128, k_top 512, f16, no mask
  c3     prefill: n_tok 512, n_kv 16384,  causal f16 mask, last 512 positions
  c4     long prefill: n_tok 2048, n_kv 131072, causal f16 mask
  c5     multi-sequence: 4 seqs x 512 queries, 4 key blocks x 262144, each
         query sees only the causal prefix of its own block
  dec1m  decode with n_kv 1048576 (the 1M-key bandwidth point)

Recipe: numpy PCG64 (default_rng(seed)); draw q, then k, then w, all in C
order.  q, k ~ N(0,1)/sqrt(D) drawn in float32 and rounded to f16 with IEEE
round-to-nearest-even for the f16 workloads; w ~ U(0,1) (divided by H except
for c1).  Mask values are f16 +0 (visible) or f16 -inf (not visible).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

F16_NEG_INF = np.uint16(0xFC00)
F16_ZERO = np.uint16(0x0000)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_tok: int
    n_kv: int
    n_head: int
    head_dim: int
    k_top: int
    dtype: str            # "f32" | "f16" | "bf16" for q and k
    w_div_h: bool         # w ~ U(0,1)/H when True, U(0,1) otherwise
    visibility: str       # "none" | "causal" | "multiseq"
    n_seq: int = 1        # number of sequences (multiseq only)

    @property
    def desc(self) -> str:
        return (f"{self.name}: n_tok={self.n_tok} n_kv={self.n_kv} H={self.n_head} "
                f"D={self.head_dim} k_top={self.k_top} {self.dtype} {self.visibility}")


WORKLOADS = {
    "c1": Workload("c1", 4, 256, 4, 32, 16, "f32", False, "causal"),
    "c2": Workload("c2", 1, 32768, 64, 128, 512, "f16", True, "none"),
    "c3": Workload("c3", 512, 16384, 64, 128, 512, "f16", True, "causal"),
    "c4": Workload("c4", 2048, 131072, 64, 128, 512, "f16", True, "causal"),
    "c5": Workload("c5", 2048, 1048576, 64, 128, 512, "f16", True, "multiseq", n_seq=4),
    "dec1m": Workload("dec1m", 1, 1048576, 64, 128, 512, "f16", True, "none"),
}


def _round_qk(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 draw -> storage dtype (bf16 is returned as its uint16 bit pattern)."""
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        # round-to-nearest-even on the dropped 16 bits (inputs are finite)
        lsb = (u >> 16) & 1
        r = (u + 0x7FFF + lsb) >> 16
        return r.astype(np.uint16)
    raise ValueError(dtype)


def draw_qkw(n_tok, n_kv, n_head, head_dim, dtype="f16", w_div_h=True, seed=0):
    """q [n_tok,H,D], k [n_kv,D] (storage dtype) and w [n_tok,H] float32."""
    rng = np.random.default_rng(seed)
    s = np.float32(1.0 / math.sqrt(head_dim))
    q = rng.standard_normal((n_tok, n_head, head_dim), dtype=np.float32) * s
    k = rng.standard_normal((n_kv, head_dim), dtype=np.float32) * s
    w = rng.random((n_tok, n_head), dtype=np.float32)
    if w_div_h:
        w = w / np.float32(n_head)
    return _round_qk(q, dtype), _round_qk(k, dtype), np.ascontiguousarray(w, dtype=np.float32)


def draw_attn(n_tok, n_kv, n_head, latent_dim, dtype="f16", seed=0):
    """Sparse-attention operands: qa [n_tok,H,L] and kv [n_kv,L], standard
    normal, in the storage dtype (bf16 as uint16 bit patterns)."""
    rng = np.random.default_rng(seed)
    qa = rng.standard_normal((n_tok, n_head, latent_dim), dtype=np.float32)
    kv = rng.standard_normal((n_kv, latent_dim), dtype=np.float32)
    return _round_qk(qa, dtype), _round_qk(kv, dtype)


def draw_selection(n_tok, n_kv, k_sel, seed=0):
    """int32 [n_tok, k_sel]: k_sel distinct random keys per query (any order),
    the shape of a full top-k selection."""
    rng = np.random.default_rng(seed)
    if k_sel > n_kv:
        raise ValueError("k_sel > n_kv")
    return np.argsort(rng.random((n_tok, n_kv), dtype=np.float32), axis=1)[:, :k_sel].astype(np.int32)


def visible_ranges(wl: Workload) -> np.ndarray | None:
    """Per-query half-open visible key range [lo, hi) as int32 [n_tok, 2], or None.

    causal:   query t sits at position n_kv - n_tok + t and sees keys s <= that.
    multiseq: query j of sequence b sits at in-block position B - Q + j of key
              block b (B keys per block, Q queries per sequence) and sees the
              causal prefix of its own block only.
    """
    if wl.visibility == "none":
        return None
    t = np.arange(wl.n_tok, dtype=np.int64)
    if wl.visibility == "causal":
        lo = np.zeros_like(t)
        hi = wl.n_kv - wl.n_tok + t + 1
    elif wl.visibility == "multiseq":
        q_per = wl.n_tok // wl.n_seq
        blk = wl.n_kv // wl.n_seq
        b = t // q_per
        j = t % q_per
        lo = b * blk
        hi = b * blk + (blk - q_per) + j + 1
    else:
        raise ValueError(wl.visibility)
    return np.stack([lo, hi], axis=1).astype(np.int32)


def mask_from_ranges(ranges: np.ndarray, n_kv: int, mask_ld: int | None = None) -> np.ndarray:
    """Dense f16 additive mask (uint16 bit patterns) [n_tok, mask_ld]: +0 inside
    [lo, hi), -inf outside (including the padding columns beyond n_kv)."""
    ld = n_kv if mask_ld is None else mask_ld
    s = np.arange(ld, dtype=np.int64)[None, :]
    vis = (s >= ranges[:, :1]) & (s < ranges[:, 1:2]) & (s < n_kv)
    return np.where(vis, F16_ZERO, F16_NEG_INF).astype(np.uint16)


def mask_from_ranges_torch(ranges, n_kv: int, device, mask_ld: int | None = None):
    """Same as mask_from_ranges, built directly in device memory (torch)."""
    import torch
    ld = n_kv if mask_ld is None else mask_ld
    r = torch.as_tensor(ranges, device=device).to(torch.int64)
    s = torch.arange(ld, device=device, dtype=torch.int64)[None, :]
    vis = (s >= r[:, :1]) & (s < r[:, 1:2]) & (s < n_kv)
    z = torch.zeros((), dtype=torch.float16, device=device)
    ninf = torch.full((), float("-inf"), dtype=torch.float16, device=device)
    return torch.where(vis, z, ninf)


def make(name: str, seed: int = 0, with_mask: bool = True):
    """All host-side inputs of a named workload.

    Returns dict(wl, q, k, w, ranges, mask). `mask` is the dense f16 mask
    (uint16 bits) when the workload has visibility structure and with_mask is
    True (never built for c5, whose dense mask would be 4 GiB; use ranges or
    mask_from_ranges_torch there)."""
    wl = WORKLOADS[name]
    q, k, w = draw_qkw(wl.n_tok, wl.n_kv, wl.n_head, wl.head_dim, wl.dtype, wl.w_div_h, seed)
    ranges = visible_ranges(wl)
    mask = None
    if ranges is not None and with_mask and wl.n_tok * wl.n_kv <= (1 << 28):
        mask = mask_from_ranges(ranges, wl.n_kv)
    return dict(wl=wl, q=q, k=k, w=w, ranges=ranges, mask=mask)
