"""CPU oracle for the fused lightning-indexer top-k (ctypes wrapper over lid_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does, and
the two share no code.  See lid_oracle.c for what is computed and which
passage of the pages each step follows.

Parity pins (tests/test_oracle*.py): a hand-worked golden example, the H=1/D=1
closed form (a plain sort), the q=0 tie case, exhaustive f16/bf16 decode
against numpy, rank-count brute force on tiny inputs, and the invariants
(masked keys never chosen, <=k_top visible keys all returned, selected >=
unselected, key permutation, inert w=0 head, linearity in w).  The shared
(per-ubatch) top-k is pinned by its one-query case (the per-query top-k), a
numpy brute force, identical queries (U = n_tok v) and the -inf rule.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lid_oracle.c")
_LIB = os.path.join(_HERE, "liblid_oracle.so")

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "f8e4m3": 3}
_lib = None


def compile_source(src: str, out: str) -> str:
    """gcc -O2 with OpenMP and no FP contraction; returns the .so path."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile lid_oracle.c into liblid_oracle.so next to it."""
    if force or not os.path.exists(_LIB):
        compile_source(_SRC, _LIB)
    return _LIB


def load_library(path: str):
    """ctypes handle of an oracle build at `path` (argument types declared)."""
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.lid_oracle_topk.restype = ctypes.c_int
    lib.lid_oracle_topk.argtypes = [i64, i64, i32, i32, i32, i32, vp, vp, vp, vp, i64, vp,
                                    vp, vp, vp, i32]
    lib.lid_oracle_scores.restype = ctypes.c_int
    lib.lid_oracle_scores.argtypes = [i64, i64, i32, i32, i32, vp, vp, vp, vp, i64, vp, vp, i32]
    lib.lid_oracle_topk_scaled.restype = ctypes.c_int
    lib.lid_oracle_topk_scaled.argtypes = [i64, i64, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, i64, vp,
                                           vp, vp, vp, i32]
    lib.lid_oracle_topk_shared.restype = ctypes.c_int
    lib.lid_oracle_topk_shared.argtypes = [i64, i64, i32, i32, i32, i32, vp, vp, vp, vp, i64, vp, vp, vp, vp, i32]
    lib.lid_oracle_sparse_attn.restype = ctypes.c_int
    lib.lid_oracle_sparse_attn.argtypes = [i64, i64, i32, i32, i32, i32, vp, vp, vp, ctypes.c_double, vp, i32]
    lib.lid_oracle_scores_scaled.restype = ctypes.c_int
    lib.lid_oracle_scores_scaled.argtypes = [i64, i64, i32, i32, i32, vp, vp, vp, vp, vp, vp, i64, vp, vp, i32]
    lib.lid_oracle_f8e4m3_to_f64.restype = ctypes.c_double
    lib.lid_oracle_f8e4m3_to_f64.argtypes = [ctypes.c_uint8]
    lib.lid_oracle_f16_to_f64.restype = ctypes.c_double
    lib.lid_oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.lid_oracle_bf16_to_f64.restype = ctypes.c_double
    lib.lid_oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _lib = load_library(_LIB)
    return _lib


class Oracle:
    """The oracle's Python API bound to one compiled library (the default
    build, or a deliberately broken copy in the mutation tests)."""

    def __init__(self, lib):
        self._lib = lib

    def topk(self, *a, **kw):
        return topk(*a, _lib=self._lib, **kw)

    def scores(self, *a, **kw):
        return scores(*a, _lib=self._lib, **kw)

    def topk_shared(self, *a, **kw):
        return topk_shared(*a, _lib=self._lib, **kw)

    def sparse_attn(self, *a, **kw):
        return sparse_attn(*a, _lib=self._lib, **kw)

    def f16_to_f64(self, bits):
        return self._lib.lid_oracle_f16_to_f64(bits)

    def bf16_to_f64(self, bits):
        return self._lib.lid_oracle_bf16_to_f64(bits)

    def f8e4m3_to_f64(self, bits):
        return self._lib.lid_oracle_f8e4m3_to_f64(bits)


def _dtype_of(x: np.ndarray, qk_dtype: str | None) -> str:
    if qk_dtype is not None:
        return qk_dtype
    if x.dtype == np.float32:
        return "f32"
    if x.dtype == np.float16:
        return "f16"
    raise ValueError("pass qk_dtype='bf16' for uint16 bf16 bit patterns, 'f8e4m3' for uint8 E4M3 bytes")


def _ptr(a):
    return None if a is None else a.ctypes.data


def _prep(q, k, w, mask, kv_range, qk_dtype, rows):
    dt = _dtype_of(q, qk_dtype)
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        q, w = q[rows], w[rows]
        mask = None if mask is None else mask[rows]
        kv_range = None if kv_range is None else kv_range[rows]
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    w = np.ascontiguousarray(w, dtype=np.float32)
    if mask is not None:
        mask = np.ascontiguousarray(mask).view(np.uint16)
    if kv_range is not None:
        kv_range = np.ascontiguousarray(kv_range, dtype=np.int32)
    return q, k, w, mask, kv_range, dt


def _scales(q_scale, k_scale, rows):
    if q_scale is None and k_scale is None:
        return None, None
    if q_scale is None or k_scale is None:
        raise ValueError("q_scale and k_scale go together")
    q_scale = np.asarray(q_scale, dtype=np.float32)
    if rows is not None:
        q_scale = q_scale[np.asarray(rows, dtype=np.int64)]
    return np.ascontiguousarray(q_scale), np.ascontiguousarray(k_scale, dtype=np.float32)


def topk(q, k, w, mask=None, kv_range=None, k_top=512, qk_dtype=None, rows=None, threads=0,
         q_scale=None, k_scale=None, _lib=None):
    """Oracle top-k.  Returns (idx int32 [n,k_top], score f32 [n,k_top], maxabs).

    rows: optional query subset (the oracle then runs only those rows).
    q_scale [n_tok, H], k_scale [n_kv] (f32): per-row scales of q and k
    (the FP8 convention; both or neither)."""
    qs, ks = _scales(q_scale, k_scale, rows)
    q, k, w, mask, kv_range, dt = _prep(q, k, w, mask, kv_range, qk_dtype, rows)
    n_tok, H, D = q.shape
    n_kv = k.shape[0]
    idx = np.empty((n_tok, k_top), dtype=np.int32)
    score = np.empty((n_tok, k_top), dtype=np.float32)
    maxabs = ctypes.c_double(0.0)
    mask_ld = 0 if mask is None else mask.shape[1]
    lib = _lib or _load()
    if qs is not None:
        rc = lib.lid_oracle_topk_scaled(n_tok, n_kv, H, D, k_top, DTYPE_CODE[dt], _ptr(q), _ptr(qs), _ptr(k),
                                        _ptr(ks), _ptr(w), _ptr(mask), mask_ld, _ptr(kv_range), _ptr(idx),
                                        _ptr(score), ctypes.addressof(maxabs), threads)
    else:
        rc = lib.lid_oracle_topk(n_tok, n_kv, H, D, k_top, DTYPE_CODE[dt], _ptr(q), _ptr(k), _ptr(w),
                                 _ptr(mask), mask_ld, _ptr(kv_range), _ptr(idx), _ptr(score),
                                 ctypes.addressof(maxabs), threads)
    if rc != 0:
        raise RuntimeError(f"lid_oracle_topk failed: {rc}")
    return idx, score, maxabs.value


def scores(q, k, w, mask=None, kv_range=None, qk_dtype=None, rows=None, threads=0, q_scale=None, k_scale=None,
           _lib=None):
    """Full masked f32 score matrix [n, n_kv] (-inf where not visible)."""
    qs, ks = _scales(q_scale, k_scale, rows)
    q, k, w, mask, kv_range, dt = _prep(q, k, w, mask, kv_range, qk_dtype, rows)
    n_tok, H, D = q.shape
    n_kv = k.shape[0]
    v = np.empty((n_tok, n_kv), dtype=np.float32)
    mask_ld = 0 if mask is None else mask.shape[1]
    lib = _lib or _load()
    if qs is not None:
        rc = lib.lid_oracle_scores_scaled(n_tok, n_kv, H, D, DTYPE_CODE[dt], _ptr(q), _ptr(qs), _ptr(k), _ptr(ks),
                                          _ptr(w), _ptr(mask), mask_ld, _ptr(kv_range), _ptr(v), threads)
    else:
        rc = lib.lid_oracle_scores(n_tok, n_kv, H, D, DTYPE_CODE[dt], _ptr(q), _ptr(k), _ptr(w),
                                   _ptr(mask), mask_ld, _ptr(kv_range), _ptr(v), threads)
    if rc != 0:
        raise RuntimeError(f"lid_oracle_scores failed: {rc}")
    return v


def topk_shared(q, k, w, mask=None, kv_range=None, k_top=512, qk_dtype=None, threads=0, _lib=None):
    """Oracle shared (per-ubatch) top-k: the k_top keys with the largest
    U[s] = sum_t v[t,s] over all queries.  Returns (idx int32 [k_top],
    score f32 [k_top], maxabs = max |U| over the selectable keys)."""
    q, k, w, mask, kv_range, dt = _prep(q, k, w, mask, kv_range, qk_dtype, None)
    n_tok, H, D = q.shape
    n_kv = k.shape[0]
    idx = np.empty(k_top, dtype=np.int32)
    score = np.empty(k_top, dtype=np.float32)
    maxabs = ctypes.c_double(0.0)
    mask_ld = 0 if mask is None else mask.shape[1]
    lib = _lib or _load()
    rc = lib.lid_oracle_topk_shared(n_tok, n_kv, H, D, k_top, DTYPE_CODE[dt], _ptr(q), _ptr(k), _ptr(w),
                                    _ptr(mask), mask_ld, _ptr(kv_range), _ptr(idx), _ptr(score),
                                    ctypes.addressof(maxabs), threads)
    if rc != 0:
        raise RuntimeError(f"lid_oracle_topk_shared failed: {rc}")
    return idx, score, maxabs.value


def sparse_attn(qa, kv, idx, scale, qk_dtype=None, threads=0, _lib=None):
    """Oracle sparse attention over the selected latent rows: o [n_tok, H, L]
    float64 = softmax(scale * qa . kv[idx]) . kv[idx] per (query, head); idx
    entries outside [0, n_kv) are skipped (none valid: o = 0)."""
    dt = _dtype_of(qa, qk_dtype)
    qa = np.ascontiguousarray(qa)
    kv = np.ascontiguousarray(kv)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    n_tok, H, L = qa.shape
    n_kv = kv.shape[0]
    k_sel = idx.shape[1] if idx.ndim == 2 else 0
    out = np.empty((n_tok, H, L), dtype=np.float64)
    lib = _lib or _load()
    rc = lib.lid_oracle_sparse_attn(n_tok, n_kv, H, L, k_sel, DTYPE_CODE[dt], _ptr(qa), _ptr(kv), _ptr(idx),
                                    float(scale), _ptr(out), threads)
    if rc != 0:
        raise RuntimeError(f"lid_oracle_sparse_attn failed: {rc}")
    return out


def f16_to_f64(bits: int) -> float:
    return _load().lid_oracle_f16_to_f64(bits)


def bf16_to_f64(bits: int) -> float:
    return _load().lid_oracle_bf16_to_f64(bits)


def f8e4m3_to_f64(bits: int) -> float:
    return _load().lid_oracle_f8e4m3_to_f64(bits)
