"""Fused lightning-indexer top-k for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI in include/lid.h (liblid.so, built in place
by sparse_attention_token_lid_amd/build.py).  This module only marshals
arguments: torch provides device memory and the current HIP stream, and every
step of scoring and selection runs in the library's HIP kernels.  There is no
CPU fallback: if liblid.so is missing, calls raise.

    idx, score = topk(q, k, w, mask=None, kv_range=None, k_top=512)

q [n_tok, H, D] and k [n_kv, D] in float16 / bfloat16 / float32, w [n_tok, H]
float32, mask [n_tok, >= n_kv] float16 (additive; -inf = not visible) or None,
kv_range [n_tok, 2] int32 half-open [lo, hi) per query or None.  Returns
idx int32 [n_tok, k_top] and score float32 [n_tok, k_top], sorted by score
descending then index ascending, padded with -1 / -inf.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblid.so")

LID_F32, LID_F16, LID_BF16, LID_F8E4M3 = 0, 1, 2, 3
PLAN_AUTO, PLAN_GENERIC, PLAN_PREFILL, PLAN_DECODE = 0, 1, 2, 3
PLAN_NAMES = {PLAN_GENERIC: "generic", PLAN_PREFILL: "prefill", PLAN_DECODE: "decode"}
STATUS = {0: "LID_OK", -1: "LID_ERR_INVALID_ARG", -2: "LID_ERR_UNSUPPORTED", -3: "LID_ERR_WORKSPACE",
          -4: "LID_ERR_HIP"}
EXPORTS = ("lid_topk", "lid_topk_noalloc", "lid_topk_fp8", "lid_topk_workspace_size", "lid_topk_plan", "lid_scores",
           "lid_topk_shared", "lid_topk_shared_workspace_size", "lid_sparse_attn",
           "lid_status_string", "lid_last_hip_error", "lid_set_profile_events", "lid_version")


class LidShape(ctypes.Structure):
    """Mirror of lid_shape (include/lid.h)."""
    _fields_ = [("n_tok", ctypes.c_int64), ("n_kv", ctypes.c_int64), ("n_head", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("k_top", ctypes.c_int32), ("qk_dtype", ctypes.c_int32),
                ("mask_ld", ctypes.c_int64), ("plan", ctypes.c_int32), ("splits", ctypes.c_int32)]


class LidError(RuntimeError):
    def __init__(self, status: int, what: str = "lid_topk"):
        self.status = status
        msg = f"{what} failed: {STATUS.get(status, status)}"
        if status == -4 and _lib is not None:
            msg += f" ({_lib.lid_last_hip_error().decode()})"
        super().__init__(msg)


_lib = None


def load():
    """The ctypes handle of liblid.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        # torch ships its own HIP runtime; importing it first makes liblid.so
        # bind to that same runtime (one runtime per process, so torch's
        # streams and memory are valid handles for the library)
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not found: run `python -m sparse_attention_token_lid_amd.build` "
                               "(or __graft_entry__.build()); there is no fallback path")
        lib = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        lib.lid_topk.restype = ctypes.c_int
        lib.lid_topk.argtypes = [ctypes.POINTER(LidShape), vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.lid_topk_noalloc.restype = ctypes.c_int
        lib.lid_topk_noalloc.argtypes = [ctypes.POINTER(LidShape), vp, vp, vp, vp, vp, vp, vp, vp]
        lib.lid_topk_workspace_size.restype = ctypes.c_size_t
        lib.lid_topk_workspace_size.argtypes = [ctypes.POINTER(LidShape)]
        lib.lid_topk_fp8.restype = ctypes.c_int
        lib.lid_topk_fp8.argtypes = [ctypes.POINTER(LidShape), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                     ctypes.c_size_t, vp]
        lib.lid_scores.restype = ctypes.c_int
        lib.lid_scores.argtypes = [ctypes.POINTER(LidShape), vp, vp, vp, vp, vp, vp, ctypes.c_int64, vp]
        lib.lid_topk_shared.restype = ctypes.c_int
        lib.lid_topk_shared.argtypes = [ctypes.POINTER(LidShape), vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.lid_topk_shared_workspace_size.restype = ctypes.c_size_t
        lib.lid_topk_shared_workspace_size.argtypes = [ctypes.POINTER(LidShape)]
        lib.lid_sparse_attn.restype = ctypes.c_int
        lib.lid_sparse_attn.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, vp, vp, vp, ctypes.c_float, vp, vp]
        lib.lid_topk_plan.restype = ctypes.c_int
        lib.lid_topk_plan.argtypes = [ctypes.POINTER(LidShape), ctypes.POINTER(ctypes.c_int32)]
        lib.lid_status_string.restype = ctypes.c_char_p
        lib.lid_status_string.argtypes = [ctypes.c_int]
        lib.lid_last_hip_error.restype = ctypes.c_char_p
        lib.lid_last_hip_error.argtypes = []
        lib.lid_set_profile_events.restype = None
        lib.lid_set_profile_events.argtypes = [vp, vp]
        lib.lid_version.restype = ctypes.c_int
        lib.lid_version.argtypes = []
        _lib = lib
    return _lib


def make_shape(n_tok, n_kv, n_head, head_dim, k_top, qk_dtype=LID_F16, mask_ld=0, plan=PLAN_AUTO, splits=0):
    return LidShape(int(n_tok), int(n_kv), int(n_head), int(head_dim), int(k_top), int(qk_dtype), int(mask_ld),
                    int(plan), int(splits))


def workspace_size(shape: LidShape) -> int:
    return int(load().lid_topk_workspace_size(ctypes.byref(shape)))


def plan_of(shape: LidShape):
    """(plan name, splits) that lid_topk would run; raises LidError if invalid."""
    sp = ctypes.c_int32(0)
    rc = load().lid_topk_plan(ctypes.byref(shape), ctypes.byref(sp))
    if rc < 0:
        raise LidError(rc, "lid_topk_plan")
    return PLAN_NAMES[rc], sp.value


def _dtype_code(t):
    import torch
    return {torch.float16: LID_F16, torch.bfloat16: LID_BF16, torch.float32: LID_F32,
            torch.float8_e4m3fn: LID_F8E4M3}[t.dtype]


def shape_for(q, k, k_top, mask=None, plan=PLAN_AUTO, splits=0) -> LidShape:
    n_tok, H, D = q.shape
    return make_shape(n_tok, k.shape[0], H, D, k_top, _dtype_code(q), mask.shape[1] if mask is not None else 0,
                      plan, splits)


def _ptr(t):
    return None if t is None else t.data_ptr()


def topk(q, k, w, mask=None, kv_range=None, k_top=512, *, plan=PLAN_AUTO, splits=0, idx=None, score=None,
         want_score=True, workspace=None, stream=None, q_scale=None, k_scale=None):
    """Fused score + mask + top-k on the GPU (see module docstring).  With
    float8_e4m3fn q and k, q_scale [n_tok, H] and k_scale [n_kv] (f32) are
    their per-row scales (lid_topk_fp8)."""
    import torch
    if q.dim() != 3 or k.dim() != 2 or w.dim() != 2:
        raise ValueError("q [n_tok,H,D], k [n_kv,D], w [n_tok,H] expected")
    n_tok, H, D = q.shape
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("lid.topk runs on the GPU only (q is on %s)" % dev)
    for name, t in (("q", q), ("k", k), ("w", w), ("mask", mask), ("kv_range", kv_range)):
        if t is not None and (t.device != dev or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous tensor on {dev}")
    if k.dtype != q.dtype or k.shape[1] != D or w.shape != (n_tok, H) or w.dtype != torch.float32:
        raise ValueError("dtype/shape mismatch among q, k, w")
    if mask is not None:
        if mask.dtype not in (torch.float16, torch.int16, torch.uint16) or mask.dim() != 2 or mask.shape[0] != n_tok:
            raise ValueError("mask must be float16 [n_tok, mask_ld]")
    if kv_range is not None and (kv_range.dtype != torch.int32 or tuple(kv_range.shape) != (n_tok, 2)):
        raise ValueError("kv_range must be int32 [n_tok, 2]")
    fp8 = q.dtype == torch.float8_e4m3fn
    if fp8:
        if q_scale is None or k_scale is None:
            raise ValueError("FP8 q and k need q_scale [n_tok, H] and k_scale [n_kv]")
        for name, t, shp in (("q_scale", q_scale, (n_tok, H)), ("k_scale", k_scale, (k.shape[0],))):
            if t.dtype != torch.float32 or tuple(t.shape) != shp or t.device != dev or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous float32 tensor {shp} on {dev}")
    elif q_scale is not None or k_scale is not None:
        raise ValueError("q_scale / k_scale go with float8_e4m3fn q and k only")
    shape = shape_for(q, k, k_top, mask, plan, splits)
    if idx is None:
        idx = torch.empty((n_tok, k_top), dtype=torch.int32, device=dev)
    if score is None and want_score:
        score = torch.empty((n_tok, k_top), dtype=torch.float32, device=dev)
    ws_bytes = workspace_size(shape)
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        # zero-filled: the decode plan keeps per-query counters at its start,
        # which must be zero before the first call (every call leaves them so)
        workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    if fp8:
        rc = load().lid_topk_fp8(ctypes.byref(shape), _ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(w),
                                 _ptr(mask), _ptr(kv_range), _ptr(idx), _ptr(score), _ptr(workspace), ws_have, stream)
    else:
        rc = load().lid_topk(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(w), _ptr(mask), _ptr(kv_range), _ptr(idx),
                             _ptr(score), _ptr(workspace), ws_have, stream)
    if rc != 0:
        raise LidError(rc)
    return idx, score


NOALLOC_SCRATCH_BYTES = 16 << 20  # the static scratch of lid_topk_noalloc, per GPU


def topk_noalloc(q, k, w, mask=None, kv_range=None, k_top=512, *, plan=PLAN_AUTO, splits=0, idx=None, score=None,
                 want_score=True, stream=None):
    """lid_topk_noalloc: the fused top-k with the library's static scratch
    instead of a workspace (no device allocation by the library; idx / score
    are allocated here unless given).  f16 / bf16 / f32 q and k."""
    import torch
    n_tok = q.shape[0]
    dev = q.device
    if q.dim() != 3 or k.dim() != 2 or w.dim() != 2 or dev.type != "cuda":
        raise ValueError("q [n_tok,H,D], k [n_kv,D], w [n_tok,H] on the GPU expected")
    for name, t in (("q", q), ("k", k), ("w", w), ("mask", mask), ("kv_range", kv_range)):
        if t is not None and (t.device != dev or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous tensor on {dev}")
    if k.dtype != q.dtype or q.dtype == torch.float8_e4m3fn or w.dtype != torch.float32:
        raise ValueError("q and k f16 / bf16 / f32 of one dtype, w float32")
    if mask is not None:
        if mask.dtype not in (torch.float16, torch.int16, torch.uint16) or mask.dim() != 2 or mask.shape[0] != n_tok:
            raise ValueError("mask must be float16 [n_tok, mask_ld]")
    if kv_range is not None and (kv_range.dtype != torch.int32 or tuple(kv_range.shape) != (n_tok, 2)):
        raise ValueError("kv_range must be int32 [n_tok, 2]")
    shape = shape_for(q, k, k_top, mask, plan, splits)
    if idx is None:
        idx = torch.empty((n_tok, k_top), dtype=torch.int32, device=dev)
    if score is None and want_score:
        score = torch.empty((n_tok, k_top), dtype=torch.float32, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = load().lid_topk_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(w), _ptr(mask), _ptr(kv_range),
                                 _ptr(idx), _ptr(score), stream)
    if rc != 0:
        raise LidError(rc, "lid_topk_noalloc")
    return idx, score


def topk_shared(q, k, w, mask=None, kv_range=None, k_top=512, *, idx=None, score=None, want_score=True,
                workspace=None, stream=None):
    """Shared (per-ubatch) top-k on the GPU: one row of the k_top keys with the
    largest U[s] = sum over all queries of the masked score (lid_topk_shared).
    Returns (idx int32 [k_top], score f32 [k_top] or None)."""
    import torch
    if q.dim() != 3 or k.dim() != 2 or w.dim() != 2:
        raise ValueError("q [n_tok,H,D], k [n_kv,D], w [n_tok,H] expected")
    n_tok, H, D = q.shape
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("lid.topk_shared runs on the GPU only (q is on %s)" % dev)
    for name, t in (("q", q), ("k", k), ("w", w), ("mask", mask), ("kv_range", kv_range)):
        if t is not None and (t.device != dev or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous tensor on {dev}")
    if k.dtype != q.dtype or k.shape[1] != D or w.shape != (n_tok, H) or w.dtype != torch.float32:
        raise ValueError("dtype/shape mismatch among q, k, w")
    if mask is not None:
        if mask.dtype not in (torch.float16, torch.int16, torch.uint16) or mask.dim() != 2 or mask.shape[0] != n_tok:
            raise ValueError("mask must be float16 [n_tok, mask_ld]")
    if kv_range is not None and (kv_range.dtype != torch.int32 or tuple(kv_range.shape) != (n_tok, 2)):
        raise ValueError("kv_range must be int32 [n_tok, 2]")
    shape = shape_for(q, k, k_top, mask)
    if idx is None:
        idx = torch.empty((k_top,), dtype=torch.int32, device=dev)
    if score is None and want_score:
        score = torch.empty((k_top,), dtype=torch.float32, device=dev)
    ws_bytes = int(load().lid_topk_shared_workspace_size(ctypes.byref(shape)))
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = load().lid_topk_shared(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(w), _ptr(mask), _ptr(kv_range),
                                _ptr(idx), _ptr(score), _ptr(workspace), ws_have, stream)
    if rc != 0:
        raise LidError(rc)
    return idx, score


def sparse_attn(qa, kv, idx, scale, *, out=None, stream=None):
    """Sparse attention over the selected latent rows (lid_sparse_attn):
    out [n_tok, H, L] f32 = softmax(scale * qa . kv[idx]) . kv[idx] per
    (query, head), over the entries of idx [n_tok, k_sel] inside [0, n_kv)."""
    import torch
    if qa.dim() != 3 or kv.dim() != 2 or idx.dim() != 2:
        raise ValueError("qa [n_tok,H,L], kv [n_kv,L], idx [n_tok,k_sel] expected")
    n_tok, H, L = qa.shape
    dev = qa.device
    if dev.type != "cuda":
        raise ValueError("lid.sparse_attn runs on the GPU only (qa is on %s)" % dev)
    for name, t in (("qa", qa), ("kv", kv), ("idx", idx)):
        if t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor on {dev}")
    if kv.dtype != qa.dtype or kv.shape[1] != L or idx.shape[0] != n_tok or idx.dtype != torch.int32:
        raise ValueError("dtype/shape mismatch among qa, kv, idx")
    if out is None:
        out = torch.empty((n_tok, H, L), dtype=torch.float32, device=dev)
    elif out.dtype != torch.float32 or tuple(out.shape) != (n_tok, H, L) or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [n_tok, H, L] tensor")
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = load().lid_sparse_attn(n_tok, kv.shape[0], H, L, idx.shape[1], _dtype_code(qa), _ptr(qa), _ptr(kv),
                                _ptr(idx), float(scale), _ptr(out), stream)
    if rc != 0:
        raise LidError(rc)
    return out


def scores(q, k, w, mask=None, kv_range=None, *, out=None, stream=None):
    """Score-only mode: the [n_tok, n_kv] f32 masked scores (-inf outside each
    query's range), the output of the fused indexer op without the top-k.
    `out` may be an f32 [n_tok, ld] tensor with ld >= n_kv."""
    import torch
    if q.dim() != 3 or k.dim() != 2 or w.dim() != 2:
        raise ValueError("q [n_tok,H,D], k [n_kv,D], w [n_tok,H] expected")
    n_tok, H, D = q.shape
    n_kv = k.shape[0]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("lid.scores runs on the GPU only (q is on %s)" % dev)
    for name, t in (("q", q), ("k", k), ("w", w), ("mask", mask), ("kv_range", kv_range)):
        if t is not None and (t.device != dev or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous tensor on {dev}")
    if k.dtype != q.dtype or k.shape[1] != D or w.shape != (n_tok, H) or w.dtype != torch.float32:
        raise ValueError("dtype/shape mismatch among q, k, w")
    if mask is not None:
        if mask.dtype not in (torch.float16, torch.int16, torch.uint16) or mask.dim() != 2 or mask.shape[0] != n_tok:
            raise ValueError("mask must be float16 [n_tok, mask_ld]")
    if kv_range is not None and (kv_range.dtype != torch.int32 or tuple(kv_range.shape) != (n_tok, 2)):
        raise ValueError("kv_range must be int32 [n_tok, 2]")
    if out is None:
        out = torch.empty((n_tok, n_kv), dtype=torch.float32, device=dev)
    if out.dtype != torch.float32 or out.dim() != 2 or out.shape[0] != n_tok or out.stride(1) != 1 \
            or out.stride(0) < n_kv:
        raise ValueError("out must be float32 [n_tok, >= n_kv] with unit column stride")
    shape = shape_for(q, k, 1, mask)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    rc = load().lid_scores(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(w), _ptr(mask), _ptr(kv_range), _ptr(out),
                           out.stride(0), stream)
    if rc != 0:
        raise LidError(rc)
    return out[:, :n_kv]


def set_profile_events(before, after):
    """Have lid_topk record two hipEvent_t handles (ints) around its scoring
    kernel; (None, None) turns this off."""
    load().lid_set_profile_events(before, after)


def hip_runtime():
    """ctypes handle of the process's HIP runtime (the one torch loaded)."""
    load()
    return ctypes.CDLL("libamdhip64.so.7")
