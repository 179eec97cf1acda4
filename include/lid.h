/*
 * lid.h -- C ABI of the fused lightning-indexer top-k for AMD Instinct MI355X
 * (gfx950).
 *
 * The operation (DeepSeek-V4-Flash lightning indexer):
 *
 *   I[t,s] = sum_h w[t,h] * max(0, sum_d q[t,h,d] * k[s,d])      (f32 accumulation)
 *   v[t,s] = I[t,s] + mask[t,s]                                    (f32; f16 mask)
 *   idx[t,:] = the k_top keys s with the largest v[t,s], ordered by v
 *              descending and, on equal v, by s ascending
 *
 * Sources: ggml-org llama.cpp issue 25468, comment "Root cause: the
 * lightning-indexer (lid_kq) score matrix" (the chain lid_kq -> relu ->
 * * weights -> sum_rows -> lid_score -> + mask -> lid_top_k, with 64 heads,
 * an f32 score and a top-512 int32 selection); the comment "Pinned: master is
 * missing the fused ggml_lightning_indexer op" (the fused op's inputs q, k,
 * weights); fairydreaming/llama.cpp PR 2 thread, last comment (the updated
 * op has no scale-factor parameters and takes an f16 mask).  Here scoring
 * and selection are one fused pass: no n_tok x n_kv score matrix, and no
 * n_tok x H x n_kv per-head matrix, is ever written.
 *
 * Conventions shared by every entry point:
 *  - Every pointer argument of lid_topk is a DEVICE pointer, owned by the
 *    caller.  The library never allocates device memory; scratch space comes
 *    in through `workspace`.
 *  - All arrays are C row-major and contiguous (mask rows have stride
 *    mask_ld).  q and k must be 16-byte aligned.
 *  - A key s is visible to query t iff lo_t <= s < hi_t and v[t,s] != -inf.
 *    Keys outside [lo_t, hi_t) never enter query t's selection; their mask
 *    entries have no effect, although the MFMA kernels may read them (only
 *    inside [0, n_kv) of row t, where a workgroup's queries' ranges overlap)
 *    so the whole [n_tok, n_kv] part of a mask must be readable.  Masked keys
 *    (-inf) are never returned.
 *  - Rows with fewer than k_top visible keys are padded with idx = -1 and
 *    score = -inf after the visible keys.
 *  - A score of -0 is reported as +0 (and ties with +0 by index).
 *  - Scale factors such as 1/sqrt(D) are not parameters: a positive scale
 *    c commutes with the ReLU (c * w * max(0,x) = (c*w) * max(0,x)), so the
 *    caller folds it into w.
 *  - lid_topk is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  It does not synchronise the host.  Identical inputs give
 *    bitwise-identical outputs.
 *  - Errors: every argument check happens before any launch; on a negative
 *    status nothing was launched and the outputs are untouched, except
 *    LID_ERR_HIP (a launch failed; outputs undefined).  There is no fallback
 *    to a path that would need an n_tok x n_kv buffer.
 *  - Calls that share one workspace must not overlap in time.
 *  - Workspace layout: every non-empty workspace starts with a 4096-byte
 *    counter region, and the plan's data follows it.  The plans that finish
 *    inside their scoring kernel (decode; prefill with a few key splits) keep
 *    32-bit completion counters there (one per query, or per block of 8
 *    queries; at most 1024); no entry point writes anything else into it.
 *    The region must be zero before the first call on a workspace; every call
 *    that completes leaves it at zero again.  So a workspace is zero-filled
 *    once and can then be reused for any later shape, plan or entry point
 *    (lid_topk, lid_topk_fp8, lid_topk_shared), also from a captured HIP
 *    graph.
 */
#ifndef LID_H
#define LID_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype of q and k.  w is always f32, mask always f16 (IEEE binary16 bits). */
typedef enum { LID_F32 = 0, LID_F16 = 1, LID_BF16 = 2, LID_F8E4M3 = 3 } lid_dtype;

typedef enum {
    LID_OK = 0,
    LID_ERR_INVALID_ARG = -1,  /* a NULL required pointer, bad size, misalignment ... */
    LID_ERR_UNSUPPORTED = -2,  /* valid request outside the library's limits (k_top > 1024 ...) */
    LID_ERR_WORKSPACE = -3,    /* workspace missing or smaller than lid_topk_workspace_size() */
    LID_ERR_HIP = -4           /* a HIP launch failed */
} lid_status;

/* Kernel plan; LID_PLAN_AUTO picks one from the shape.  The others force a
 * plan (for tests); a forced plan that cannot run the shape returns
 * LID_ERR_UNSUPPORTED. */
typedef enum {
    LID_PLAN_AUTO = 0,
    LID_PLAN_GENERIC = 1,   /* vector-ALU scoring, any H, D and dtype */
    LID_PLAN_PREFILL = 2,   /* MFMA scoring, key tiles shared through LDS by a block of queries */
    LID_PLAN_DECODE = 3     /* MFMA scoring, keys split across many workgroups per query */
} lid_plan;

typedef struct {
    int64_t n_tok;     /* queries, >= 0 (0: nothing to do)                    */
    int64_t n_kv;      /* keys, 0 <= n_kv <= 2^31 - 1                          */
    int32_t n_head;    /* H >= 1                                               */
    int32_t head_dim;  /* D >= 1                                               */
    int32_t k_top;     /* 1 <= k_top <= 1024                                   */
    int32_t qk_dtype;  /* lid_dtype of q and k                                 */
    int64_t mask_ld;   /* row stride of mask in elements, >= n_kv; ignored if mask == NULL */
    int32_t plan;      /* lid_plan; LID_PLAN_AUTO normally                     */
    int32_t splits;    /* key splits per query; 0 = chosen by the library      */
} lid_shape;

/* Bytes of device workspace lid_topk needs for this shape (0 is possible:
 * then workspace may be NULL).  Returns 0 for an invalid shape as well;
 * lid_topk reports the error.  Depends only on the shape fields. */
size_t lid_topk_workspace_size(const lid_shape* shape);

/* The fused score + mask + top-k.
 *   q         [n_tok, H, D]     qk_dtype
 *   k         [n_kv, D]         qk_dtype
 *   w         [n_tok, H]        f32, any sign
 *   mask      [n_tok, mask_ld]  f16 additive mask, or NULL (no mask)
 *   kv_range  [n_tok, 2]        int32 half-open [lo, hi) per query, or NULL
 *                               (= [0, n_kv)); clamped to [0, n_kv); lo >= hi
 *                               is an empty range
 *   idx       [n_tok, k_top]    int32 output
 *   score     [n_tok, k_top]    f32 output (the v of each returned key), or NULL
 *   workspace device scratch of >= lid_topk_workspace_size(shape) bytes,
 *             8-byte aligned, its first 4096 bytes zero before its first use
 *             (see above)
 *   stream    hipStream_t
 * Inputs must be finite (q, k, w); a NaN or +inf score is not detected. */
int lid_topk(const lid_shape* shape, const void* q, const void* k, const float* w,
             const uint16_t* mask, const int32_t* kv_range, int32_t* idx, float* score,
             void* workspace, size_t workspace_bytes, void* stream);

/* lid_topk without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc.  It computes exactly what lid_topk
 * computes (the same kernels; bitwise-identical results) and allocates
 * nothing: its scratch is a static device array of 16 MiB (16777216 bytes),
 * one per GPU the library runs on, held until the process ends.  Its address
 * is looked up (hipGetSymbolAddress) on the first call on each device, with
 * the caller's current device, which must be the device of `stream`.
 *   arguments  as for lid_topk (all device pointers, caller-owned)
 *   returns    LID_ERR_WORKSPACE, before any launch, for a shape whose
 *              lid_topk_workspace_size exceeds 16 MiB (e.g. a prefill plan
 *              with many key splits and queries); other errors as lid_topk
 * Every call on one GPU uses that GPU's one array: each call clears the
 * array's counter region itself (a small kernel on `stream` before the
 * scoring kernel), but calls that overlap in time on one GPU (on different
 * streams or host threads) race on the array and give undefined results. */
int lid_topk_noalloc(const lid_shape* shape, const void* q, const void* k, const float* w,
                     const uint16_t* mask, const int32_t* kv_range, int32_t* idx, float* score,
                     void* stream);

/* Score-only mode: the output of the pages' fused indexer op itself, without
 * the top-k.  ggml-org llama.cpp issue 25468, comment "Pinned: master is
 * missing the fused ggml_lightning_indexer op", gives that op's inputs (q, k,
 * weights) and its [n_kv, n_tok] score output (ggml order; here row t of a C
 * [n_tok, n_kv] array); fairydreaming/llama.cpp pull request 2 (last
 * comment) drops its scale factors and adds the f16 mask.  So
 *   scores[t * scores_ld + s] = sum_h w[t,h] * max(0, q[t,h,:] . k[s,:])
 *                               + mask[t,s]      for s in the query's range,
 *                               -inf             elsewhere (s < n_kv),
 * the same v that lid_topk selects from (same kernels, f32 accumulation).
 *   q, k, w, mask, kv_range  as for lid_topk (k_top, plan and splits of the
 *                            shape are ignored)
 *   scores     [n_tok, scores_ld] f32 output, scores_ld >= n_kv; columns
 *              n_kv .. scores_ld - 1 are not written
 * This is the n_tok x n_kv buffer that lid_topk never forms: 4 B per pair
 * (c4-sized: 1 GiB).  No workspace.  Asynchronous on `stream`. */
int lid_scores(const lid_shape* shape, const void* q, const void* k, const float* w,
               const uint16_t* mask, const int32_t* kv_range, float* scores, int64_t scores_ld,
               void* stream);

/* The fused score + mask + top-k with FP8 q and k (shape->qk_dtype ==
 * LID_F8E4M3): q and k hold OCP FP8 E4M3 bytes (E4M3FN: bias 7, no
 * infinities, S.1111.111 NaN), dequantised per row,
 *   q[t,h,:] = e4m3(q8[t,h,:]) * q_scale[t,h],   k[s,:] = e4m3(k8[s,:]) * k_scale[s],
 * and then scored and selected exactly as lid_topk does.  The pages quantise
 * the DeepSeek-V4 indexer to FP4 after a Hadamard rotation (ggml-org
 * llama.cpp PR 22378, the batched-prefill commit) and its KV cache to FP8
 * E4M3 (the DSV4 CUDA-kernel plan, "dsv4_fp8_kv_quantize"), but give no scale
 * convention for the indexer: this per-row one is this library's.
 *   q_scale  [n_tok, H] f32, > 0 and finite
 *   k_scale  [n_kv]     f32, > 0 and finite
 * Other arguments as for lid_topk (workspace: lid_topk_workspace_size of the
 * same shape).  H = 64, D = 128 runs on the MFMA kernels (128 bytes per key
 * instead of 256): the decode kernel for at most 4 queries
 * (v_mfma_f32_32x32x64_f8f6f4), the prefill kernel otherwise
 * (v_mfma_f32_16x16x128_f8f6f4, the whole head dimension per instruction);
 * other shapes run on the vector-ALU kernel. */
int lid_topk_fp8(const lid_shape* shape, const void* q, const float* q_scale, const void* k,
                 const float* k_scale, const float* w, const uint16_t* mask,
                 const int32_t* kv_range, int32_t* idx, float* score, void* workspace,
                 size_t workspace_bytes, void* stream);

/* Shared (per-ubatch) top-k: ONE selection of k_top keys for all the queries
 * of the call, by the summed score
 *   U[s] = sum_t v[t,s]       (v as for lid_topk: the masked f32 score; a key
 *                              outside query t's range, or masked for it, has
 *                              v = -inf, and then U[s] = -inf: not selectable)
 *   idx[:] = the k_top keys with the largest U, ordered by U descending and,
 *            on equal U, by key index ascending; score[:] = their U.
 * ggml-org llama.cpp PR 22378, the batched-prefill commit: the indexer's
 * per-query scores are summed over the ubatch (and heads) and one ubatch-wide
 * top-k is taken, which every query of the ubatch then uses (the pages call it
 * an approximation whose loss is small for adjacent prefill tokens); the
 * commit that reverts collapse-Q writes it as top_k(sum_q relu(kv*q)*w).
 * U is accumulated in f32 over the queries in a fixed order (deterministic);
 * with no queries (n_tok = 0) U = 0 for every key.
 *   q, k, w, mask, kv_range  as for lid_topk; H = 64, D = 128, f16 or bf16
 *                            (other shapes and dtypes: LID_ERR_UNSUPPORTED)
 *   idx       [k_top]  int32 output (-1 after the selectable keys)
 *   score     [k_top]  f32 output (-inf after them), or NULL
 *   workspace device scratch of >= lid_topk_shared_workspace_size(shape)
 *             bytes, 8-byte aligned: after the 4096-byte counter region
 *             (left untouched, so that a zeroed workspace can be shared with
 *             lid_topk), the partial sums of U per key and query chunk
 *             (O(n_kv), not O(n_tok * n_kv)) and, above 16384 keys, the
 *             sorted lists of the key chunks
 * k_top, plan and splits: k_top as for lid_topk; plan and splits are ignored.
 * Asynchronous on `stream`; errors as for lid_topk. */
size_t lid_topk_shared_workspace_size(const lid_shape* shape);
int lid_topk_shared(const lid_shape* shape, const void* q, const void* k, const float* w,
                    const uint16_t* mask, const int32_t* kv_range, int32_t* idx, float* score,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Sparse attention over the selected keys: the consumer of the top-k.  For
 * query t and head h, over the entries j of idx[t,:] with 0 <= idx[t,j] <
 * n_kv (others, such as lid_topk's -1 padding, are skipped; a repeated index
 * counts once per entry):
 *   s_j    = scale * sum_d qa[t,h,d] * kv[idx[t,j], d]
 *   out[t,h,:] = sum_j softmax_j(s) * kv[idx[t,j], :]     (0 if no entry is valid)
 * Issue 25468, "Root cause" comment: each CSA layer's top-512 selection of
 * the compressed KV rows feeds that layer's attention; ggml-org llama.cpp PR
 * 22378, the flash-attention unblock commit: the MLA latent KV row is 512
 * wide and attention is softmax(Q K^T) V.  The absorbed-MLA form is read: one
 * latent row serves as key and as value (the query has been multiplied into
 * the latent space beforehand by the caller).
 *   qa    [n_tok, n_head, latent_dim]  qk_dtype (LID_F16 or LID_BF16)
 *   kv    [n_kv, latent_dim]           qk_dtype
 *   idx   [n_tok, k_sel]               int32 (any values; out of range = skipped)
 *   out   [n_tok, n_head, latent_dim]  f32 output
 * All device pointers, caller-owned, contiguous; qa, kv and out 16-byte
 * aligned.  8 <= latent_dim <= 1024 with latent_dim % 8 == 0 (larger:
 * LID_ERR_UNSUPPORTED); k_sel >= 0; scale finite (1/sqrt(latent_dim) for the
 * usual scaling: not implied).  Scores, the running maximum, the softmax
 * denominator and the weighted sum are f32.  Asynchronous on `stream`, no
 * workspace, deterministic; errors as for lid_topk.  The profile events of
 * lid_set_profile_events bracket its one kernel. */
int lid_sparse_attn(int64_t n_tok, int64_t n_kv, int32_t n_head, int32_t latent_dim, int32_t k_sel,
                    int32_t qk_dtype, const void* qa, const void* kv, const int32_t* idx, float scale,
                    float* out, void* stream);

/* The plan lid_topk would run for `shape` (a lid_plan value), and through
 * `splits_out` (may be NULL) its key splits per query; negative lid_status if
 * the shape is invalid or unsupported. */
int lid_topk_plan(const lid_shape* shape, int32_t* splits_out);

/* Static text for a status code. */
const char* lid_status_string(int status);

/* Measurement hook.  With non-NULL hipEvent_t handles, every later lid_topk
 * (and lid_scores) records `before_scoring` on its stream right before it
 * launches its scoring kernel and `after_scoring` right after, so
 * hipEventElapsedTime gives that kernel's duration; the split merge (if
 * any) and the score-only mode's fill outside the ranges fall outside.  NULL, NULL turns
 * it off.  Process-wide setting, not synchronised: set it from one thread. */
void lid_set_profile_events(void* before_scoring, void* after_scoring);

/* Text of the HIP error behind the last LID_ERR_HIP returned to this
 * thread ("no error" if there was none).  Static storage; never NULL. */
const char* lid_last_hip_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int lid_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LID_H */
