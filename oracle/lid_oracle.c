/*
 * lid_oracle.c -- plain, slow CPU oracle for the fused lightning-indexer top-k.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code, header or table with the HIP library.
 *
 * What it computes (the plain definition, in the order the pages give it):
 *
 *  1. Per-head scores and the head reduction.  ggml-org llama.cpp issue 25468,
 *     comment "Root cause: the lightning-indexer (lid_kq) score matrix ...",
 *     chain diagram: lid_kq = mul_mat(indexer_k, indexer_q) -> relu -> * weights
 *     -> sum_rows = lid_score.  Written out for query t and key s:
 *         I[t,s] = sum_h w[t,h] * max(0, sum_d q[t,h,d] * k[s,d])
 *     accumulated here in double precision from the exactly decoded inputs.
 *  2. No scale factors inside the op: fairydreaming/llama.cpp PR 2 thread, last
 *     comment (scale-factor parameters removed, an f16 mask parameter added).
 *  3. The mask is added after the head reduction, to the f32 score
 *     (issue 25468, same chain: lid_score -> + mask -> lid_top_k).  lid_score is
 *     an f32 tensor (64 MiB = 32768 x 512 x 4 B in that comment), so the score
 *     is rounded to f32 once and the f16 mask value is added in f32.  A result
 *     of -inf marks a key that may not be chosen (padding masked with -INFINITY,
 *     ggml-org llama.cpp PR 22378, kq_mask padding commit).
 *  4. Per-token top-k: the k_top best keys per query (lid_top_k is
 *     [512 x n_tok] int32, 1 MiB, same comment), ordered by score descending
 *     and, among equal f32 scores, by key index ascending.
 *
 * FP8 inputs (lid_oracle_topk_scaled / lid_oracle_scores_scaled).  The pages'
 * DeepSeek-V4 path quantises the indexer to FP4 after a Hadamard rotation
 * (ggml-org llama.cpp PR 22378, the batched-prefill commit) and its KV cache
 * to FP8 E4M3 (the DSV4 CUDA-kernel plan, section "dsv4_fp8_kv_quantize"),
 * but gives no scale convention for the indexer, so a synthetic one is used:
 * q and k are OCP FP8 E4M3 bytes with a positive f32 scale per
 * query head row and per key row, q[t,h,:] = e4m3(q8[t,h,:]) * q_scale[t,h],
 * k[s,:] = e4m3(k8[s,:]) * k_scale[s]; these dequantised values (exact in
 * double) then go through steps 1-4 unchanged.
 *
 * Readings where the pages are silent: -0 scores are treated as +0; fewer
 * than k_top visible keys pad the row with index -1 / score -inf; an optional
 * per-query half-open key range [lo, hi) restricts the keys scored (keys
 * outside it are never scored and their mask is never read).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_F8E4M3 = 3 };
enum { ORC_OK = 0, ORC_EINVAL = -1, ORC_ENONFINITE = -2, ORC_ENOMEM = -3 };

/* IEEE binary16 -> double, written from the format definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double lid_oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 -> double: the upper 16 bits of an IEEE binary32. */
double lid_oracle_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP FP8 E4M3 (E4M3FN) -> double, written from the format definition:
 * 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits; exponent field 0 is
 * subnormal (m * 2^-9); no infinities; S.1111.111 is NaN. */
double lid_oracle_f8e4m3_to_f64(uint8_t x)
{
    int sign = (x >> 7) & 1;
    int e = (x >> 3) & 0xF;
    int m = x & 0x7;
    double v;
    if (e == 0)
        v = ldexp((double)m, -9);                  /* subnormal: (m/8) * 2^-6 */
    else if (e == 15 && m == 7)
        v = NAN;
    else
        v = ldexp((double)(8 + m), e - 10);        /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

static double decode(const void* p, int dtype, int64_t i)
{
    switch (dtype) {
    case ORC_F32: return (double)((const float*)p)[i];
    case ORC_F16: return lid_oracle_f16_to_f64(((const uint16_t*)p)[i]);
    case ORC_F8E4M3: return lid_oracle_f8e4m3_to_f64(((const uint8_t*)p)[i]);
    default:      return lid_oracle_bf16_to_f64(((const uint16_t*)p)[i]);
    }
}

typedef struct { float v; int64_t s; } cand;

/* score descending, then key index ascending */
static int cand_cmp(const void* a, const void* b)
{
    const cand* x = (const cand*)a;
    const cand* y = (const cand*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->s < y->s) ? -1 : (x->s > y->s);
}

/* I[t,s] of step 1 for one query (decoded rows qd [H*D], wd [H]) and key row kd [D]. */
static double head_reduced_score(const double* qd, const double* wd, const double* kd,
                                 int H, int D)
{
    double I = 0.0;
    for (int h = 0; h < H; ++h) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += qd[(int64_t)h * D + d] * kd[d];
        if (dot > 0.0)              /* ReLU: a non-positive dot contributes nothing */
            I += wd[h] * dot;
    }
    return I;
}

/* Visible key range of query t: [lo, hi) clamped to [0, n_kv); empty if lo >= hi. */
static void key_range(const int32_t* kv_range, int64_t t, int64_t n_kv,
                      int64_t* lo, int64_t* hi)
{
    int64_t a = 0, b = n_kv;
    if (kv_range) {
        a = kv_range[2 * t];
        b = kv_range[2 * t + 1];
        if (a < 0) a = 0;
        if (b > n_kv) b = n_kv;
        if (b < a) b = a;
    }
    *lo = a;
    *hi = b;
}

/* Steps 2-3: masked f32 score of a pair, canonicalised so that -0 becomes +0.
 * Returns 0, or ORC_ENONFINITE if the score is NaN or +inf. */
static int masked_score(double I, const uint16_t* mask, int64_t mask_ld, int64_t t,
                        int64_t s, float* out)
{
    float v = (float)I;
    if (mask)
        v = v + (float)lid_oracle_f16_to_f64(mask[t * mask_ld + s]);
    if (isnan(v) || (isinf(v) && v > 0))
        return ORC_ENONFINITE;
    *out = v + 0.0f;
    return 0;
}

static int check_args(int64_t n_tok, int64_t n_kv, int32_t H, int32_t D, int32_t dtype,
                      const void* q, const void* k, const float* w, int64_t mask_ld,
                      const uint16_t* mask)
{
    if (n_tok < 0 || n_kv < 0 || n_kv > INT32_MAX || H <= 0 || D <= 0)
        return ORC_EINVAL;
    if (dtype != ORC_F32 && dtype != ORC_F16 && dtype != ORC_BF16 && dtype != ORC_F8E4M3)
        return ORC_EINVAL;
    if ((n_tok > 0 && (!q || !w)) || (n_kv > 0 && !k))
        return ORC_EINVAL;
    if (mask && mask_ld < n_kv)
        return ORC_EINVAL;
    return ORC_OK;
}

/* Decoded key rows, each times its scale when k_scale is given. */
static double* decode_keys(const void* k, int dtype, int64_t n_kv, int D, const float* k_scale)
{
    double* kd = (double*)malloc(sizeof(double) * (size_t)(n_kv > 0 ? n_kv : 1) * (size_t)D);
    if (!kd) return NULL;
    for (int64_t i = 0; i < n_kv * D; ++i) {
        kd[i] = decode(k, dtype, i);
        if (k_scale)
            kd[i] *= (double)k_scale[i / D];
    }
    return kd;
}

/*
 * Top-k of the masked score per query.
 *   q        [n_tok, H, D]   dtype (f32 / f16 bits / bf16 bits)
 *   k        [n_kv, D]       dtype
 *   w        [n_tok, H]      f32
 *   mask     [n_tok, mask_ld] f16 bits, or NULL
 *   kv_range [n_tok, 2]      int32 half-open [lo, hi), or NULL (all keys)
 *   idx_out  [n_tok, k_top]  int32;  score_out [n_tok, k_top] f32 (may be NULL)
 *   maxabs_out: max |I[t,s]| over every visible pair (may be NULL)
 *   n_threads: OpenMP threads (<= 0: runtime default)
 */
static int topk_impl(int64_t n_tok, int64_t n_kv, int32_t H, int32_t D, int32_t k_top,
                     int32_t dtype, const void* q, const void* k, const float* w,
                     const uint16_t* mask, int64_t mask_ld, const int32_t* kv_range,
                     int32_t* idx_out, float* score_out, double* maxabs_out, int32_t n_threads,
                     const float* q_scale, const float* k_scale)
{
    int rc = check_args(n_tok, n_kv, H, D, dtype, q, k, w, mask_ld, mask);
    if (rc) return rc;
    if (k_top <= 0 || !idx_out) return ORC_EINVAL;

    double* kd = decode_keys(k, dtype, n_kv, D, k_scale);
    if (!kd) return ORC_ENOMEM;

    double maxabs = 0.0;
    int err = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(max : maxabs) reduction(min : err)
    for (int64_t t = 0; t < n_tok; ++t) {
        double* qd = (double*)malloc(sizeof(double) * (size_t)H * (size_t)D);
        double* wd = (double*)malloc(sizeof(double) * (size_t)H);
        int64_t lo, hi;
        key_range(kv_range, t, n_kv, &lo, &hi);
        cand* c = (cand*)malloc(sizeof(cand) * (size_t)(hi - lo > 0 ? hi - lo : 1));
        if (!qd || !wd || !c) {
            err = ORC_ENOMEM;
            free(qd); free(wd); free(c);
            continue;
        }
        for (int64_t i = 0; i < (int64_t)H * D; ++i) {
            qd[i] = decode(q, dtype, t * H * D + i);
            if (q_scale)
                qd[i] *= (double)q_scale[t * H + i / D];
        }
        for (int h = 0; h < H; ++h)
            wd[h] = (double)w[t * H + h];

        int64_t n = 0;
        for (int64_t s = lo; s < hi; ++s) {
            double I = head_reduced_score(qd, wd, kd + s * D, H, D);
            float v;
            if (masked_score(I, mask, mask_ld, t, s, &v)) { err = ORC_ENONFINITE; break; }
            if (isinf(v))                      /* -inf: masked, never chosen */
                continue;
            if (fabs(I) > maxabs) maxabs = fabs(I);
            c[n].v = v;
            c[n].s = s;
            ++n;
        }
        qsort(c, (size_t)n, sizeof(cand), cand_cmp);
        for (int32_t j = 0; j < k_top; ++j) {
            int valid = j < n;
            idx_out[t * k_top + j] = valid ? (int32_t)c[j].s : -1;
            if (score_out)
                score_out[t * k_top + j] = valid ? c[j].v : -INFINITY;
        }
        free(qd); free(wd); free(c);
    }
    free(kd);
    if (maxabs_out) *maxabs_out = maxabs;
    return err;
}

int lid_oracle_topk(int64_t n_tok, int64_t n_kv, int32_t H, int32_t D, int32_t k_top,
                    int32_t dtype, const void* q, const void* k, const float* w,
                    const uint16_t* mask, int64_t mask_ld, const int32_t* kv_range,
                    int32_t* idx_out, float* score_out, double* maxabs_out, int32_t n_threads)
{
    return topk_impl(n_tok, n_kv, H, D, k_top, dtype, q, k, w, mask, mask_ld, kv_range, idx_out,
                     score_out, maxabs_out, n_threads, NULL, NULL);
}

/* The same with per-row scales on q ([n_tok, H] f32) and k ([n_kv] f32). */
int lid_oracle_topk_scaled(int64_t n_tok, int64_t n_kv, int32_t H, int32_t D, int32_t k_top,
                           int32_t dtype, const void* q, const float* q_scale, const void* k,
                           const float* k_scale, const float* w, const uint16_t* mask,
                           int64_t mask_ld, const int32_t* kv_range, int32_t* idx_out,
                           float* score_out, double* maxabs_out, int32_t n_threads)
{
    if (!q_scale || !k_scale) return ORC_EINVAL;
    return topk_impl(n_tok, n_kv, H, D, k_top, dtype, q, k, w, mask, mask_ld, kv_range, idx_out,
                     score_out, maxabs_out, n_threads, q_scale, k_scale);
}

/*
 * The full masked score matrix v[t,s] (f32, -inf where not visible) -- the
 * output of the pages' un-selected fused op (issue 25468, comment "Pinned:
 * master is missing the fused ggml_lightning_indexer op": output shape
 * [n_kv, n_tok] in ggml order).  For small problems only: it is n_tok x n_kv.
 */
static int scores_impl(int64_t n_tok, int64_t n_kv, int32_t H, int32_t D, int32_t dtype,
                       const void* q, const void* k, const float* w,
                       const uint16_t* mask, int64_t mask_ld, const int32_t* kv_range,
                       float* v_out, int32_t n_threads, const float* q_scale, const float* k_scale)
{
    int rc = check_args(n_tok, n_kv, H, D, dtype, q, k, w, mask_ld, mask);
    if (rc) return rc;
    if (!v_out) return ORC_EINVAL;
    double* kd = decode_keys(k, dtype, n_kv, D, k_scale);
    if (!kd) return ORC_ENOMEM;
    int err = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(min : err)
    for (int64_t t = 0; t < n_tok; ++t) {
        double* qd = (double*)malloc(sizeof(double) * (size_t)H * (size_t)D);
        double* wd = (double*)malloc(sizeof(double) * (size_t)H);
        if (!qd || !wd) { err = ORC_ENOMEM; free(qd); free(wd); continue; }
        for (int64_t i = 0; i < (int64_t)H * D; ++i) {
            qd[i] = decode(q, dtype, t * H * D + i);
            if (q_scale)
                qd[i] *= (double)q_scale[t * H + i / D];
        }
        for (int h = 0; h < H; ++h)
            wd[h] = (double)w[t * H + h];
        int64_t lo, hi;
        key_range(kv_range, t, n_kv, &lo, &hi);
        for (int64_t s = 0; s < n_kv; ++s) {
            float v = -INFINITY;
            if (s >= lo && s < hi) {
                double I = head_reduced_score(qd, wd, kd + s * D, H, D);
                if (masked_score(I, mask, mask_ld, t, s, &v)) { err = ORC_ENONFINITE; v = NAN; }
            }
            v_out[t * n_kv + s] = v;
        }
        free(qd); free(wd);
    }
    free(kd);
    return err;
}

int lid_oracle_scores(int64_t n_tok, int64_t n_kv, int32_t H, int32_t D, int32_t dtype,
                      const void* q, const void* k, const float* w,
                      const uint16_t* mask, int64_t mask_ld, const int32_t* kv_range,
                      float* v_out, int32_t n_threads)
{
    return scores_impl(n_tok, n_kv, H, D, dtype, q, k, w, mask, mask_ld, kv_range, v_out, n_threads,
                       NULL, NULL);
}

int lid_oracle_scores_scaled(int64_t n_tok, int64_t n_kv, int32_t H, int32_t D, int32_t dtype,
                             const void* q, const float* q_scale, const void* k,
                             const float* k_scale, const float* w, const uint16_t* mask,
                             int64_t mask_ld, const int32_t* kv_range, float* v_out,
                             int32_t n_threads)
{
    if (!q_scale || !k_scale) return ORC_EINVAL;
    return scores_impl(n_tok, n_kv, H, D, dtype, q, k, w, mask, mask_ld, kv_range, v_out, n_threads,
                       q_scale, k_scale);
}

/*
 * Shared (per-ubatch) top-k: one selection for all the queries of a ubatch.
 * ggml-org llama.cpp PR 22378, the batched-prefill commit: the indexer's
 * per-query scores are summed over the ubatch's queries (and heads) and a
 * single ubatch-wide top-k is taken, which every query then uses; the later
 * commit that reverts collapse-Q writes this summed form as
 * top_k(sum_q relu(kv * q) * w).  Written out:
 *     U[s] = sum_t v[t,s]
 * where v[t,s] is the masked f32 score of steps 1-3 (the value the per-query
 * top-k selects from), and a term of -inf (key outside query t's range, or
 * masked for it) makes U[s] = -inf: the key is not selectable.  The terms are
 * summed in double, U is rounded to f32 once, and the k_top keys with the
 * largest U are returned, ordered by U descending and, on equal U, by index
 * ascending (the per-query conventions of step 4).  A ubatch without queries
 * sums nothing: U = 0 for every key.
 *   idx_out [k_top] int32, score_out [k_top] f32 (may be NULL),
 *   maxabs_out: max |U[s]| over the selectable keys (may be NULL).
 */
int lid_oracle_topk_shared(int64_t n_tok, int64_t n_kv, int32_t H, int32_t D, int32_t k_top,
                           int32_t dtype, const void* q, const void* k, const float* w,
                           const uint16_t* mask, int64_t mask_ld, const int32_t* kv_range,
                           int32_t* idx_out, float* score_out, double* maxabs_out,
                           int32_t n_threads)
{
    int rc = check_args(n_tok, n_kv, H, D, dtype, q, k, w, mask_ld, mask);
    if (rc) return rc;
    if (k_top <= 0 || !idx_out) return ORC_EINVAL;
    double* kd = decode_keys(k, dtype, n_kv, D, NULL);
    double* qd = (double*)malloc(sizeof(double) * (size_t)(n_tok > 0 ? n_tok : 1) * (size_t)H * (size_t)D);
    double* wd = (double*)malloc(sizeof(double) * (size_t)(n_tok > 0 ? n_tok : 1) * (size_t)H);
    cand* c = (cand*)malloc(sizeof(cand) * (size_t)(n_kv > 0 ? n_kv : 1));
    int64_t* lo = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_tok > 0 ? n_tok : 1));
    int64_t* hi = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_tok > 0 ? n_tok : 1));
    uint8_t* ok = (uint8_t*)malloc((size_t)(n_kv > 0 ? n_kv : 1));
    if (!kd || !qd || !wd || !c || !lo || !hi || !ok) {
        free(kd); free(qd); free(wd); free(c); free(lo); free(hi); free(ok);
        return ORC_ENOMEM;
    }
    for (int64_t i = 0; i < n_tok * H * D; ++i)
        qd[i] = decode(q, dtype, i);
    for (int64_t i = 0; i < n_tok * H; ++i)
        wd[i] = (double)w[i];
    for (int64_t t = 0; t < n_tok; ++t)
        key_range(kv_range, t, n_kv, &lo[t], &hi[t]);

    int err = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel for schedule(dynamic, 64) reduction(min : err)
    for (int64_t s = 0; s < n_kv; ++s) {
        double U = 0.0;
        int selectable = 1;
        for (int64_t t = 0; t < n_tok && selectable; ++t) {
            if (s < lo[t] || s >= hi[t]) { selectable = 0; break; }   /* v = -inf */
            double I = head_reduced_score(qd + t * H * D, wd + t * H, kd + s * D, H, D);
            float v;
            if (masked_score(I, mask, mask_ld, t, s, &v)) { err = ORC_ENONFINITE; selectable = 0; break; }
            if (isinf(v)) { selectable = 0; break; }                 /* -inf term */
            U += (double)v;
        }
        ok[s] = (uint8_t)selectable;
        c[s].v = (float)U + 0.0f;
        c[s].s = s;
    }
    double maxabs = 0.0;
    int64_t n = 0;
    for (int64_t s = 0; s < n_kv; ++s) {
        if (!ok[s]) continue;
        if (fabs((double)c[s].v) > maxabs) maxabs = fabs((double)c[s].v);
        c[n++] = c[s];
    }
    qsort(c, (size_t)n, sizeof(cand), cand_cmp);
    for (int32_t j = 0; j < k_top; ++j) {
        int valid = j < n;
        idx_out[j] = valid ? (int32_t)c[j].s : -1;
        if (score_out)
            score_out[j] = valid ? c[j].v : -INFINITY;
    }
    free(kd); free(qd); free(wd); free(c); free(lo); free(hi); free(ok);
    if (maxabs_out) *maxabs_out = maxabs;
    return err;
}

/*
 * Sparse attention over the selected keys (the consumer of the top-k).
 * Issue 25468, "Root cause" comment: each CSA layer's score chain ends in a
 * per-token top-512 selection of the compressed KV rows; ggml-org llama.cpp
 * PR 22378, the flash-attention unblock commit: V4's MLA latent KV has K
 * width 512, and attention is Q K^T -> softmax -> * V, where masked (-inf)
 * slots contribute nothing.  Reading (the pages give no other attention
 * shape): the absorbed-MLA form, in which one latent row of width L serves
 * as both key and value, so for query t and head h
 *     s_j    = scale * sum_d qa[t,h,d] * kv[idx[t,j], d]
 *     o[t,h] = sum_j exp(s_j - max_j s) kv[idx[t,j]] / sum_j exp(s_j - max_j s)
 * over the entries j of the selection with 0 <= idx[t,j] < n_kv (others,
 * such as the top-k's -1 padding, are skipped; a repeated index counts each
 * time); a selection with no valid entry gives o = 0.  In double throughout.
 *   qa [n_tok, H, L], kv [n_kv, L] (dtype), idx [n_tok, k_sel] int32,
 *   out [n_tok, H, L] double.
 */
int lid_oracle_sparse_attn(int64_t n_tok, int64_t n_kv, int32_t H, int32_t L, int32_t k_sel, int32_t dtype,
                           const void* qa, const void* kv, const int32_t* idx, double scale, double* out,
                           int32_t n_threads)
{
    if (n_tok < 0 || n_kv < 0 || H <= 0 || L <= 0 || k_sel < 0 || !out)
        return ORC_EINVAL;
    if (dtype != ORC_F32 && dtype != ORC_F16 && dtype != ORC_BF16)
        return ORC_EINVAL;
    if ((n_tok > 0 && (!qa || (k_sel > 0 && !idx))) || (n_kv > 0 && !kv))
        return ORC_EINVAL;
    double* kd = decode_keys(kv, dtype, n_kv, L, NULL);
    if (!kd) return ORC_ENOMEM;
    int err = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(min : err)
    for (int64_t th = 0; th < n_tok * H; ++th) {
        const int64_t t = th / H;
        double* q = (double*)malloc(sizeof(double) * (size_t)L);
        double* s = (double*)malloc(sizeof(double) * (size_t)(k_sel > 0 ? k_sel : 1));
        if (!q || !s) { err = ORC_ENOMEM; free(q); free(s); continue; }
        for (int32_t d = 0; d < L; ++d)
            q[d] = decode(qa, dtype, th * L + d);
        double mx = -INFINITY;
        for (int32_t j = 0; j < k_sel; ++j) {
            const int32_t r = idx[t * k_sel + j];
            if (r < 0 || r >= n_kv) { s[j] = -INFINITY; continue; }
            double dot = 0.0;
            for (int32_t d = 0; d < L; ++d)
                dot += q[d] * kd[(int64_t)r * L + d];
            s[j] = scale * dot;
            if (s[j] > mx) mx = s[j];
        }
        double* o = out + th * L;
        for (int32_t d = 0; d < L; ++d) o[d] = 0.0;
        if (mx > -INFINITY) {
            double den = 0.0;
            for (int32_t j = 0; j < k_sel; ++j) {
                if (s[j] == -INFINITY) continue;
                const double p = exp(s[j] - mx);
                const int32_t r = idx[t * k_sel + j];
                den += p;
                for (int32_t d = 0; d < L; ++d)
                    o[d] += p * kd[(int64_t)r * L + d];
            }
            for (int32_t d = 0; d < L; ++d) o[d] /= den;
        }
        free(q); free(s);
    }
    free(kd);
    return err;
}
