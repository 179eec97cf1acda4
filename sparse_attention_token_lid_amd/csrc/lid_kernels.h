// lid_kernels.h -- internal interface between the C-ABI host code and the
// HIP kernels of the fused lightning-indexer top-k.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lid {

// Arguments shared by every kernel (passed by value).
struct KArgs {
  const void* q;            // [n_tok, H, D] f32 / f16 bits / bf16 bits
  const void* k;            // [n_kv, D]
  const float* w;           // [n_tok, H]
  const float* q_scale;     // FP8 (dtype 3): [n_tok, H] per-row scale of q, else null
  const float* k_scale;     // FP8 (dtype 3): [n_kv] per-row scale of k, else null
  const uint16_t* mask;     // [n_tok, mask_ld] f16 bits, or null
  const int32_t* kv_range;  // [n_tok, 2], or null
  int32_t* idx;             // [n_tok, K]
  float* score;             // [n_tok, K], or null
  uint64_t* lists;          // [n_tok, P, K] per-split sorted candidate keys (P > 1); decode summary
                            // forms: [n_tok, P, C] split summaries (C = 16 or 8)
  uint32_t* raw;            // decode, raw form: [n_tok, raw_ld] ordered scores (0 = no key)
  float* scores;            // score-only mode: [n_tok, scores_ld] f32 output; shared top-k:
                            // [query chunks, scores_ld] partial sums over the ubatch
  int64_t scores_ld;
  uint32_t* counters;       // finished-workgroup counters (zero between launches): decode [n_tok],
                            // prefill with a fused finish [query blocks]
  int64_t n_tok, n_kv, mask_ld, raw_ld;
  int32_t H, D, K, P;
  int32_t cap;              // per-wave candidate buffer capacity (entries)
  int32_t dtype;            // 0 f32, 1 f16, 2 bf16, 3 FP8 E4M3 (with q_scale, k_scale)
  int32_t fuse;             // prefill, P > 1: the last workgroup of a query block finishes the
                            // query's top-k from the split lists: 1 = sorted lists merged,
                            // 2 = unsorted lists selected from (P K <= 64 kFuseSelectRows)
};

// Shapes the MFMA kernels are written for.
constexpr int kMfmaHeads = 64;
constexpr int kMfmaDim = 128;
constexpr int kPrefillTile = 128;      // keys per LDS tile
constexpr int kDecodeMaxKeys = 8192;   // keys one decode workgroup scores (LDS bound)
constexpr int kRawMax = 32768;         // decode, raw form: longest visible range per query
constexpr int kDecodeTopsC = 16;       // decode, summary forms: keys in each split's summary (16, or 8)
constexpr int kDecodeTopsMax = 4096;   // decode, summary forms: most summary keys per query (P C)
constexpr int kSharedGroupKeys = 512;  // shared top-k: keys per scoring workgroup (64 per wavefront)
constexpr int kSharedSelectKeys = 16384;  // shared top-k: most keys for the one-workgroup selection
constexpr int kSharedListKeys = 4096;  // shared top-k: keys per selection workgroup (one sorted list each)
constexpr int kFuseMaxSplits = 16;     // prefill: most splits merged inside the scoring kernel
constexpr int kFuseSelectRows = 32;    // prefill: the finish selects from P K <= 64 x this keys
constexpr int kFuseMergeSplits = 4;   // prefill: up to this many splits, sorted lists are merged
                                      // (their bucket passes plus the register merges cost less
                                      // than radix cuts plus one selection over P K keys)

// Raises a kernel's dynamic-LDS limit to `bytes` on the current device, once
// per (kernel, device); thread-safe.
hipError_t set_lds_limit(const void* kernel, int bytes);

// Launchers (return hipSuccess or the launch error).
hipError_t launch_prefill(const KArgs& a, int nw, hipStream_t st);
hipError_t launch_prefill_scores(const KArgs& a, hipStream_t st);  // score-only mode, 8 queries per workgroup
hipError_t launch_scores_fill(const KArgs& a, hipStream_t st);     // -inf outside each query's range
hipError_t launch_generic_scores(const KArgs& a, hipStream_t st);  // score-only mode, any shape
size_t prefill_lds_bytes(int nw, int cap);

// decode finish forms: 0 sorted split lists, 1 raw scores, 2 / 3 split summaries of 16 / 8 keys
hipError_t launch_decode(const KArgs& a, int keys_per_wg, int ch, int form, hipStream_t st);
size_t decode_lds_bytes(int keys_per_wg, int K, int P, int ch, int form);

// shared (per-ubatch) top-k: partial sums of U over nqc query chunks into
// a.scores [nqc, scores_ld], then a.P sorted lists of a.K keys (or, when a.P
// == 1, the output row itself)
hipError_t launch_shared_scores(const KArgs& a, int qchunk, int nqc, hipStream_t st);
hipError_t launch_shared_lists(const KArgs& a, int nqc, hipStream_t st);
size_t shared_lists_lds_bytes(int K);
size_t shared_select_lds_bytes(int K);
hipError_t launch_shared_select(const KArgs& a, int nqc, hipStream_t st);
hipError_t launch_shared_merge(const KArgs& a, int ch, hipStream_t st);  // a.P lists of a.K -> the output row
size_t shared_merge_lds_bytes(int P, int K, int ch);

// sparse attention over the selected latent rows (dtype: 1 f16, 2 bf16; L <= 1024, L % 8 == 0)
hipError_t launch_sparse_attn(const void* qa, const void* kv, const int32_t* idx, float* out, int64_t n_tok,
                              int64_t n_kv, int H, int L, int k_sel, int dtype, float scale, hipStream_t st);

hipError_t launch_merge(const KArgs& a, int ch, hipStream_t st);
size_t merge_lds_bytes(int P, int K, int ch);

hipError_t launch_generic(const KArgs& a, hipStream_t st);
size_t generic_lds_bytes(int cap);

}  // namespace lid
