// lid_api.hip -- the C ABI (include/lid.h): argument checks, plan choice,
// workspace sizing and kernel launches.  No device memory is allocated here;
// nothing synchronises the host.
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <set>
#include <utility>

#include "lid.h"
#include "lid_device.h"
#include "lid_kernels.h"

// The static scratch of lid_topk_noalloc: a device array of fixed size, one
// copy per GPU (each at its own address), held until the process ends.  Host
// code never uses the array's name as an address (on the host it is a
// stand-in, not device memory): the address comes from hipGetSymbolAddress,
// looked up once per device with that device current, and is kept per device
// (scratch_address below).
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

using namespace lid;

constexpr int kMaxTopK = 1024;
constexpr int kMaxSplits = 1024;
constexpr int kDecodeMaxTok = 4;       // auto plan: at most this many queries use the decode kernel
constexpr int kDecodeKeysPerSplit = 128;
constexpr int64_t kCUs = 256;          // MI355X compute units
constexpr int kDecodeMaxSplits = 256;  // bounds the decode workspace independently of n_kv
constexpr size_t kMaxLds = 160 * 1024;
constexpr int kTreeCapHost = 512;     // k_top range of the decode merge tree: next_pow2(k_top) == 512
// Every workspace starts with a counter region of this fixed size; the data
// of every plan follows it.  The finishing counters of the split plans live
// there (at most kMaxCounters of them), every call leaves them at zero, and no
// entry point writes anything else into the region: so a workspace that was
// zeroed once stays valid for any later shape, plan or entry point.
constexpr size_t kCounterRegion = 4096;
constexpr int64_t kMaxCounters = (int64_t)(kCounterRegion / 4);

struct Plan {
  int kind;         // lid_plan (never AUTO)
  int P;            // key splits per query
  int nw;           // prefill: wavefronts (queries) per workgroup
  int cap;          // per-wave candidate capacity
  int keys_per_wg;  // decode: LDS key slots per workgroup
  int ch;           // merge: entries per list per round
  int form;         // decode finish: 0 sorted split lists, 1 raw scores (the last workgroup
                    // selects from all of them), 2 / 3 split summaries (the best 16 / 8 keys of
                    // every split; a split is scored again if its summary is too short)
  int fuse;         // prefill, P > 1: the scoring kernel finishes from the split lists itself
                    // (1: merging sorted lists, 2: selecting from unsorted ones)
  int64_t raw_ld;   // decode, raw form: scores per query row
  size_t ws;        // workspace bytes (0, or kCounterRegion + the plan's data)
  bool counters;    // the plan keeps finishing counters in the counter region
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

std::mutex g_attr_mu;
std::set<std::pair<const void*, int>> g_attr_done;  // (kernel, device) with the LDS limit raised

thread_local hipError_t g_last_hip_error = hipSuccess;
hipEvent_t g_prof_before = nullptr;  // recorded around the scoring kernel when set
hipEvent_t g_prof_after = nullptr;

int hip_fail(hipError_t e) {
  g_last_hip_error = e;
  return LID_ERR_HIP;
}

int merge_chunk(int P, int K) {
  // read about 4K entries in the first round, at least 4 per list
  int ch = next_pow2((int)cdiv(4LL * K, P));
  if (ch < 4) ch = 4;
  if (ch > next_pow2(K)) ch = next_pow2(K);
  while (ch > 4 && (size_t)P * ch > 8192) ch >>= 1;
  return ch;
}

int check_shape(const lid_shape* s) {
  if (!s) return LID_ERR_INVALID_ARG;
  if (s->n_tok < 0 || s->n_kv < 0 || s->n_kv > INT32_MAX || s->n_tok > INT32_MAX) return LID_ERR_INVALID_ARG;
  if (s->n_head < 1 || s->head_dim < 1 || s->k_top < 1) return LID_ERR_INVALID_ARG;
  if (s->qk_dtype != LID_F32 && s->qk_dtype != LID_F16 && s->qk_dtype != LID_BF16 && s->qk_dtype != LID_F8E4M3)
    return LID_ERR_INVALID_ARG;
  if (s->plan < LID_PLAN_AUTO || s->plan > LID_PLAN_DECODE || s->splits < 0) return LID_ERR_INVALID_ARG;
  if (s->k_top > kMaxTopK || s->splits > kMaxSplits) return LID_ERR_UNSUPPORTED;
  return LID_OK;
}

int make_plan(const lid_shape* s, Plan* pl) {
  int rc = check_shape(s);
  if (rc) return rc;
  const int K = s->k_top;
  const bool mfma_shape = s->n_head == kMfmaHeads && s->head_dim == kMfmaDim;
  const bool fp8 = s->qk_dtype == LID_F8E4M3;
  const bool mfma_ok = (s->qk_dtype == LID_F16 || s->qk_dtype == LID_BF16 || fp8) && mfma_shape;
  memset(pl, 0, sizeof(*pl));
  pl->cap = prefill_cap(K);  // per-wave candidate slots (lid_budget.h)
  int kind = s->plan;
  if (kind == LID_PLAN_AUTO) {
    if (!mfma_ok) kind = LID_PLAN_GENERIC;
    else if (s->n_tok <= kDecodeMaxTok && cdiv(s->n_kv, kDecodeMaxSplits) <= kDecodeMaxKeys) kind = LID_PLAN_DECODE;
    else kind = LID_PLAN_PREFILL;
  }
  if ((kind == LID_PLAN_PREFILL || kind == LID_PLAN_DECODE) && !mfma_ok) return LID_ERR_UNSUPPORTED;
  pl->kind = kind;

  if (kind == LID_PLAN_GENERIC) {
    int64_t want = cdiv(s->n_kv, 8192);
    pl->P = s->splits ? s->splits : (int)(want < 1 ? 1 : (want > 64 ? 64 : want));
    if (generic_lds_bytes(pl->cap) > kMaxLds) return LID_ERR_UNSUPPORTED;
  } else if (kind == LID_PLAN_PREFILL) {
    pl->nw = (K <= 512) ? 8 : 4;
    const int64_t tiles = cdiv(s->n_kv, kPrefillTile);
    int P = s->splits;
    if (!P) {
      // enough (query block, split) workgroups for one per CU, but never a
      // split shorter than 2048 keys
      const int64_t nqb = s->n_tok > 0 ? cdiv(s->n_tok, pl->nw) : 1;
      int64_t want = cdiv(kCUs, nqb);
      const int64_t min_tiles = 2048 / kPrefillTile;
      const int64_t cap = tiles / min_tiles > 1 ? tiles / min_tiles : 1;
      want = want < cap ? want : cap;
      P = (int)(want < 1 ? 1 : (want > 64 ? 64 : want));
    }
    pl->P = P;
    if (prefill_lds_bytes(pl->nw, pl->cap) + 2 * (size_t)kPrefillTile * kMfmaDim * 2 > kMaxLds)
      return LID_ERR_UNSUPPORTED;
    if (P > 1) {
      // workspace: the split lists after the counter region; with few splits
      // the last workgroup of a query block merges them, counted by one
      // counter per query block (the register merge needs next_pow2(K) in
      // 256..1024 and an even K); otherwise the merge kernel does it
      const int n2 = next_pow2(K);
      const bool fusable = P <= kFuseMaxSplits && n2 >= 256 && n2 <= 1024 && K % 2 == 0 &&
                           cdiv(s->n_tok, pl->nw) <= kMaxCounters;
      pl->fuse = !fusable ? 0 : (P > kFuseMergeSplits && (int64_t)P * K <= 64 * kFuseSelectRows ? 2 : 1);
      pl->counters = pl->fuse != 0;
      pl->ws = kCounterRegion + (size_t)s->n_tok * P * K * sizeof(uint64_t);
      if (!pl->fuse) {
        pl->ch = merge_chunk(P, K);
        if (merge_lds_bytes(P, K, pl->ch) > kMaxLds) return LID_ERR_UNSUPPORTED;
      }
    }
  } else {  // decode
    int P = s->splits;
    if (!P) {
      int64_t want = cdiv(s->n_kv, kDecodeKeysPerSplit);
      P = (int)(want < 1 ? 1 : (want > kDecodeMaxSplits ? kDecodeMaxSplits : want));
    }
    pl->P = P;
    if (s->n_tok > kMaxCounters) return LID_ERR_UNSUPPORTED;  // one finishing counter per query
    int64_t kp = cdiv(cdiv(s->n_kv, 32), P) * 32;
    if (kp < 32) kp = 32;
    if (kp > kDecodeMaxKeys) return LID_ERR_UNSUPPORTED;
    pl->keys_per_wg = (int)kp;
    const int64_t span = cdiv(s->n_kv, 32) * 32;  // longest visible range, in 32-key blocks
    // summaries of C keys per split when the finish's selection applies and
    // 4 K <= P C <= 4096 (then a split rarely holds more than C of the
    // answer): C = 8 when the splits are that many, else 16; otherwise raw
    // scores for short ranges, sorted split lists for long ones
    int tc = 0;
    if (P >= 2 && next_pow2(K) == kTreeCapHost) {
      for (int c : {8, kDecodeTopsC})
        if (!tc && (int64_t)P * c >= 4LL * K && (int64_t)P * c <= kDecodeTopsMax) tc = c;
    }
    pl->form = tc == 8 ? 3 : (tc ? 2 : (span <= kRawMax ? 1 : 0));
    if (P > 1 && pl->form == 0) pl->ch = merge_chunk(P, K);
    if (decode_lds_bytes(pl->keys_per_wg, K, P, pl->ch, pl->form) > kMaxLds) return LID_ERR_UNSUPPORTED;
    // workspace: one counter per query in the counter region, then the raw
    // scores, the per-split lists or the summaries
    pl->counters = true;
    if (pl->form == 1) {
      pl->raw_ld = cdiv(span, 64) * 64;
      pl->ws = kCounterRegion + (size_t)s->n_tok * pl->raw_ld * sizeof(uint32_t);
    } else if (pl->form >= 2) {
      pl->ws = kCounterRegion + (size_t)s->n_tok * P * tc * sizeof(uint64_t);
    } else {
      pl->ws = kCounterRegion + (P > 1 ? (size_t)s->n_tok * P * K * sizeof(uint64_t) : 0);
    }
  }
  if (pl->P > 1 && kind == LID_PLAN_GENERIC) {
    pl->ch = merge_chunk(pl->P, K);
    if (merge_lds_bytes(pl->P, K, pl->ch) > kMaxLds) return LID_ERR_UNSUPPORTED;
    pl->ws = kCounterRegion + (size_t)s->n_tok * pl->P * K * sizeof(uint64_t);
  }
  // grid sizes must fit a 32-bit grid
  const int64_t blocks = (kind == LID_PLAN_PREFILL) ? cdiv(s->n_tok, pl->nw) * pl->P
                         : (kind == LID_PLAN_DECODE) ? s->n_tok * pl->P
                                                     : cdiv(s->n_tok * pl->P, 4);
  if (blocks > INT32_MAX) return LID_ERR_UNSUPPORTED;
  return LID_OK;
}

}  // namespace

namespace lid {
hipError_t set_lds_limit(const void* kernel, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_attr_mu);
  if (g_attr_done.count({kernel, dev})) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) g_attr_done.insert({kernel, dev});
  return e;
}
}  // namespace lid

extern "C" {

size_t lid_topk_workspace_size(const lid_shape* shape) {
  Plan pl;
  if (make_plan(shape, &pl) != LID_OK) return 0;
  return pl.ws;
}

int lid_topk_plan(const lid_shape* shape, int32_t* splits_out) {
  Plan pl;
  int rc = make_plan(shape, &pl);
  if (rc != LID_OK) return rc;
  if (splits_out) *splits_out = pl.P;
  return pl.kind;
}

}  // extern "C"

namespace {

// zeroes n 32-bit words (the counter region of the static scratch: a kernel,
// not hipMemsetAsync, so that a captured graph replays it reliably)
__global__ void zero_words_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// clear_counters: zero the workspace's counter region on the stream before
// the scoring kernel (the static scratch keeps whatever the previous call on
// the device left there)
int topk_impl(const lid_shape* shape, const void* q, const float* q_scale, const void* k, const float* k_scale,
              const float* w, const uint16_t* mask, const int32_t* kv_range, int32_t* idx, float* score,
              void* workspace, size_t workspace_bytes, void* stream, bool clear_counters = false) {
  Plan pl;
  int rc = make_plan(shape, &pl);
  if (rc != LID_OK) return rc;
  const lid_shape& s = *shape;
  if ((s.qk_dtype == LID_F8E4M3) != (q_scale != nullptr && k_scale != nullptr)) return LID_ERR_INVALID_ARG;
  if (s.n_tok == 0) return LID_OK;
  if (!q || !w || !idx || (s.n_kv > 0 && !k)) return LID_ERR_INVALID_ARG;
  if (mask && s.mask_ld < s.n_kv) return LID_ERR_INVALID_ARG;
  if (pl.kind != LID_PLAN_GENERIC &&
      ((reinterpret_cast<uintptr_t>(q) & 15) || (reinterpret_cast<uintptr_t>(k) & 15)))
    return LID_ERR_INVALID_ARG;
  if (pl.ws > 0 && (!workspace || workspace_bytes < pl.ws)) return LID_ERR_WORKSPACE;
  if (pl.ws > 0 && (reinterpret_cast<uintptr_t>(workspace) & 7)) return LID_ERR_INVALID_ARG;

  KArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.w = w;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.mask = mask;
  a.kv_range = kv_range;
  a.idx = idx;
  a.score = score;
  if (pl.ws > 0) {
    unsigned char* data = reinterpret_cast<unsigned char*>(workspace) + kCounterRegion;
    a.counters = pl.counters ? reinterpret_cast<uint32_t*>(workspace) : nullptr;
    a.lists = reinterpret_cast<uint64_t*>(data);
    a.raw = reinterpret_cast<uint32_t*>(data);
    a.raw_ld = pl.raw_ld;
  }
  a.n_tok = s.n_tok;
  a.n_kv = s.n_kv;
  a.mask_ld = mask ? s.mask_ld : 0;
  a.H = s.n_head;
  a.D = s.head_dim;
  a.K = s.k_top;
  a.P = pl.P;
  a.cap = pl.cap;
  a.dtype = s.qk_dtype;
  a.fuse = pl.fuse;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);

  hipError_t e;
  if (clear_counters && pl.counters) {
    hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3((unsigned)kMaxCounters), 0, st,
                       reinterpret_cast<uint32_t*>(workspace), (int)kMaxCounters);
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e);
  }
  if (g_prof_before && (e = hipEventRecord(g_prof_before, st)) != hipSuccess) return hip_fail(e);
  if (pl.kind == LID_PLAN_PREFILL) e = launch_prefill(a, pl.nw, st);
  else if (pl.kind == LID_PLAN_DECODE) e = launch_decode(a, pl.keys_per_wg, pl.ch, pl.form, st);
  else e = launch_generic(a, st);
  if (e != hipSuccess) return hip_fail(e);
  if (g_prof_after && (e = hipEventRecord(g_prof_after, st)) != hipSuccess) return hip_fail(e);
  if (pl.P > 1 && pl.kind != LID_PLAN_DECODE && !pl.fuse) {
    e = launch_merge(a, pl.ch, st);
    if (e != hipSuccess) return hip_fail(e);
  }
  return LID_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device; null until looked up

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int lid_topk(const lid_shape* shape, const void* q, const void* k, const float* w, const uint16_t* mask,
             const int32_t* kv_range, int32_t* idx, float* score, void* workspace, size_t workspace_bytes,
             void* stream) {
  return topk_impl(shape, q, nullptr, k, nullptr, w, mask, kv_range, idx, score, workspace, workspace_bytes, stream);
}

int lid_topk_fp8(const lid_shape* shape, const void* q, const float* q_scale, const void* k, const float* k_scale,
                 const float* w, const uint16_t* mask, const int32_t* kv_range, int32_t* idx, float* score,
                 void* workspace, size_t workspace_bytes, void* stream) {
  if (!shape || shape->qk_dtype != LID_F8E4M3 || !q_scale || !k_scale) return LID_ERR_INVALID_ARG;
  return topk_impl(shape, q, q_scale, k, k_scale, w, mask, kv_range, idx, score, workspace, workspace_bytes, stream);
}

int lid_topk_noalloc(const lid_shape* shape, const void* q, const void* k, const float* w, const uint16_t* mask,
                     const int32_t* kv_range, int32_t* idx, float* score, void* stream) {
  Plan pl;
  int rc = make_plan(shape, &pl);
  if (rc != LID_OK) return rc;
  if (pl.ws > kScratchBytes) return LID_ERR_WORKSPACE;  // needs more than the static scratch holds
  void* ws = nullptr;
  if (pl.ws > 0 && shape->n_tok > 0) {
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return hip_fail(e);
  }
  return topk_impl(shape, q, nullptr, k, nullptr, w, mask, kv_range, idx, score, ws, ws ? kScratchBytes : 0, stream,
                   true);
}

int lid_scores(const lid_shape* shape, const void* q, const void* k, const float* w, const uint16_t* mask,
               const int32_t* kv_range, float* scores, int64_t scores_ld, void* stream) {
  if (!shape) return LID_ERR_INVALID_ARG;
  if (shape->qk_dtype == LID_F8E4M3) return LID_ERR_UNSUPPORTED;  // (no scale arguments here)
  // the scoring plan: the prefill kernel's key splits (k_top does not matter)
  lid_shape ps = *shape;
  ps.k_top = 512;
  ps.plan = LID_PLAN_AUTO;
  ps.splits = 0;
  const bool mfma = (ps.qk_dtype == LID_F16 || ps.qk_dtype == LID_BF16) && ps.n_head == kMfmaHeads &&
                    ps.head_dim == kMfmaDim && shape->plan != LID_PLAN_GENERIC;
  ps.plan = mfma ? LID_PLAN_PREFILL : LID_PLAN_GENERIC;
  Plan pl;
  int rc = make_plan(&ps, &pl);
  if (rc != LID_OK) return rc;
  const lid_shape& s = *shape;
  if (s.n_tok == 0 || s.n_kv == 0) return LID_OK;
  if (!q || !k || !w || !scores || scores_ld < s.n_kv) return LID_ERR_INVALID_ARG;
  if (mask && s.mask_ld < s.n_kv) return LID_ERR_INVALID_ARG;
  if (mfma && ((reinterpret_cast<uintptr_t>(q) & 15) || (reinterpret_cast<uintptr_t>(k) & 15)))
    return LID_ERR_INVALID_ARG;
  if (!mfma && s.n_tok * cdiv(s.n_kv, 256) > INT32_MAX) return LID_ERR_UNSUPPORTED;

  KArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.w = w;
  a.mask = mask;
  a.kv_range = kv_range;
  a.scores = scores;
  a.scores_ld = scores_ld;
  a.n_tok = s.n_tok;
  a.n_kv = s.n_kv;
  a.mask_ld = mask ? s.mask_ld : 0;
  a.H = s.n_head;
  a.D = s.head_dim;
  a.K = ps.k_top;
  a.P = pl.P;
  a.cap = pl.cap;
  a.dtype = s.qk_dtype;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (mfma && kv_range && (e = launch_scores_fill(a, st)) != hipSuccess) return hip_fail(e);
  if (g_prof_before && (e = hipEventRecord(g_prof_before, st)) != hipSuccess) return hip_fail(e);
  e = mfma ? launch_prefill_scores(a, st) : launch_generic_scores(a, st);
  if (e != hipSuccess) return hip_fail(e);
  if (g_prof_after && (e = hipEventRecord(g_prof_after, st)) != hipSuccess) return hip_fail(e);
  return LID_OK;
}

}  // extern "C"

// ------------------------------------------------------------------ shared top-k
namespace {

struct SharedPlan {
  int nqc;        // query chunks (partial sums per key)
  int qchunk;     // queries per chunk
  int P;          // selection workgroups (sorted lists) over the keys
  int ch;         // merge chunk when P > 1
  bool one;       // one workgroup selects from every key (no lists, no merge)
  size_t ws;      // workspace bytes
  size_t ws_lists;  // offset of the lists
};

int make_shared_plan(const lid_shape* s, SharedPlan* sp) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (s->qk_dtype != LID_F16 && s->qk_dtype != LID_BF16) return LID_ERR_UNSUPPORTED;
  if (s->n_head != kMfmaHeads || s->head_dim != kMfmaDim) return LID_ERR_UNSUPPORTED;
  memset(sp, 0, sizeof(*sp));
  const int64_t groups = cdiv(s->n_kv, kSharedGroupKeys);
  // enough (key group, query chunk) workgroups for one per CU
  int64_t nqc = groups > 0 ? cdiv(kCUs, groups) : 1;
  nqc = nqc < 16 ? nqc : 16;
  nqc = nqc < (s->n_tok > 0 ? s->n_tok : 1) ? nqc : (s->n_tok > 0 ? s->n_tok : 1);
  sp->nqc = (int)(nqc < 1 ? 1 : nqc);
  sp->qchunk = (int)(s->n_tok > 0 ? cdiv(s->n_tok, sp->nqc) : 1);
  sp->one = s->n_kv <= kSharedSelectKeys && shared_select_lds_bytes(s->k_top) <= kMaxLds;
  const int64_t P = sp->one ? 1 : cdiv(s->n_kv, kSharedListKeys);
  if (P > kMaxSplits) return LID_ERR_UNSUPPORTED;
  sp->P = (int)(P < 1 ? 1 : P);
  if (!sp->one && shared_lists_lds_bytes(s->k_top) > kMaxLds) return LID_ERR_UNSUPPORTED;
  if (sp->P > 1) {
    sp->ch = merge_chunk(sp->P, s->k_top);
    if (shared_merge_lds_bytes(sp->P, s->k_top, sp->ch) > kMaxLds) return LID_ERR_UNSUPPORTED;
  }
  if (groups * sp->nqc > INT32_MAX) return LID_ERR_UNSUPPORTED;
  // after the counter region (not used here, but kept out of, so that one
  // workspace can serve lid_topk and lid_topk_shared): the partial sums, then
  // the lists
  sp->ws_lists = kCounterRegion + (size_t)cdiv((int64_t)sp->nqc * s->n_kv * 4, 256) * 256;
  sp->ws = sp->ws_lists + (sp->P > 1 ? (size_t)sp->P * s->k_top * sizeof(uint64_t) : 0);
  return LID_OK;
}

}  // namespace

extern "C" {

size_t lid_topk_shared_workspace_size(const lid_shape* shape) {
  SharedPlan sp;
  if (!shape || make_shared_plan(shape, &sp) != LID_OK) return 0;
  return sp.ws;
}

int lid_topk_shared(const lid_shape* shape, const void* q, const void* k, const float* w, const uint16_t* mask,
                    const int32_t* kv_range, int32_t* idx, float* score, void* workspace, size_t workspace_bytes,
                    void* stream) {
  if (!shape) return LID_ERR_INVALID_ARG;
  SharedPlan sp;
  int rc = make_shared_plan(shape, &sp);
  if (rc != LID_OK) return rc;
  const lid_shape& s = *shape;
  if (!idx || (s.n_tok > 0 && (!q || !w)) || (s.n_kv > 0 && !k)) return LID_ERR_INVALID_ARG;
  if (mask && s.mask_ld < s.n_kv) return LID_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(q) & 15) || (reinterpret_cast<uintptr_t>(k) & 15)) return LID_ERR_INVALID_ARG;
  if (sp.ws > 0 && (!workspace || workspace_bytes < sp.ws)) return LID_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 7) return LID_ERR_INVALID_ARG;

  KArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.w = w;
  a.mask = mask;
  a.kv_range = kv_range;
  a.idx = idx;
  a.score = score;
  a.scores = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(workspace) + kCounterRegion);
  a.scores_ld = s.n_kv;
  a.lists = reinterpret_cast<uint64_t*>(reinterpret_cast<unsigned char*>(workspace) + sp.ws_lists);
  a.n_tok = s.n_tok;
  a.n_kv = s.n_kv;
  a.mask_ld = mask ? s.mask_ld : 0;
  a.H = s.n_head;
  a.D = s.head_dim;
  a.K = s.k_top;
  a.P = sp.P;
  a.dtype = s.qk_dtype;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (g_prof_before && (e = hipEventRecord(g_prof_before, st)) != hipSuccess) return hip_fail(e);
  if ((e = launch_shared_scores(a, sp.qchunk, sp.nqc, st)) != hipSuccess) return hip_fail(e);
  if (g_prof_after && (e = hipEventRecord(g_prof_after, st)) != hipSuccess) return hip_fail(e);
  if (sp.one) {
    if ((e = launch_shared_select(a, sp.nqc, st)) != hipSuccess) return hip_fail(e);
  } else if ((e = launch_shared_lists(a, sp.nqc, st)) != hipSuccess) {
    return hip_fail(e);
  }
  if (sp.P > 1) {
    if ((e = launch_shared_merge(a, sp.ch, st)) != hipSuccess) return hip_fail(e);
  }
  return LID_OK;
}

int lid_sparse_attn(int64_t n_tok, int64_t n_kv, int32_t n_head, int32_t latent_dim, int32_t k_sel,
                    int32_t qk_dtype, const void* qa, const void* kv, const int32_t* idx, float scale, float* out,
                    void* stream) {
  if (n_tok < 0 || n_kv < 0 || n_kv > INT32_MAX || n_head < 1 || latent_dim < 8 || k_sel < 0)
    return LID_ERR_INVALID_ARG;
  if (latent_dim % 8 != 0 || !(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
    return LID_ERR_INVALID_ARG;
  if (qk_dtype != LID_F16 && qk_dtype != LID_BF16) return LID_ERR_UNSUPPORTED;
  if (latent_dim > 1024) return LID_ERR_UNSUPPORTED;
  if (n_tok == 0) return LID_OK;
  // 256-lane workgroups, one per query and 64 heads (latent width 512, MFMA) or 4 heads
  // (other widths): the grid's lane count must fit 32 bits
  const int64_t heads_per_wg = latent_dim == 512 ? 64 : 4;
  if (n_tok * ((n_head + heads_per_wg - 1) / heads_per_wg) > (int64_t)(1u << 24) - 1) return LID_ERR_UNSUPPORTED;
  if (!qa || !out || (k_sel > 0 && !idx) || (n_kv > 0 && k_sel > 0 && !kv)) return LID_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(qa) & 15) || (reinterpret_cast<uintptr_t>(kv) & 15) ||
      (reinterpret_cast<uintptr_t>(out) & 15) || (reinterpret_cast<uintptr_t>(idx) & 3))
    return LID_ERR_INVALID_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // with no keys every entry is invalid: the result is that of an empty selection
  const int ks = n_kv == 0 ? 0 : k_sel;
  hipError_t e;
  if (g_prof_before && (e = hipEventRecord(g_prof_before, st)) != hipSuccess) return hip_fail(e);
  if ((e = launch_sparse_attn(qa, kv, idx, out, n_tok, n_kv, n_head, latent_dim, ks, qk_dtype, scale, st)) !=
      hipSuccess)
    return hip_fail(e);
  if (g_prof_after && (e = hipEventRecord(g_prof_after, st)) != hipSuccess) return hip_fail(e);
  return LID_OK;
}

const char* lid_status_string(int status) {
  switch (status) {
    case LID_OK: return "ok";
    case LID_ERR_INVALID_ARG: return "invalid argument";
    case LID_ERR_UNSUPPORTED: return "unsupported shape or option";
    case LID_ERR_WORKSPACE: return "workspace missing or too small";
    case LID_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

void lid_set_profile_events(void* before_scoring, void* after_scoring) {
  g_prof_before = reinterpret_cast<hipEvent_t>(before_scoring);
  g_prof_after = reinterpret_cast<hipEvent_t>(after_scoring);
}

const char* lid_last_hip_error(void) { return hipGetErrorString(g_last_hip_error); }

int lid_version(void) { return 100; }

}  // extern "C"
