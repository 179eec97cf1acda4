// k_scores.hip -- the score-only mode's helpers: the vector-ALU kernel for
// shapes the MFMA kernel does not take, and the fill of the positions the
// MFMA kernel does not visit.
//
// What is computed is the fused op's output in ggml-org llama.cpp issue 25468
// ("Pinned" comment: the indexer scores of every key for every query token,
// [n_kv, n_tok] in ggml order, i.e. row t of a C [n_tok, n_kv] array), with
// the updated API of fairydreaming/llama.cpp pull request 2 (last comment:
// no scale factors, an f16 mask added to the score): v[t, s] =
// sum_h w[t, h] * max(0, q[t, h, :] . k[s, :]) + mask[t, s], and -inf for keys
// outside the query's [lo, hi) range.
#include "lid_device.h"
#include "lid_kernels.h"

namespace lid {
namespace {

__device__ __forceinline__ float load_el(const void* p, int64_t i, int dtype) {
  if (dtype == 0) return reinterpret_cast<const float*>(p)[i];
  const uint16_t b = reinterpret_cast<const uint16_t*>(p)[i];
  if (dtype == 1) return f16_bits_to_f32(b);
  return __uint_as_float((uint32_t)b << 16);
}

__device__ __forceinline__ void query_range(const KArgs& a, int64_t t, int64_t& lo, int64_t& hi) {
  lo = 0;
  hi = a.n_kv;
  if (a.kv_range) {
    const int64_t l0 = a.kv_range[2 * t], h0 = a.kv_range[2 * t + 1];
    lo = l0 < 0 ? 0 : l0;
    hi = h0 > a.n_kv ? a.n_kv : h0;
    if (hi < lo) hi = lo;
  }
}

// One thread per (query, key): f32 fused multiply-adds, heads in order.
__global__ __launch_bounds__(256) void generic_scores_kernel(KArgs a, uint32_t chunks) {
  const int64_t t = blockIdx.x / chunks;
  const int64_t s = (int64_t)(blockIdx.x % chunks) * 256 + threadIdx.x;
  if (s >= a.n_kv) return;
  int64_t lo, hi;
  query_range(a, t, lo, hi);
  float v = -__builtin_inff();
  if (s >= lo && s < hi) {
    const int H = a.H, D = a.D;
    float I = 0.f;
    for (int h = 0; h < H; ++h) {
      float dot = 0.f;
      const int64_t qo = (t * H + h) * (int64_t)D;
      for (int d = 0; d < D; ++d) dot = __builtin_fmaf(load_el(a.q, qo + d, a.dtype), load_el(a.k, s * D + d, a.dtype), dot);
      I = __builtin_fmaf(a.w[t * H + h], relu(dot), I);
    }
    const float mv = a.mask ? f16_bits_to_f32(a.mask[t * a.mask_ld + s]) : 0.f;
    v = (I + mv) + 0.0f;
  }
  a.scores[t * a.scores_ld + s] = v;
}

// -inf at every key outside the query's range (one workgroup per query).
__global__ __launch_bounds__(256) void scores_fill_kernel(KArgs a) {
  const int64_t t = blockIdx.x;
  int64_t lo, hi;
  query_range(a, t, lo, hi);
  float* row = a.scores + t * a.scores_ld;
  for (int64_t s = threadIdx.x; s < lo; s += 256) __builtin_nontemporal_store(-__builtin_inff(), row + s);
  for (int64_t s = hi + threadIdx.x; s < a.n_kv; s += 256) __builtin_nontemporal_store(-__builtin_inff(), row + s);
}

}  // namespace

hipError_t launch_generic_scores(const KArgs& a, hipStream_t st) {
  const uint32_t chunks = (uint32_t)((a.n_kv + 255) / 256);  // the host checks chunks * n_tok < 2^31
  hipLaunchKernelGGL(generic_scores_kernel, dim3((unsigned)(chunks * a.n_tok)), dim3(256), 0, st, a, chunks);
  return hipGetLastError();
}

hipError_t launch_scores_fill(const KArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(scores_fill_kernel, dim3((unsigned)a.n_tok), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lid
