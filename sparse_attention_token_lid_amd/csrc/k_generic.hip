// k_generic.hip -- vector-ALU scoring for any head count, head size and dtype
// (f32, f16, bf16, FP8 E4M3 with per-row scales), with the same streaming
// top-k as the MFMA kernels.
//
// The score is the indexer chain of ggml-org llama.cpp issue 25468 ("Root
// cause" comment): I = sum_h w_h * max(0, q_h . k), plus the f16 mask.  One
// wavefront owns one (query, key split) pair; each lane scores one key per
// step with f32 fused multiply-adds, and the 64 scores of a step go into the
// wavefront's top-k buffer.  This path exists for shapes the MFMA kernels do
// not cover (and for f32 inputs); it is correct for all of them, not fast.
#include "lid_device.h"
#include "lid_kernels.h"

namespace lid {
namespace {

constexpr int NWG = 4;  // wavefronts per workgroup

__device__ __forceinline__ float load_qk(const void* p, int64_t i, int dtype) {
  if (dtype == 0) return reinterpret_cast<const float*>(p)[i];
  if (dtype == 3) return e4m3_to_f32(reinterpret_cast<const uint8_t*>(p)[i]);
  const uint16_t b = reinterpret_cast<const uint16_t*>(p)[i];
  if (dtype == 1) return f16_bits_to_f32(b);
  return __uint_as_float((uint32_t)b << 16);
}

__global__ __launch_bounds__(NWG * 64) void generic_kernel(KArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int wv = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t* cand = reinterpret_cast<uint64_t*>(smem) + (size_t)wv * a.cap;
  uint32_t* hist = reinterpret_cast<uint32_t*>(reinterpret_cast<uint64_t*>(smem) + (size_t)NWG * a.cap) + wv * 256;

  const int64_t item = (int64_t)blockIdx.x * NWG + wv;
  const int P = a.P;
  if (item >= a.n_tok * P) return;  // whole wavefront; no block barriers below
  const int64_t t = item / P;
  const int p = (int)(item - t * P);

  int64_t lo = 0, hi = a.n_kv;
  if (a.kv_range) {
    int64_t l0 = a.kv_range[2 * t], h0 = a.kv_range[2 * t + 1];
    lo = l0 < 0 ? 0 : l0;
    hi = h0 > a.n_kv ? a.n_kv : h0;
    if (hi < lo) hi = lo;
  }
  const int64_t len = hi - lo;
  const int64_t c0 = lo + len * p / P, c1 = lo + len * (p + 1) / P;

  WaveTopK st;
  wave_topk_init(st, cand, hist, a.K, a.cap);
  const int H = a.H, D = a.D;
  for (int64_t s0 = c0; s0 < c1; s0 += kWave) {
    const int64_t s = s0 + lane;
    const bool inr = s < c1;
    float v = -__builtin_inff();
    if (inr) {
      float I = 0.f;
      for (int h = 0; h < H; ++h) {
        float dot = 0.f;
        const int64_t qo = (t * H + h) * (int64_t)D;
        for (int d = 0; d < D; ++d) dot = __builtin_fmaf(load_qk(a.q, qo + d, a.dtype), load_qk(a.k, s * D + d, a.dtype), dot);
        // FP8: positive per-row scales commute with the ReLU
        const float wh = a.dtype == 3 ? a.w[t * H + h] * a.q_scale[t * H + h] : a.w[t * H + h];
        I = __builtin_fmaf(wh, relu(dot), I);
      }
      if (a.dtype == 3) I *= a.k_scale[s];
      float mv = a.mask ? f16_bits_to_f32(a.mask[t * a.mask_ld + s]) : 0.f;
      v = (I + mv) + 0.0f;
    }
    const bool valid = inr && v != -__builtin_inff();
    wave_topk_insert(st, make_key(v, (uint32_t)s), valid);
  }
  wave_topk_finish(st);
  if (P == 1)
    wave_write_row(st.buf, a.K, a.idx + t * a.K, a.score ? a.score + t * a.K : nullptr, nullptr);
  else
    wave_write_row(st.buf, a.K, nullptr, nullptr, a.lists + ((size_t)t * P + p) * a.K);
}

}  // namespace

size_t generic_lds_bytes(int cap) { return (size_t)NWG * cap * 8 + (size_t)NWG * 256 * 4; }

hipError_t launch_generic(const KArgs& a, hipStream_t st) {
  hipError_t e = set_lds_limit(reinterpret_cast<const void*>(&generic_kernel), 160 * 1024);
  if (e != hipSuccess) return e;
  const int64_t items = a.n_tok * a.P;
  dim3 grid((unsigned)((items + NWG - 1) / NWG));
  hipLaunchKernelGGL(generic_kernel, grid, dim3(NWG * 64), generic_lds_bytes(a.cap), st, a);
  return hipGetLastError();
}

}  // namespace lid
