// k_prefill.hip -- MFMA scoring + fused epilogue + streaming top-k for a block
// of queries (the prefill shape: many query tokens, H = 64 heads, D = 128).
//
// What is computed follows the indexer chain of ggml-org llama.cpp issue
// 25468 ("Root cause" comment): per-head scores q.k, ReLU, times the head
// weight, summed over heads, plus the f16 mask, then a per-token top-k.  The
// per-head score tile never leaves registers and the head-reduced score of a
// (query, key) pair is consumed by the top-k the moment it exists, so neither
// the n_tok x H x n_kv nor the n_tok x n_kv matrix is ever written.
//
// Work decomposition.  A workgroup owns NW consecutive queries (one wavefront
// per query) and one of P contiguous chunks of the key range those queries can
// see.  Key tiles of 64 keys x 128 dims (16 KiB) are staged through LDS once
// per workgroup and shared by its NW wavefronts (double buffered).  With P a
// multiple of 8 the chunk index is blockIdx % P, so every workgroup that runs
// on one XCD (blocks are dealt round-robin to the 8 XCDs) reads the same 1/P
// of the keys and that slice stays in the XCD's own L2.
//
// Per wavefront and tile: S = Q_t (64 heads x 128) . K_tile^T with
// v_mfma_f32_32x32x16 (f16 or bf16 in, f32 accumulate): 2 row blocks of 32
// heads x 2 column blocks of 32 keys x 8 k-steps.  Heads run along the MFMA
// rows, so each lane holds 16 heads of one key and the head reduction
// sum_h w_h * max(S_h, 0) is 32 fused multiply-adds in registers plus one
// permlane32 swap that also turns the two 32-key halves into one 64-lane
// vector (lane l <-> key tile_base + l).
//
// The k-index of the MFMA is mapped to the head dimension as
// d = 64 * (lane / 32) + 8 * kstep + i, so each lane's 8 k-steps cover 128
// contiguous bytes of a q or k row.
#include "lid_device.h"
#include "lid_kernels.h"

namespace lid {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int DT> struct Mfma;
template <> struct Mfma<1> {
  typedef f16x8 T;
  static __device__ __forceinline__ f32x16 run(T a, T b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<2> {
  typedef bf16x8 T;
  static __device__ __forceinline__ f32x16 run(T a, T b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

constexpr int H = kMfmaHeads;
constexpr int D = kMfmaDim;
constexpr int TN = kPrefillTile;
constexpr int kTileBytes = TN * D * 2;       // 16 KiB
constexpr int kChunksPerTile = kTileBytes / 16;  // 16-byte chunks

__device__ __forceinline__ int swz(int row, int ch) { return row * D + ((ch ^ (row & 15)) << 3); }

template <int NW, int DT>
__global__ __launch_bounds__(NW * 64, 8 / NW) void prefill_kernel(KArgs a) {
  using M = Mfma<DT>;
  using T = typename M::T;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* ktile = reinterpret_cast<uint16_t*>(smem);  // [2][TN*D]
  uint64_t* cand = reinterpret_cast<uint64_t*>(smem + 2 * kTileBytes);
  uint32_t* hist = reinterpret_cast<uint32_t*>(cand + (size_t)NW * a.cap);
  int64_t* rlo = reinterpret_cast<int64_t*>(hist + NW * 256);
  int64_t* rhi = rlo + NW;

  const int wv = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 5, m = lane & 31;
  const int P = a.P;
  const int p = (int)(blockIdx.x % (unsigned)P);
  const int64_t qb = blockIdx.x / (unsigned)P;
  const int64_t t = qb * NW + wv;
  const bool has_q = t < a.n_tok;

  // visible range of this wave's query
  int64_t lo = 0, hi = 0;
  if (has_q) {
    lo = 0;
    hi = a.n_kv;
    if (a.kv_range) {
      int64_t l0 = a.kv_range[2 * t], h0 = a.kv_range[2 * t + 1];
      lo = l0 < 0 ? 0 : l0;
      hi = h0 > a.n_kv ? a.n_kv : h0;
      if (hi < lo) hi = lo;
    }
  }
  if (lane == 0) { rlo[wv] = lo; rhi[wv] = hi; }
  __syncthreads();
  int64_t ulo = INT64_MAX, uhi = 0;
  for (int w2 = 0; w2 < NW; ++w2) {
    if (rhi[w2] > rlo[w2]) {
      ulo = rlo[w2] < ulo ? rlo[w2] : ulo;
      uhi = rhi[w2] > uhi ? rhi[w2] : uhi;
    }
  }
  if (ulo >= uhi) { ulo = 0; uhi = 0; }
  const int64_t T0 = ulo / TN;
  const int64_t nt = (uhi + TN - 1) / TN - T0;
  const int64_t c0 = T0 + nt * p / P;
  const int64_t c1 = T0 + nt * (p + 1) / P;
  const int64_t wlo = lo > c0 * TN ? lo : c0 * TN;
  const int64_t whi = hi < c1 * TN ? hi : c1 * TN;

  // this wave's query in MFMA A-operand layout, and its head weights
  T A[2][8];
  float wr[2][16];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + (has_q ? t : 0) * H * D;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u32x4 v = {0, 0, 0, 0};
        if (has_q) v = *reinterpret_cast<const u32x4*>(qrow + (32 * rb + m) * D + 64 * g + 8 * j);
        A[rb][j] = __builtin_bit_cast(T, v);
      }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        int h = 32 * rb + 8 * (jj >> 2) + 4 * g + (jj & 3);
        wr[rb][jj] = has_q ? a.w[t * H + h] : 0.f;
      }
  }

  WaveTopK st;
  wave_topk_init(st, cand + (size_t)wv * a.cap, hist + wv * 256, a.K, a.cap);

  // cooperative global -> LDS copy of one key tile (16-byte chunks, XOR-swizzled)
  constexpr int PER_T = kChunksPerTile / (NW * 64);
  static_assert(PER_T * NW * 64 == kChunksPerTile, "tile copy must divide evenly");
  u32x4 stage[PER_T];
  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k);
  auto gload = [&](int64_t tile) {
#pragma unroll
    for (int r = 0; r < PER_T; ++r) {
      int c = threadIdx.x + r * NW * 64;
      int row = c >> 4, ch = c & 15;
      int64_t s = tile * TN + row;
      u32x4 v = {0, 0, 0, 0};
      if (s < a.n_kv) v = *reinterpret_cast<const u32x4*>(kbase + s * D + ch * 8);
      stage[r] = v;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < PER_T; ++r) {
      int c = threadIdx.x + r * NW * 64;
      int row = c >> 4, ch = c & 15;
      *reinterpret_cast<u32x4*>(ktile + buf * TN * D + swz(row, ch)) = stage[r];
    }
  };

  const int64_t ntile = c1 - c0;
  if (ntile > 0) {
    gload(c0);
    sstore(0);
  }
  __syncthreads();
  for (int64_t it = 0; it < ntile; ++it) {
    const int64_t tile = c0 + it;
    const int cur = (int)(it & 1);
    if (it + 1 < ntile) gload(tile + 1);
    const int64_t s0 = tile * TN;
    if (has_q && s0 < whi && s0 + TN > wlo) {
      const int64_t s = s0 + lane;
      const bool inr = s >= wlo && s < whi;
      float mv = 0.f;
      if (a.mask && inr) mv = f16_bits_to_f32(a.mask[t * a.mask_ld + s]);
      f32x16 acc[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[kb][rb][e] = 0.f;
      const uint16_t* kt = ktile + cur * TN * D;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int row = 32 * kb + m;
          T b = __builtin_bit_cast(T, *reinterpret_cast<const u32x4*>(kt + swz(row, 8 * g + j)));
          acc[kb][0] = M::run(A[0][j], b, acc[kb][0]);
          acc[kb][1] = M::run(A[1][j], b, acc[kb][1]);
        }
      }
      float part[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float sum = 0.f;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int e = 0; e < 16; ++e) sum = __builtin_fmaf(wr[rb][e], __builtin_fmaxf(acc[kb][rb][e], 0.f), sum);
        part[kb] = sum;
      }
      // lanes 0-31: key half 0 (both head halves summed), lanes 32-63: key half 1
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[1]), false, false);
      const float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      const float v = (tot + mv) + 0.0f;
      const bool valid = inr && v != -__builtin_inff();
      wave_topk_insert(st, make_key(v, (uint32_t)s), valid);
    }
    if (it + 1 < ntile) sstore(cur ^ 1);
    __syncthreads();
  }

  if (has_q) {
    wave_topk_finish(st);
    if (P == 1)
      wave_write_row(st.buf, a.K, a.idx + t * a.K, a.score ? a.score + t * a.K : nullptr, nullptr);
    else
      wave_write_row(st.buf, a.K, nullptr, nullptr, a.lists + ((size_t)t * P + p) * a.K);
  }
}

template <int NW, int DT>
hipError_t launch_one(const KArgs& a, hipStream_t st) {
  const size_t lds = prefill_lds_bytes(NW, a.cap);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<NW, DT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t nqb = (a.n_tok + NW - 1) / NW;
  dim3 grid((unsigned)(nqb * a.P));
  hipLaunchKernelGGL((prefill_kernel<NW, DT>), grid, dim3(NW * 64), lds, st, a);
  return hipGetLastError();
}

}  // namespace

size_t prefill_lds_bytes(int nw, int cap) {
  return 2 * (size_t)kTileBytes + (size_t)nw * cap * 8 + (size_t)nw * 256 * 4 + 2 * (size_t)nw * 8;
}

hipError_t launch_prefill(const KArgs& a, int nw, hipStream_t st) {
  if (a.dtype == 1) return nw == 8 ? launch_one<8, 1>(a, st) : launch_one<4, 1>(a, st);
  return nw == 8 ? launch_one<8, 2>(a, st) : launch_one<4, 2>(a, st);
}

}  // namespace lid
