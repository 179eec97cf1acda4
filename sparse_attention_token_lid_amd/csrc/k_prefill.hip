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

  // Key tiles go straight from global memory to LDS (global_load_lds_dwordx4:
  // each lane's 16 bytes land at LDS base + 16 * lane, so one instruction
  // fills 1 KiB = 4 rows).  The XOR swizzle of the LDS layout is applied by
  // permuting which 16-byte chunk each lane fetches.  Rows past n_kv are
  // clamped to the last key (never scored), so the loads need no branches.
  constexpr int kInstPerTile = kTileBytes / 1024;           // 16
  constexpr int kInstPerWave = kInstPerTile / NW;
  static_assert(kInstPerWave * NW == kInstPerTile, "tile copy must divide evenly");
  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k);
  const int64_t last_key = a.n_kv - 1;
  auto gload = [&](int64_t tile, int buf) {
#pragma unroll
    for (int r = 0; r < kInstPerWave; ++r) {
      const int q = wv * kInstPerWave + r;          // 1 KiB piece of the tile
      const int row = 4 * q + (lane >> 4);
      const int ch = (lane & 15) ^ (row & 15);
      int64_t s = tile * TN + row;
      s = s < last_key ? s : last_key;
      __builtin_amdgcn_global_load_lds(kbase + s * D + ch * 8, ktile + buf * TN * D + q * 512, 16, 0, 0);
    }
  };
  // this wave's mask values for one tile (lane l <-> key tile*64 + l); read one
  // tile ahead so that no wait on global memory sits in front of the MFMAs
  const bool wave_has_keys = has_q && whi > wlo;
  const uint16_t* mrow = a.mask ? a.mask + (has_q ? t : 0) * a.mask_ld : nullptr;
  auto mload = [&](int64_t tile) -> uint16_t {
    if (!mrow || !wave_has_keys) return 0;
    int64_t s = tile * TN + lane;
    s = s < wlo ? wlo : (s >= whi ? whi - 1 : s);
    return __builtin_nontemporal_load(mrow + s);
  };

  // Software pipeline over 32-key halves.  Step "A" of tile i issues the 16
  // MFMAs of keys 0-31 while the VALU epilogue of tile i-1's keys 32-63 runs;
  // then tile i-1's 64 scores enter the top-k; step "B" issues the MFMAs of
  // keys 32-63 while the epilogue of keys 0-31 runs.  Neither half waits for
  // its own MFMAs, so the matrix pipe stays busy during the epilogue.
  // Head reduction of one 32-key half.  The summation order (four partial
  // sums, combined as (s0 + s1) + (s2 + s3)) is the same here and inside
  // step(), so a key's score does not depend on where its tile falls.
  auto epilogue = [&](const f32x16 (&acc)[2]) -> float {
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      s0 = __builtin_fmaf(wr[0][2 * j], relu(acc[0][2 * j]), s0);
      s1 = __builtin_fmaf(wr[1][2 * j], relu(acc[1][2 * j]), s1);
      s2 = __builtin_fmaf(wr[0][2 * j + 1], relu(acc[0][2 * j + 1]), s2);
      s3 = __builtin_fmaf(wr[1][2 * j + 1], relu(acc[1][2 * j + 1]), s3);
    }
    return (s0 + s1) + (s2 + s3);
  };
  // One pipeline step: the 16 MFMAs of key half `kb` of tile `kt` into acc,
  // with the epilogue of `prev` (the half scored one step earlier) spread
  // between them, 4 VALU ops after each MFMA; B fragments are read from LDS
  // two k-steps ahead.  The order is pinned with scheduling barriers.
  auto step = [&](const uint16_t* kt, int kb, f32x16 (&acc)[2], const f32x16 (&prev)[2]) -> float {
    const int row = 32 * kb + m;
    auto frag = [&](int j) { return __builtin_bit_cast(T, *reinterpret_cast<const u32x4*>(kt + swz(row, 8 * g + j))); };
    const f32x16 zero = {};
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    T bq[3];
    bq[0] = frag(0);
    bq[1] = frag(1);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j + 2 < 8) bq[(j + 2) % 3] = frag(j + 2);
      const T b = bq[j % 3];
      // (the empty asm statements keep each group of epilogue ops next to its
      // MFMA; without them instruction selection moves the whole epilogue
      // behind the last MFMA)
      acc[0] = M::run(A[0][j], b, j == 0 ? zero : acc[0]);
      s0 = __builtin_fmaf(wr[0][2 * j], relu(prev[0][2 * j]), s0);
      s1 = __builtin_fmaf(wr[1][2 * j], relu(prev[1][2 * j]), s1);
      asm volatile("" : "+v"(s0), "+v"(s1));
      __builtin_amdgcn_sched_barrier(0);
      acc[1] = M::run(A[1][j], b, j == 0 ? zero : acc[1]);
      s2 = __builtin_fmaf(wr[0][2 * j + 1], relu(prev[0][2 * j + 1]), s2);
      s3 = __builtin_fmaf(wr[1][2 * j + 1], relu(prev[1][2 * j + 1]), s3);
      asm volatile("" : "+v"(s2), "+v"(s3));
      __builtin_amdgcn_sched_barrier(0);
    }
    return (s0 + s1) + (s2 + s3);
  };
  auto insert_tile = [&](int64_t s0, float p0, float p1, uint16_t mb, bool live) {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
    const float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const int64_t s = s0 + lane;
    const float v = (tot + f16_bits_to_f32(mb)) + 0.0f;
    const bool valid = live && s >= wlo && s < whi && v != -__builtin_inff();
    wave_topk_insert(st, make_key(v, (uint32_t)s), valid);
  };

  const int64_t ntile = c1 - c0;
  uint16_t mbits = 0;
  if (ntile > 0) {
    mbits = mload(c0);
    gload(c0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 accA[2], accB[2];
#pragma unroll
  for (int e = 0; e < 16; ++e) { accB[0][e] = 0.f; accB[1][e] = 0.f; }
  float part0 = 0.f;
  uint16_t mprev = 0;
  for (int64_t it = 0; it < ntile; ++it) {
    const int64_t tile = c0 + it;
    const uint16_t* kt = ktile + (int)(it & 1) * TN * D;
    const uint16_t mcur = mbits;
    if (it + 1 < ntile) {
      mbits = mload(tile + 1);
      gload(tile + 1, (int)((it + 1) & 1));
    }
    // step A: MFMAs of keys 0-31 of this tile || epilogue of keys 32-63 of the previous tile
    const float part1 = step(kt, 0, accA, accB);
    insert_tile((tile - 1) * TN, part0, part1, mprev, it > 0);
    // step B: MFMAs of keys 32-63 || epilogue of keys 0-31
    part0 = step(kt, 1, accB, accA);
    mprev = mcur;
    __builtin_amdgcn_s_waitcnt(0);  // this thread's part of the next tile has landed in LDS
    __syncthreads();
  }
  if (ntile > 0) insert_tile((c1 - 1) * TN, part0, epilogue(accB), mprev, true);

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
