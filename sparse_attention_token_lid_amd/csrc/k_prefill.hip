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
// see.  Key tiles of 128 keys x 128 dims (32 KiB) are staged through LDS once
// per workgroup and shared by its NW wavefronts (double buffered, one barrier
// per tile).
//
// Per wavefront and 32-key half of a tile: S = Q_t (64 heads x 128) . K^T with
// v_mfma_f32_32x32x16 (f16 or bf16 in, f32 accumulate): 2 row blocks of 32
// heads x 8 k-steps.  Heads run along the MFMA
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
constexpr int TN = kPrefillTile;              // keys per tile (4 halves of 32)
constexpr int kTileBytes = TN * D * 2;         // 32 KiB
constexpr int kHalfBytes = 32 * D * 2;         // 8 KiB

__device__ __forceinline__ int swz(int row, int ch) { return row * D + ((ch ^ (row & 15)) << 3); }

template <int NW, int DT>
__global__ __launch_bounds__(NW * 64, 8 / NW) void prefill_kernel(KArgs a) {
  using M = Mfma<DT>;
  using T = typename M::T;
  // The two key-tile buffers are separate LDS objects, so the compiler can
  // tell that the asynchronous global->LDS copy into one buffer does not alias
  // reads of the other (otherwise it waits for the copy before every LDS read).
  __shared__ __attribute__((aligned(16))) uint16_t ktile0[TN * D];
  __shared__ __attribute__((aligned(16))) uint16_t ktile1[TN * D];
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint64_t* cand = reinterpret_cast<uint64_t*>(smem);
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
  const int c0 = (int)(T0 + nt * p / P);
  const int c1 = (int)(T0 + nt * (p + 1) / P);
  // this wave's visible keys inside the chunk (32-bit: n_kv < 2^31)
  const int wlo = (int)(lo > (int64_t)c0 * TN ? lo : (int64_t)c0 * TN);
  const int whi = (int)(hi < (int64_t)c1 * TN ? hi : (int64_t)c1 * TN);

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
  // permuting which 16-byte chunk each lane fetches.  Rows past n_kv (only in
  // the last tile) are clamped to the last key; they are never scored.
  constexpr int kInstPerWave = kTileBytes / 1024 / NW;
  static_assert(kInstPerWave * NW * 1024 == kTileBytes, "tile copy must divide evenly");
  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k);
  const int n_kv = (int)a.n_kv;
  auto gload = [&](int tile, int buf) {
    const bool tail = (tile + 1) * TN > n_kv;
#pragma unroll
    for (int r = 0; r < kInstPerWave; ++r) {
      const int q = wv * kInstPerWave + r;          // 1 KiB piece of the tile
      const int row = 4 * q + (lane >> 4);
      const int ch = (lane & 15) ^ (row & 15);
      int s = tile * TN + row;
      if (tail) s = s < n_kv - 1 ? s : n_kv - 1;
      uint16_t* dst = (buf ? ktile1 : ktile0) + q * 512;
      __builtin_amdgcn_global_load_lds(kbase + (size_t)s * D + ch * 8, dst, 16, 0, 0);
    }
  };
  // this wave's mask values for 64 keys (lane l <-> key s0 + l), read one
  // tile ahead so that no wait on global memory sits in front of the MFMAs
  const bool wave_has_keys = has_q && whi > wlo;
  const uint16_t* mrow = (a.mask && wave_has_keys) ? a.mask + t * a.mask_ld : nullptr;
  auto mload = [&](int s0) -> uint16_t {
    if (!mrow) return 0;
    int s = s0 + lane;
    s = s < n_kv - 1 ? s : n_kv - 1;
    return __builtin_nontemporal_load(mrow + s);
  };

  // LDS byte offset of B fragment j for this lane inside a 32-key half
  uint32_t foff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) foff[j] = (uint32_t)(m * (D * 2) + (((8 * g + j) ^ (m & 15)) << 4));

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
  // One pipeline step: the 16 MFMAs of half `hq` of the tile in LDS buffer
  // `buf` into acc, with the epilogue of `prev` (the half scored one step
  // earlier) spread between them, 4 VALU ops after each MFMA; B fragments are
  // read from LDS two k-steps ahead.  The order is pinned with scheduling
  // barriers (the empty asm statements keep each group of epilogue ops next
  // to its MFMA; without them instruction selection moves the whole epilogue
  // behind the last MFMA).
  auto step = [&](int buf, int hq, f32x16 (&acc)[2], const f32x16 (&prev)[2]) -> float {
    const unsigned char* kt = reinterpret_cast<const unsigned char*>(buf ? ktile1 : ktile0) + hq * kHalfBytes;
    auto frag = [&](int j) { return __builtin_bit_cast(T, *reinterpret_cast<const u32x4*>(kt + foff[j])); };
    const f32x16 zero = {};
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    T bq[3];
    bq[0] = frag(0);
    bq[1] = frag(1);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j + 2 < 8) bq[(j + 2) % 3] = frag(j + 2);
      const T b = bq[j % 3];
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
  // 64 scores (two halves) into the top-k.  Most keys cannot enter once the
  // buffer has been cut (v < score of tau): one f32 compare and a ballot
  // dismiss them before any 64-bit key is formed.
  auto insert_unit = [&](int s0, float p0, float p1, uint16_t mb, bool live) {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
    const float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const int s = s0 + lane;
    const float v = (tot + f16_bits_to_f32(mb)) + 0.0f;
    const bool vis = live && s >= wlo && s < whi && v != -__builtin_inff() && v >= st.tau_v;
    if (ballot(vis) == 0ull) return;
    wave_topk_insert(st, make_key(v, (uint32_t)s), vis);
  };

  const int ntile = c1 - c0;
  uint16_t mn0 = 0, mn1 = 0;  // mask bits of the next tile (keys 0-63, 64-127)
  if (ntile > 0) {
    mn0 = mload(c0 * TN);
    mn1 = mload(c0 * TN + 64);
    gload(c0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 accA[2], accB[2];
#pragma unroll
  for (int e = 0; e < 16; ++e) { accB[0][e] = 0.f; accB[1][e] = 0.f; }
  float part0 = 0.f, part1 = 0.f, part2 = 0.f;
  uint16_t mprev1 = 0;
  // Pipeline over the four 32-key halves of each tile: step h issues the
  // MFMAs of half h and finishes the epilogue of the half before it; every
  // second step hands 64 finished scores to the top-k.
  auto tile_body = [&](int it, int buf) {
    const int tile = c0 + it;
    const uint16_t mc0 = mn0, mc1 = mn1;
    if (it + 1 < ntile) {
      mn0 = mload((tile + 1) * TN);
      mn1 = mload((tile + 1) * TN + 64);
      gload(tile + 1, buf ^ 1);
    }
    const float part3 = step(buf, 0, accA, accB);
    insert_unit((tile - 1) * TN + 64, part2, part3, mprev1, it > 0);
    part0 = step(buf, 1, accB, accA);
    part1 = step(buf, 2, accA, accB);
    insert_unit(tile * TN, part0, part1, mc0, true);
    part2 = step(buf, 3, accB, accA);
    mprev1 = mc1;
    __builtin_amdgcn_s_waitcnt(0);  // this thread's part of the next tile has landed in LDS
    __syncthreads();
  };
  for (int it = 0; it < ntile; it += 2) {
    tile_body(it, 0);
    if (it + 1 >= ntile) break;
    tile_body(it + 1, 1);
  }
  if (ntile > 0) insert_unit((c1 - 1) * TN + 64, part2, epilogue(accB), mprev1, true);

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
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 2 * kTileBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t nqb = (a.n_tok + NW - 1) / NW;
  dim3 grid((unsigned)(nqb * a.P));
  hipLaunchKernelGGL((prefill_kernel<NW, DT>), grid, dim3(NW * 64), lds, st, a);
  return hipGetLastError();
}

}  // namespace

// dynamic part only; the two key tiles (2 x 32 KiB) are static LDS
size_t prefill_lds_bytes(int nw, int cap) {
  return (size_t)nw * cap * 8 + (size_t)nw * 256 * 4 + 2 * (size_t)nw * 8;
}

hipError_t launch_prefill(const KArgs& a, int nw, hipStream_t st) {
  if (a.dtype == 1) return nw == 8 ? launch_one<8, 1>(a, st) : launch_one<4, 1>(a, st);
  return nw == 8 ? launch_one<8, 2>(a, st) : launch_one<4, 2>(a, st);
}

}  // namespace lid
