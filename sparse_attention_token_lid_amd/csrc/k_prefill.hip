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
// per tile).  With P > 1 each wavefront leaves its split's k_top best in the
// workspace, and the last workgroup of a query block to finish turns the P
// lists of each of its queries into the output row (wave_select_lists or
// wave_merge_lists; with more than 16 splits the merge kernel does it).
//
// Per wavefront and 16-key block of a tile: S = Q_t (64 heads x 128) . K^T
// with v_mfma_f32_16x16x32 (f16 or bf16 in, f32 accumulate): 4 row blocks of
// 16 heads x 4 k-steps.  Heads run along the MFMA rows, so each lane holds 16
// heads of one key, and the head reduction sum_h w_h * max(S_h, 0) is 16
// fused multiply-adds in registers per block; the four lane groups of a block
// are summed by three permlane swaps per 64 keys, which also leave key
// s0 + l of a 64-key unit in lane l.  On gfx950 this MFMA shape runs at a
// higher sustained clock than 32x32x16 under the same data (the chip is power
// limited here), which is why the kernel uses it.
//
// The k-index of the MFMA is mapped to the head dimension as
// d = 32 * (lane / 16) + 8 * kstep + i, so each lane's 4 k-steps cover 64
// contiguous bytes of a q or k row.
#include "lid_device.h"
#include "lid_kernels.h"

namespace lid {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int DT> struct Mfma;
template <> struct Mfma<1> {
  typedef f16x8 T;
  static __device__ __forceinline__ f32x4 run(T a, T b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<2> {
  typedef bf16x8 T;
  static __device__ __forceinline__ f32x4 run(T a, T b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
// OCP FP8 E4M3 in both operands, K = 128 per instruction: the whole head
// dimension in one MFMA (format codes 0, 0; no block scales).  Lane l holds
// row l % 16 and the 32 bytes k = 32 (l / 16) ... + 31.
typedef int i32x8 __attribute__((ext_vector_type(8)));
template <> struct Mfma<3> {
  typedef i32x8 T;
  static __device__ __forceinline__ f32x4 run(T a, T b, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
};
__device__ __forceinline__ i32x8 join8(u32x4 lo, u32x4 hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

constexpr int H = kMfmaHeads;
constexpr int D = kMfmaDim;
constexpr int TN = kPrefillTile;              // keys per tile (8 blocks of 16)
constexpr int kTileBytes = TN * D * 2;         // 32 KiB (one LDS tile buffer; FP8 tiles use half)
// bytes per key row: 256 (f16 / bf16) or 128 (FP8)
template <int DT> constexpr int row_bytes() { return DT == 3 ? D : 2 * D; }

// The k_top best of the P sorted split lists of one query (row t of
// a.lists: P lists of K keys, descending, 0 = empty), merged by one wavefront
// in registers and written as the output row.  N = 64 E >= K entries per
// run, lane L holding elements E L .. E L + E - 1.  Two sorted runs merge in
// one step: the N largest of runs A and B are max(A[i], B[N - 1 - i]), a
// bitonic sequence, which the last log2(N) stages of the bitonic network
// sort.  The lists were written by other workgroups, possibly on other XCDs:
// they are read with agent-scope atomic loads, which bypass the caches that
// are not coherent between XCDs.
template <int E>
__device__ __forceinline__ void wave_merge_lists(const KArgs& a, int64_t t) {
  constexpr int N = kWave * E;
  const int lane = lane_id();
  const int P = a.P, K = a.K;
  const uint64_t* lists = a.lists + (size_t)t * P * K;
  // 16-byte loads through a buffer resource (entries past K read as 0; K is
  // even, so no load straddles the end) with the cache policy of an
  // agent-scope atomic load (sc1).  Lane L reads its E entries E L ..
  // E L + E - 1, or for a reversed run the entries N - E (L + 1) ..
  // N - 1 - E L in reverse order.
  auto load = [&](int p, bool reversed, uint64_t (&x)[E]) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint64_t*>(lists + (size_t)p * K), (short)0, K * 8, 0x00020000);
    const int j0 = reversed ? E * (kWave - 1 - lane) : E * lane;
#pragma unroll
    for (int c = 0; c < E / 2; ++c) {
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (j0 + 2 * c) * 8, 0, 16));
      const uint64_t e0 = ((uint64_t)v[1] << 32) | v[0], e1 = ((uint64_t)v[3] << 32) | v[2];
      if (reversed) { x[E - 1 - 2 * c] = e0; x[E - 2 - 2 * c] = e1; }
      else { x[2 * c] = e0; x[2 * c + 1] = e1; }
    }
  };
  // all loads of a batch of up to 8 runs are in flight before its merges
  constexpr int B = E >= 16 ? 4 : 8;
  uint64_t acc[E];
  load(0, false, acc);
  for (int p0 = 1; p0 < P; p0 += B) {
    uint64_t run[B][E];
#pragma unroll
    for (int b = 0; b < B; ++b)
      if (p0 + b < P) load(p0 + b, true, run[b]);
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (p0 + b < P) {
#pragma unroll
        for (int s = 0; s < E; ++s) acc[s] = acc[s] > run[b][s] ? acc[s] : run[b][s];
        wave_bitonic_merge_reg<E, N, N / 2>(acc, lane);
      }
    }
  }
#pragma unroll
  for (int s = 0; s < E; ++s) {
    const int e = E * lane + s;
    if (e < K) {
      a.idx[t * K + e] = key_index(acc[s]);
      if (a.score) a.score[t * K + e] = key_score(acc[s]);
    }
  }
}

// The k_top best of the P unsorted split lists of one query (row t of
// a.lists: P x K keys, 0 = empty; P K <= 64 R), by one wavefront: all keys
// are read into registers at once (16-byte agent-coherent loads as above),
// the K-th largest is found by radix passes over the registers, the K best
// are compacted into the wave's LDS buffer, sorted there through registers
// and written as the output row.
template <int R, int E>
__device__ __forceinline__ void wave_select_lists(const KArgs& a, int64_t t, WaveTopK& st) {
  const int lane = lane_id();
  const int n = a.P * a.K;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint64_t*>(a.lists + (size_t)t * n), (short)0, n * 8, 0x00020000);
  uint64_t x[R];
#pragma unroll
  for (int c = 0; c < R / 2; ++c) {
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (lane + kWave * c) * 16, 0, 16));
    x[2 * c] = ((uint64_t)v[1] << 32) | v[0];
    x[2 * c + 1] = ((uint64_t)v[3] << 32) | v[2];
  }
  uint32_t c = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) c += x[r] ? 1u : 0u;
  const uint32_t present = __builtin_amdgcn_readfirstlane(wave_sum_u32(c));
  const uint64_t kap = present > (uint32_t)a.K ? wave_cut_reg<R, true>(x, (uint32_t)a.K, st.hist) : 1ull;
  const int m = wave_compact_reg<R>(x, kap, st.buf);
  wave_sort_desc_reg<E>(st.buf, m);
  wave_write_row(st.buf, a.K, a.idx + t * a.K, a.score ? a.score + t * a.K : nullptr, nullptr);
}

// The k_top best of the P split lists of one query (P K <= 64 kFuseSelectRows
// keys, 0 = empty), sorted, into the output row by one bucket pass
// (wave_bucket_topk): all keys are read into registers at once (16-byte
// agent-coherent loads, as above), the wave's candidate buffer holds the
// pass's segments and `bins` its buckets.  Returns false (nothing written)
// when a bucket overflows; the caller then selects by radix passes.
__device__ __forceinline__ bool wave_bucket_lists(const KArgs& a, int64_t t, WaveTopK& st, uint32_t* bins,
                                                  uint32_t* meta) {
  constexpr int R = kFuseSelectRows;
  const int lane = lane_id();
  const int n = a.P * a.K, K = a.K;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint64_t*>(a.lists + (size_t)t * n), (short)0, n * 8, 0x00020000);
  uint64_t x[R];
#pragma unroll
  for (int c = 0; c < R / 2; ++c) {
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (lane + kWave * c) * 16, 0, 16));
    x[2 * c] = ((uint64_t)v[1] << 32) | v[0];
    x[2 * c + 1] = ((uint64_t)v[3] << 32) | v[2];
  }
  int32_t* irow = a.idx + t * K;
  float* srow = a.score ? a.score + t * K : nullptr;
  const int m = wave_bucket_topk<R, 512>(x, K, bins, st.buf, meta, [&](int pos, uint64_t key) {
    irow[pos] = key_index(key);
    if (srow) srow[pos] = key_score(key);
  });
  if (m < 0) return false;
  for (int i = m + lane; i < K; i += kWave) {
    irow[i] = -1;
    if (srow) srow[i] = -__builtin_inff();
  }
  return true;
}

// SC: score-only mode.  Every (query, key) score of the workgroup's chunk
// is written to a.scores (f32, row stride a.scores_ld; -inf outside the
// query's range or under a -inf mask) instead of entering a top-k: the output
// of the pages' fused op, from the same tiles, MFMAs and epilogue.
template <int NW, int DT, bool MK, bool SC>
__global__ __launch_bounds__(NW * 64, 8 / NW) void prefill_kernel(KArgs a) {
  using M = Mfma<DT>;
  using T = typename M::T;
  constexpr bool F8 = DT == 3;
  static_assert(!(F8 && SC), "no FP8 score-only mode");
  constexpr int RB = row_bytes<DT>();          // bytes per key row
  constexpr int KS = F8 ? 1 : 4;               // MFMA k-steps per 16-key block
  constexpr int kTB = TN * RB;                 // bytes per key tile
  constexpr int kBlockBytes = 16 * RB;         // bytes per 16-key block
  // The two key-tile buffers are separate LDS objects, so the compiler can
  // tell that the asynchronous global->LDS copy into one buffer does not alias
  // reads of the other (otherwise it waits for the copy before every LDS read).
  __shared__ __attribute__((aligned(16))) uint16_t ktile0[TN * D];
  __shared__ __attribute__((aligned(16))) uint16_t ktile1[TN * D];
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint64_t* cand = reinterpret_cast<uint64_t*>(smem);
  uint32_t* hist = reinterpret_cast<uint32_t*>(cand + (size_t)NW * a.cap);
  uint32_t* cflag = hist + NW * 256;  // [2][NW] compaction requests
  uint32_t& s_last = cflag[2 * NW];  // this workgroup is the last of its query block to finish

  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int lane = threadIdx.x & (kWave - 1);
  const int G = lane >> 4, r16 = lane & 15;
  const int P = a.P;
  // Workgroups go to the 8 XCDs round-robin (block b to XCD b % 8).  The
  // (query block, split) pairs are numbered so that each XCD gets a
  // contiguous run of them: the P splits of a query block share one XCD and
  // its L2, which then fetches their queries from HBM once, not P times; and
  // consecutive query blocks, which see nearly the same keys (causal) or the
  // same sequence's key block (several sequences in one batch), share one, so
  // an XCD's L2 streams only the keys its own queries see.
  uint32_t g;
  {
    const uint32_t T = gridDim.x, x = blockIdx.x % 8u, i = blockIdx.x / 8u;
    const uint32_t Q = T / 8u, Rm = T % 8u;
    g = x * Q + (x < Rm ? x : Rm) + i;
  }
  const int p = (int)(g % (unsigned)P);
  const int64_t qb = g / (unsigned)P;
  const int64_t t = qb * NW + wv;
  const bool has_q = t < a.n_tok;

  // visible range of query t2 (empty past n_tok)
  auto qrange = [&](int64_t t2, int64_t& l, int64_t& h) {
    l = 0;
    h = 0;
    if (t2 >= a.n_tok) return;
    h = a.n_kv;
    if (a.kv_range) {
      const int64_t l0 = a.kv_range[2 * t2], h0 = a.kv_range[2 * t2 + 1];
      l = l0 < 0 ? 0 : l0;
      h = h0 > a.n_kv ? a.n_kv : h0;
      if (h < l) h = l;
    }
  };
  // this wave's range, and the union of the block's ranges, which every
  // wave computes itself (wave-uniform loads; no LDS exchange and no
  // barrier, so the first tile's copy is issued next to the q loads)
  int64_t lo, hi;
  qrange(t, lo, hi);
  int64_t ulo = INT64_MAX, uhi = 0;
  for (int w2 = 0; w2 < NW; ++w2) {
    int64_t l2, h2;
    qrange(qb * NW + w2, l2, h2);
    if (h2 > l2) {
      ulo = l2 < ulo ? l2 : ulo;
      uhi = h2 > uhi ? h2 : uhi;
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

  // this wave's query in MFMA A-operand layout (A[rb][j]: head 16 rb + lane % 16,
  // dims 32 (lane / 16) + 8 j ... + 7; FP8: A[rb][0] holds dims 32 (lane / 16)
  // ... + 31) and the weights of the heads its accumulators hold (wr[rb][e]:
  // head 16 rb + 4 (lane / 16) + e; FP8: times the head's q scale, which is
  // positive and so commutes with the ReLU)
  T A[4][KS];
  float wr[4][4];
  if constexpr (F8) {
    const unsigned char* qrow = reinterpret_cast<const unsigned char*>(a.q) + (has_q ? t : 0) * H * D;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      u32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
      if (has_q) {
        lo = *reinterpret_cast<const u32x4*>(qrow + (16 * rb + r16) * D + 32 * G);
        hi = *reinterpret_cast<const u32x4*>(qrow + (16 * rb + r16) * D + 32 * G + 16);
      }
      A[rb][0] = join8(lo, hi);
    }
    // the weights and q scales of row t (row 0 without a query: every load
    // is issued before any is used, then zeroed)
    const int64_t tw = has_q ? t : 0;
    float wv[4][4], qv[4][4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int h = 16 * rb + 4 * G + e;
        wv[rb][e] = a.w[tw * H + h];
        qv[rb][e] = a.q_scale[tw * H + h];
      }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int e = 0; e < 4; ++e) wr[rb][e] = has_q ? wv[rb][e] * qv[rb][e] : 0.f;
  } else {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + (has_q ? t : 0) * H * D;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        u32x4 v = {0, 0, 0, 0};
        if (has_q) v = *reinterpret_cast<const u32x4*>(qrow + (16 * rb + r16) * D + 32 * G + 8 * j);
        A[rb][j] = __builtin_bit_cast(T, v);
      }
    // the weights of row t (row 0 without a query, whose A operand is zero
    // and whose range is empty, so they never reach a score), loaded with no
    // select behind them: a select right behind each load made the compiler
    // wait for it, and for the q loads before it, one load at a time
    const int64_t tw = has_q ? t : 0;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int e = 0; e < 4; ++e) wr[rb][e] = a.w[tw * H + 16 * rb + 4 * G + e];
  }

  // |S| form of the head reduction (f16 and FP8 keys).  max(S, 0) is
  // (S + |S|) / 2, so sum_h w_h max(S_h, 0) = sum_h (w_h / 2) |S_h| + qt . k
  // with qt = (1/2) sum_h w_h q_h (FP8: w_h times the head's q scale and q_h
  // the E4M3 values; the k scale multiplies both terms).  |S_h| is a free
  // source modifier of the FMA, so the per-head work is one FMA instead of a
  // v_med3 and an FMA.  The linear term of the workgroup's NW queries is one
  // more 16-row MFMA block (f16, 16x16x32) per 16 keys for the whole
  // workgroup: row 2 i + p holds part p of qt_i 2^e_i split into f16 high and
  // low parts (22 bits of it; e_i puts its largest entry in [2^14, 2^15)),
  // built in LDS (als: 16 rows of 128 dims, 16-byte chunk c of row r at
  // chunk c ^ r) and held in registers (read again after a compaction, which
  // is the kernel's register peak and so runs without them).  Wavefront b % NW computes the term for block b of
  // every tile and hands it to the others through LDS: lin[tile parity]
  // [query][key of the tile].  bf16 keys keep the v_med3 form (their parts
  // would need three bf16 rows), and so does the f16 kernel with 4
  // wavefronts (k_top > 512), which has no registers for the term's A operand.
  constexpr bool AB = DT == 3 || (DT == 1 && NW == 8);
  float* lin = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(cflag) + 2 * NW * 4 + 16);
  unsigned char* als = reinterpret_cast<unsigned char*>(lin + 2 * NW * TN);
  int* les = reinterpret_cast<int*>(als + 16 * D * 2);  // e of each query
  f16x8 AL[4];   // the A operand in registers (row r16, dims 32 G + 8 j ... + 7)
  // this lane's row of the linear term's A operand, dims 32 G + 8 j ... + 7
  auto al_frag = [&](int j) -> f16x8 {
    return *reinterpret_cast<const f16x8*>(als + r16 * 2 * D + ((4 * G + j) ^ r16) * 16);
  };
  float lsc[2];  // 2^-e of queries 2 G and 2 G + 1, the rows lane group G holds in the lin result
  if constexpr (AB) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int e = 0; e < 4; ++e) wr[rb][e] *= 0.5f;
    // qt of this wave's query: each lane sums its heads 16 rb + r16 (the A
    // layout) over dims 32 G ... + 31, then the 16 lanes of its group add up
    // (xor butterfly: every lane of the group ends with the same sums)
    const int64_t tw = has_q ? t : 0;
    float wa[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      float wt = a.w[tw * H + 16 * rb + r16];
      if constexpr (F8) wt *= a.q_scale[tw * H + 16 * rb + r16];
      wa[rb] = has_q ? wt : 0.f;
    }
    float qt[32];
    float mx = 0.f;
#pragma unroll
    for (int c = 0; c < 32; ++c) qt[c] = 0.f;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      if constexpr (F8) {
        // E4M3 -> f32 in hardware (exact), two bytes per conversion
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const auto lo2 = __builtin_amdgcn_cvt_pk_f32_fp8(A[rb][0][e], false);
          const auto hi2 = __builtin_amdgcn_cvt_pk_f32_fp8(A[rb][0][e], true);
          qt[4 * e] = __builtin_fmaf(wa[rb], lo2[0], qt[4 * e]);
          qt[4 * e + 1] = __builtin_fmaf(wa[rb], lo2[1], qt[4 * e + 1]);
          qt[4 * e + 2] = __builtin_fmaf(wa[rb], hi2[0], qt[4 * e + 2]);
          qt[4 * e + 3] = __builtin_fmaf(wa[rb], hi2[1], qt[4 * e + 3]);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 32; ++c) qt[c] = __builtin_fmaf(wa[rb], (float)A[rb][c >> 3][c & 7], qt[c]);
      }
    }
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      float x = qt[c];
      x += __uint_as_float(xor_lane_u32<1>(__float_as_uint(x)));
      x += __uint_as_float(xor_lane_u32<2>(__float_as_uint(x)));
      x += __uint_as_float(xor_lane_u32<4>(__float_as_uint(x)));
      x += __uint_as_float(xor_lane_u32<8>(__float_as_uint(x)));
      qt[c] = 0.5f * x;
      mx = __builtin_fmaxf(mx, __builtin_fabsf(qt[c]));
    }
    mx = __builtin_fmaxf(mx, __uint_as_float(xor_lane_u32<16>(__float_as_uint(mx))));
    mx = __builtin_fmaxf(mx, __uint_as_float(xor_lane_u32<32>(__float_as_uint(mx))));
    int e = 0;
    if (mx > 0.f) {
      e = 15 - __builtin_amdgcn_frexp_expf(mx);
      e = e < -120 ? -120 : (e > 120 ? 120 : e);
    }
    // rows 2 wv (high parts, lane r16 = 0 of each group) and 2 wv + 1 (low
    // parts, r16 = 1) of als, dims 32 G ... + 31 (chunks 4 G ... + 3); with
    // NW < 8, wave 0 also clears the rows of the missing queries
    if (r16 < 2) {
      const int row = 2 * wv + r16;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f16x8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float x = __builtin_ldexpf(qt[8 * j + i], e);
          const _Float16 h = (_Float16)x;
          v[i] = r16 == 0 ? h : (_Float16)(x - (float)h);
        }
        *reinterpret_cast<f16x8*>(als + row * 2 * D + ((4 * G + j) ^ row) * 16) = v;
      }
    }
    if (NW < 8 && wv == 0 && r16 >= 2 * NW) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<u32x4*>(als + r16 * 2 * D + ((4 * G + j) ^ r16) * 16) = u32x4{0, 0, 0, 0};
    }
    if (lane == 0) les[wv] = e;
  }

  // Streaming top-k state.  Scores enter on an f32 test alone (v >= tau_v,
  // where tau_v is the score of the k_top-th best key at the last
  // compaction): every key that beats tau passes it, and the few that tie
  // tau_v without beating tau only take buffer space until the next
  // compaction.  tau_v starts at -FLT_MAX, so masked keys (-inf) never enter.
  WaveTopK st;
  wave_topk_init(st, cand + (size_t)wv * a.cap, hist + wv * 256, a.K, a.cap);
  st.tau_v = -3.402823466e38f;

  // Key tiles go straight from global memory to LDS (global_load_lds_dwordx4:
  // each lane's 16 bytes land at LDS base + 16 * lane, so one instruction
  // fills 1 KiB = 4 rows).  The XOR swizzle of the LDS layout is applied by
  // permuting which 16-byte chunk each lane fetches; the per-lane byte offsets
  // inside a tile are fixed, so a load is a scalar tile base plus one of them.
  // Rows past n_kv (only in the last tile) are clamped to the last key; they
  // are never scored.  The copy is issued through dma_row4() (inline asm):
  // when the compiler sees an LDS DMA in flight it stops counting outstanding
  // LDS reads and waits for all of them before every fragment use, so the
  // copy is kept out of its view and waited for explicitly (vmcnt(0) before
  // the barrier that ends a tile).
  // (FP8 rows are 128 bytes: one instruction copies 8 rows, and the 16-byte
  // chunk c of row r lives at chunk c ^ (r & 7).)
  constexpr int LPR = RB / 16;                 // lanes (16-byte chunks) per row
  constexpr int RPI = kWave / LPR;             // rows per 1 KiB instruction
  constexpr int kInstPerWave = kTB / 1024 / NW;
  static_assert(kInstPerWave * NW * 1024 == kTB, "tile copy must divide evenly");
  const unsigned char* kbytes = reinterpret_cast<const unsigned char*>(a.k);
  const int n_kv = (int)a.n_kv;
  uint32_t goff[kInstPerWave];
#pragma unroll
  for (int r = 0; r < kInstPerWave; ++r) {
    const int row = RPI * (wv * kInstPerWave + r) + lane / LPR;
    goff[r] = (uint32_t)(row * RB + (((lane % LPR) ^ (row % LPR)) << 4));
  }
  auto gload = [&](int tile, int buf) {
    const unsigned char* tb = kbytes + (size_t)tile * kTB;
    const uint32_t lds0 = (uint32_t)(uintptr_t)((buf ? ktile1 : ktile0) + wv * kInstPerWave * 512);
    if ((tile + 1) * TN <= n_kv) {
#pragma unroll
      for (int r = 0; r < kInstPerWave; ++r) dma_row4(tb, goff[r], lds0 + 1024 * r);
    } else {
      const int last = n_kv - 1 - tile * TN;  // last valid row of the tile
#pragma unroll
      for (int r = 0; r < kInstPerWave; ++r) {
        const int row = (int)(goff[r] / RB);
        const uint32_t off = row <= last ? goff[r] : goff[r] - (uint32_t)((row - last) * RB);
        dma_row4(tb, off, lds0 + 1024 * r);
      }
    }
  };
  // this wave's mask values for 64 keys (lane l <-> key s0 + l), read one
  // tile ahead so that no wait on global memory sits in front of the MFMAs.
  // Every wave issues the load, so that exactly kAfterCopy loads follow each
  // copy: a wave without a query or keys reads row 0, and its values are
  // never used (its range test sets every key to -inf).  The loaded value is
  // returned untouched: any use of it here would make the compiler wait for
  // the load at once.
  const bool wave_has_keys = has_q && whi > wlo;
  const uint16_t* mrow = MK ? a.mask + (wave_has_keys ? t * a.mask_ld : 0) : nullptr;
  auto mload = [&](int s0) -> uint16_t {
    if constexpr (!MK) return 0;
    int s = s0 + lane;
    s = s < n_kv - 1 ? s : n_kv - 1;
    return __builtin_nontemporal_load(mrow + s);
  };
  // FP8: this wave's k scales for 64 keys (lane l <-> key s0 + l), read one
  // tile ahead like the mask (by every wave, likewise)
  auto kload = [&](int s0) -> float {
    if constexpr (!F8) return 1.f;
    int s = s0 + lane;
    s = s < n_kv - 1 ? s : n_kv - 1;
    return a.k_scale[s];
  };

  // LDS byte offset of B fragment j (key row lane % 16 of a block, dims
  // 32 (lane / 16) + 8 j ... + 7) inside a 16-key block; FP8: the two 16-byte
  // halves of the fragment (dims 32 (lane / 16) ... + 31)
  uint32_t foff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    foff[j] = F8 ? (uint32_t)(r16 * RB + (((2 * G + (j & 1)) ^ (r16 & 7)) << 4))
                 : (uint32_t)(r16 * RB + (((4 * G + j) ^ r16) << 4));
  auto frag = [&](const unsigned char* kt, int j) -> T {
    if constexpr (F8)
      return join8(*reinterpret_cast<const u32x4*>(kt + foff[0]), *reinterpret_cast<const u32x4*>(kt + foff[1]));
    else
      return __builtin_bit_cast(T, *reinterpret_cast<const u32x4*>(kt + foff[j]));
  };
  auto frags = [&](int buf, int blk, T (&bq)[KS]) {
    const unsigned char* kt = reinterpret_cast<const unsigned char*>(buf ? ktile1 : ktile0) + blk * kBlockBytes;
#pragma unroll
    for (int j = 0; j < KS; ++j) bq[j] = frag(kt, j);
  };

  // the per-head term: |S| (weights halved, linear term added per key) or max(S, 0)
  auto hterm = [](float x) -> float {
    if constexpr (AB) return __builtin_fabsf(x);
    else return relu(x);
  };

  // Head reduction of one 16-key block, this lane's 16 heads, as one chain
  // of fused multiply-adds in element order i = 4 rb + e (16 cycles apart in
  // step(), so the chain never waits).  step() below uses the same order, so
  // a key's score does not depend on where its block falls.  The chain starts
  // from +0 and every term is added with round-to-nearest, so a zero sum is
  // +0, never -0.
  auto epilogue = [&](const f32x4 (&acc)[4]) -> float {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s = __builtin_fmaf(wr[i >> 2][i & 3], hterm(acc[i >> 2][i & 3]), s);
    return s;
  };

  // Hand-off of 64 finished keys (four 16-key blocks: this lane's partial
  // sums p[0..3], unit base s0) to the top-k, done in slices between the
  // MFMAs of the following step.  Two permlane32 swaps add lane groups {0,2}
  // and {1,3}, one permlane16 swap adds the pairs, leaving key s0 + l in
  // lane l.  Keys outside this wave's visible range are set to -inf with a
  // lane mask built on the scalar unit; the rest pass on v >= tau_v.  If any
  // lane passes, all 64 lanes store: passing keys at count + (rank among the
  // passing lanes), the others at count + n + lane, past the new count, where
  // they are dead (the buffer always has 128 free slots here: see
  // flag_need()).
  // Adding the f16 mask to a sum that is never -0 cannot give -0 either, so
  // v needs no further canonicalisation.
  struct Unit {
    float p[4];
    int s0;
    uint16_t mb;
    float ks;    // FP8: the key's scale (lane l <-> key s0 + l)
    bool live;
    int lo;      // |S| form: LDS offset (floats) of this wave's 64 linear terms in lin
  };
  struct Slice {  // values carried between the slices of one hand-off
    uint32_t x0, x1, y0, y1;
    float v, mf, ln;
  };
  // Hand-off modes: kFull (all slices); kEarly, the lane combine alone
  // (slices 0-5 leave the unit's head-reduced sums in z.v and its mask
  // values in z.mf); kLate, the rest (slices 0, 5, 6, 7: linear term, k
  // scale, mask, range, insert).  The |S| form splits the unit of keys 0-63
  // so: combined before the tile barrier, finished after it, which keeps
  // two values per lane across the barrier instead of four partial sums.
  constexpr int kFull = 0, kEarly = 1, kLate = 2;
  auto insert_slice = [&](const Unit& u, int i, int mode, Slice& z) {
    const bool comb = mode != kLate, fin = mode != kEarly;
    if (i == 0) {
      if (AB && fin) z.ln = lin[u.lo + lane];  // used in slice 5
      if (comb) {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(u.p[0]), __float_as_uint(u.p[2]), false, false);
        z.x0 = r[0]; z.x1 = r[1];
        asm volatile("" : "+v"(z.x0), "+v"(z.x1));
      }
    } else if (i == 1) {
      if (comb) {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(u.p[1]), __float_as_uint(u.p[3]), false, false);
        z.y0 = r[0]; z.y1 = r[1];
        asm volatile("" : "+v"(z.y0), "+v"(z.y1));
      }
    } else if (i == 2) {
      if (comb) {
        z.x0 = __float_as_uint(__uint_as_float(z.x0) + __uint_as_float(z.x1));
        asm volatile("" : "+v"(z.x0));
      }
    } else if (i == 3) {
      if (comb) {
        z.y0 = __float_as_uint(__uint_as_float(z.y0) + __uint_as_float(z.y1));
        asm volatile("" : "+v"(z.y0));
      }
    } else if (i == 4) {
      if (comb) {
        auto r = __builtin_amdgcn_permlane16_swap(z.x0, z.y0, false, false);
        z.x0 = r[0]; z.x1 = r[1];
        asm volatile("" : "+v"(z.x0), "+v"(z.x1));
        if (MK) {
          z.mf = f16_bits_to_f32(u.mb);
          asm volatile("" : "+v"(z.mf));
        }
      }
    } else if (i == 5) {
      if (comb) z.v = __uint_as_float(z.x0) + __uint_as_float(z.x1);
      if (fin) {
        if (AB) z.v = z.v + z.ln;
        if (F8) z.v = z.v * u.ks;
      }
      asm volatile("" : "+v"(z.v));
    } else if (i == 6 && fin) {
      if (MK) z.v = z.v + z.mf;
      // lanes whose key lies outside [wlo, whi) (or all, for a dead unit)
      const int l0 = wlo - u.s0, l1 = whi - u.s0;
      const uint64_t below_hi = l1 >= kWave ? ~0ull : (l1 <= 0 ? 0ull : (1ull << l1) - 1);
      const uint64_t below_lo = l0 >= kWave ? ~0ull : (l0 <= 0 ? 0ull : (1ull << l0) - 1);
      const uint64_t inr = u.live ? (below_hi & ~below_lo) : 0ull;
      z.v = lane_select(inr, z.v, -__builtin_inff());
      asm volatile("" : "+v"(z.v));
    } else if (i == 7 && fin && SC) {
      // 64 consecutive keys per store: 256 contiguous bytes of the row
      const int s = u.s0 + lane;
      if (u.live && has_q && s < n_kv) __builtin_nontemporal_store(z.v, a.scores + t * a.scores_ld + s);
    } else if (i == 7 && fin) {
      const bool pass = z.v >= st.tau_v;
      const uint64_t m = ballot(pass);
      if (m != 0ull) {
        const uint32_t n = (uint32_t)__popcll(m);
        const uint32_t c = (uint32_t)st.count;
        const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, c));
        const uint32_t pos = __float_as_uint(lane_select(m, __uint_as_float(rank), __uint_as_float(c + n + (uint32_t)lane)));
        const uint32_t b = __float_as_uint(z.v);
        const uint32_t khi = b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);  // ord_f32
        const uint32_t klo = ~(uint32_t)(u.s0 + lane);
        st.buf[pos] = ((uint64_t)khi << 32) | klo;
        st.count = (int)(c + n);
      }
    }
  };
  // Make room for one more unit: compaction to the k_top best when fewer than
  // 128 free slots remain (rare once the stream is long).
  auto room = [&]() __attribute__((always_inline)) {
    if (SC) return;
    st.count = __builtin_amdgcn_readfirstlane(st.count);  // keep it scalar (see uniform_u64)
    if (prefill_room(st.count, st.cap)) wave_topk_trim(st);
  };
  // Compactions are synchronised across the workgroup: a wave that could not
  // take a whole further tile (two units) raises its flag before the tile
  // barrier, and after the barrier every wave with more than k_top candidates
  // compacts.  The waves meet at every tile barrier anyway, so one wave
  // compacting alone would hold all of them; together they pay for it once.
  // The flags are double buffered by tile parity: a wave can only rewrite a
  // slot after the next barrier, which every reader of it has passed.
  auto flag_need = [&](int it) {
    if (SC) return;
    if (lane == 0) cflag[(it & 1) * NW + wv] = prefill_flag(st.count, st.cap) ? 1u : 0u;
  };
  // `after` runs behind a compaction: it reads the next tile's first
  // fragments and the linear term's A operand again, so that they need no
  // registers while the compaction runs (it is the kernel's register peak).
  auto sync_compact = [&](int it, auto&& after) {
    if (SC) return;
    uint32_t any = 0;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) any |= cflag[(it & 1) * NW + w2];
    if (__builtin_amdgcn_readfirstlane(any)) {
      st.count = __builtin_amdgcn_readfirstlane(st.count);
      wave_topk_trim(st);
      after();
    }
  };

  // The linear term of one 16-key block for the workgroup's queries (|S|
  // form), computed by every wave at the same steps of a tile for its own
  // block(s) wv + NW k, so that no step branches on the wave index (a branch
  // there makes the compiler drain every LDS read at its join).  The block's
  // fragments are read from the tile in LDS (lin_load, early in a step) and
  // fed to four MFMAs at the step's end (lin_mma): B as f16 (FP8: converted
  // exactly, the k dimension mapped as in the FP8 MFMA, lane group G holding
  // dims 32 G ... + 31, which the A rows follow).  Lanes of group G then
  // store queries 2 G and 2 G + 1 (high + low part, times 2^-e) for key
  // 16 blk + r16, one step later.
  struct LinIn {
    T b[KS];
  };
  auto lin_load = [&](int buf, int blk, LinIn& li) {
    const unsigned char* kt = reinterpret_cast<const unsigned char*>(buf ? ktile1 : ktile0) + blk * kBlockBytes;
#pragma unroll
    for (int j = 0; j < KS; ++j) li.b[j] = frag(kt, j);
  };
  auto lin_mma = [&](const LinIn& li) -> f32x4 {
    f16x8 bl[4];
    if constexpr (F8) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const uint32_t wd = (uint32_t)li.b[0][2 * j + m];  // bytes 8 j + 4 m ... + 3
          const auto lo2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wd, 1.f, false);
          const auto hi2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wd, 1.f, true);
          bl[j][4 * m] = lo2[0];
          bl[j][4 * m + 1] = lo2[1];
          bl[j][4 * m + 2] = hi2[0];
          bl[j][4 * m + 3] = hi2[1];
        }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) bl[j] = __builtin_bit_cast(f16x8, li.b[j]);
    }
    f32x4 c = {};
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x32_f16(AL[j], bl[j], c, 0, 0, 0);
    return c;
  };
  f32x4 lacc[2];  // linear terms of this wave's blocks, between their MFMAs and their store
  auto lin_store = [&](const f32x4& c, int par, int blk) {
    if (2 * G < NW) {
      float* dst = lin + (par * NW + 2 * G) * TN + 16 * blk + r16;
      dst[0] = (c[0] + c[1]) * lsc[0];
      dst[TN] = (c[2] + c[3]) * lsc[1];
    }
  };

  // One pipeline step: the 16 MFMAs of the block whose B fragments are in bq
  // into acc, with the head reduction of `prev` (the block scored one step
  // earlier) spread between them, two VALU ops after each MFMA, the B
  // fragments of the next block read from LDS into nxt (if load_next; all four
  // behind the first MFMAs, so they have landed when the next step starts), and
  // the slices of a pending top-k hand-off (if u is given).  The order is
  // pinned with scheduling barriers (the empty asm statements keep each group
  // of ops next to its MFMA; without them instruction selection moves the
  // whole epilogue behind the last MFMA).
  auto step = [&](const T (&bq)[KS], T (&nxt)[KS], bool load_next, int nbuf, int nblk, f32x4 (&acc)[4],
                  const f32x4 (&prev)[4], const Unit* u, int umode, Slice& z, int lk, int ls, auto&& mid) -> float {
    const unsigned char* kn = reinterpret_cast<const unsigned char*>(nbuf ? ktile1 : ktile0) + nblk * kBlockBytes;
    const f32x4 zero = {};
    float sum = 0.f;
    // linear term (|S| form): lk >= 0 reads block wv + NW lk of this tile
    // here and issues its MFMAs at the end of the step (into lacc[lk]); ls >=
    // 0 stores lacc[ls] at the end of the step
    LinIn li;
    if (AB && lk >= 0) lin_load(nbuf, wv + NW * lk, li);
    if constexpr (F8) {
      // four MFMAs (one per row block of 16 heads, the whole head dimension
      // each), four terms of the head reduction and two hand-off slices after
      // each; the next block's fragment is read behind the first
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        acc[rb] = M::run(A[rb][0], bq[0], zero);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * rb + e;
          sum = __builtin_fmaf(wr[i >> 2][i & 3], hterm(prev[i >> 2][i & 3]), sum);
          asm volatile("" : "+v"(sum));
        }
        if (load_next && rb == 0) nxt[0] = frag(kn, 0);
        if (u) {
          insert_slice(*u, 2 * rb, umode, z);
          insert_slice(*u, 2 * rb + 1, umode, z);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (rb == 0) mid();
        if (rb == 3 && AB && ls >= 0) lin_store(lacc[ls], nbuf, wv + NW * ls);
        if (rb == 3 && AB && lk >= 0) lacc[lk] = lin_mma(li);
      }
    } else {
#pragma unroll
      for (int j = 0; j < KS; ++j) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const int i = 4 * j + rb;
          acc[rb] = M::run(A[rb][j], bq[j], j == 0 ? zero : acc[rb]);
          sum = __builtin_fmaf(wr[i >> 2][i & 3], hterm(prev[i >> 2][i & 3]), sum);
          asm volatile("" : "+v"(sum));
          if (load_next && j == 0) nxt[rb] = frag(kn, rb);
          if (u) insert_slice(*u, i, umode, z);
          __builtin_amdgcn_sched_barrier(0);
          if (i == 3) mid();
          if (i == 15 && AB && ls >= 0) lin_store(lacc[ls], nbuf, wv + NW * ls);
          if (i == 15 && AB && lk >= 0) lacc[lk] = lin_mma(li);
        }
      }
    }
    return sum;
  };

  const int ntile = c1 - c0;
  // vector memory loads issued after a tile's copy (mask entries, k scales)
  // and the s_waitcnt that waits for everything but them (vmcnt = that count;
  // expcnt and lgkmcnt at their maxima: no wait)
  constexpr int kAfterCopy = (MK ? 2 : 0) + (F8 ? 2 : 0);
  constexpr int kWaitCopy = (kAfterCopy & 0xF) | ((kAfterCopy >> 4) << 14) | (7 << 4) | (15 << 8);
  // mask bits (keys 0-63, 64-127) and FP8 k scales of a tile, one register
  // set per tile parity: a tile's set is loaded at the previous tile's start
  // and read where its hand-offs need it (step 6, and after step 7), so the
  // loads have almost two tiles to arrive; the next tile's loads go to the
  // other set, whose values were copied into the hand-offs by then
  uint16_t mset[2][2] = {{0, 0}, {0, 0}};
  float kset[2][2] = {{1.f, 1.f}, {1.f, 1.f}};
  if (ntile > 0) {
    mset[0][0] = mload(c0 * TN);
    mset[0][1] = mload(c0 * TN + 64);
    kset[0][0] = kload(c0 * TN);
    kset[0][1] = kload(c0 * TN + 64);
    gload(c0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if constexpr (AB) {
#pragma unroll
    for (int j = 0; j < 4; ++j) AL[j] = al_frag(j);
    lsc[0] = 2 * G < NW ? __builtin_ldexpf(1.f, -les[2 * G]) : 0.f;
    lsc[1] = 2 * G + 1 < NW ? __builtin_ldexpf(1.f, -les[2 * G + 1]) : 0.f;
  }
  f32x4 accA[4], accB[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int e = 0; e < 4; ++e) { accA[rb][e] = 0.f; accB[rb][e] = 0.f; }
  T bq0[KS], bq1[KS];
  if (ntile > 0) frags(0, 0, bq0);
  const auto no_mid = [] {};
  Unit u0, u1;  // keys 0-63 and 64-127 of a tile
  Slice z0, zt;  // the hand-off of u0 (kept from its early to its late part), any other
  z0.v = 0.f;
  z0.mf = 0.f;
  u1.p[0] = u1.p[1] = u1.p[2] = 0.f;
  u1.mb = 0;
  u1.ks = 1.f;
  u1.lo = 0;
  u0.p[0] = u0.p[1] = u0.p[2] = u0.p[3] = 0.f;
  u0.s0 = 0;
  u0.mb = 0;
  u0.ks = 1.f;
  u0.live = false;
  u0.lo = 0;
  // Pipeline over the eight 16-key blocks of each tile: step b issues the
  // MFMAs of block b and finishes the head reduction of block b - 1.  The 64
  // scores of blocks 0-3 are handed to the top-k during the step of block 5,
  // those of blocks 4-7 during the step of block 1 of the next tile.  In the
  // |S| form both wait for the tile barrier, which makes every wave's linear
  // terms of the tile visible: blocks 0-3 go during the step of block 1 of
  // the next tile (their unit's fields are rewritten only after it), blocks
  // 4-7 during the step of block 2.
  // The tile barrier sits inside the step of block 7, after its first four
  // MFMAs (block 7's fragments are in registers by then, so every wave is
  // done reading this tile's buffer): right after it each wave reads block
  // 0 of the next tile, and those reads complete behind block 7's remaining
  // twelve MFMAs instead of stalling every wave at the start of the tile.
  // bq0 holds block 0's fragments when a tile starts.
  auto tile_body = [&](int it, int buf) {
    const int tile = c0 + it;
    const bool more = it + 1 < ntile;
    if (more) {
      // the copy first: the tile barrier then waits for it alone, while the
      // mask entries and k scales of the next tile (from HBM, used only a
      // tile later) may still be in flight (kAfterCopy loads)
      gload(tile + 1, buf ^ 1);
      mset[buf ^ 1][0] = mload((tile + 1) * TN);
      mset[buf ^ 1][1] = mload((tile + 1) * TN + 64);
      kset[buf ^ 1][0] = kload((tile + 1) * TN);
      kset[buf ^ 1][1] = kload((tile + 1) * TN + 64);
    }
    u1.p[3] = step(bq0, bq1, true, buf, 1, accA, accB, nullptr, kFull, zt, -1, -1, no_mid);
    u1.s0 = (tile - 1) * TN + 64;
    u1.live = it > 0;
    u0.p[0] = step(bq1, bq0, true, buf, 2, accB, accA, AB ? &u0 : &u1, AB ? kLate : kFull, AB ? z0 : zt, -1, -1, no_mid);
    u0.p[1] = step(bq0, bq1, true, buf, 3, accA, accB, AB ? &u1 : nullptr, kFull, zt, -1, -1, no_mid);
    u0.p[2] = step(bq1, bq0, true, buf, 4, accB, accA, nullptr, kFull, zt, 0, -1, no_mid);
    u0.p[3] = step(bq0, bq1, true, buf, 5, accA, accB, nullptr, kFull, zt, NW < 8 ? 1 : -1, 0, no_mid);
    u0.s0 = tile * TN;
    u0.mb = mset[buf][0];
    u0.ks = kset[buf][0];
    u0.live = true;
    u0.lo = (buf * NW + wv) * TN;
    u1.p[0] = step(bq1, bq0, true, buf, 6, accB, accA, &u0, AB ? kEarly : kFull, z0, -1, -1, no_mid);
    u1.p[1] = step(bq0, bq1, true, buf, 7, accA, accB, nullptr, kFull, zt, -1, NW < 8 ? 1 : -1, no_mid);
    u1.p[2] = step(bq1, bq0, false, buf, 0, accB, accA, nullptr, kFull, zt, -1, -1, [&] {
      flag_need(it);
      // this wave's part of the next tile has landed in LDS: every vector
      // memory operation but the kAfterCopy issued after the copy is done
      // (they complete in order; the compiler's own waits before the mask
      // and scale values are used do not count the copy, so they can only
      // wait longer, never too little)
      __builtin_amdgcn_s_waitcnt(kWaitCopy);
      __syncthreads();
      if (more) frags(buf ^ 1, 0, bq0);
    });
    u1.mb = mset[buf][1];
    u1.ks = kset[buf][1];
    u1.lo = (buf * NW + wv) * TN + 64;
    sync_compact(it, [&] {
      if (more) frags(buf ^ 1, 0, bq0);
      if constexpr (AB) {
#pragma unroll
        for (int j = 0; j < 4; ++j) AL[j] = al_frag(j);
      }
    });
  };
  for (int it = 0; it < ntile; it += 2) {
    tile_body(it, 0);
    if (it + 1 >= ntile) break;
    tile_body(it + 1, 1);
  }
  if (ntile > 0) {
    u1.p[3] = epilogue(accB);
    u1.s0 = (c1 - 1) * TN + 64;
    u1.live = true;
    if (AB) {
      room();
#pragma unroll
      for (int i = 0; i < 8; ++i) insert_slice(u0, i, kLate, z0);
    }
    room();
#pragma unroll
    for (int i = 0; i < 8; ++i) insert_slice(u1, i, kFull, zt);
  }

  if (SC) return;  // score-only mode: nothing to finish

  // The key tiles are free now (every wave has passed the last tile
  // barrier): each wave takes 8 KiB of them for its bucket pass, 2 x 512
  // bins and the segment bounds of up to 1024 keys.
  constexpr int kBins = 512;
  constexpr int kWaveLds = 8192;
  static_assert(NW * kWaveLds <= 2 * kTileBytes, "bucket bins fit the key tiles");
  unsigned char* wlds = reinterpret_cast<unsigned char*>(wv * kWaveLds < kTileBytes ? ktile0 : ktile1) +
                        (wv * kWaveLds) % kTileBytes;
  uint32_t* bins = reinterpret_cast<uint32_t*>(wlds);
  uint32_t* meta = bins + 2 * kBins;
  static_assert(2 * kBins * 4 + (512 + kWaveBucketMax) * 4 <= kWaveLds, "segment bounds fit");
  const int K = a.K;
  int32_t* irow = a.idx + t * K;
  float* srow = a.score ? a.score + t * K : nullptr;
  uint64_t* lrow = a.lists + ((size_t)t * P + p) * K;
  // Where a sorted result is needed (the query's row with one split; sorted
  // split lists for the merges), the K best come from one bucket pass over
  // the buffer read into registers (it then serves as the pass's segments),
  // instead of a radix cut and a sort network: into the output row, or as
  // this split's list (agent-scope stores when the last workgroup of the
  // query block reads it in this kernel).  A bucket that overflows sends the
  // wave to the radix cut and sort below.  Unsorted split lists (a.fuse ==
  // 2) keep the radix cut alone, which is cheaper than the pass there.
  bool finished = false;
  if (has_q && a.fuse != 2 && st.cap <= kWave * kReduceRegRows && K <= 512) {
    uint64_t x[kReduceRegRows];
#pragma unroll
    for (int r = 0; r < kReduceRegRows; ++r) x[r] = lane + kWave * r < st.count ? st.buf[lane + kWave * r] : 0ull;
    const int m = wave_bucket_topk<kReduceRegRows, kBins>(x, K, bins, st.buf, meta, [&](int pos, uint64_t key) {
      if (P == 1) {
        irow[pos] = key_index(key);
        if (srow) srow[pos] = key_score(key);
      } else if (a.fuse) {
        __hip_atomic_store(lrow + pos, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        lrow[pos] = key;
      }
    });
    if (m >= 0) {
      for (int i = m + lane; i < K; i += kWave) {
        if (P == 1) {
          irow[i] = -1;
          if (srow) srow[i] = -__builtin_inff();
        } else if (a.fuse) {
          __hip_atomic_store(lrow + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          lrow[i] = 0ull;
        }
      }
      finished = true;
    }
  }

  if (finished) {
  } else if (has_q && a.fuse == 2) {
    // unsorted split list: the K best (all present keys if fewer), 0-padded
    wave_topk_reduce(st);
    uint64_t* out = a.lists + ((size_t)t * P + p) * a.K;
    for (int i = lane; i < a.K; i += kWave)
      __hip_atomic_store(out + i, i < st.count ? st.buf[i] : 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (has_q) {
    wave_topk_finish(st);
    if (P == 1) {
      wave_write_row(st.buf, a.K, a.idx + t * a.K, a.score ? a.score + t * a.K : nullptr, nullptr);
    } else if (!a.fuse) {
      wave_write_row(st.buf, a.K, nullptr, nullptr, a.lists + ((size_t)t * P + p) * a.K);
    } else {
      uint64_t* out = a.lists + ((size_t)t * P + p) * a.K;
      for (int i = lane; i < a.K; i += kWave)
        __hip_atomic_store(out + i, st.buf[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (P > 1 && a.fuse) {
    // Publish this split's lists, then let the last workgroup of the query
    // block merge them: every store has completed (vmcnt(0)) before the
    // workgroup's barrier and the counter increment (agent scope, wrapping at
    // P, so it is back at zero after the launch).
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
      s_last = __builtin_amdgcn_atomic_inc32(a.counters + qb, (unsigned)(P - 1), __ATOMIC_RELAXED, "agent") ==
                       (unsigned)(P - 1) ? 1u : 0u;
    __syncthreads();
    if (s_last && has_q) {
      const int n2 = next_pow2(a.K);
      if (a.fuse == 2 && a.K <= 512 && wave_bucket_lists(a, t, st, bins, meta)) {
        // done by the bucket pass
      } else if (a.fuse == 2) {
        if (n2 == 256) wave_select_lists<kFuseSelectRows, 4>(a, t, st);
        else if (n2 == 512) wave_select_lists<kFuseSelectRows, 8>(a, t, st);
        else wave_select_lists<kFuseSelectRows, 16>(a, t, st);
      } else {
        if (n2 == 256) wave_merge_lists<4>(a, t);
        else if (n2 == 512) wave_merge_lists<8>(a, t);
        else wave_merge_lists<16>(a, t);
      }
    }
  }
}

template <int NW, int DT, bool MK, bool SC = false>
hipError_t launch_one(const KArgs& a, hipStream_t st) {
  const size_t lds = prefill_lds_bytes(NW, a.cap);
  hipError_t e = set_lds_limit(reinterpret_cast<const void*>(&prefill_kernel<NW, DT, MK, SC>),
                               160 * 1024 - 2 * kTileBytes);
  if (e != hipSuccess) return e;
  const int64_t nqb = (a.n_tok + NW - 1) / NW;
  dim3 grid((unsigned)(nqb * a.P));
  hipLaunchKernelGGL((prefill_kernel<NW, DT, MK, SC>), grid, dim3(NW * 64), lds, st, a);
  return hipGetLastError();
}

}  // namespace

// dynamic part only; the two key tiles (2 x 32 KiB) are static LDS
size_t prefill_lds_bytes(int nw, int cap) {
  return (size_t)nw * cap * 8 + (size_t)nw * 256 * 4 + 2 * (size_t)nw * 4 + 16 + 2 * (size_t)nw * TN * 4 +
         16 * D * 2 + 4 * (size_t)nw;
}

hipError_t launch_prefill(const KArgs& a, int nw, hipStream_t st) {
  const bool mk = a.mask != nullptr;
  if (a.dtype == 3) {
    if (nw == 8) return mk ? launch_one<8, 3, true>(a, st) : launch_one<8, 3, false>(a, st);
    return mk ? launch_one<4, 3, true>(a, st) : launch_one<4, 3, false>(a, st);
  }
  if (a.dtype == 1) {
    if (nw == 8) return mk ? launch_one<8, 1, true>(a, st) : launch_one<8, 1, false>(a, st);
    return mk ? launch_one<4, 1, true>(a, st) : launch_one<4, 1, false>(a, st);
  }
  if (nw == 8) return mk ? launch_one<8, 2, true>(a, st) : launch_one<8, 2, false>(a, st);
  return mk ? launch_one<4, 2, true>(a, st) : launch_one<4, 2, false>(a, st);
}

hipError_t launch_prefill_scores(const KArgs& a, hipStream_t st) {
  const bool mk = a.mask != nullptr;
  if (a.dtype == 1) return mk ? launch_one<8, 1, true, true>(a, st) : launch_one<8, 1, false, true>(a, st);
  return mk ? launch_one<8, 2, true, true>(a, st) : launch_one<8, 2, false, true>(a, st);
}

}  // namespace lid
