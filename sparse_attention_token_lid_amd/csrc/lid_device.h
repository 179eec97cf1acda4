// lid_device.h -- device-side building blocks shared by the lightning-indexer
// kernels: the selection key, wavefront helpers, the per-wavefront streaming
// top-k, and block-wide select / compact / sort.
//
// Selection key.  The top-k keeps, per query, the k_top largest masked scores
// v, ties broken by the smaller key index (ggml-org llama.cpp issue 25468,
// "Root cause" comment: lid_score -> + mask -> lid_top_k, a per-token top-512).
// Both parts are packed into one unsigned 64-bit key so that a single integer
// comparison decides the order:
//     key = (ord(v) << 32) | (~s)          larger key = better
// where ord() maps f32 to an unsigned integer in the same order (negative
// values bit-inverted, positive values with the sign bit set) and ~s ranks a
// smaller index higher.  s < 2^31, so every real key has bit 31 set and the
// value 0 is free to mean "empty".
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lid_budget.h"

namespace lid {

constexpr int kWave = 64;

__device__ __forceinline__ uint32_t ord_f32(float v) {
  uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float unord_f32(uint32_t o) {
  uint32_t b = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(b);
}
__device__ __forceinline__ uint64_t make_key(float v, uint32_t s) {
  return ((uint64_t)ord_f32(v) << 32) | (uint64_t)(~s);
}
__device__ __forceinline__ int32_t key_index(uint64_t key) {
  return key ? (int32_t)(~(uint32_t)key) : -1;
}
__device__ __forceinline__ float key_score(uint64_t key) {
  return key ? unord_f32((uint32_t)(key >> 32)) : -__builtin_inff();
}

// max(x, 0) for finite x as one v_med3_f32 (clamp to [0, FLT_MAX]); fmaxf
// (or a med3 against +inf, which the compiler folds back into fmaxf) would add
// a NaN-quieting canonicalisation of every MFMA result first.
__device__ __forceinline__ float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.0f, 3.402823466e38f); }

// OCP FP8 E4M3 (E4M3FN) byte -> f32 (exact), from the format definition:
// sign, 4 exponent bits (bias 7), 3 fraction bits; exponent 0 is subnormal
// (m * 2^-9); S.1111.111 is NaN; no infinities.
__device__ __forceinline__ float e4m3_to_f32(uint8_t x) {
  const uint32_t sg = (uint32_t)(x & 0x80) << 24, e = (x >> 3) & 15, m = x & 7;
  float v;
  if (e == 0) v = (float)m * 0.001953125f;                                 // m * 2^-9
  else if (e == 15 && m == 7) v = __uint_as_float(0x7FC00000u);
  else v = __uint_as_float(((e + 120u) << 23) | (m << 20));               // (1 + m/8) 2^(e-7)
  return __uint_as_float(__float_as_uint(v) | sg);
}

// f16 mask bits -> f32 (exact)
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  _Float16 x = __builtin_bit_cast(_Float16, h);
  return (float)x;
}

// ---------------------------------------------------------------- wave helpers
// One global_load_lds_dwordx4: lane l copies 16 bytes from gbase + voff into
// LDS byte address lds_addr + 16 l (lds_addr wave-uniform).  M0, which
// carries the LDS address, is saved and restored around it.  The caller waits
// for completion with s_waitcnt vmcnt(0).
__device__ __forceinline__ void dma_row4(const void* gbase, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(gbase), "s"(lds_addr)
      : "memory");
}

// out[lane] = bit lane of m ? a : b (one v_cndmask_b32 on a scalar lane mask)
__device__ __forceinline__ float lane_select(uint64_t m, float a, float b) {
  float r;
  asm("v_cndmask_b32 %0, %1, %2, %3" : "=v"(r) : "v"(b), "v"(a), "s"(m));
  return r;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// number of set bits of `m` below this lane
__device__ __forceinline__ int mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Partner value of this lane's x in the xor-J butterfly (J < 64), with
// VALU-only exchanges: DPP quad_perm (xor 1, 2), row_shl/row_shr (xor 4),
// row_ror:8 (xor 8), v_permlane16_swap (xor 16), v_permlane32_swap (xor 32).
template <int J>
__device__ __forceinline__ uint32_t xor_lane_u32(uint32_t x) {
  const int L = lane_id();
  if constexpr (J == 1) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
  } else if constexpr (J == 2) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
  } else if constexpr (J == 4) {
    const uint32_t up = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x104, 0xF, 0xF, true);  // row_shl:4
    const uint32_t dn = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x114, 0xF, 0xF, true);  // row_shr:4
    return (L & 4) ? dn : up;
  } else if constexpr (J == 8) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, true);  // row_ror:8
  } else if constexpr (J == 16) {
    auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (L & 16) ? r[0] : r[1];
  } else {
    static_assert(J == 32, "xor distance");
    auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (L & 32) ? r[0] : r[1];
  }
}

template <int J>
__device__ __forceinline__ uint64_t xor_lane_u64(uint64_t x) {
  return ((uint64_t)xor_lane_u32<J>((uint32_t)(x >> 32)) << 32) | xor_lane_u32<J>((uint32_t)x);
}

// Butterfly reductions over the 64 lanes (every lane gets the result).
template <typename Op>
__device__ __forceinline__ uint64_t wave_reduce_u64(uint64_t x, Op op) {
  x = op(x, xor_lane_u64<1>(x));
  x = op(x, xor_lane_u64<2>(x));
  x = op(x, xor_lane_u64<4>(x));
  x = op(x, xor_lane_u64<8>(x));
  x = op(x, xor_lane_u64<16>(x));
  x = op(x, xor_lane_u64<32>(x));
  return x;
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t x) {
  return wave_reduce_u64(x, [](uint64_t a, uint64_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ uint64_t wave_and_u64(uint64_t x) {
  return wave_reduce_u64(x, [](uint64_t a, uint64_t b) { return a & b; });
}
__device__ __forceinline__ uint64_t wave_or_u64(uint64_t x) {
  return wave_reduce_u64(x, [](uint64_t a, uint64_t b) { return a | b; });
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  x += xor_lane_u32<1>(x);
  x += xor_lane_u32<2>(x);
  x += xor_lane_u32<4>(x);
  x += xor_lane_u32<8>(x);
  x += xor_lane_u32<16>(x);
  x += xor_lane_u32<32>(x);
  return x;
}
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t x, Op op) {
  x = op(x, xor_lane_u32<1>(x));
  x = op(x, xor_lane_u32<2>(x));
  x = op(x, xor_lane_u32<4>(x));
  x = op(x, xor_lane_u32<8>(x));
  x = op(x, xor_lane_u32<16>(x));
  x = op(x, xor_lane_u32<32>(x));
  return x;
}
__device__ __forceinline__ uint32_t wave_and_u32(uint32_t x) {
  return wave_reduce_u32(x, [](uint32_t a, uint32_t b) { return a & b; });
}
__device__ __forceinline__ uint32_t wave_or_u32(uint32_t x) {
  return wave_reduce_u32(x, [](uint32_t a, uint32_t b) { return a | b; });
}
// Inclusive prefix sum over the 64 lanes with DPP row shifts and row
// broadcasts (no LDS traffic): within each row of 16 lanes, then rows 0-1
// into row 1 / rows 2-3 into row 3 (row_bcast:15), then rows 0-1 into 2-3.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// ------------------------------------------------ radix digit search (shared)
// Given a 256-bin histogram of the current digit (in LDS) and the rank `need`
// (1-based, counted from the largest), find digit d with
//   above(d) = sum_{d' > d} hist[d'] < need <= above(d) + hist[d].
// Executed by one full wavefront; results are wave-uniform.
struct DigitPick { uint32_t d, above, cnt; };

__device__ __forceinline__ DigitPick pick_digit(const uint32_t* hist, uint32_t need) {
  const int lane = lane_id();
  // lane L holds bins 255-4L, 254-4L, 253-4L, 252-4L (descending digits)
  uint32_t c0 = hist[255 - 4 * lane], c1 = hist[254 - 4 * lane];
  uint32_t c2 = hist[253 - 4 * lane], c3 = hist[252 - 4 * lane];
  uint32_t s = c0 + c1 + c2 + c3;
  uint32_t incl = wave_incl_scan_u32(s);
  uint32_t excl = incl - s;
  uint64_t m = ballot(excl < need && need <= incl);
  int fl = __ffsll((unsigned long long)m) - 1;  // need <= total, so m != 0
  DigitPick r;
  uint32_t d = 0, above = 0, cnt = 0;
  if (lane == fl) {
    uint32_t a = excl;
    if (a + c0 >= need)            { d = 255 - 4 * lane; above = a; cnt = c0; }
    else if (a + c0 + c1 >= need)  { d = 254 - 4 * lane; above = a + c0; cnt = c1; }
    else if (a + c0 + c1 + c2 >= need) { d = 253 - 4 * lane; above = a + c0 + c1; cnt = c2; }
    else                           { d = 252 - 4 * lane; above = a + c0 + c1 + c2; cnt = c3; }
  }
  r.d = (uint32_t)__builtin_amdgcn_readlane((int)d, fl);
  r.above = (uint32_t)__builtin_amdgcn_readlane((int)above, fl);
  r.cnt = (uint32_t)__builtin_amdgcn_readlane((int)cnt, fl);
  return r;
}

// ------------------------------------------------- per-wavefront streaming top-k
// One wavefront owns one query's candidate buffer `buf` (LDS, capacity `cap`
// >= K + 128).  Candidates with key > tau are appended; when the buffer would
// overflow it is cut back to its K best (radix select of the K-th largest key,
// which becomes the new tau).  Every key is unique, so "the K best" is exact.

// K-th largest key (1 <= K <= n) among buf[0..n); all keys nonzero and unique.
__device__ inline uint64_t wave_kth_largest(const uint64_t* buf, int n, int K, uint32_t* hist) {
  const int lane = lane_id();
  uint64_t a = ~0ull, o = 0ull;
  for (int i = lane; i < n; i += kWave) {
    uint64_t e = buf[i];
    a &= e;
    o |= e;
  }
  a = wave_and_u64(a);
  o = wave_or_u64(o);
  uint64_t diff = a ^ o;
  if (diff == 0) return a;  // n == 1
  int top = 63 - __clzll((long long)diff);  // highest bit that differs between keys
  uint64_t pmask = (top == 63) ? 0ull : ~((2ull << top) - 1ull);
  uint64_t prefix = a & pmask;
  uint32_t need = (uint32_t)K;
  int shift = top - 7;
  for (;;) {
    int sh = shift > 0 ? shift : 0;
    for (int i = lane; i < 256; i += kWave) hist[i] = 0;
    __builtin_amdgcn_wave_barrier();
    for (int i = lane; i < n; i += kWave) {
      uint64_t e = buf[i];
      if ((e & pmask) == prefix) atomicAdd(&hist[(uint32_t)(e >> sh) & 0xFFu], 1u);
    }
    __builtin_amdgcn_wave_barrier();
    DigitPick p = pick_digit(hist, need);
    need -= p.above;
    prefix |= (uint64_t)p.d << sh;
    pmask |= 0xFFull << sh;
    if (p.cnt == need || sh == 0) break;
    shift -= 8;
  }
  // selected = { e >= prefix }: exactly K keys; the K-th largest is their minimum
  uint64_t mn = ~0ull;
  for (int i = lane; i < n; i += kWave) {
    uint64_t e = buf[i];
    if (e >= prefix && e < mn) mn = e;
  }
  return wave_min_u64(mn);
}

// Keep the keys >= kappa (in place, order kept); returns the new count.
__device__ inline int wave_compact(uint64_t* buf, int n, uint64_t kappa) {
  const int lane = lane_id();
  int base = 0;
  for (int i0 = 0; i0 < n; i0 += kWave) {
    int i = i0 + lane;
    uint64_t e = (i < n) ? buf[i] : 0ull;
    bool keep = (i < n) && e >= kappa;
    uint64_t m = ballot(keep);
    if (keep) buf[base + mbcnt(m)] = e;
    base += __popcll(m);
  }
  return base;
}

struct WaveTopK {
  uint64_t* buf;   // LDS candidate buffer of this wave
  uint32_t* hist;  // LDS 256-bin histogram of this wave
  int count;       // wave-uniform
  int K;
  int cap;
  uint64_t tau;    // insert iff key > tau
  float tau_v;     // score part of tau (-inf while tau == 0): v < tau_v can never enter
};

__device__ __forceinline__ void wave_topk_init(WaveTopK& st, uint64_t* buf, uint32_t* hist, int K, int cap) {
  st.buf = buf; st.hist = hist; st.count = 0; st.K = K; st.cap = cap; st.tau = 0ull;
  st.tau_v = -__builtin_inff();
}

// The results are wave-uniform; readfirstlane says so to the compiler, which
// otherwise keeps the count in a vector register (its loops over the buffer
// have per-lane trip counts) and turns every later test of it into
// exec-masked code.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// The same cut with the buffer read once into registers (R per lane, entry
// lane + 64 r in x[r]): the AND/OR statistics, the radix passes (8-bit
// digits counted into the wave's LDS histogram), the minimum of the selected
// keys and the compaction all work on the registers, so the buffer is read
// once and written once.  Needs cap <= 64 R.  EXACT = false is the cheaper
// trim used while the stream runs: the passes stop as soon as keeping the
// whole bucket that holds the K-th key keeps at most kTrimSlack keys beyond K,
// and the threshold becomes that bucket's floor (still <= the K-th key, so
// nothing that can reach the final top-K is dropped).
// Threshold of the K best among the nonzero keys x (R per lane, unique),
// which must number more than K: the K-th largest key (EXACT), or the floor
// of the 8-bit radix bucket that holds it once that bucket adds at most
// kTrimSlack keys beyond K (!EXACT).  hist: the wave's 256-bin LDS histogram.
template <int R, bool EXACT>
__device__ __forceinline__ uint64_t wave_cut_reg(const uint64_t (&x)[R], uint32_t K, uint32_t* hist) {
  const int lane = lane_id();
  uint64_t an = ~0ull, on = 0ull;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    an &= x[r] ? x[r] : ~0ull;
    on |= x[r];
  }
  an = uniform_u64(wave_and_u64(an));
  on = uniform_u64(wave_or_u64(on));
  if (an == on) return an;  // a single key
  const int top = 63 - __clzll((long long)(an ^ on));
  uint64_t pmask = (top == 63) ? 0ull : ~((2ull << top) - 1ull);
  uint64_t prefix = an & pmask;
  uint32_t need = K;
  int shift = top - 7;
  for (;;) {
    const int sh = shift > 0 ? shift : 0;
#pragma unroll
    for (int i = 0; i < 256 / kWave; ++i) hist[lane + kWave * i] = 0u;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (x[r] && (x[r] & pmask) == prefix) atomicAdd(&hist[(uint32_t)(x[r] >> sh) & 0xFFu], 1u);
    __builtin_amdgcn_wave_barrier();
    const DigitPick pk = pick_digit(hist, need);
    need -= pk.above;
    prefix |= (uint64_t)pk.d << sh;
    pmask |= 0xFFull << sh;
    if (pk.cnt == need || sh == 0) break;
    if (!EXACT && pk.cnt - need <= (uint32_t)kTrimSlack) return prefix;  // the bucket's floor
    shift -= 8;
  }
  // the selected keys are those >= prefix (exactly K); the K-th is their minimum
  uint64_t mn = ~0ull;
#pragma unroll
  for (int r = 0; r < R; ++r) mn = (x[r] != 0ull && x[r] >= prefix && x[r] < mn) ? x[r] : mn;
  return uniform_u64(wave_min_u64(mn));
}

// The nonzero keys >= kap of x (R per lane) into buf[0..), any order; returns
// how many (wave-uniform).
template <int R>
__device__ __forceinline__ int wave_compact_reg(const uint64_t (&x)[R], uint64_t kap, uint64_t* buf) {
  int base = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool keep = x[r] != 0ull && x[r] >= kap;
    const uint64_t m = ballot(keep);
    if (keep) buf[base + mbcnt(m)] = x[r];
    base += __popcll(m);
  }
  return __builtin_amdgcn_readfirstlane(base);
}

template <int R, bool EXACT>
__device__ __forceinline__ void wave_topk_reduce_reg(WaveTopK& st) {
  const int lane = lane_id();
  const int n = st.count;
  uint64_t x[R];
#pragma unroll
  for (int r = 0; r < R; ++r) x[r] = (lane + kWave * r < n) ? st.buf[lane + kWave * r] : 0ull;
  const uint64_t kap = wave_cut_reg<R, EXACT>(x, (uint32_t)st.K, st.hist);
  st.count = wave_compact_reg<R>(x, kap, st.buf);
  st.tau = kap;
  st.tau_v = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(key_score(kap))));
}

constexpr int kReduceRegRows = 19;  // register cut for buffers of up to 1216 entries (k_top <= 512)

__device__ __forceinline__ void wave_topk_reduce(WaveTopK& st) {
  if (st.count > st.K && st.cap <= kWave * kReduceRegRows) {
    wave_topk_reduce_reg<kReduceRegRows, true>(st);
    return;
  }
  if (st.count > st.K) {
    const uint64_t kap = uniform_u64(wave_kth_largest(st.buf, st.count, st.K, st.hist));
    st.count = __builtin_amdgcn_readfirstlane(wave_compact(st.buf, st.count, kap));
    st.tau = kap;
    st.tau_v = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(key_score(kap))));
  }
}

// Cut the buffer to between K and K + kTrimSlack keys (all keys that can still
// reach the final top-K stay): the cheaper cut for compactions inside the
// stream; the final one uses wave_topk_reduce.
__device__ __forceinline__ void wave_topk_trim(WaveTopK& st) {
  if (st.cap <= kWave * kReduceRegRows) {
    if (prefill_trim(st.count, st.K)) wave_topk_reduce_reg<kReduceRegRows, false>(st);
    return;
  }
  wave_topk_reduce(st);
}

// Offer one key per lane (valid == false: no candidate on this lane).
__device__ __forceinline__ void wave_topk_insert(WaveTopK& st, uint64_t key, bool valid) {
  bool p = valid && key > st.tau;
  uint64_t m = ballot(p);
  if (m == 0ull) return;
  int n = __popcll(m);
  if (st.count + n > st.cap) {
    wave_topk_reduce(st);
    p = valid && key > st.tau;
    m = ballot(p);
    n = __popcll(m);
  }
  if (p) st.buf[st.count + mbcnt(m)] = key;
  st.count += n;
}

// Bitonic sort of buf[0..n2) descending (n2 a power of two), one wavefront.
__device__ inline void wave_sort_desc(uint64_t* buf, int n2) {
  const int lane = lane_id();
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = lane; i < (n2 >> 1); i += kWave) {
        int a = 2 * i - (i & (j - 1));
        int b = a + j;
        uint64_t x = buf[a], y = buf[b];
        bool desc = (a & k) == 0;
        if (desc ? (x < y) : (x > y)) { buf[a] = y; buf[b] = x; }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

__host__ __device__ constexpr int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Descending bitonic sort of 64 E keys held in registers by one wavefront,
// lane L holding elements E L .. E L + E - 1 in x[0..E).  A compare-exchange
// at element distance j < E stays inside one lane's registers; one at
// distance j >= E pairs lanes L and L ^ (j / E), exchanged with DPP or a
// permlane swap.  No LDS and no barrier; E independent chains per stage.
// Lane exchange for the paired compare-exchange below: lanes with
// (lane & D) == 0 end up holding slot s's pair (own element in a, partner in
// b), the others slot t's pair (partner in a, own element in b), and the same
// call applied to the results puts every element back.  D = 16 and 32 use
// the permlane swaps; D = 4 and 8 two bank-masked DPP moves (the banks of 4
// lanes with bit D set, resp. clear, take the row-shifted value).
template <int D>
__device__ __forceinline__ void pair_exchange(uint32_t& a, uint32_t& b) {
  if constexpr (D == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = r[0];
    b = r[1];
  } else if constexpr (D == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = r[0];
    b = r[1];
  } else {
    static_assert(D == 4 || D == 8, "paired exchange distance");
    constexpr int kShr = D == 4 ? 0x114 : 0x118;  // row_shr:D (lane L reads L - D)
    constexpr int kShl = D == 4 ? 0x104 : 0x108;  // row_shl:D (lane L reads L + D)
    constexpr int kHi = D == 4 ? 0xA : 0xC;       // banks whose lanes have bit D set
    const uint32_t a2 = (uint32_t)__builtin_amdgcn_update_dpp((int)a, (int)b, kShr, 0xF, kHi, false);
    const uint32_t b2 = (uint32_t)__builtin_amdgcn_update_dpp((int)b, (int)a, kShl, 0xF, 0xF ^ kHi, false);
    a = a2;
    b = b2;
  }
}

template <int E, int K, int J>
__device__ __forceinline__ void wave_bitonic_stage_reg(uint64_t (&x)[E], int lane) {
  if constexpr (J < E) {
#pragma unroll
    for (int s = 0; s < E; ++s) {
      if (s & J) continue;
      bool desc;  // the run holding element E lane + s is sorted descending
      if constexpr (K < E) desc = (s & K) == 0;
      else desc = (lane & (K / E)) == 0;
      const uint64_t a = x[s], b = x[s | J];
      const bool sw = (a < b) == desc;  // equal keys (empty slots) need no swap
      x[s] = sw ? b : a;
      x[s | J] = sw ? a : b;
    }
  } else if constexpr (E >= 2 && (J / E == 4 || J / E == 8 || J / E == 16 || J / E == 32)) {
    // slots s and s + E / 2 travel together: one exchange gathers both
    // elements of a pair in one lane, which compare-exchanges them in
    // registers, and the same exchange returns them
    constexpr int D = J / E;
#pragma unroll
    for (int s = 0; s < E / 2; ++s) {
      uint32_t alo = (uint32_t)x[s], ahi = (uint32_t)(x[s] >> 32);
      uint32_t blo = (uint32_t)x[s + E / 2], bhi = (uint32_t)(x[s + E / 2] >> 32);
      pair_exchange<D>(alo, blo);
      pair_exchange<D>(ahi, bhi);
      const uint64_t a = ((uint64_t)ahi << 32) | alo, b = ((uint64_t)bhi << 32) | blo;  // lower, upper element
      bool desc;  // K >= 2 J >= 2 E here: the direction follows the lower element's lane
      if constexpr (K / E >= kWave) desc = true;
      else desc = (lane & (K / E)) == 0;
      const bool sw = (a < b) == desc;
      const uint64_t a2 = sw ? b : a, b2 = sw ? a : b;
      alo = (uint32_t)a2; ahi = (uint32_t)(a2 >> 32);
      blo = (uint32_t)b2; bhi = (uint32_t)(b2 >> 32);
      pair_exchange<D>(alo, blo);
      pair_exchange<D>(ahi, bhi);
      x[s] = ((uint64_t)ahi << 32) | alo;
      x[s + E / 2] = ((uint64_t)bhi << 32) | blo;
    }
  } else {
    constexpr int D = J / E;
    const bool low = (lane & D) == 0;  // this lane holds the lower element of each pair
#pragma unroll
    for (int s = 0; s < E; ++s) {
      const uint64_t y = xor_lane_u64<D>(x[s]);
      bool desc;
      if constexpr (K < E) desc = (s & K) == 0;
      else desc = (lane & (K / E)) == 0;
      const bool take_max = desc == low;
      x[s] = (take_max == (x[s] > y)) ? x[s] : y;
    }
  }
}
template <int E, int K, int J>
__device__ __forceinline__ void wave_bitonic_merge_reg(uint64_t (&x)[E], int lane) {
  wave_bitonic_stage_reg<E, K, J>(x, lane);
  if constexpr (J > 1) wave_bitonic_merge_reg<E, K, J / 2>(x, lane);
}
template <int E, int K = 2>
__device__ __forceinline__ void wave_sort_reg(uint64_t (&x)[E], int lane) {
  wave_bitonic_merge_reg<E, K, K / 2>(x, lane);
  if constexpr (K < kWave * E) wave_sort_reg<E, K * 2>(x, lane);
}

// buf[0..64 E) sorted descending in place through registers (entries at or
// past n are taken as empty keys).
template <int E>
__device__ __forceinline__ void wave_sort_desc_reg(uint64_t* buf, int n) {
  const int lane = lane_id();
  uint64_t x[E];
#pragma unroll
  for (int s = 0; s < E; ++s) x[s] = (E * lane + s < n) ? buf[E * lane + s] : 0ull;
  wave_sort_reg<E>(x, lane);
#pragma unroll
  for (int s = 0; s < E; ++s) buf[E * lane + s] = x[s];
  __builtin_amdgcn_wave_barrier();
}

// Cut to the K best, sort descending and pad with empty keys to K entries.
// Needs cap >= next_pow2(K).  Result in buf[0..K).
__device__ inline void wave_topk_finish(WaveTopK& st) {
  wave_topk_reduce(st);
  const int n2 = next_pow2(st.K);
  if (n2 == 256) { wave_sort_desc_reg<4>(st.buf, st.count); return; }
  if (n2 == 512) { wave_sort_desc_reg<8>(st.buf, st.count); return; }
  if (n2 == 1024) { wave_sort_desc_reg<16>(st.buf, st.count); return; }
  for (int i = st.count + lane_id(); i < n2; i += kWave) st.buf[i] = 0ull;
  __builtin_amdgcn_wave_barrier();
  wave_sort_desc(st.buf, n2);
}

// Write K sorted keys as the final (idx, score) row, or as a candidate list.
__device__ inline void wave_write_row(const uint64_t* buf, int K, int32_t* idx_row, float* score_row,
                                      uint64_t* list_row) {
  for (int i = lane_id(); i < K; i += kWave) {
    uint64_t key = buf[i];
    if (list_row) {
      list_row[i] = key;
    } else {
      idx_row[i] = key_index(key);
      if (score_row) score_row[i] = key_score(key);
    }
  }
}

// --------------------------------------------- wavefront bucket pass (top-K)
// Maximum and minimum over the wavefront.  Every partner value is taken once,
// by all lanes, before the comparison (a lane exchange evaluated inside a
// divergent select would read 0 from the lanes the select masked off).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  uint32_t y;
  y = xor_lane_u32<1>(x);
  x = __builtin_elementwise_max(x, y);
  y = xor_lane_u32<2>(x);
  x = __builtin_elementwise_max(x, y);
  y = xor_lane_u32<4>(x);
  x = __builtin_elementwise_max(x, y);
  y = xor_lane_u32<8>(x);
  x = __builtin_elementwise_max(x, y);
  y = xor_lane_u32<16>(x);
  x = __builtin_elementwise_max(x, y);
  y = xor_lane_u32<32>(x);
  x = __builtin_elementwise_max(x, y);
  return x;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) { return ~wave_max_u32(~x); }

// The K best of one wavefront's nonzero keys x (R per lane, unique), in
// descending order, by one bucket pass, without a radix select or a sort
// network.  The bucket of a key is floor((v - vmin) * NB / (vmax - vmin)),
// clamped to NB - 1, over the keys' score range: each step of that map (a
// subtraction of one value, a product with one positive factor, a
// truncation) is monotone in the score v, so a larger key never lands in a
// lower bucket and equal scores share one.  The bucket counts, scanned in
// descending order, give each bucket its first output position; the keys of
// every bucket that starts below K are scattered into a segment of `seg`
// (with the segment's bounds beside each key in `meta`), and a key's place
// inside its bucket is its rank among that segment's keys (full 64-bit
// comparison: equal scores go by index).  out(pos, key) is called once for
// every pos < m = min(K, number of keys), by some lane of the wavefront.
// Returns m, or -1 (wave-uniform; out never called) when a bucket that
// starts below K holds more than kWaveBucketMax keys, for the caller's
// general path.  LDS of this wavefront: bins 2 NB u32; seg K + kWaveBucketMax
// + 8 u64 (it may be the buffer x was read from); meta K + kWaveBucketMax u32.
constexpr int kWaveBucketMax = 64;

template <int R, int NB, typename Out>
__device__ __forceinline__ int wave_bucket_topk(const uint64_t (&x)[R], int K, uint32_t* bins, uint64_t* seg,
                                                uint32_t* meta, Out&& out) {
  static_assert(NB % (4 * kWave) == 0, "whole 16-byte bin groups per lane");
  constexpr int PER = NB / kWave;  // bins per lane in the scan
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const int lane = lane_id();
  uint32_t* cnt = bins;       // counts, then fill cursors
  uint32_t* start = bins + NB;
  // 1. score range and count of the present keys; counts cleared
  uint32_t omin = ~0u, omax = 0u, c = 0u;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t h = (uint32_t)(x[r] >> 32);
    omin = (x[r] && h < omin) ? h : omin;
    omax = (x[r] && h > omax) ? h : omax;
    c += x[r] ? 1u : 0u;
  }
  omin = __builtin_amdgcn_readfirstlane(wave_min_u32(omin));
  omax = __builtin_amdgcn_readfirstlane(wave_max_u32(omax));
  const uint32_t n = __builtin_amdgcn_readfirstlane(wave_sum_u32(c));
#pragma unroll
  for (int i = 0; i < PER / 4; ++i) *reinterpret_cast<u32x4_t*>(cnt + 4 * (lane + kWave * i)) = u32x4_t{0u, 0u, 0u, 0u};
  // finite scores only (-inf keys are never candidates); a range that is 0,
  // infinite or so small that the factor overflows puts every key in bucket 0
  const float vmin = unord_f32(omin);
  const float range = unord_f32(omax) - vmin;
  float scale = range > 0.f ? (float)NB / range : 0.f;
  scale = (scale < 3.0e38f && range < 3.0e38f) ? scale : 0.f;
  auto bucket = [&](uint64_t key) -> uint32_t {
    const uint32_t b = (uint32_t)((unord_f32((uint32_t)(key >> 32)) - vmin) * scale);
    return b < (uint32_t)(NB - 1) ? b : (uint32_t)(NB - 1);
  };
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // 2. bucket counts
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (x[r]) atomicAdd(&cnt[bucket(x[r])], 1u);
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // 3. lane L owns buckets NB - 1 - PER L - e (e < PER), in descending order
  uint32_t hc[PER], sum = 0u;
#pragma unroll
  for (int i = 0; i < PER / 4; ++i) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(cnt + NB - PER * (lane + 1) + 4 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) hc[PER - 1 - (4 * i + j)] = v[j];
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) sum += hc[e];
  uint32_t o = wave_incl_scan_u32(sum) - sum;
  uint32_t used = 0u, mx = 0u;  // end of the last bucket that starts below K; the largest such bucket
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int b = NB - 1 - PER * lane - e;
    start[b] = o;
    cnt[b] = o;
    const bool below = o < (uint32_t)K;
    used = below && o + hc[e] > used ? o + hc[e] : used;
    mx = below && hc[e] > mx ? hc[e] : mx;
    o += hc[e];
  }
  if (__builtin_amdgcn_readfirstlane(wave_max_u32(mx)) > (uint32_t)kWaveBucketMax) return -1;
  used = __builtin_amdgcn_readfirstlane(wave_max_u32(used));
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // 4. the keys of the buckets that start below K, each into its segment,
  //    with the segment's bounds (a bucket ends where the next lower one
  //    starts; the lowest ends at n)
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (x[r]) {
      const uint32_t d = bucket(x[r]);
      const uint32_t st = start[d];
      if (st < (uint32_t)K) {
        const uint32_t en = d > 0 ? start[d - 1] : n;
        const uint32_t slot = atomicAdd(&cnt[d], 1u);
        seg[slot] = x[r];
        meta[slot] = st | (en << 16);
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // 5. a key's place: its bucket's start plus its rank inside the bucket.
  //    The lanes walk the filled slots [0, used), two at a time; the first 8
  //    entries of a key's segment are read at once, entries past its end are
  //    ignored.
  auto place = [&](uint32_t i) {
    const uint64_t key = seg[i];
    const uint32_t mt = meta[i];
    const uint32_t st = mt & 0xFFFFu, en = mt >> 16;
    uint64_t sv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) sv[j] = seg[st + j];
    uint32_t pos = st;
#pragma unroll
    for (int j = 0; j < 8; ++j) pos += (st + j < en && sv[j] > key) ? 1u : 0u;
    for (uint32_t j = st + 8; j < en; ++j) pos += seg[j] > key ? 1u : 0u;
    if (pos < (uint32_t)K) out((int)pos, key);
  };
  for (uint32_t i = (uint32_t)lane; i < used; i += 2 * kWave) {
    place(i);
    if (i + kWave < used) place(i + kWave);
  }
  return n < (uint32_t)K ? (int)n : K;
}

// ------------------------------------------------------------ block-wide ops
// All threads of the block call these (blockDim.x = BS, a multiple of 64,
// 128 <= BS <= 1024).  Barriers are the expensive part, so each helper uses
// as few as it can.

struct BlockShared {
  uint32_t hist[3][256];  // radix histograms (triple buffered)
  int32_t wsum[16];       // per-wavefront partial sums
  uint64_t red_and, red_or, red_min;
  uint32_t nz;
  uint32_t pick_d, pick_above, pick_cnt;
};

// Exclusive prefix sum of one int per thread over the block; *total gets the sum.
__device__ inline int block_excl_scan(int x, int* total, BlockShared& sh) {
  const int lane = lane_id(), wv = threadIdx.x / kWave, nw = blockDim.x / kWave;
  const int incl = (int)wave_incl_scan_u32((uint32_t)x);
  if (lane == kWave - 1) sh.wsum[wv] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w2 = 0; w2 < nw; ++w2) {
    const int c = sh.wsum[w2];
    base += (w2 < wv) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return base + incl - x;
}

// One compare-exchange stage (k, j) of a descending bitonic sort with one
// element per thread; partners in other wavefronts (j >= 64) meet in LDS
// (ping-pong halves of tmp, one barrier per stage).
template <int K, int J>
__device__ __forceinline__ void bitonic_stage(uint64_t& x, uint64_t* tmp, int& flip) {
  const int i = threadIdx.x;
  uint64_t y;
  if constexpr (J >= kWave) {
    uint64_t* t = tmp + flip * blockDim.x;
    flip ^= 1;
    t[i] = x;
    __syncthreads();
    y = t[i ^ J];
  } else {
    y = xor_lane_u64<J>(x);
  }
  const bool take_max = ((i & K) == 0) == ((i & J) == 0);
  x = (take_max == (x > y)) ? x : y;
}
template <int K, int J>
__device__ __forceinline__ void bitonic_merge_steps(uint64_t& x, uint64_t* tmp, int& flip) {
  bitonic_stage<K, J>(x, tmp, flip);
  if constexpr (J > 1) bitonic_merge_steps<K, J / 2>(x, tmp, flip);
}
template <int N2, int K = 2>
__device__ __forceinline__ void bitonic_all(uint64_t& x, uint64_t* tmp, int& flip) {
  bitonic_merge_steps<K, K / 2>(x, tmp, flip);
  if constexpr (K < N2) bitonic_all<N2, K * 2>(x, tmp, flip);
}

// Bitonic sort of buf[0..N2) descending (N2 a power of two <= blockDim.x),
// fully unrolled; tmp holds 2 * blockDim.x entries.
template <int N2>
__device__ inline void block_sort_desc_n(uint64_t* buf, uint64_t* tmp) {
  const int i = threadIdx.x;
  uint64_t x = (i < N2) ? buf[i] : 0ull;
  int flip = 0;
  if constexpr (N2 > 1) bitonic_all<N2>(x, tmp, flip);
  __syncthreads();
  if (i < N2) buf[i] = x;
  __syncthreads();
}

// Bitonic sort through LDS only (any n2 <= 2048), for sizes beyond blockDim.
__device__ inline void block_sort_desc_lds(uint64_t* buf, int n2) {
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < (n2 >> 1); i += blockDim.x) {
        int a = 2 * i - (i & (j - 1));
        int b = a + j;
        uint64_t x = buf[a], y = buf[b];
        bool desc = (a & k) == 0;
        if (desc ? (x < y) : (x > y)) { buf[a] = y; buf[b] = x; }
      }
      __syncthreads();
    }
  }
}

// K-th largest among the nonzero keys of arr[0..n) (all nonzero keys unique);
// needs K <= nonzero count.  Starts at the highest bit where keys differ
// (a, o = AND / OR of the nonzero keys) and resolves 8 bits per pass.  Every
// wavefront reads the histogram and picks the digit itself, and the three
// histogram buffers rotate (pass p fills buffer p % 3 and clears buffer
// (p + 2) % 3, last read in pass p - 1), so one barrier per pass suffices.
__device__ inline uint64_t block_kth_largest(const uint64_t* arr, int n, int K, uint64_t a, uint64_t o,
                                             BlockShared& sh) {
  const uint64_t diff = a ^ o;
  if (diff == 0ull) return a;
  const int top = 63 - __clzll((long long)diff);
  uint64_t pmask = (top == 63) ? 0ull : ~((2ull << top) - 1ull);
  uint64_t prefix = a & pmask;
  uint32_t need = (uint32_t)K;
  int shift = top - 7;
  for (int pass = 0;; ++pass) {
    const int sh8 = shift > 0 ? shift : 0;
    uint32_t* hist = sh.hist[pass % 3];
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const uint64_t e = arr[i];
      if (e && (e & pmask) == prefix) atomicAdd(&hist[(uint32_t)(e >> sh8) & 0xFFu], 1u);
    }
    __syncthreads();
    const DigitPick pk = pick_digit(hist, need);
    for (int i = threadIdx.x; i < 256; i += blockDim.x) sh.hist[(pass + 2) % 3][i] = 0;
    need -= pk.above;
    prefix |= (uint64_t)pk.d << sh8;
    pmask |= 0xFFull << sh8;
    if (pk.cnt == need || sh8 == 0) break;
    shift -= 8;
  }
  // every key >= prefix is selected (exactly K of them); the K-th is their minimum
  uint64_t mn = ~0ull;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const uint64_t e = arr[i];
    if (e >= prefix && e < mn) mn = e;
  }
  mn = wave_min_u64(mn);
  if (lane_id() == 0) atomicMin((unsigned long long*)&sh.red_min, mn);
  __syncthreads();
  return sh.red_min;
}

// Copy the nonzero keys >= kappa of src[0..n) to dst[0..) in order (each
// thread owns one contiguous slice); returns the count.  No overlap allowed.
__device__ inline int block_compact(const uint64_t* src, int n, uint64_t kappa, uint64_t* dst, BlockShared& sh) {
  const int per = (n + (int)blockDim.x - 1) / (int)blockDim.x;
  const int lo = threadIdx.x * per;
  const int hi = lo + per < n ? lo + per : n;
  int c = 0;
  for (int i = lo; i < hi; ++i) {
    const uint64_t e = src[i];
    c += (e != 0ull && e >= kappa);
  }
  int total;
  int pos = block_excl_scan(c, &total, sh);
  for (int i = lo; i < hi; ++i) {
    const uint64_t e = src[i];
    if (e != 0ull && e >= kappa) dst[pos++] = e;
  }
  __syncthreads();
  return total;
}

// AND / OR / count of the nonzero keys of arr[0..n); also zeroes the radix
// histograms and the min slot for block_kth_largest.
__device__ inline uint32_t block_key_stats(const uint64_t* arr, int n, uint64_t* a_out, uint64_t* o_out,
                                           BlockShared& sh) {
  if (threadIdx.x == 0) { sh.red_and = ~0ull; sh.red_or = 0ull; sh.red_min = ~0ull; sh.nz = 0; }
  for (int i = threadIdx.x; i < 3 * 256; i += blockDim.x) (&sh.hist[0][0])[i] = 0;
  __syncthreads();
  uint64_t a = ~0ull, o = 0ull;
  uint32_t c = 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const uint64_t e = arr[i];
    if (e) { a &= e; o |= e; ++c; }
  }
  a = wave_and_u64(a);
  o = wave_or_u64(o);
  c = wave_sum_u32(c);
  if (lane_id() == 0) {
    atomicAnd((unsigned long long*)&sh.red_and, a);
    atomicOr((unsigned long long*)&sh.red_or, o);
    atomicAdd(&sh.nz, c);
  }
  __syncthreads();
  *a_out = sh.red_and;
  *o_out = sh.red_or;
  return sh.nz;
}

// Descending sort of buf[0..n2) for a power of two n2 <= 1024: the unrolled
// register network when n2 <= blockDim.x, else the LDS network.
__device__ __forceinline__ void block_sort_desc(uint64_t* buf, int n2, uint64_t* tmp) {
  if (n2 > (int)blockDim.x) { block_sort_desc_lds(buf, n2); return; }
  switch (n2) {
    case 1: break;
    case 2: block_sort_desc_n<2>(buf, tmp); break;
    case 4: block_sort_desc_n<4>(buf, tmp); break;
    case 8: block_sort_desc_n<8>(buf, tmp); break;
    case 16: block_sort_desc_n<16>(buf, tmp); break;
    case 32: block_sort_desc_n<32>(buf, tmp); break;
    case 64: block_sort_desc_n<64>(buf, tmp); break;
    case 128: block_sort_desc_n<128>(buf, tmp); break;
    case 256: block_sort_desc_n<256>(buf, tmp); break;
    case 512: block_sort_desc_n<512>(buf, tmp); break;
    default: block_sort_desc_n<1024>(buf, tmp); break;
  }
}

// The K best nonzero keys of arr[0..n) into sel[0..K), sorted descending and
// padded with empty keys; sel has room for next_pow2(K) entries, tmp for
// 2 * blockDim.x.  sel must not overlap arr.
__device__ inline void block_select_sorted(const uint64_t* arr, int n, int K, uint64_t* sel, uint64_t* tmp,
                                           BlockShared& sh) {
  uint64_t a, o;
  const uint32_t nz = block_key_stats(arr, n, &a, &o, sh);
  uint64_t kappa = 1ull;
  if ((int)nz > K) kappa = block_kth_largest(arr, n, K, a, o, sh);
  const int m = block_compact(arr, n, kappa, sel, sh);
  const int n2 = next_pow2(K);
  for (int i = m + threadIdx.x; i < n2; i += blockDim.x) sel[i] = 0ull;
  __syncthreads();
  block_sort_desc(sel, n2, tmp);
}

}  // namespace lid
