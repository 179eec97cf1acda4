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

// f16 mask bits -> f32 (exact)
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  _Float16 x = __builtin_bit_cast(_Float16, h);
  return (float)x;
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// number of set bits of `m` below this lane
__device__ __forceinline__ int mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int mask) {
  uint32_t lo = __shfl_xor((uint32_t)x, mask);
  uint32_t hi = __shfl_xor((uint32_t)(x >> 32), mask);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t x) {
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t y = shfl_xor_u64(x, o);
    x = y < x ? y : x;
  }
  return x;
}
__device__ __forceinline__ uint64_t wave_and_u64(uint64_t x) {
  for (int o = 32; o > 0; o >>= 1) x &= shfl_xor_u64(x, o);
  return x;
}
__device__ __forceinline__ uint64_t wave_or_u64(uint64_t x) {
  for (int o = 32; o > 0; o >>= 1) x |= shfl_xor_u64(x, o);
  return x;
}
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
  const int lane = lane_id();
  for (int o = 1; o < kWave; o <<= 1) {
    uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
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
  r.d = __shfl(d, fl);
  r.above = __shfl(above, fl);
  r.cnt = __shfl(cnt, fl);
  return r;
}

// ------------------------------------------------- per-wavefront streaming top-k
// One wavefront owns one query's candidate buffer `buf` (LDS, capacity `cap`
// >= K + 64).  Candidates with key > tau are appended; when the buffer would
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
};

__device__ __forceinline__ void wave_topk_init(WaveTopK& st, uint64_t* buf, uint32_t* hist, int K, int cap) {
  st.buf = buf; st.hist = hist; st.count = 0; st.K = K; st.cap = cap; st.tau = 0ull;
}

__device__ __forceinline__ void wave_topk_reduce(WaveTopK& st) {
  if (st.count > st.K) {
    uint64_t kap = wave_kth_largest(st.buf, st.count, st.K, st.hist);
    st.count = wave_compact(st.buf, st.count, kap);
    st.tau = kap;
  }
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

// Cut to the K best, sort descending and pad with empty keys to K entries.
// Needs cap >= next_pow2(K).  Result in buf[0..K).
__device__ inline void wave_topk_finish(WaveTopK& st) {
  wave_topk_reduce(st);
  const int n2 = next_pow2(st.K);
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

// ------------------------------------------------------------ block-wide ops
// All threads of the block call these (blockDim.x = BS, a multiple of 64).

struct BlockShared {
  uint32_t hist[256];
  uint32_t wcount[16];
  uint64_t red_and, red_or, red_min;
  uint32_t nz;
  uint32_t pick_d, pick_above, pick_cnt;
};

// Number of nonzero keys in arr[0..n).
__device__ inline uint32_t block_count_nonzero(const uint64_t* arr, int n, BlockShared& sh) {
  if (threadIdx.x == 0) sh.nz = 0;
  __syncthreads();
  uint32_t c = 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) c += arr[i] != 0ull;
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
  if (lane_id() == 0) atomicAdd(&sh.nz, c);
  __syncthreads();
  uint32_t r = sh.nz;
  __syncthreads();
  return r;
}

// K-th largest among the nonzero keys of arr[0..n) (requires K <= nonzero count).
__device__ inline uint64_t block_kth_largest(const uint64_t* arr, int n, int K, BlockShared& sh) {
  const int lane = lane_id();
  if (threadIdx.x == 0) { sh.red_and = ~0ull; sh.red_or = 0ull; sh.red_min = ~0ull; }
  __syncthreads();
  uint64_t a = ~0ull, o = 0ull;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    uint64_t e = arr[i];
    if (e) { a &= e; o |= e; }
  }
  a = wave_and_u64(a);
  o = wave_or_u64(o);
  if (lane == 0) { atomicAnd((unsigned long long*)&sh.red_and, a); atomicOr((unsigned long long*)&sh.red_or, o); }
  __syncthreads();
  a = sh.red_and;
  o = sh.red_or;
  uint64_t diff = a ^ o;
  if (diff == 0ull) { __syncthreads(); return a; }
  int top = 63 - __clzll((long long)diff);
  uint64_t pmask = (top == 63) ? 0ull : ~((2ull << top) - 1ull);
  uint64_t prefix = a & pmask;
  uint32_t need = (uint32_t)K;
  int shift = top - 7;
  for (;;) {
    int sh8 = shift > 0 ? shift : 0;
    for (int i = threadIdx.x; i < 256; i += blockDim.x) sh.hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      uint64_t e = arr[i];
      if (e && (e & pmask) == prefix) atomicAdd(&sh.hist[(uint32_t)(e >> sh8) & 0xFFu], 1u);
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
      DigitPick p = pick_digit(sh.hist, need);
      if (threadIdx.x == 0) { sh.pick_d = p.d; sh.pick_above = p.above; sh.pick_cnt = p.cnt; }
    }
    __syncthreads();
    uint32_t d = sh.pick_d, above = sh.pick_above, cnt = sh.pick_cnt;
    __syncthreads();
    need -= above;
    prefix |= (uint64_t)d << sh8;
    pmask |= 0xFFull << sh8;
    if (cnt == need || sh8 == 0) break;
    shift -= 8;
  }
  uint64_t mn = ~0ull;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    uint64_t e = arr[i];
    if (e >= prefix && e < mn) mn = e;
  }
  mn = wave_min_u64(mn);
  if (lane == 0) atomicMin((unsigned long long*)&sh.red_min, mn);
  __syncthreads();
  uint64_t r = sh.red_min;
  __syncthreads();
  return r;
}

// Copy the keys of src[0..n) that are >= kappa (and nonzero) to dst[0..),
// keeping their order; returns the number copied.  src and dst must not overlap.
__device__ inline int block_compact(const uint64_t* src, int n, uint64_t kappa, uint64_t* dst, BlockShared& sh) {
  const int wv = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  int base = 0;
  for (int i0 = 0; i0 < n; i0 += blockDim.x) {
    int i = i0 + threadIdx.x;
    uint64_t e = (i < n) ? src[i] : 0ull;
    bool keep = (i < n) && e != 0ull && e >= kappa;
    uint64_t m = ballot(keep);
    if (lane_id() == 0) sh.wcount[wv] = __popcll(m);
    __syncthreads();
    int before = 0, total = 0;
    for (int w2 = 0; w2 < nw; ++w2) {
      int c = sh.wcount[w2];
      before += (w2 < wv) ? c : 0;
      total += c;
    }
    if (keep) dst[base + before + mbcnt(m)] = e;
    base += total;
    __syncthreads();
  }
  return base;
}

// Bitonic sort of buf[0..n2) descending, whole block.
__device__ inline void block_sort_desc(uint64_t* buf, int n2) {
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

// Select the K best nonzero keys of arr[0..n) into sel[0..K) sorted
// descending, padded with empty keys (sel has room for next_pow2(K)).
__device__ inline void block_select_sorted(const uint64_t* arr, int n, int K, uint64_t* sel, BlockShared& sh) {
  uint32_t nz = block_count_nonzero(arr, n, sh);
  uint64_t kappa = 1ull;
  if ((int)nz > K) kappa = block_kth_largest(arr, n, K, sh);
  int m = block_compact(arr, n, kappa, sel, sh);
  const int n2 = next_pow2(K);
  for (int i = m + threadIdx.x; i < n2; i += blockDim.x) sel[i] = 0ull;
  __syncthreads();
  block_sort_desc(sel, n2);
}

}  // namespace lid
