// lid_select.h -- block-wide exact selection with the keys held in
// registers (used by the decode kernel and the merge; workgroups of kSelThreads
// threads).  A radix select with 8-bit digits from the highest bit in which
// the keys differ: the keys are counted into a shared LDS histogram and every
// wavefront finds the digit that holds the K-th largest key from it; no LDS
// array of keys is rescanned per pass and a pass costs one barrier.
#pragma once
#include "lid_device.h"

namespace lid {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / kWave;
// LDS the helpers need besides their key arrays: histograms and a small
// reduction area.
constexpr size_t kSelHistBytes = 2 * kSelWaves * 256 * 4;
constexpr size_t kSelRedBytes = (4 * kSelWaves + 8) * 4;

// Radix select over values held in registers, R per thread (0 = absent):
// returns b with at least K present values >= b and b <= the K-th largest
// present value (exactly the K-th largest when the values are unique), or 1
// when fewer than K values are present.  8-bit digits from the highest bit in
// which the values differ; one shared 256-bin LDS histogram per pass (three
// rotate, each cleared two passes ahead), and every wavefront finds the digit
// from it itself, so a pass costs a single barrier.  hw is unused (kept for
// the callers' layout).
template <typename KT, int R>
__device__ __forceinline__ KT block_kth_largest_reg(const KT (&xin)[R], uint32_t K, uint32_t* hw, BlockShared* sh,
                                                    uint32_t* red) {
  (void)hw;
  (void)red;
  constexpr int BITS = 8 * (int)sizeof(KT);
  const int tid = threadIdx.x;
  // a private copy, made opaque at every pass so that per-key conditions are
  // recomputed (cheap) instead of being kept live as lane masks across passes
  KT x[R];
#pragma unroll
  for (int i = 0; i < R; ++i) x[i] = xin[i];
  KT an = ~(KT)0, on = 0;
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    an &= x[i] ? x[i] : ~(KT)0;
    on |= x[i];
    c += x[i] ? 1u : 0u;
  }
  if constexpr (BITS == 64) {
    an = wave_and_u64(an);
    on = wave_or_u64(on);
  } else {
    an = wave_and_u32(an);
    on = wave_or_u32(on);
  }
  c = wave_sum_u32(c);
  if (tid == 0) { sh->red_and = ~0ull; sh->red_or = 0ull; sh->nz = 0u; }
  for (int i = tid; i < 3 * 256; i += kSelThreads) (&sh->hist[0][0])[i] = 0u;
  __syncthreads();
  if ((tid & (kWave - 1)) == 0) {
    atomicAnd((unsigned long long*)&sh->red_and, (unsigned long long)an);
    atomicOr((unsigned long long*)&sh->red_or, (unsigned long long)on);
    atomicAdd(&sh->nz, c);
  }
  __syncthreads();
  an = (KT)sh->red_and;
  on = (KT)sh->red_or;
  c = sh->nz;
  if (c < K) return (KT)1;
  if (an == on) return an;
  const int top = BITS - 1 - (BITS == 64 ? __clzll((long long)(uint64_t)(an ^ on)) : __builtin_clz((uint32_t)(an ^ on)));
  KT prefix = top == BITS - 1 ? (KT)0 : (an & ~(((KT)2 << top) - (KT)1));
  uint32_t need = K;
  int hi_bit = top;  // undecided bits: [hi_bit .. 0]
  for (int pass = 0;; ++pass) {
    const int nb = hi_bit + 1 < 8 ? hi_bit + 1 : 8;
    const int shft = hi_bit + 1 - nb;
    const uint32_t dmask = (1u << nb) - 1u;
    uint32_t* h = sh->hist[pass % 3];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if constexpr (sizeof(KT) == 8) {
        uint32_t lo = (uint32_t)x[i], hi = (uint32_t)(x[i] >> 32);
        asm volatile("" : "+v"(lo), "+v"(hi));
        x[i] = ((KT)hi << 32) | lo;
      } else {
        asm volatile("" : "+v"(x[i]));
      }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const bool in = x[i] != 0 && (hi_bit >= BITS - 1 || (x[i] >> (hi_bit + 1)) == (prefix >> (hi_bit + 1)));
      if (in) atomicAdd(&h[(uint32_t)(x[i] >> shft) & dmask], 1u);
    }
    __syncthreads();
    // digits above dmask stay zero, so the 256-bin search sees the nb-bit digit
    const DigitPick pk = pick_digit(h, need);
    for (int i = tid; i < 256; i += kSelThreads) sh->hist[(pass + 2) % 3][i] = 0u;
    prefix |= (KT)pk.d << shft;
    need -= pk.above;
    if (pk.cnt == need || shft == 0) return prefix;  // lower bits zero: the bucket and above
    hi_bit = shft - 1;
  }
}

// The K best of arr[0..n) (n <= R * kSelThreads; unique keys, 0 = empty), in
// no particular order, into dst; returns how many (min(K, keys present)).
template <int R>
__device__ __forceinline__ int block_select_compact_reg(const uint64_t* arr, int n, int K, uint64_t* dst,
                                                        uint32_t* hw, BlockShared* sh, uint32_t* red) {
  const int tid = threadIdx.x;
  uint64_t k[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int j = i * kSelThreads + tid;
    k[i] = j < n ? arr[j] : 0ull;
  }
  const uint64_t thr = n > K ? block_kth_largest_reg<uint64_t, R>(k, (uint32_t)K, hw, sh, red) : 1ull;
#pragma unroll
  for (int i = 0; i < R; ++i) {  // opaque: see block_kth_largest_reg
    uint32_t lo = (uint32_t)k[i], hi = (uint32_t)(k[i] >> 32);
    asm volatile("" : "+v"(lo), "+v"(hi));
    k[i] = ((uint64_t)hi << 32) | lo;
  }
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < R; ++i) c += (k[i] != 0ull && k[i] >= thr) ? 1u : 0u;
  int total;
  int pos = block_excl_scan((int)c, &total, *sh);
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (k[i] != 0ull && k[i] >= thr) dst[pos++] = k[i];
  __syncthreads();
  return total;
}

// The K best of arr[0..n), sorted descending and padded with empty keys to
// next_pow2(K), into sel (tmp: 2 kSelThreads entries for the sort).
template <int R>
__device__ __forceinline__ void block_select_sorted_reg(const uint64_t* arr, int n, int K, uint64_t* sel,
                                                        uint64_t* tmp, uint32_t* hw, BlockShared* sh, uint32_t* red) {
  const int m = block_select_compact_reg<R>(arr, n, K, sel, hw, sh, red);
  const int n2 = next_pow2(K);
  for (int i = m + (int)threadIdx.x; i < n2; i += kSelThreads) sel[i] = 0ull;
  __syncthreads();
  block_sort_desc(sel, n2, tmp);
}

// The same with the register count chosen from n at run time (n is
// block-uniform), so a small set is not scanned through empty slots.
__device__ __forceinline__ int block_select_compact_any(const uint64_t* arr, int n, int K, uint64_t* dst, uint32_t* hw,
                                                        BlockShared* sh, uint32_t* red) {
  if (n <= 2 * kSelThreads) return block_select_compact_reg<2>(arr, n, K, dst, hw, sh, red);
  if (n <= 4 * kSelThreads) return block_select_compact_reg<4>(arr, n, K, dst, hw, sh, red);
  if (n <= 8 * kSelThreads) return block_select_compact_reg<8>(arr, n, K, dst, hw, sh, red);
  if (n <= 16 * kSelThreads) return block_select_compact_reg<16>(arr, n, K, dst, hw, sh, red);
  return block_select_compact_reg<18>(arr, n, K, dst, hw, sh, red);  // n <= 18 kSelThreads (callers check)
}
__device__ __forceinline__ void block_select_sorted_any(const uint64_t* arr, int n, int K, uint64_t* sel,
                                                        uint64_t* tmp, uint32_t* hw, BlockShared* sh, uint32_t* red) {
  const int m = block_select_compact_any(arr, n, K, sel, hw, sh, red);
  const int n2 = next_pow2(K);
  for (int i = m + (int)threadIdx.x; i < n2; i += kSelThreads) sel[i] = 0ull;
  __syncthreads();
  block_sort_desc(sel, n2, tmp);
}

// ---------------------------------------------------------- merge-tree top-K
// The K best (next_pow2(K) == kTreeCap) of buf[0..m), m <= 8 * 64 E, sorted
// descending, by the block's 8 wavefronts without a radix select: each
// wavefront sorts a chunk of 64 E keys in registers (wave_sort_reg), then
// three levels merge pairs of sorted runs through LDS, one barrier each.
// Two sorted runs A, B of length L give one bitonic sequence C: A followed by
// B reversed when 2 L <= kTreeCap, else max(A[i], B[L - 1 - i]), which holds
// the kTreeCap best of both.  The W wavefronts of a merge split its output
// into W blocks: the first log2(W) half-cleaner stages of the bitonic merge
// act on the columns C[i + u N / W], u < W, which each wavefront evaluates
// straight from LDS, keeping the value of its own block; its block is then
// bitonic and is sorted by the remaining stages in registers.  buf holds the
// candidates (8 * 64 E entries, those at or past m read as empty) and alt is
// LDS for 2048 more; the result goes straight to the output row, or, when
// out is given, to out[0..kTreeCap) in LDS (visible after the call).
constexpr int kTreeCap = 512;

template <int EB, int W, int LIN, bool CAPPED>
__device__ __forceinline__ void wave_merge_block(const uint64_t* A, const uint64_t* B, int j, uint64_t (&x)[EB]) {
  constexpr int NB = kWave * EB;  // outputs per wavefront
  const int lane = lane_id();
#pragma unroll
  for (int s = 0; s < EB; ++s) {
    uint64_t v[W];
#pragma unroll
    for (int u = 0; u < W; ++u) {
      const int i = u * NB + EB * lane + s;  // position in C
      if constexpr (CAPPED) {
        const uint64_t a = A[i], b = B[LIN - 1 - i];
        v[u] = a > b ? a : b;
      } else {
        v[u] = i < LIN ? A[i] : B[2 * LIN - 1 - i];
      }
    }
#pragma unroll
    for (int h = W / 2; h >= 1; h /= 2)
#pragma unroll
      for (int u = 0; u < W; ++u)
        if (!(u & h)) {
          const uint64_t hi = v[u] > v[u + h] ? v[u] : v[u + h];
          const uint64_t lo = v[u] > v[u + h] ? v[u + h] : v[u];
          v[u] = hi;
          v[u + h] = lo;
        }
    uint64_t r = v[0];
#pragma unroll
    for (int u = 1; u < W; ++u) r = j == u ? v[u] : r;
    x[s] = r;
  }
  wave_bitonic_merge_reg<EB, NB, NB / 2>(x, lane);
}

// Level LVL (1..3): 8 >> LVL merges of the runs in src (length LIN, stride
// SIN), W = 2^LVL wavefronts each, into dst (length LOUT, stride LOUT), or the
// output row at the last level.
template <int E, int LVL>
__device__ __forceinline__ void tree_level(const uint64_t* src, uint64_t* dst, uint64_t* other, int K,
                                           int32_t* idx_row, float* score_row, uint64_t* out) {
  constexpr int CH = kWave * E;
  constexpr int LIN = (CH << (LVL - 1)) < kTreeCap ? (CH << (LVL - 1)) : kTreeCap;
  constexpr int SIN = LVL == 1 ? CH : LIN;
  constexpr bool CAPPED = 2 * LIN > kTreeCap;
  constexpr int LOUT = CAPPED ? kTreeCap : 2 * LIN;
  constexpr int W = 1 << LVL;
  constexpr int EB = LOUT / W / kWave;
  static_assert(EB >= 1 && EB * kWave * W == LOUT, "block split");
  const int wv = threadIdx.x / kWave, lane = lane_id();
  const int g = wv / W, j = wv % W;
  uint64_t x[EB];
  wave_merge_block<EB, W, LIN, CAPPED>(src + (2 * g) * SIN, src + (2 * g + 1) * SIN, j, x);
  if constexpr (LVL == 3) {
#pragma unroll
    for (int s = 0; s < EB; ++s) {
      const int i = j * kWave * EB + EB * lane + s;
      if (out) {
        out[i] = x[s];
      } else if (i < K) {
        idx_row[i] = key_index(x[s]);
        if (score_row) score_row[i] = key_score(x[s]);
      }
    }
    if (out) __syncthreads();
  } else {
#pragma unroll
    for (int s = 0; s < EB; ++s) dst[g * LOUT + j * kWave * EB + EB * lane + s] = x[s];
    __syncthreads();
    tree_level<E, LVL + 1>(dst, other, dst, K, idx_row, score_row, out);
  }
}

template <int E>
__device__ __forceinline__ void block_topk_tree(uint64_t* buf, uint64_t* alt, int m, int K, int32_t* idx_row,
                                                float* score_row, uint64_t* out) {
  static_assert(kSelThreads == 8 * kWave, "eight wavefronts");
  constexpr int CH = kWave * E;
  const int wv = threadIdx.x / kWave, lane = lane_id();
  uint64_t x[E];
#pragma unroll
  for (int s = 0; s < E; ++s) {
    const int i = wv * CH + E * lane + s;
    x[s] = i < m ? buf[i] : 0ull;
  }
  wave_sort_reg<E>(x, lane);
  // each wavefront rewrites only the chunk it read itself
#pragma unroll
  for (int s = 0; s < E; ++s) buf[wv * CH + E * lane + s] = x[s];
  __syncthreads();
  tree_level<E, 1>(buf, alt, buf, K, idx_row, score_row, out);
}

// Dispatch on m (block-uniform): the smallest chunk that holds m / 8.
__device__ __forceinline__ void block_topk_tree_any(uint64_t* buf, uint64_t* alt, int m, int K, int32_t* idx_row,
                                                    float* score_row, uint64_t* out = nullptr) {
  if (m <= 8 * 128) block_topk_tree<2>(buf, alt, m, K, idx_row, score_row, out);
  else if (m <= 8 * 256) block_topk_tree<4>(buf, alt, m, K, idx_row, score_row, out);
  else block_topk_tree<8>(buf, alt, m, K, idx_row, score_row, out);
}

// ------------------------------------------------------------ one bucket pass
// Block-wide top-K by one bucket pass (workgroups of kSelThreads threads).
// The K best of the keys held in registers, R per thread (key i is
// x[i / kSelThreads] of thread i % kSelThreads; 0 = empty), sorted
// descending into the output row (idx_row / score_row, padded with -1 / -inf
// up to K) and, if best is given, into best[0..npad) padded with 0.
// The bucket of a key is floor((v - vmin) * 2048 / (vmax - vmin)), clamped
// to 2047, over the candidates' score range [vmin, vmax]: each step of that
// (a subtraction of one value, a product with one positive factor, a
// truncation) is monotone in v, so a larger key never lands in a lower
// bucket and equal scores share one.  A block scan over the 2048 bucket
// counts, in descending bucket order, gives each bucket its first output
// position; the keys of every bucket that starts below K are scattered into
// a segment of their own, and a key's place inside its bucket is its rank
// among that segment's keys (full 64-bit comparison: equal scores go by
// index).  Keys placed at K or later are dropped.  No radix passes and no
// sort network: six barriers.  Returns false before writing anything outside
// its scratch (block-uniform) when a bucket holds more than kBlockBucketMax keys
// (many equal or nearly equal scores); the caller then takes the general
// selection.  Scratch: H, S [kBlockBuckets] u32, seg [K + kBlockBucketMax] u64, red
// [5 kSelWaves] u32.
constexpr int kBlockBucketBits = 11;
constexpr int kBlockBuckets = 1 << kBlockBucketBits;
constexpr int kBlockBucketMax = 64;
static_assert(kBlockBuckets == 4 * kSelThreads, "four buckets per thread in the scan");

template <int R>
__device__ __forceinline__ bool block_bucket_topk(const uint64_t (&x)[R], int K, uint64_t* best, int npad, uint32_t* H,
                                                  uint32_t* S, uint64_t* seg, uint32_t* red, int32_t* idx_row,
                                                  float* score_row) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  constexpr int BS = kSelThreads, NW = kSelWaves;
  const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave;
  // 1. smallest and largest score word of the present keys, their count;
  //    the bucket counts cleared
  uint32_t omin = ~0u, omax = 0u, c = 0u;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t h = (uint32_t)(x[r] >> 32);
    omin = (x[r] && h < omin) ? h : omin;
    omax = (x[r] && h > omax) ? h : omax;
    c += x[r] ? 1u : 0u;
  }
  omin = ~wave_max_u32(~omin);
  omax = wave_max_u32(omax);
  c = wave_sum_u32(c);
  if (lane == 0) { red[wv] = omin; red[NW + wv] = omax; red[2 * NW + wv] = c; }
  *reinterpret_cast<u32x4*>(H + 4 * tid) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  omin = ~0u;
  omax = 0u;
  uint32_t n = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    omin = red[w] < omin ? red[w] : omin;
    omax = red[NW + w] > omax ? red[NW + w] : omax;
    n += red[2 * NW + w];
  }
  // scores are finite (-inf keys are never candidates); a range that is 0,
  // infinite, or so small that the factor overflows puts every key in bucket 0
  const float vmin = unord_f32(omin);
  const float range = unord_f32(omax) - vmin;
  float scale = range > 0.f ? (float)kBlockBuckets / range : 0.f;
  scale = (scale < 3.0e38f && range < 3.0e38f) ? scale : 0.f;
  auto digit = [&](uint64_t key) -> uint32_t {
    const uint32_t b = (uint32_t)((unord_f32((uint32_t)(key >> 32)) - vmin) * scale);
    return b < (uint32_t)(kBlockBuckets - 1) ? b : (uint32_t)(kBlockBuckets - 1);
  };
  // 2. bucket counts
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (x[r]) atomicAdd(&H[digit(x[r])], 1u);
  __syncthreads();
  // 3. thread tid owns buckets kBlockBuckets - 1 - 4 tid - e (e < 4): descending digits
  uint32_t hc[4], sum = 0u, mx = 0u;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hc[e] = H[kBlockBuckets - 1 - 4 * tid - e];
    sum += hc[e];
    mx = hc[e] > mx ? hc[e] : mx;
  }
  const uint32_t incl = wave_incl_scan_u32(sum);
  mx = wave_max_u32(mx);
  if (lane == kWave - 1) red[3 * NW + wv] = incl;
  if (lane == 0) red[4 * NW + wv] = mx;
  __syncthreads();
  uint32_t base = 0u, maxc = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    base += w < wv ? red[3 * NW + w] : 0u;
    maxc = red[4 * NW + w] > maxc ? red[4 * NW + w] : maxc;
  }
  if (maxc > (uint32_t)kBlockBucketMax) return false;
  uint32_t o = base + incl - sum;
  uint32_t used = 0u;  // end of the segments: the last bucket that starts below K ends there
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int b = kBlockBuckets - 1 - 4 * tid - e;
    S[b] = o;  // first position of the bucket
    H[b] = o;  // its fill cursor
    used = o < (uint32_t)K && o + hc[e] > used ? o + hc[e] : used;
    o += hc[e];
  }
  used = wave_max_u32(used);
  if (lane == 0) red[wv] = used;  // (slots 0 .. NW - 1 were last read before the previous barrier)
  __syncthreads();
  used = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) used = red[w] > used ? red[w] : used;
  // 4. the keys of the buckets that start below K, each bucket into its
  //    segment (slots < K + kBlockBucketMax)
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (x[r]) {
      const uint32_t d = digit(x[r]);
      if (S[d] < (uint32_t)K) seg[atomicAdd(&H[d], 1u)] = x[r];
    }
  }
  __syncthreads();
  // 5. a key's place is its bucket's start plus its rank inside the bucket.
  //    The threads walk the filled segment slots [0, used) (the keys that
  //    can be placed below K, about one per thread); the first 8 entries of a
  //    key's segment are read at once (entries past its end are ignored, and
  //    every read stays inside seg's K + kBlockBucketMax + 8 entries).  The placed
  //    keys go to best and straight to the output row as well.
  for (uint32_t i = (uint32_t)tid; i < used; i += BS) {
    const uint64_t key = seg[i];
    const uint32_t d = digit(key);
    const uint32_t st = S[d], en = H[d];
    uint64_t sv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) sv[j] = seg[st + j];
    uint32_t pos = st;
#pragma unroll
    for (int j = 0; j < 8; ++j) pos += (st + j < en && sv[j] > key) ? 1u : 0u;
    for (uint32_t j = st + 8; j < en; ++j) pos += seg[j] > key ? 1u : 0u;
    if (pos < (uint32_t)K) {
      if (best) best[pos] = key;
      idx_row[pos] = key_index(key);
      if (score_row) score_row[pos] = key_score(key);
    }
  }
  const int nsel = n < (uint32_t)K ? (int)n : K;
  for (int i = nsel + tid; i < (best && npad > K ? npad : K); i += BS) {
    if (best) best[i] = 0ull;
    if (i < K) {
      idx_row[i] = -1;
      if (score_row) score_row[i] = -__builtin_inff();
    }
  }
  __syncthreads();
  return true;
}

}  // namespace lid
