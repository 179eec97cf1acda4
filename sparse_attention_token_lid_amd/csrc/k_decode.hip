// k_decode.hip -- the few-query (decode) shape: one or a few query tokens
// against a long key range, H = 64 heads, D = 128, in one kernel launch.
//
// Scoring is the same fused chain as the prefill kernel (per-head q.k, ReLU,
// head weight, head sum, f16 mask; ggml-org llama.cpp issue 25468, "Root
// cause" comment), but the parallelism comes from the keys: the visible range
// of each query is cut into P contiguous splits, one workgroup per
// (query, split).  Each wavefront streams its own 32-key blocks (8 KiB): the
// loads are fully coalesced (64 lanes x 16 B = 1 KiB of consecutive bytes per
// instruction), land in registers while the previous block is scored, and go
// through a private LDS slot (XOR-swizzled) that turns them into the MFMA
// B-operand layout.
//
// The per-query top-k is finished by whichever workgroup of the query ends
// last (a device-scope counter in the workspace, incremented with a wrapping
// atomicInc, so it is back at zero after every launch).  Two forms:
//  * raw (the query's range fits kRawMax positions): every workgroup writes
//    its 32-bit ordered scores to the workspace and the last one selects the
//    k_top best of all of them from registers: a lower bound of the k_top-th
//    score (from the per-thread top two; 11-bit radix digit passes with
//    per-wavefront LDS histograms when that bound is too loose) cuts them to
//    at most a few thousand candidates, which the merge tree of lid_select.h
//    selects and sorts exactly;
//  * lists: every workgroup selects the k_top best of its split (register
//    radix select + bitonic sort) and writes them as a sorted list; the last
//    one finishes from the P lists (lid_merge.h).
#include "lid_device.h"
#include "lid_kernels.h"
#include "lid_merge.h"
#include "lid_select.h"

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
// OCP FP8 E4M3 in both operands, K = 64 per instruction (format codes 0, 0;
// no block scales)
typedef int i32x8 __attribute__((ext_vector_type(8)));
template <> struct Mfma<3> {
  typedef i32x8 T;
  static __device__ __forceinline__ f32x16 run(T a, T b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
};

constexpr int H = kMfmaHeads;
constexpr int D = kMfmaDim;
constexpr int NW = 8;     // wavefronts per workgroup
constexpr int BS = NW * kWave;
constexpr int KB = 32;    // keys per MFMA column block
constexpr int kBlockBytes = KB * D * 2;          // 8 KiB per wavefront slot
constexpr int kStageBytes = NW * kBlockBytes;    // 64 KiB
static_assert(BS == kMergeThreads && BS == kSelThreads, "the last workgroup runs the merge");
static_assert(kRawMax == BS * 64, "raw selection holds 64 positions per thread");

constexpr int kRows = kRawMax / BS;   // positions per thread in the raw selection
constexpr int kDigitBits = 11;        // radix digit of the raw selection
constexpr int kBins = 1 << kDigitBits;
constexpr int kCandMax = 4096;        // candidates gathered into LDS for the exact select
#ifndef LID_DECODE_DEPTH
#define LID_DECODE_DEPTH 2
#endif
constexpr int kDepth = LID_DECODE_DEPTH;  // key blocks per wave in registers (1 scored + kDepth - 1 loading)
static_assert(kCandMax == 8 * kTreeCap, "the merge tree takes up to 8 chunks of kTreeCap candidates");

__device__ __forceinline__ int swz(int row, int ch) { return row * D + ((ch ^ (row & 15)) << 3); }

// ----------------------------------------------------------------- raw select
// Block-wide reductions over one value per thread.
__device__ inline uint32_t block_sum_u32(uint32_t x, uint32_t* red) {
  const int lane = lane_id(), wv = threadIdx.x / kWave;
  x = wave_sum_u32(x);
  if (lane == 0) red[wv] = x;
  __syncthreads();
  uint32_t s = 0;
#pragma unroll
  for (int w2 = 0; w2 < NW; ++w2) s += red[w2];
  __syncthreads();
  return s;
}
__device__ inline uint32_t block_and_u32(uint32_t x, uint32_t* red) {
  const int lane = lane_id(), wv = threadIdx.x / kWave;
  x = wave_and_u32(x);
  if (lane == 0) red[wv] = x;
  __syncthreads();
  uint32_t s = ~0u;
#pragma unroll
  for (int w2 = 0; w2 < NW; ++w2) s &= red[w2];
  __syncthreads();
  return s;
}
__device__ inline uint32_t block_or_u32(uint32_t x, uint32_t* red) {
  const int lane = lane_id(), wv = threadIdx.x / kWave;
  x = wave_or_u32(x);
  if (lane == 0) red[wv] = x;
  __syncthreads();
  uint32_t s = 0;
#pragma unroll
  for (int w2 = 0; w2 < NW; ++w2) s |= red[w2];
  __syncthreads();
  return s;
}

// Position of slot r of this thread in the raw row: 16-byte loads, thread
// tid reading positions 2048 i + 4 tid + e for slot r = 4 i + e.
__device__ __forceinline__ int raw_pos(int r, int tid) { return (r >> 2) * (4 * BS) + 4 * tid + (r & 3); }

// The k_top best of the query's n ordered scores a.raw[row t][0..n) (0 = no
// key there; position p is key lo + p), sorted, written as the output row.
// A lower bound of the k_top-th score cuts the n values down to at most
// kCandMax candidates (v >= thr, which hold the k_top best), which are
// gathered as 64-bit keys (score, index) and selected exactly (the merge
// tree when next_pow2(k_top) == 512).  The bound comes from the per-thread
// top two values; when it leaves too many candidates, 11-bit radix digit
// passes over the score word with per-wavefront LDS histograms find one.  If
// a single score value is shared by more than kCandMax positions at the
// threshold, the tied positions are taken in index order instead.
__device__ __forceinline__ void select_raw(const KArgs& a, int64_t t, int n, int64_t lo, unsigned char* smem) {
  const int tid = threadIdx.x, wv = tid / kWave;
  const int K = a.K, n2 = next_pow2(K);
  uint32_t* hw = reinterpret_cast<uint32_t*>(smem);                    // [NW][kBins]
  uint64_t* cand = reinterpret_cast<uint64_t*>(hw + NW * kBins);        // [kCandMax]
  uint64_t* sel = cand + kCandMax;                                      // [n2]
  uint64_t* tmp = sel + n2;                                             // [2 BS]
  BlockShared* sh = reinterpret_cast<BlockShared*>(tmp + 2 * BS);
  uint32_t* red = reinterpret_cast<uint32_t*>(sh + 1);                  // [4 NW + 8]

  // agent-coherent (sc1) 16-byte loads; positions >= n read as 0 (the buffer
  // resource ends there)
  const uint32_t* row = a.raw + (size_t)t * a.raw_ld;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(row), (short)0, n * 4, 0x00020000);
  uint32_t v[kRows];
#pragma unroll
  for (int i = 0; i < kRows / 4; ++i) {
    const u32x4 x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (i * 4 * BS + 4 * tid) * 4, 0, 16));
    v[4 * i] = x[0]; v[4 * i + 1] = x[1]; v[4 * i + 2] = x[2]; v[4 * i + 3] = x[3];
  }
  // Each phase below re-derives its per-slot conditions from v; making v
  // opaque between phases keeps the compiler from carrying 64 lane masks
  // (128 scalar registers) from one phase to the next.
  auto opaque = [&]() {
#pragma unroll
    for (int r = 0; r < kRows; ++r) asm volatile("" : "+v"(v[r]));
  };
  opaque();
  uint32_t c = 0, m1 = 0u, m2 = 0u;
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const uint32_t x = v[r];
    c += x < 1u ? x : 1u;  // present (integer min: no lane mask)
    m2 = x > m1 ? m1 : (x > m2 ? x : m2);
    m1 = x > m1 ? x : m1;
  }
  const uint32_t present = block_sum_u32(c, red);

  // Candidates are the values >= thr (thr >= 1, so only present ones); the
  // gather writes them wave by wave: wcount[] holds each wave's count for
  // the threshold in wthr, and the waves' offsets follow from it.
  uint32_t* wcount = red + 4 * NW;  // [NW]
  auto count_waves = [&](uint32_t th) -> uint32_t {  // block total; wcount[] filled
    opaque();
    uint32_t c2 = 0;
#pragma unroll
    for (int r = 0; r < kRows; ++r) c2 += (uint32_t)__popcll(ballot(v[r] >= th));
    if (lane_id() == 0) wcount[wv] = c2;
    __syncthreads();
    uint32_t tot = 0;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) tot += wcount[w2];
    return tot;
  };
  uint32_t thr = 1u;        // candidates: v >= thr
  bool tie_path = false;    // the k_top-th score is shared by too many positions
  bool have_thr = present <= (uint32_t)K;  // then every present value is a candidate
  bool counted = false;     // wcount[] holds the counts for thr
  if (!have_thr) {
    // Lower bound of the k_top-th score: the k_top-th largest of the
    // per-thread top-2 values (k_top of them are >= it, and it is one of the
    // values); it usually leaves a few hundred candidates.
    const uint32_t top2[2] = {m1, m2};
    const uint32_t lb = block_kth_largest_reg<uint32_t, 2>(top2, (uint32_t)K, hw, sh, red);
    if (count_waves(lb) <= (uint32_t)kCandMax) {
      thr = lb;
      have_thr = true;
      counted = true;
    } else {
      __syncthreads();  // wcount[] is read by every wave before it is reused
    }
  }
  if (!have_thr) {
    opaque();
    uint32_t an = ~0u, on = 0u;
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      an &= v[r] ? v[r] : ~0u;
      on |= v[r];
    }
    an = block_and_u32(an, red);
    on = block_or_u32(on, red);
    if (an == on) {
      thr = an;
      tie_path = present > (uint32_t)kCandMax;
    } else {
      // digits below the bits all present values share
      int top = 31 - __builtin_clz(an ^ on);
      uint32_t prefix = top == 31 ? 0u : (an & ~((2u << top) - 1u));
      uint32_t need = (uint32_t)K;
      uint32_t gt = 0;  // values above the current digit bucket
      for (;;) {
        const int nb = top + 1 < kDigitBits ? top + 1 : kDigitBits;
        const int shft = top + 1 - nb;
        const uint32_t dmask = (1u << nb) - 1u;
        const int msh = top + 1;  // bits at and above msh are fixed (== prefix)
        for (int i = tid; i < NW * kBins; i += BS) hw[i] = 0u;
        __syncthreads();
        opaque();
        uint32_t* h = hw + wv * kBins;
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
          const bool in = v[r] != 0u && (msh >= 32 || (v[r] >> msh) == (prefix >> msh));
          if (in) atomicAdd(&h[(v[r] >> shft) & dmask], 1u);
        }
        __syncthreads();
        // bins in descending digit order: thread tid owns digits d0 - j, j < kPer
        constexpr int kPer = kBins / BS;
        const int d0 = (int)dmask - kPer * tid;
        uint32_t cb[kPer];
        uint32_t s4 = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const int d = d0 - j;
          uint32_t x = 0;
          if (d >= 0) {
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) x += hw[w2 * kBins + d];
          }
          cb[j] = x;
          s4 += x;
        }
        int tot;
        const uint32_t excl = (uint32_t)block_excl_scan((int)s4, &tot, *sh);
        if (excl < need && need <= excl + s4) {
          uint32_t above = excl;
#pragma unroll
          for (int j = 0; j < kPer; ++j) {
            if (above + cb[j] >= need) {
              sh->pick_d = (uint32_t)(d0 - j);
              sh->pick_above = above;
              sh->pick_cnt = cb[j];
              break;
            }
            above += cb[j];
          }
        }
        __syncthreads();
        const uint32_t d = sh->pick_d, above = sh->pick_above, dcnt = sh->pick_cnt;
        __syncthreads();
        prefix |= d << shft;
        need -= above;
        gt += above;
        if (gt + dcnt <= (uint32_t)kCandMax) {
          thr = prefix;  // lower bits zero: every value of the bucket and above
          break;
        }
        if (shft == 0) {  // one exact score value, too many positions
          thr = prefix;
          tie_path = true;
          break;
        }
        top = shft - 1;
      }
    }
  }

  // gather the candidates as 64-bit keys (score word, ~index)
  int m = 0;
  if (!tie_path) {
    thr = thr > 1u ? thr : 1u;  // absent positions hold 0 and never qualify
    const uint32_t total = counted ? [&] {
      uint32_t tot = 0;
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) tot += wcount[w2];
      return tot;
    }() : count_waves(thr);
    uint32_t base = 0;  // this wave's offset: the counts of the waves before it
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) base += w2 < wv ? wcount[w2] : 0u;
    base = __builtin_amdgcn_readfirstlane(base);
    opaque();
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const bool c = v[r] >= thr;
      const uint64_t mk = ballot(c);
      if (c) {
        const uint32_t s = (uint32_t)(lo + raw_pos(r, tid));
        cand[base + __builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u))] =
            ((uint64_t)v[r] << 32) | (uint64_t)(~s);
      }
      base += (uint32_t)__popcll(mk);
    }
    m = (int)total;
  } else {
    // everything above thr, then the first `need` positions (in index order)
    // that score exactly thr: the cut position is found by bisection
    auto gather = [&](auto pred, int base) -> int {
      uint64_t bits = 0ull;
#pragma unroll
      for (int r = 0; r < kRows; ++r) bits |= (uint64_t)(pred(r) ? 1u : 0u) << r;
      int total;
      int pos = base + block_excl_scan(__popcll(bits), &total, *sh);
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        if ((bits >> r) & 1ull) {
          const uint32_t s = (uint32_t)(lo + raw_pos(r, tid));
          cand[pos++] = ((uint64_t)v[r] << 32) | (uint64_t)(~s);
        }
      }
      return base + total;
    };
    const int above = gather([&](int r) { return v[r] > thr; }, 0);
    const uint32_t need = (uint32_t)(K - above);
    int x0 = 0, x1 = n;  // smallest x with #{tied positions < x} >= need
    while (x0 < x1) {
      const int mid = (x0 + x1) / 2;
      uint32_t cc = 0;
#pragma unroll
      for (int r = 0; r < kRows; ++r) cc += (v[r] == thr && raw_pos(r, tid) < mid) ? 1u : 0u;
      if (block_sum_u32(cc, red) >= need) x1 = mid;
      else x0 = mid + 1;
    }
    m = gather([&](int r) { return v[r] == thr && raw_pos(r, tid) < x0; }, above);
  }
  __syncthreads();
  if (next_pow2(K) == kTreeCap) {
    // the digit histograms are free now: they hold the merge levels
    block_topk_tree_any(cand, reinterpret_cast<uint64_t*>(hw), m, K, a.idx + t * K, a.score ? a.score + t * K : nullptr);
    return;
  }
  block_select_sorted_reg<kCandMax / BS>(cand, m, K, sel, tmp, hw, sh, red);
  for (int i = tid; i < K; i += BS) {
    a.idx[t * K + i] = key_index(sel[i]);
    if (a.score) a.score[t * K + i] = key_score(sel[i]);
  }
}

// ------------------------------------------------------------------- kernel
template <int DT, bool RAW>
__global__ __launch_bounds__(BS, 1) void decode_kernel(KArgs a, int keys_per_wg, int ch) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* stage_all = reinterpret_cast<uint16_t*>(smem);           // [NW][KB * D]
  uint64_t* arr = reinterpret_cast<uint64_t*>(smem + kStageBytes);   // [keys_per_wg] (lists form)
  uint64_t* sel = arr + keys_per_wg;                                 // [next_pow2(K)]
  uint64_t* tmp = sel + next_pow2(a.K);                              // [2 * BS]
  BlockShared* sh = reinterpret_cast<BlockShared*>(tmp + 2 * BS);
  uint32_t* s_last = reinterpret_cast<uint32_t*>(sh + 1);

  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 5, m = lane & 31;
  const int P = a.P;
  const int p = (int)(blockIdx.x % (unsigned)P);
  const int64_t t = blockIdx.x / (unsigned)P;

  int64_t lo = 0, hi = a.n_kv;
  if (a.kv_range) {
    int64_t l0 = a.kv_range[2 * t], h0 = a.kv_range[2 * t + 1];
    lo = l0 < 0 ? 0 : l0;
    hi = h0 > a.n_kv ? a.n_kv : h0;
    if (hi < lo) hi = lo;
  }
  const int64_t nblk = (hi - lo + KB - 1) / KB;
  const int64_t b0 = nblk * p / P, b1 = nblk * (p + 1) / P;
  const int nkeys = (int)((b1 - b0) * KB);  // <= keys_per_wg (host-checked)

  const int64_t last_row = hi - 1;
  uint32_t* raw = RAW ? a.raw + (size_t)t * a.raw_ld : nullptr;
  auto load_mask = [&](int64_t b) -> uint16_t {
    if (!a.mask) return 0;
    int64_t s = lo + b * KB + m;
    s = s < last_row ? s : last_row;
    return __builtin_nontemporal_load(a.mask + t * a.mask_ld + s);
  };
  // the masked score v of key s (lane m of the block's first half) goes out
  auto emit = [&](int64_t b, int64_t s, float v) {
    if (g == 0) {
      const bool valid = s < hi && v != -__builtin_inff();
      if (RAW) __hip_atomic_store(&raw[b * KB + m], valid ? ord_f32(v) : 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else arr[(b - b0) * KB + m] = valid ? make_key(v, (uint32_t)s) : 0ull;
    }
  };
  // the head reduction of a 32-key block: sum_h w_h relu(acc) over this
  // lane's 32 heads, then the other 32 (the lanes 32 apart)
  auto head_sum = [&](const f32x16& acc0, const f32x16& acc1, const float (&wr)[2][16]) -> float {
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      part = __builtin_fmaf(wr[0][e], relu(acc0[e]), part);
      part = __builtin_fmaf(wr[1][e], relu(acc1[e]), part);
    }
    return part + __uint_as_float(xor_lane_u32<32>(__float_as_uint(part)));
  };

  if constexpr (DT != 3) {
    using M = Mfma<DT>;
    using T = typename M::T;
    T A[2][8];
    float wr[2][16];
    {
      const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + t * H * D;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          A[rb][j] = __builtin_bit_cast(T, *reinterpret_cast<const u32x4*>(qrow + (32 * rb + m) * D + 64 * g + 8 * j));
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) wr[rb][jj] = a.w[t * H + 32 * rb + 8 * (jj >> 2) + 4 * g + (jj & 3)];
    }

    // Key rows past the split (or past n_kv) are clamped to the split's last
    // row and never stored, so every load is unconditional.  Instruction i of a
    // block load reads bytes [1024 i, 1024 i + 1024) of the block: lane l gets
    // row 4 i + l / 16, 16-byte chunk l % 16.
    const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k);
    uint16_t* stage = stage_all + wv * (KB * D);
    auto load_blk = [&](int64_t b, u32x4 (&f)[8]) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int64_t s = lo + b * KB + 4 * i + (lane >> 4);
        s = s < last_row ? s : last_row;
        f[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + s * D + (lane & 15) * 8));
      }
    };
    auto score_blk = [&](int64_t b, const u32x4 (&f)[8], uint16_t mbits) {
      const int64_t s = lo + b * KB + m;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<u32x4*>(stage + swz(4 * i + (lane >> 4), lane & 15)) = f[i];
      f32x16 acc0, acc1;
#pragma unroll
      for (int e = 0; e < 16; ++e) { acc0[e] = 0.f; acc1[e] = 0.f; }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        T bf = __builtin_bit_cast(T, *reinterpret_cast<const u32x4*>(stage + swz(m, 8 * g + j)));
        acc0 = M::run(A[0][j], bf, acc0);
        acc1 = M::run(A[1][j], bf, acc1);
      }
      const float tot = head_sum(acc0, acc1, wr);
      emit(b, s, (tot + f16_bits_to_f32(mbits)) + 0.0f);
    };

    // A ring of kDepth register sets: while a block is scored, the loads of
    // the next kDepth - 1 blocks of this wave are in flight.
    if (hi > lo) {
      u32x4 f[kDepth][8];
      uint16_t mk[kDepth];
      const int64_t bs = b0 + wv;
#pragma unroll
      for (int d = 0; d < kDepth - 1; ++d) {
        const int64_t b = bs + d * NW;
        mk[d] = 0;
        if (b < b1) { mk[d] = load_mask(b); load_blk(b, f[d]); }
      }
      for (int64_t b = bs; b < b1; b += kDepth * NW) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
          const int64_t bc = b + d * NW;  // scored now, from slot d
          if (bc >= b1) break;
          const int64_t bl = bc + (kDepth - 1) * NW;  // loaded now, into the slot freed last
          if (bl < b1) { mk[(d + kDepth - 1) % kDepth] = load_mask(bl); load_blk(bl, f[(d + kDepth - 1) % kDepth]); }
          score_blk(bc, f[d], mk[d]);
        }
      }
    }
  } else {
    // FP8 E4M3 q and k with per-row scales (q_scale [n_tok, H], k_scale
    // [n_kv], positive): S[h,s] = q_scale[t,h] k_scale[s] (q8 . k8), and since
    // the scales are positive, I = k_scale[s] sum_h (w[t,h] q_scale[t,h])
    // relu(q8 . k8).  The MFMA k-index maps to the head dimension as
    // d = 64 (lane / 32) + 32 j + i (j the instruction, i < 32 the byte).
    // Key rows are 128 bytes: a 32-key block is 4 KiB, and the ring holds
    // twice as many blocks, so as many bytes are in flight as for f16.
    using M = Mfma<3>;
    M::T A[2][2];
    float wr[2][16];
    {
      const unsigned char* qrow = reinterpret_cast<const unsigned char*>(a.q) + t * H * D;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const unsigned char* p = qrow + (32 * rb + m) * D + 64 * g + 32 * j;
          const u32x4 lo4 = *reinterpret_cast<const u32x4*>(p), hi4 = *reinterpret_cast<const u32x4*>(p + 16);
          A[rb][j] = M::T{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3], (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
        }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const int h = 32 * rb + 8 * (jj >> 2) + 4 * g + (jj & 3);
          wr[rb][jj] = a.w[t * H + h] * a.q_scale[t * H + h];
        }
    }
    constexpr int kRow8 = D;                  // bytes per key row
    constexpr int kDepth8 = 2 * kDepth;
    const unsigned char* kb8 = reinterpret_cast<const unsigned char*>(a.k);
    unsigned char* stage8 = reinterpret_cast<unsigned char*>(stage_all) + wv * (KB * kRow8);
    // LDS: 16-byte chunk c of row r at r * 128 + ((c ^ (r & 7)) << 4)
    auto swz8 = [](int r, int c) { return r * kRow8 + ((c ^ (r & 7)) << 4); };
    // instruction i of a block load: lane l reads row 8 i + l / 8, chunk l % 8
    auto load_blk8 = [&](int64_t b, u32x4 (&f)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int64_t s = lo + b * KB + 8 * i + (lane >> 3);
        s = s < last_row ? s : last_row;
        f[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb8 + s * kRow8 + (lane & 7) * 16));
      }
    };
    auto score_blk8 = [&](int64_t b, const u32x4 (&f)[4], uint16_t mbits) {
      const int64_t s = lo + b * KB + m;
      const float ks = a.k_scale[s < last_row ? s : last_row];
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(stage8 + swz8(8 * i + (lane >> 3), lane & 7)) = f[i];
      f32x16 acc0, acc1;
#pragma unroll
      for (int e = 0; e < 16; ++e) { acc0[e] = 0.f; acc1[e] = 0.f; }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = 4 * g + 2 * j;
        const u32x4 b0v = *reinterpret_cast<const u32x4*>(stage8 + swz8(m, c));
        const u32x4 b1v = *reinterpret_cast<const u32x4*>(stage8 + swz8(m, c + 1));
        const M::T bf = {(int)b0v[0], (int)b0v[1], (int)b0v[2], (int)b0v[3], (int)b1v[0], (int)b1v[1], (int)b1v[2], (int)b1v[3]};
        acc0 = M::run(A[0][j], bf, acc0);
        acc1 = M::run(A[1][j], bf, acc1);
      }
      const float tot = head_sum(acc0, acc1, wr);
      emit(b, s, (tot * ks + f16_bits_to_f32(mbits)) + 0.0f);
    };
    if (hi > lo) {
      u32x4 f[kDepth8][4];
      uint16_t mk[kDepth8];
      const int64_t bs = b0 + wv;
#pragma unroll
      for (int d = 0; d < kDepth8 - 1; ++d) {
        const int64_t b = bs + d * NW;
        mk[d] = 0;
        if (b < b1) { mk[d] = load_mask(b); load_blk8(b, f[d]); }
      }
      for (int64_t b = bs; b < b1; b += kDepth8 * NW) {
#pragma unroll
        for (int d = 0; d < kDepth8; ++d) {
          const int64_t bc = b + d * NW;
          if (bc >= b1) break;
          const int64_t bl = bc + (kDepth8 - 1) * NW;
          if (bl < b1) { mk[(d + kDepth8 - 1) % kDepth8] = load_mask(bl); load_blk8(bl, f[(d + kDepth8 - 1) % kDepth8]); }
          score_blk8(bc, f[d], mk[d]);
        }
      }
    }
  }
  __syncthreads();

  if (!RAW) {
    // the stage buffers are free now: histograms and reduction slots
    uint32_t* shw = reinterpret_cast<uint32_t*>(smem);
    uint32_t* sred = reinterpret_cast<uint32_t*>(smem + kSelHistBytes);
    if (nkeys <= 8 * BS)
      block_select_sorted_reg<8>(arr, nkeys, a.K, sel, tmp, shw, sh, sred);
    else
      block_select_sorted_reg<kDecodeMaxKeys / BS>(arr, nkeys, a.K, sel, tmp, shw, sh, sred);
    if (P == 1) {  // the only split: its list is the answer
      for (int i = threadIdx.x; i < a.K; i += BS) {
        a.idx[t * a.K + i] = key_index(sel[i]);
        if (a.score) a.score[t * a.K + i] = key_score(sel[i]);
      }
      return;
    }
    uint64_t* out = a.lists + ((size_t)t * P + p) * a.K;
    for (int i = threadIdx.x; i < a.K; i += BS)
      __hip_atomic_store(&out[i], sel[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // Publish this split's part, then let the last workgroup of the query
  // finish.  The parts are written and read with agent-scope atomic stores
  // and loads (coherent across the XCDs' separate L2 caches without writing
  // back or invalidating them, which device-scope fences would do); every
  // store has completed (vmcnt(0)) before the counter moves.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    s_last[0] = __builtin_amdgcn_atomic_inc32(a.counters + t, (unsigned)(P - 1), __ATOMIC_RELAXED, "agent") ==
                        (unsigned)(P - 1) ? 1u : 0u;
  __syncthreads();
  if (!s_last[0]) return;
  if (RAW)
    select_raw(a, t, (int)(nblk * KB), lo, smem);
  else
    finish_lists(a, ch, t, smem);
}

template <int DT, bool RAW>
hipError_t launch_one(const KArgs& a, int keys_per_wg, int ch, hipStream_t st) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<DT, RAW>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid((unsigned)(a.n_tok * a.P));
  hipLaunchKernelGGL((decode_kernel<DT, RAW>), grid, dim3(BS), decode_lds_bytes(keys_per_wg, a.K, a.P, ch, RAW), st,
                     a, keys_per_wg, ch);
  return hipGetLastError();
}

}  // namespace

size_t decode_lds_bytes(int keys_per_wg, int K, int P, int ch, bool raw) {
  const size_t scoring = (size_t)kStageBytes + (size_t)keys_per_wg * 8 + (size_t)next_pow2(K) * 8 + 2 * BS * 8 +
                         sizeof(BlockShared) + 16;
  size_t finish;
  if (raw)
    finish = (size_t)NW * kBins * 4 + (size_t)kCandMax * 8 + (size_t)next_pow2(K) * 8 + 2 * BS * 8 +
             sizeof(BlockShared) + (4 * NW + 8) * 4;
  else
    finish = P > 1 ? finish_lds_need(P, K, ch) : 0;
  return scoring > finish ? scoring : finish;
}

hipError_t launch_decode(const KArgs& a, int keys_per_wg, int ch, bool raw, hipStream_t st) {
  if (a.dtype == 1) return raw ? launch_one<1, true>(a, keys_per_wg, ch, st) : launch_one<1, false>(a, keys_per_wg, ch, st);
  if (a.dtype == 3) return raw ? launch_one<3, true>(a, keys_per_wg, ch, st) : launch_one<3, false>(a, keys_per_wg, ch, st);
  return raw ? launch_one<2, true>(a, keys_per_wg, ch, st) : launch_one<2, false>(a, keys_per_wg, ch, st);
}

}  // namespace lid
