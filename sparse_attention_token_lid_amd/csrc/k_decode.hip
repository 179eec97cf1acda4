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
constexpr int kRingDepth = LID_DECODE_DEPTH;  // key blocks per wave in registers (1 scored + the rest loading)
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
// Forms of the per-query finish (chosen by the host, see lid_api.hip).
constexpr int kFormLists = 0;  // every split writes its sorted k_top best; the last merges them
constexpr int kFormRaw = 1;    // every split writes raw ordered scores; the last selects from all
constexpr int kFormTops = 2;   // every split writes its sorted 16 best; the last merges them and
                               // re-scores a split only when its summary is too short
constexpr int kFormTops8 = 3;  // the same with summaries of 8 keys (twice as many splits)
template <int FORM> constexpr int tops_c() { return FORM == kFormTops8 ? 8 : 16; }  // keys per summary
static_assert(NW * 16 == 2 * kWave && NW * 8 == kWave, "a split summary combines two or one keys per lane");
constexpr int kTopsArrMin = NW * kWave;  // summaries + wavefront buffers (C + (64 - C) per wavefront)

// LDS of the tops form.  The stage region (scoring) also holds the merge
// tree's candidates and its second buffer; `arr` holds the wave summaries and
// the wavefronts' candidate buffers in the scoring pass, and a re-scored
// split in the finish.
struct TopsLds {
  size_t arr, best, sh, red, lastc, flags, ints, total;
};
__host__ __device__ inline TopsLds tops_lds(int keys_per_wg, int P) {  // (either summary size)
  static_assert((size_t)kStageBytes >= (4096 + 2048) * 8, "tree buffers fit the stage region");
  static_assert(2 * kTreeCap + 2 * BS <= 2048, "the block sort's keys and scratch fit the second buffer");
  TopsLds L;
  size_t o = kStageBytes;
  L.arr = o;
  o += (size_t)(keys_per_wg > kTopsArrMin ? keys_per_wg : kTopsArrMin) * 8;
  L.best = o;
  o += (size_t)kTreeCap * 8;
  L.sh = o;
  o += (sizeof(BlockShared) + 15) & ~(size_t)15;
  L.red = o;
  o += (size_t)(4 * NW + 8) * 4;
  o = (o + 7) & ~(size_t)7;
  L.lastc = o;
  o += (size_t)P * 8;
  L.flags = o;
  o += (size_t)P;
  o = (o + 15) & ~(size_t)15;
  L.ints = o;
  o += 32;
  L.total = o;
  return L;
}

// A wavefront's running best kTopsC keys while it streams: the kept keys
// (lanes 0 .. kTopsC-1 of `top`, descending, 0 = empty), their smallest
// (th), and a buffer of up to kTopsBuf candidates above th in LDS.  A block's
// keys (in lanes 32..63; lanes 0..31 hold the same keys) that beat th are
// appended to the buffer; when it would overflow, the kept keys and the
// buffer are sorted in registers (one key per lane) and the best kTopsC kept,
// which raises th.  On random data a wavefront sorts a few times per split.
struct TopsState {
  uint64_t top;    // lanes 0 .. kTopsC-1
  uint64_t th;     // wave-uniform: the kTopsC-th kept key (0 while fewer are kept)
  int nbuf;        // wave-uniform
  uint64_t* buf;   // [kTopsBuf] this wavefront's LDS buffer
};
template <int kTopsC>
__device__ __forceinline__ void tops_flush(TopsState& st, int lane) {
  __builtin_amdgcn_wave_barrier();
  uint64_t x[1] = {lane < kTopsC ? st.top : (lane - kTopsC < st.nbuf ? st.buf[lane - kTopsC] : 0ull)};
  wave_sort_reg<1>(x, lane);
  st.top = x[0];
  st.nbuf = 0;
  const uint32_t thi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x[0] >> 32), kTopsC - 1);
  const uint32_t tlo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x[0], kTopsC - 1);
  st.th = ((uint64_t)thi << 32) | tlo;
  __builtin_amdgcn_wave_barrier();
}
template <int kTopsC>
__device__ __forceinline__ void tops_insert(TopsState& st, uint64_t key, int lane) {
  constexpr int kTopsBuf = kWave - kTopsC;  // candidate slots per wavefront
  bool c = lane >= 32 && key > st.th;
  uint64_t mk = ballot(c);
  if (mk == 0ull) return;
  int n = __popcll(mk);
  if (st.nbuf + n > kTopsBuf) {
    tops_flush<kTopsC>(st, lane);
    c = lane >= 32 && key > st.th;
    mk = ballot(c);
    if (mk == 0ull) return;
    n = __popcll(mk);
  }
  if (c) st.buf[st.nbuf + mbcnt(mk)] = key;
  st.nbuf += n;
}

// ------------------------------------------ summary finish: one bucket pass
// (block_bucket_topk of lid_select.h)
static_assert(BS == kSelThreads && NW == kSelWaves, "the block bucket pass runs on this workgroup shape");

template <int DT, int FORM>
__global__ __launch_bounds__(BS, 1) void decode_kernel(KArgs a, int keys_per_wg, int ch) {
  constexpr bool TOPS = FORM == kFormTops || FORM == kFormTops8;
  constexpr int kTopsC = tops_c<FORM>();
  constexpr int kTopsBuf = kWave - kTopsC;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* stage_all = reinterpret_cast<uint16_t*>(smem);           // [NW][KB * D]
  uint64_t* arr = reinterpret_cast<uint64_t*>(smem + kStageBytes);   // [keys_per_wg] (lists form)
  uint64_t* sel = arr + keys_per_wg;                                 // [next_pow2(K)]
  uint64_t* tmp = sel + next_pow2(a.K);                              // [2 * BS]
  BlockShared* sh = reinterpret_cast<BlockShared*>(tmp + 2 * BS);
  uint32_t* s_last = reinterpret_cast<uint32_t*>(sh + 1);
  // next 32-key block of the current range for the wavefront that asks first
  int* s_next = TOPS ? reinterpret_cast<int*>(smem + tops_lds(keys_per_wg, a.P).ints + 24)
                                  : reinterpret_cast<int*>(s_last + 1);

  const int tid = threadIdx.x;
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

  // Scores the 32-key blocks [rb0, rb1) of this query's range: wavefront wv
  // takes blocks rb0 + wv, rb0 + wv + NW, ...  For every block, every lane
  // calls sink(b, s, v) with the masked score v of key s = lo + 32 b + lane %
  // 32 (both halves of the wavefront hold the same 32 scores; s may be past
  // hi for the padded tail of the range).  DEPTH: key blocks per wavefront
  // in registers (one scored, the others loading).
  auto score_range = [&](auto depth, int64_t rb0, int64_t rb1, auto&& sink) {
    constexpr int kDepth = decltype(depth)::value;
    // the query row, opaque per call: keeps the q and w loads (96 registers)
    // inside the call instead of live across a caller's loop
    int64_t tq = t;
    asm volatile("" : "+s"(tq));
    // The key rows and mask entries of blocks [rb0, rb1) are read through
    // buffer resources based at the first row: the hardware returns 0 for
    // bytes past the range end (the tail of the last block, and the ring's
    // look-ahead past the last block; never kept) without reading memory, so
    // a block needs one 32-bit offset and no clamping, and the loads are
    // unconditional (a load under a branch makes the compiler wait for every
    // load in flight where the paths join).  Offsets stay below 2^22: at most
    // kDecodeMaxKeys + 32 NW (kDepth + 1) rows.  Without a mask the mask buffer
    // is empty: its loads read nothing and give 0.
    const int64_t row0 = lo + rb0 * KB;
    int64_t nrows = (rb1 - rb0) * KB;
    nrows = nrows < hi - row0 ? nrows : hi - row0;
    nrows = nrows > 0 ? nrows : 0;
    constexpr int kRowBytes = DT == 3 ? D : 2 * D;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(reinterpret_cast<const unsigned char*>(a.k) + row0 * kRowBytes), (short)0,
        (int)(nrows * kRowBytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.mask ? a.mask + t * a.mask_ld + row0 : reinterpret_cast<const uint16_t*>(a.w)),
        (short)0, a.mask ? (int)(nrows * 2) : 0, 0x00020000);
    constexpr int kNT = 2;  // non-temporal: the keys are read once
    // Blocks are handed out dynamically: wavefront w starts with block rb0 +
    // w, then takes the next one from the workgroup's LDS counter whenever it
    // loads, so faster wavefronts score more blocks (with a fixed share, the
    // slowest wavefront of the slowest workgroup set the kernel's end, about
    // 9 us after the typical one on the 1M-key decode).  Which wavefront
    // scores a block does not change any result.  Past the range end the
    // counter hands out blocks >= rb1, whose loads read nothing.
    if (threadIdx.x == 0) *s_next = NW;
    __syncthreads();
    auto grab = [&]() -> int64_t {
      int v = 0;
      if (lane == 0) v = __hip_atomic_fetch_add(s_next, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      return rb0 + __builtin_amdgcn_readfirstlane(v);
    };
    auto load_mask = [&](int64_t b) -> uint16_t {
      return __builtin_amdgcn_raw_buffer_load_b16(mrs, (uint32_t)((b - rb0) * KB + m) * 2u, 0, kNT);
    };
    if constexpr (DT != 3) {
      using M = Mfma<DT>;
      using T = typename M::T;
      T A[2][8];
      float wr[2][16];
      {
        const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + tq * H * D;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            A[rb][j] = __builtin_bit_cast(T, *reinterpret_cast<const u32x4*>(qrow + (32 * rb + m) * D + 64 * g + 8 * j));
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) wr[rb][jj] = a.w[tq * H + 32 * rb + 8 * (jj >> 2) + 4 * g + (jj & 3)];
      }

      // Instruction i of a block load reads bytes [1024 i, 1024 i + 1024) of
      // the block: lane l gets row 4 i + l / 16, 16-byte chunk l % 16.
      uint16_t* stage = stage_all + wv * (KB * D);
      auto load_blk = [&](int64_t b, u32x4 (&f)[8]) {
        const uint32_t off = (uint32_t)(b - rb0) * (KB * 2 * D) + (uint32_t)lane * 16u;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          f[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off + 1024u * i, 0, kNT));
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
        sink(b, s, (tot + f16_bits_to_f32(mbits)) + 0.0f);
      };

      // A ring of kDepth register sets: while a block is scored, the loads of
      // the next kDepth - 1 blocks of this wave are in flight.  A slot whose
      // block lies past the range loads from beyond the buffer's range
      // (zeros, no memory access) and is never scored: every load is
      // unconditional.
      const int64_t bs = rb0 + wv;
      if constexpr (kDepth == 1) {
        // no ring: load a block, score it, then take the next
        if (hi > lo) {
          u32x4 f[8];
          for (int64_t b = bs; b < rb1; b = grab()) {
            const uint16_t mb = load_mask(b);
            load_blk(b, f);
            score_blk(b, f, mb);
          }
        }
      } else if (hi > lo && bs < rb1) {
        static_assert(kDepth >= 2, "ring depth");
        u32x4 f[kDepth][8];
        uint16_t mk[kDepth];
        int64_t bid[kDepth];
#pragma unroll
        for (int d = 0; d < kDepth - 1; ++d) {
          bid[d] = d == 0 ? bs : grab();
          mk[d] = load_mask(bid[d]);
          load_blk(bid[d], f[d]);
        }
        for (bool more = true; more;) {
#pragma unroll
          for (int d = 0; d < kDepth; ++d) {
            if (bid[d] >= rb1) { more = false; break; }  // slot d holds the block scored now
            const int dl = (d + kDepth - 1) % kDepth;  // the slot freed last: load the next block
            bid[dl] = grab();
            mk[dl] = load_mask(bid[dl]);
            load_blk(bid[dl], f[dl]);
            score_blk(bid[d], f[d], mk[d]);
          }
        }
      }
    } else {
      // FP8 E4M3 q and k with per-row scales (q_scale [n_tok, H], k_scale
      // [n_kv], positive): S[h,s] = q_scale[t,h] k_scale[s] (q8 . k8), and
      // since the scales are positive, I = k_scale[s] sum_h (w[t,h]
      // q_scale[t,h]) relu(q8 . k8).  The MFMA k-index maps to the head
      // dimension as d = 64 (lane / 32) + 32 j + i (j the instruction, i < 32
      // the byte).  Key rows are 128 bytes: a 32-key block is 4 KiB; the q
      // fragments stay in registers and the ring holds up to four blocks.
      using M = Mfma<3>;
      M::T A[2][2];
      float wr[2][16];
      {
        const unsigned char* qrow = reinterpret_cast<const unsigned char*>(a.q) + tq * H * D;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const unsigned char* pq = qrow + (32 * rb + m) * D + 64 * g + 32 * j;
            const u32x4 lo4 = *reinterpret_cast<const u32x4*>(pq), hi4 = *reinterpret_cast<const u32x4*>(pq + 16);
            A[rb][j] = M::T{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3], (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
          }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) {
            const int h = 32 * rb + 8 * (jj >> 2) + 4 * g + (jj & 3);
            wr[rb][jj] = a.w[tq * H + h] * a.q_scale[tq * H + h];
          }
      }
      constexpr int kRow8 = D;                  // bytes per key row
      constexpr int kDepth8 = 2 * (kDepth < 2 ? kDepth : 2);  // (q stays in registers here)
      unsigned char* stage8 = reinterpret_cast<unsigned char*>(stage_all) + wv * (KB * kRow8);
      // LDS: 16-byte chunk c of row r at r * 128 + ((c ^ (r & 7)) << 4)
      auto swz8 = [](int r, int c) { return r * kRow8 + ((c ^ (r & 7)) << 4); };
      // instruction i of a block load: lane l reads row 8 i + l / 8, chunk l % 8
      auto load_blk8 = [&](int64_t b, u32x4 (&f)[4]) {
        const uint32_t off = (uint32_t)(b - rb0) * (KB * kRow8) + (uint32_t)lane * 16u;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          f[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off + 1024u * i, 0, kNT));
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
        sink(b, s, (tot * ks + f16_bits_to_f32(mbits)) + 0.0f);
      };
      const int64_t bs = rb0 + wv;
      if (hi > lo && bs < rb1) {
        u32x4 f[kDepth8][4];
        uint16_t mk[kDepth8];
        int64_t bid[kDepth8];
#pragma unroll
        for (int d = 0; d < kDepth8 - 1; ++d) {
          bid[d] = d == 0 ? bs : grab();
          mk[d] = load_mask(bid[d]);
          load_blk8(bid[d], f[d]);
        }
        for (bool more = true; more;) {
#pragma unroll
          for (int d = 0; d < kDepth8; ++d) {
            if (bid[d] >= rb1) { more = false; break; }
            const int dl = (d + kDepth8 - 1) % kDepth8;
            bid[dl] = grab();
            mk[dl] = load_mask(bid[dl]);
            load_blk8(bid[dl], f[dl]);
            score_blk8(bid[d], f[d], mk[d]);
          }
        }
      }
    }
  };
  auto valid_key = [&](int64_t s, float v) -> uint64_t {
    return (s < hi && v != -__builtin_inff()) ? make_key(v, (uint32_t)s) : 0ull;
  };

  if constexpr (FORM == kFormRaw) {
    uint32_t* raw = a.raw + (size_t)t * a.raw_ld;
    score_range(std::integral_constant<int, kRingDepth>{}, b0, b1, [&](int64_t b, int64_t s, float v) {
      if (g == 0)
        __hip_atomic_store(&raw[b * KB + m], (s < hi && v != -__builtin_inff()) ? ord_f32(v) : 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    });
  } else if constexpr (FORM == kFormLists) {
    score_range(std::integral_constant<int, kRingDepth>{}, b0, b1, [&](int64_t b, int64_t s, float v) {
      if (g == 0) arr[(b - b0) * KB + m] = valid_key(s, v);
    });
  } else {
    // every wavefront keeps its best kTopsC keys while it streams; the
    // workgroup's summary is the best kTopsC of the wavefronts' ones
    const TopsLds L = tops_lds(keys_per_wg, P);
    uint64_t* tw = reinterpret_cast<uint64_t*>(smem + L.arr);  // [NW][kTopsC], then [NW][kTopsBuf]
    TopsState st{0ull, 0ull, 0, tw + NW * kTopsC + wv * kTopsBuf};
    score_range(std::integral_constant<int, kRingDepth>{}, b0, b1,
                [&](int64_t b, int64_t s, float v) { tops_insert<kTopsC>(st, valid_key(s, v), lane); });
    if (st.nbuf) tops_flush<kTopsC>(st, lane);
    if (lane < kTopsC) tw[wv * kTopsC + lane] = st.top;
    __syncthreads();
    if (wv == 0) {
      uint64_t* out = a.lists + ((size_t)t * P + p) * kTopsC;
      if constexpr (NW * kTopsC == 2 * kWave) {
        uint64_t x[2] = {tw[2 * lane], tw[2 * lane + 1]};
        wave_sort_reg<2>(x, lane);
        if (lane < kTopsC / 2) {
          __hip_atomic_store(&out[2 * lane], x[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(&out[2 * lane + 1], x[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      } else {
        uint64_t x[1] = {tw[lane]};
        wave_sort_reg<1>(x, lane);
        if (lane < kTopsC) __hip_atomic_store(&out[lane], x[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  __syncthreads();

  if constexpr (FORM == kFormLists) {
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
  uint32_t* s_flag = s_last;
  if constexpr (TOPS) s_flag = reinterpret_cast<uint32_t*>(smem + tops_lds(keys_per_wg, P).ints);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    s_flag[0] = __builtin_amdgcn_atomic_inc32(a.counters + t, (unsigned)(P - 1), __ATOMIC_RELAXED, "agent") ==
                        (unsigned)(P - 1) ? 1u : 0u;
  __syncthreads();
  if (!s_flag[0]) return;
  if constexpr (FORM == kFormRaw) {
    select_raw(a, t, (int)(nblk * KB), lo, smem);
  } else if constexpr (FORM == kFormLists) {
    finish_lists(a, ch, t, smem);
  } else {
    // The K best of the query from the P summaries (each the sorted kTopsC
    // best keys of one split).  The K best candidates, sorted (radix cut and
    // block sort, or the merge tree for at most 1024), have a K-th key tau
    // that bounds the answer from below.  A split whose kTopsC-th key is
    // above tau may hold further keys above tau: the one with the highest
    // such key is scored again into LDS, its K best replace its summary
    // among the candidates, and the selection runs again, until no summary
    // is cut short above tau (every key of the answer is then a candidate).
    // Each split is re-scored at most once.
    const int K = a.K;
    const TopsLds L = tops_lds(keys_per_wg, P);
    uint64_t* cand = reinterpret_cast<uint64_t*>(smem);               // [4096] (stage region)
    uint64_t* alt = cand + 4096;                                       // [2048]
    uint64_t* ex = reinterpret_cast<uint64_t*>(smem + L.arr);          // [keys_per_wg] a re-scored split
    uint64_t* best = reinterpret_cast<uint64_t*>(smem + L.best);       // [kTreeCap]
    BlockShared* shs = reinterpret_cast<BlockShared*>(smem + L.sh);
    uint32_t* red = reinterpret_cast<uint32_t*>(smem + L.red);
    uint64_t* lastc = reinterpret_cast<uint64_t*>(smem + L.lastc);     // [P] kTopsC-th key per summary
    uint8_t* done = smem + L.flags;                                    // [P] split re-scored
    unsigned long long* s_emax = reinterpret_cast<unsigned long long*>(smem + L.ints + 8);
    int* s_pick = reinterpret_cast<int*>(smem + L.ints + 16);
    const uint64_t* sums = a.lists + (size_t)t * P * kTopsC;
    const int m0 = P * kTopsC;  // <= 4096 (host-checked)
    // the candidates, in registers (for the bucket pass) and in LDS
    // First round: the bucket pass over the candidates in registers (the
    // stage region past the candidates and the merge tree's buffer holds its
    // two bucket arrays), unless a bucket is too full; then, and after a
    // re-scored split, the radix select and sort or the merge tree.
    uint32_t* bH = reinterpret_cast<uint32_t*>(smem + 6144 * 8);
    uint32_t* bS = bH + kBlockBuckets;
    static_assert(6144 * 8 + 2 * kBlockBuckets * 4 <= kStageBytes, "bucket arrays fit the stage region");
    static_assert(kTreeCap + kBlockBucketMax + 8 <= 2048, "the bucket segments fit the merge tree's buffer");
    auto load_and_bucket = [&](auto rr) -> bool {
      constexpr int R = decltype(rr)::value;
      // every load is issued before any value is used (clamped index; the
      // entries past m0 are replaced by 0 afterwards), so the R round trips
      // overlap instead of following one another
      uint64_t xk[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int i = r * BS + tid;
        xk[r] = __hip_atomic_load(&sums[i < m0 ? i : 0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int i = r * BS + tid;
        xk[r] = i < m0 ? xk[r] : 0ull;
        if (i < m0) {
          cand[i] = xk[r];
          if (i % kTopsC == kTopsC - 1) lastc[i / kTopsC] = xk[r];
        }
      }
      for (int i = tid; i < P; i += BS) done[i] = 0;
      if (tid == 0) *s_emax = 0ull;
      __syncthreads();
      return block_bucket_topk<R>(xk, K, best, kTreeCap, bH, bS, alt, red, a.idx + t * K, a.score ? a.score + t * K : nullptr);
    };
    bool have_best = m0 <= 4 * BS ? load_and_bucket(std::integral_constant<int, 4>{})
                                  : load_and_bucket(std::integral_constant<int, 4096 / BS>{});
    bool row_written = have_best;  // the bucket pass wrote the output row as well
    int mc = m0;
    for (;;) {
      if (have_best) {
        have_best = false;
      } else if (mc > 2 * kTreeCap) {
        // more than 1024 candidates: a register radix select cuts them to the K
        // best, which one key per thread then sorts (block bitonic sort, six
        // LDS stages for 512 keys); measured faster than the merge tree there
        uint64_t* selk = alt;                 // [kTreeCap]
        uint64_t* tmps = alt + 2 * kTreeCap;  // [2 BS]
        const int ns = block_select_compact_any(cand, mc, K, selk, nullptr, shs, red);  // registers sized to mc
        for (int i = ns + tid; i < kTreeCap; i += BS) selk[i] = 0ull;
        __syncthreads();
        block_sort_desc(selk, kTreeCap, tmps);
        for (int i = tid; i < kTreeCap; i += BS) best[i] = selk[i];
        __syncthreads();
      } else {
        block_topk_tree_any(cand, alt, mc, K, nullptr, nullptr, best);
      }
      const uint64_t tau = best[K - 1];
      uint64_t e = 0ull;
      for (int i = tid; i < P; i += BS)
        if (!done[i] && lastc[i] > tau && lastc[i] > e) e = lastc[i];
      e = wave_reduce_u64(e, [](uint64_t x, uint64_t y) { return x > y ? x : y; });
      if (lane == 0 && e) atomicMax(s_emax, (unsigned long long)e);
      __syncthreads();
      const uint64_t emax = *s_emax;
      if (emax == 0ull) break;
      for (int i = tid; i < P; i += BS)
        if (!done[i] && lastc[i] == emax) *s_pick = i;
      __syncthreads();
      const int pe = *s_pick;
      if (tid == 0) { done[pe] = 1; *s_emax = 0ull; }
      row_written = false;
      const int64_t eb0 = nblk * pe / P, eb1 = nblk * (pe + 1) / P;
      const int64_t slo = lo + eb0 * KB, shi = lo + eb1 * KB;  // the split's keys
      score_range(std::integral_constant<int, 1>{}, eb0, eb1, [&](int64_t b, int64_t s, float v) {
        if (g == 0) ex[(b - eb0) * KB + m] = valid_key(s, v);
      });
      __syncthreads();
      // the other splits' keys among the K best, then the split's own K best
      const uint64_t bk = tid < K ? best[tid] : 0ull;
      const int64_t bs = (int64_t)key_index(bk);
      const bool keep = bk != 0ull && (bs < slo || bs >= shi);
      int nb;
      const int pos = block_excl_scan(keep ? 1 : 0, &nb, *shs);
      if (keep) cand[pos] = bk;
      const int ns = block_select_compact_any(ex, (int)((eb1 - eb0) * KB), K, cand + nb, nullptr, shs, red);
      mc = nb + ns;
    }
    if (!row_written) {
      for (int i = tid; i < K; i += BS) {
        a.idx[t * K + i] = key_index(best[i]);
        if (a.score) a.score[t * K + i] = key_score(best[i]);
      }
    }
  }
}

template <int DT, int FORM>
hipError_t launch_one(const KArgs& a, int keys_per_wg, int ch, hipStream_t st) {
  hipError_t e = set_lds_limit(reinterpret_cast<const void*>(&decode_kernel<DT, FORM>), 160 * 1024);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)(a.n_tok * a.P));
  hipLaunchKernelGGL((decode_kernel<DT, FORM>), grid, dim3(BS), decode_lds_bytes(keys_per_wg, a.K, a.P, ch, FORM), st,
                     a, keys_per_wg, ch);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const KArgs& a, int keys_per_wg, int ch, int form, hipStream_t st) {
  if (form == kFormRaw) return launch_one<DT, kFormRaw>(a, keys_per_wg, ch, st);
  if (form == kFormTops) return launch_one<DT, kFormTops>(a, keys_per_wg, ch, st);
  if (form == kFormTops8) return launch_one<DT, kFormTops8>(a, keys_per_wg, ch, st);
  return launch_one<DT, kFormLists>(a, keys_per_wg, ch, st);
}

}  // namespace

size_t decode_lds_bytes(int keys_per_wg, int K, int P, int ch, int form) {
  if (form == kFormTops || form == kFormTops8) return tops_lds(keys_per_wg, P).total;
  const bool raw = form == kFormRaw;
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

hipError_t launch_decode(const KArgs& a, int keys_per_wg, int ch, int form, hipStream_t st) {
  if (a.dtype == 1) return launch_dt<1>(a, keys_per_wg, ch, form, st);
  if (a.dtype == 3) return launch_dt<3>(a, keys_per_wg, ch, form, st);
  return launch_dt<2>(a, keys_per_wg, ch, form, st);
}

}  // namespace lid
