// k_shared.hip -- the shared (per-ubatch) top-k: one selection of k_top keys
// for all the queries of a ubatch, by
//     U[s] = sum_t v[t,s]
// with v the masked score of the per-query op, and -inf when any query of the
// ubatch does not see the key (outside its range, or masked).  ggml-org
// llama.cpp PR 22378, the batched-prefill commit: the indexer's per-query
// scores are summed over the ubatch (and heads) and one ubatch-wide top-k is
// taken; the later commit that reverts collapse-Q writes it as
// top_k(sum_q relu(kv * q) * w).
//
// Two kernels, then (several key chunks) a merge of the sorted lists:
//  * shared_scores_kernel: one workgroup per (group of 512 keys, chunk of
//    queries).  The output is per key, so the keys are the resident operand:
//    each wavefront holds 64 keys (four 16-key blocks) as MFMA B fragments in
//    registers for the whole kernel, and the queries of the chunk stream
//    past them through LDS, four at a time (64 KiB of q rows and their head
//    weights per batch, copied by global_load_lds_dwordx4 into one of two
//    buffers while the other is read; 16-byte chunks XOR-swizzled per row).
//    Per query a wavefront runs 64 v_mfma_f32_16x16x32 (4 key blocks x 4 head
//    blocks x 4 k-steps) with the q fragments in registers; the head
//    reduction sum_h w_h * max(S_h, 0) of a block runs between the MFMAs of
//    the next block, and the next query's fragments are read from LDS behind
//    the last block's MFMAs.  A query's 64 scores (lane l <-> key l after
//    three lane swaps) get the mask and the range test and are added to the
//    lane's running sum, query by query in order; the chunk's sums are
//    written as partial sums [QC, n_kv].  No LDS reduction between
//    wavefronts: each owns its keys.
//  * shared_select_kernel (up to 16384 keys): one workgroup adds the QC
//    partial sums of every key and takes the k_top best by one block bucket
//    pass, straight into the output.
//  * otherwise shared_lists_kernel: one workgroup per 4096 keys: U = the QC partial
//    sums added in chunk order (so the result does not depend on timing),
//    as 64-bit keys (ordered U, ~index; 0 = not selectable); the k_top best
//    are selected and sorted, into the output when one workgroup covers
//    every key, else into a list for the merge.
//  * shared_merge_kernel: the round-based list merge of lid_merge.h (each
//    list here may hold a large share of the answer, so the merge reads
//    about 4 k_top entries in its first round instead of short prefixes).
#include "lid_device.h"
#include "lid_kernels.h"
#include "lid_merge.h"
#include "lid_select.h"

namespace lid {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int DT> struct MfmaS;
template <> struct MfmaS<1> {
  typedef f16x8 T;
  static __device__ __forceinline__ f32x4 run(T a, T b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct MfmaS<2> {
  typedef bf16x8 T;
  static __device__ __forceinline__ f32x4 run(T a, T b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

constexpr int H = kMfmaHeads;
constexpr int D = kMfmaDim;
constexpr int NW = 8;
constexpr int BS = NW * kWave;
constexpr int WK = 64;                      // keys per wavefront
constexpr int KG = kSharedGroupKeys;        // keys per scoring workgroup
constexpr int QB = 4;                       // queries per staged batch
constexpr int kQBytes = H * D * 2;          // one query's q rows (16 KiB)
constexpr int kBufBytes = QB * kQBytes + 1024;  // a batch: q rows, then 4 x 256 B of head weights
constexpr size_t kScoresLds = 2 * (size_t)kBufBytes;
constexpr int kListKeys = kSharedListKeys;
static_assert(KG == NW * WK, "one 64-key slice per wavefront");
static_assert(QB * kQBytes / 1024 % NW == 0, "the q copy divides over the wavefronts");
static_assert(BS == kSelThreads, "the list kernel runs the block selection");
static_assert(kSharedSelectKeys % BS == 0, "whole registers of keys per thread");

template <int DT, bool MK, bool RG>
__global__ __launch_bounds__(BS, 1) void shared_scores_kernel(KArgs a, int qchunk) {
  constexpr bool AB = true;  // the |S| form of the head reduction (below; kept switchable)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  using M = MfmaS<DT>;
  using T = typename M::T;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  const int G = lane >> 4, r16 = lane & 15;
  // (key group, query chunk) pairs numbered so that each XCD (blocks go to
  // the 8 XCDs round-robin) gets a contiguous run: the key groups of one
  // query chunk share an XCD, whose L2 then fetches the chunk's q rows once.
  const int64_t ngroups = (a.n_kv + KG - 1) / KG;
  uint32_t gi;
  {
    const uint32_t T = gridDim.x, x = blockIdx.x % 8u, i = blockIdx.x / 8u;
    const uint32_t Q = T / 8u, Rm = T % 8u;
    gi = x * Q + (x < Rm ? x : Rm) + i;
  }
  const int64_t kg = gi % ngroups, qc = gi / ngroups;
  const int64_t t0 = qc * qchunk;
  const int64_t t1 = t0 + qchunk < a.n_tok ? t0 + qchunk : a.n_tok;
  const int ks0 = (int)(kg * KG) + wv * WK;  // this wavefront's first key (n_kv < 2^31)
  const int n_kv = (int)a.n_kv;

  // The wavefront's 64 keys as B fragments: Bk[b][j] holds key ks0 + 16 b +
  // lane % 16, dims 32 (lane / 16) + 8 j ... + 7 (the k-index mapping of
  // the prefill kernel).  Keys past n_kv are zeros; their sums are not kept.
  T Bk[4][4];
  {
    const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.k);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int s = ks0 + 16 * b + r16;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (s < n_kv) v = *reinterpret_cast<const u32x4*>(kb + (size_t)s * D + 32 * G + 8 * j);
        Bk[b][j] = __builtin_bit_cast(T, v);
      }
    }
  }

  // Running sums over the chunk's queries.  P[b]: key block b's head-reduced
  // score summed over the queries, for this lane's key (16 b + lane % 16) and
  // head group (lane / 16); the four head groups are added once at the end.
  // msum: the mask entries of this lane's key (ks0 + lane), summed.  A -inf
  // mask entry makes the sum -inf, and so U[s] (I is finite).  [L, R): the
  // keys every query of the chunk sees (the intersection of the ranges).
  float P[4] = {0.f, 0.f, 0.f, 0.f};
  float msum = 0.f;
  int L = 0, R = n_kv;
  const int nq = t1 > t0 ? (int)(t1 - t0) : 0;
  if (nq > 0) {
    // Batch copy: 64 instructions of 1 KiB (4 head rows of one query) per
    // batch, 8 per wavefront, plus one for the 4 weight rows (wavefront 0).
    // LDS chunk position p of head row h holds q chunk p ^ (h % 16).  Queries
    // past the chunk copy the chunk's last query (never read).
    const unsigned char* qbytes = reinterpret_cast<const unsigned char*>(a.q);
    const unsigned char* wbytes = reinterpret_cast<const unsigned char*>(a.w);
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    auto stage = [&](int bi, int buf) {
      const int64_t tb = t0 + (int64_t)bi * QB;
      const int last = (int)(t1 - 1 - tb);  // last valid query of the batch, relative
      const uint32_t lb = lds0 + (uint32_t)(buf * kBufBytes);
#pragma unroll
      for (int r = 0; r < QB * kQBytes / 1024 / NW; ++r) {
        const int i = wv * (QB * kQBytes / 1024 / NW) + r;  // 1 KiB piece: query i / 16, head rows 4 (i % 16) ...
        const int qi = i / 16 < last ? i / 16 : last;
        const int h = 4 * (i % 16) + lane / 16;
        const uint32_t off = (uint32_t)(qi * kQBytes + h * 2 * D + (((lane & 15) ^ (h & 15)) << 4));
        dma_row4(qbytes + tb * kQBytes, off, lb + 1024u * (uint32_t)i);
      }
      if (wv == 0) {
        const int qi = lane / 16 < last ? lane / 16 : last;
        dma_row4(wbytes + tb * H * 4, (uint32_t)(qi * H * 4 + (lane & 15) * 16), lb + QB * kQBytes);
      }
    };
    // A fragments of query qi of a buffer: head 16 rb + lane % 16, dims
    // 32 (lane / 16) + 8 j ... + 7; and the weights of the heads this lane's
    // accumulators hold (16 rb + 4 (lane / 16) + e)
    auto afrag = [&](int buf, int qi, int rb, int j) -> T {
      const unsigned char* p = smem + buf * kBufBytes + qi * kQBytes + (16 * rb + r16) * 2 * D + (((4 * G + j) ^ r16) << 4);
      return __builtin_bit_cast(T, *reinterpret_cast<const u32x4*>(p));
    };
    auto wload = [&](int buf, int qi, float (&wq)[4][4]) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(smem + buf * kBufBytes + QB * kQBytes + qi * H * 4 + (16 * rb + 4 * G) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) wq[rb][e] = v[e];
      }
    };
    // the mask entry of query t for this lane's key and the query's range
    // (read a batch ahead, unconditionally: t is clamped into the chunk)
    auto clampq = [&](int64_t t) -> int64_t { return t < t1 ? t : t1 - 1; };
    auto mload = [&](int64_t t) -> uint16_t {
      if (!MK) return 0;
      int s = ks0 + lane;
      s = s < n_kv - 1 ? s : n_kv - 1;
      return __builtin_nontemporal_load(a.mask + t * a.mask_ld + s);
    };
    auto rload = [&](int64_t t, int (&r)[2]) {
      if (RG) {
        // wave-uniform: scalar loads (into SGPRs, read-only data)
        typedef const __attribute__((address_space(4))) int* cint_p;
        const cint_p kr = (cint_p)(a.kv_range);
        r[0] = kr[2 * t];
        r[1] = kr[2 * t + 1];
      } else {
        r[0] = 0;
        r[1] = n_kv;
      }
    };

    // |S| form: U = (1/2) (sum_t sum_h w |S| + Qt . k) with Qt = sum_t sum_h
    // w_th q_th over the chunk (max(S, 0) = (S + |S|) / 2), so each head term
    // is one FMA with |.| as a source modifier and the linear part is one dot
    // product per key at the end.  Qt is accumulated from the staged q rows:
    // wavefront wv takes dims 32 G + 8 (wv % 4) ... + 7 of heads 16 rb + r16
    // for rb = 2 (wv / 4), 2 (wv / 4) + 1 (its LDS addresses depend on wv, so
    // no step branches on it), summed over the chunk's queries in order.
    const int qtj = wv & 3, qtr = 2 * (wv >> 2);
    auto hterm = [](float x) -> float {
      if constexpr (AB) return __builtin_fabsf(x);
      else return relu(x);
    };
    float qacc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qacc[e] = 0.f;
    T qa0, qa1;
    float qw0 = 0.f, qw1 = 0.f;
    auto qt_load = [&](int buf, int qi) {
      qa0 = afrag(buf, qi, qtr, qtj);
      qa1 = afrag(buf, qi, qtr + 1, qtj);
      const float* wrow = reinterpret_cast<const float*>(smem + buf * kBufBytes + QB * kQBytes + qi * H * 4);
      qw0 = wrow[16 * qtr + r16];
      qw1 = wrow[16 * (qtr + 1) + r16];
    };
    auto qt_add = [&](int e) {
      qacc[e] = __builtin_fmaf(qw0, (float)qa0[e], qacc[e]);
      qacc[e] = __builtin_fmaf(qw1, (float)qa1[e], qacc[e]);
    };

    T A[4][4];        // the current query's q fragments
    float wq[2][4][4];  // head weights of the even / odd queries of the chunk
    f32x4 accA[4], accB[4];
    const f32x4 zero = {};
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) { accA[rb] = zero; accB[rb] = zero; }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int e = 0; e < 4; ++e) { wq[0][rb][e] = 0.f; wq[1][rb][e] = 0.f; }

    // One step: the 16 MFMAs of key block b into acc, with the head
    // reduction of `prev` (the block scored one step earlier, weights wp)
    // added into its running sum `ps` in between, one op pair per MFMA, and
    // after MFMA i the callback after(i) (the next query's fragment reads,
    // the batch barrier).
    auto step = [&](int b, f32x4 (&acc)[4], const f32x4 (&prev)[4], const float (&wp)[4][4], float& ps,
                    auto&& after) {
      float sum = ps;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const int i = 4 * j + rb;
          acc[rb] = M::run(A[rb][j], Bk[b][j], j == 0 ? zero : acc[rb]);
          sum = __builtin_fmaf(wp[i >> 2][i & 3], hterm(prev[i >> 2][i & 3]), sum);
          asm volatile("" : "+v"(sum));
          after(i);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      ps = sum;
    };
    const auto nothing = [](int) {};

    const int nb = (nq + QB - 1) / QB;
    uint16_t mkn[QB];   // mask entries of the next batch's queries
    int rqn[QB][2];     // and their ranges
    stage(0, 0);
#pragma unroll
    for (int i = 0; i < QB; ++i) {
      mkn[i] = mload(clampq(t0 + i));
      rload(clampq(t0 + i), rqn[i]);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int j = 0; j < 4; ++j) A[rb][j] = afrag(0, 0, rb, j);
    wload(0, 0, wq[0]);

    for (int bi = 0; bi < nb; ++bi) {
      const int buf = bi & 1;
      const int64_t tb = t0 + (int64_t)bi * QB;
      const int nqb = nq - bi * QB < QB ? nq - bi * QB : QB;
      const bool more = bi + 1 < nb;
      // this batch's mask entries and ranges (read one batch earlier) into the
      // running sum and the intersection; past the chunk the query index was
      // clamped to the chunk's last query, whose range it repeats and whose
      // mask entry is not added twice
#pragma unroll
      for (int i = 0; i < QB; ++i) {
        if (MK && i < nqb) msum = msum + f16_bits_to_f32(mkn[i]);
        if (RG) {
          const int lo = __builtin_amdgcn_readfirstlane(rqn[i][0]), hi = __builtin_amdgcn_readfirstlane(rqn[i][1]);
          L = lo > L ? lo : L;
          R = hi < R ? hi : R;
        }
      }
      if (more) {
        stage(bi + 1, buf ^ 1);
#pragma unroll
        for (int i = 0; i < QB; ++i) {
          mkn[i] = mload(clampq(tb + QB + i));
          rload(clampq(tb + QB + i), rqn[i]);
        }
      }
      // QB is even, so a query's parity in the chunk is qi's
#pragma unroll
      for (int qi = 0; qi < QB; ++qi) {
        if (qi >= nqb) break;
        const bool last_q = qi + 1 == nqb;
        // the next query's slot (after the chunk's last query: any valid
        // slot; the reads are not used)
        const int nbuf = last_q && more ? buf ^ 1 : buf;
        const int nqi = last_q ? 0 : qi + 1;
        float (&wc)[4][4] = wq[qi & 1];        // this query's weights
        float (&wo)[4][4] = wq[(qi & 1) ^ 1];  // the previous query's, then the next one's
        step(0, accA, accB, wo, P[3], nothing);
        step(1, accB, accA, wc, P[0], [&](int i) {
          if (!AB) return;
          if (i == 0) qt_load(buf, qi);
          else if (i >= 8) qt_add(i - 8);
        });
        step(2, accA, accB, wc, P[1], nothing);
        // the last block: the next query's fragments are read behind its
        // MFMAs: the first k-step's four (and the weights) after the first
        // four MFMAs, the others each right after the last use of the
        // register it replaces.  At the end of a batch the barrier comes
        // first, since the next batch's buffer is read.  Both cases issue the
        // same LDS reads in the same order, so the compiler can count them.
        step(3, accB, accA, wc, P[2], [&](int i) {
          const int rb = i & 3, j = i >> 2;
          if (i == 3) {
            if (last_q) {
              __builtin_amdgcn_s_waitcnt(0);  // this wavefront's part of the next batch has landed
              __syncthreads();
            }
#pragma unroll
            for (int r2 = 0; r2 < 4; ++r2) A[r2][0] = afrag(nbuf, nqi, r2, 0);
            wload(nbuf, nqi, wo);
          } else if (j > 0) {
            A[rb][j] = afrag(nbuf, nqi, rb, j);
          }
        });
      }
    }
    // the last query's last block (the chunk's last query has parity
    // (nq - 1) & 1)
    {
      const float (&wl)[4][4] = wq[(nq - 1) & 1];
      float sum = P[3];
#pragma unroll
      for (int i = 0; i < 16; ++i) sum = __builtin_fmaf(wl[i >> 2][i & 3], hterm(accB[i >> 2][i & 3]), sum);
      P[3] = sum;
    }
    if constexpr (AB) {
    // The linear part: the 16 lanes of a group hold the same dims of
    // different heads (xor butterfly adds them), the wavefronts' parts meet
    // in LDS (the staging buffers are free once every wavefront is past its
    // last query), and each lane adds Qt . k over its group's 32 dims to its
    // keys' sums; the lane combine below adds the groups.
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = qacc[e];
      x += __uint_as_float(xor_lane_u32<1>(__float_as_uint(x)));
      x += __uint_as_float(xor_lane_u32<2>(__float_as_uint(x)));
      x += __uint_as_float(xor_lane_u32<4>(__float_as_uint(x)));
      x += __uint_as_float(xor_lane_u32<8>(__float_as_uint(x)));
      qacc[e] = x;
    }
    float* part = reinterpret_cast<float*>(smem);  // [wavefront][dim]
    if (r16 == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) part[wv * D + 32 * G + 8 * qtj + e] = qacc[e];
    }
    __syncthreads();
    float qt[4][8];  // Qt at dims 32 G + 8 j + e: heads 0-31 from wavefront j, 32-63 from 4 + j
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) qt[j][e] = part[j * D + 32 * G + 8 * j + e] + part[(4 + j) * D + 32 * G + 8 * j + e];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      float d = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) d = __builtin_fmaf(qt[j][e], (float)Bk[b][j][e], d);
      P[b] += d;
    }
    }
  }
  // Add the four head groups of each key: two permlane32 swaps add lane
  // groups {0, 2} and {1, 3}, one permlane16 swap adds the pairs, leaving
  // key ks0 + l in lane l; then the mask sum, and -inf for keys outside the
  // chunk's common range.
  float usum;
  {
    const auto r0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(P[0]), __float_as_uint(P[2]), false, false);
    const auto r1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(P[1]), __float_as_uint(P[3]), false, false);
    const uint32_t x = __float_as_uint(__uint_as_float(r0[0]) + __uint_as_float(r0[1]));
    const uint32_t y = __float_as_uint(__uint_as_float(r1[0]) + __uint_as_float(r1[1]));
    const auto r2 = __builtin_amdgcn_permlane16_swap(x, y, false, false);
    usum = __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
    if (AB) usum = 0.5f * usum;  // |S| form: twice the sum
    usum = usum + msum;
    const int s = ks0 + lane;
    if (s < L || s >= R) usum = -__builtin_inff();
  }
  if (ks0 + lane < n_kv) a.scores[qc * a.scores_ld + ks0 + lane] = usum;
}

__global__ __launch_bounds__(BS, 1) void shared_lists_kernel(KArgs a, int nqc) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint64_t* arr = reinterpret_cast<uint64_t*>(smem);        // [kListKeys]
  uint64_t* sel = arr + kListKeys;                          // [next_pow2(K)]
  uint64_t* tmp = sel + next_pow2(a.K);                     // [2 BS]
  BlockShared* sh = reinterpret_cast<BlockShared*>(tmp + 2 * BS);
  uint32_t* red = reinterpret_cast<uint32_t*>(sh + 1);      // [4 NW + 8]
  const int64_t c0 = (int64_t)blockIdx.x * kListKeys;
  const int64_t rest = a.n_kv - c0;
  const int n = (int)(rest < kListKeys ? (rest > 0 ? rest : 0) : kListKeys);
  for (int i = threadIdx.x; i < kListKeys; i += BS) {
    uint64_t key = 0ull;
    if (i < n) {
      const int64_t s = c0 + i;
      float u = a.scores[s];
      for (int c = 1; c < nqc; ++c) u += a.scores[c * a.scores_ld + s];
      if (u != -__builtin_inff()) key = make_key(u + 0.0f, (uint32_t)s);
    }
    arr[i] = key;
  }
  __syncthreads();
  block_select_sorted_reg<kListKeys / BS>(arr, n, a.K, sel, tmp, nullptr, sh, red);
  if (a.P == 1) {
    for (int i = threadIdx.x; i < a.K; i += BS) {
      a.idx[i] = key_index(sel[i]);
      if (a.score) a.score[i] = key_score(sel[i]);
    }
    return;
  }
  uint64_t* out = a.lists + (size_t)blockIdx.x * a.K;
  for (int i = threadIdx.x; i < a.K; i += BS) out[i] = sel[i];
}

// Up to kSharedSelectKeys keys: one workgroup does the whole selection.  U
// is the QC partial sums added in chunk order (as in the list kernel), 32
// keys per thread in registers; the k_top best go straight to the output by
// one block bucket pass (block_bucket_topk), or, when a bucket overflows
// (many equal or nearly equal sums), by the radix select and sort over the
// keys copied to LDS.
__global__ __launch_bounds__(BS, 1) void shared_select_kernel(KArgs a, int nqc) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int R = kSharedSelectKeys / BS;
  const int tid = threadIdx.x;
  const int n = (int)a.n_kv, K = a.K;
  // the partial sums, one chunk row at a time: all R loads of a row are in
  // flight together (keys past n read key n - 1; their sums are not used)
  float u[R];
#pragma unroll
  for (int r = 0; r < R; ++r) u[r] = 0.f;
  for (int c = 0; c < (n > 0 ? nqc : 0); ++c) {  // (no keys: nothing to read)
    const float* row = a.scores + (int64_t)c * a.scores_ld;
    float v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = r * BS + tid;
      v[r] = row[i < n ? i : n - 1];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) u[r] = c == 0 ? v[r] : u[r] + v[r];
  }
  uint64_t x[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = r * BS + tid;
    x[r] = (i < n && u[r] != -__builtin_inff()) ? make_key(u[r] + 0.0f, (uint32_t)i) : 0ull;
  }
  uint32_t* H = reinterpret_cast<uint32_t*>(smem);
  uint32_t* S = H + kBlockBuckets;
  uint64_t* seg = reinterpret_cast<uint64_t*>(S + kBlockBuckets);
  uint32_t* bred = reinterpret_cast<uint32_t*>(seg + K + kBlockBucketMax + 8);
  if (block_bucket_topk<R>(x, K, nullptr, 0, H, S, seg, bred, a.idx, a.score)) return;
  __syncthreads();  // every thread is done with the bucket scratch
  uint64_t* arr = reinterpret_cast<uint64_t*>(smem);  // [kSharedSelectKeys]
  uint64_t* sel = arr + kSharedSelectKeys;            // [next_pow2(K)]
  uint64_t* tmp = sel + next_pow2(K);                 // [2 BS]
  BlockShared* sh = reinterpret_cast<BlockShared*>(tmp + 2 * BS);
  uint32_t* red = reinterpret_cast<uint32_t*>(sh + 1);  // [4 NW + 8]
#pragma unroll
  for (int r = 0; r < R; ++r) arr[r * BS + tid] = x[r];
  __syncthreads();
  block_select_sorted_reg<R>(arr, n, K, sel, tmp, nullptr, sh, red);
  for (int i = tid; i < K; i += BS) {
    a.idx[i] = key_index(sel[i]);
    if (a.score) a.score[i] = key_score(sel[i]);
  }
}

__global__ __launch_bounds__(kMergeThreads) void shared_merge_kernel(KArgs a, int ch) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  merge_lists(a, ch, 0, smem);
}

}  // namespace

size_t shared_select_lds_bytes(int K) {
  const size_t fallback = (size_t)kSharedSelectKeys * 8 + (size_t)next_pow2(K) * 8 + 2 * BS * 8 + sizeof(BlockShared) +
                          (4 * NW + 8) * 4;
  const size_t bucket = 2 * (size_t)kBlockBuckets * 4 + ((size_t)K + kBlockBucketMax + 8) * 8 + 5 * NW * 4;
  return fallback > bucket ? fallback : bucket;
}

hipError_t launch_shared_select(const KArgs& a, int nqc, hipStream_t st) {
  hipError_t e = set_lds_limit(reinterpret_cast<const void*>(&shared_select_kernel), 160 * 1024);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(shared_select_kernel, dim3(1), dim3(BS), shared_select_lds_bytes(a.K), st, a, nqc);
  return hipGetLastError();
}

size_t shared_lists_lds_bytes(int K) {
  return (size_t)kListKeys * 8 + (size_t)next_pow2(K) * 8 + 2 * BS * 8 + sizeof(BlockShared) + (4 * NW + 8) * 4;
}

template <int DT, bool MK, bool RG>
hipError_t launch_scores_one(const KArgs& a, int qchunk, dim3 grid, hipStream_t st) {
  hipError_t e = set_lds_limit(reinterpret_cast<const void*>(&shared_scores_kernel<DT, MK, RG>), (int)kScoresLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((shared_scores_kernel<DT, MK, RG>), grid, dim3(BS), kScoresLds, st, a, qchunk);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_scores_dt(const KArgs& a, int qchunk, dim3 grid, hipStream_t st) {
  const bool mk = a.mask != nullptr, rg = a.kv_range != nullptr;
  if (mk) return rg ? launch_scores_one<DT, true, true>(a, qchunk, grid, st) : launch_scores_one<DT, true, false>(a, qchunk, grid, st);
  return rg ? launch_scores_one<DT, false, true>(a, qchunk, grid, st) : launch_scores_one<DT, false, false>(a, qchunk, grid, st);
}

hipError_t launch_shared_scores(const KArgs& a, int qchunk, int nqc, hipStream_t st) {
  const int64_t ngroups = (a.n_kv + KG - 1) / KG;
  if (ngroups == 0) return hipSuccess;
  const dim3 grid((unsigned)(ngroups * nqc));
  return a.dtype == 2 ? launch_scores_dt<2>(a, qchunk, grid, st) : launch_scores_dt<1>(a, qchunk, grid, st);
}

size_t shared_merge_lds_bytes(int P, int K, int ch) { return merge_lds_need(P, K, ch); }

hipError_t launch_shared_merge(const KArgs& a, int ch, hipStream_t st) {
  hipError_t e = set_lds_limit(reinterpret_cast<const void*>(&shared_merge_kernel), 160 * 1024);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(shared_merge_kernel, dim3(1), dim3(kMergeThreads), shared_merge_lds_bytes(a.P, a.K, ch), st, a,
                     ch);
  return hipGetLastError();
}

hipError_t launch_shared_lists(const KArgs& a, int nqc, hipStream_t st) {
  hipError_t e = set_lds_limit(reinterpret_cast<const void*>(&shared_lists_kernel), 160 * 1024);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(shared_lists_kernel, dim3((unsigned)a.P), dim3(BS), shared_lists_lds_bytes(a.K), st, a, nqc);
  return hipGetLastError();
}

}  // namespace lid
