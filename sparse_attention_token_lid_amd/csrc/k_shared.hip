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
//  * shared_scores_kernel: one workgroup per (group of 256 keys, chunk of
//    queries).  The key group is staged once in LDS (16-byte chunks
//    XOR-swizzled per row); wavefront w takes queries w, w + 8, ... of the
//    chunk, scores the 256 keys with 32x32x16 MFMAs (q fragments in
//    registers, the same layout as the decode kernel, the next query's
//    loaded while the current one is scored), applies ReLU, the
//    head weights, the head sum and the mask, and adds v into one f32 sum
//    per key (in its own LDS row).  The eight wavefronts' sums are added in
//    wavefront order and written as the chunk's partial sums [QC, n_kv].
//  * shared_lists_kernel: one workgroup per 4096 keys: U = the QC partial
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
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int DT> struct MfmaS;
template <> struct MfmaS<1> {
  typedef f16x8 T;
  static __device__ __forceinline__ f32x16 run(T a, T b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct MfmaS<2> {
  typedef bf16x8 T;
  static __device__ __forceinline__ f32x16 run(T a, T b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

constexpr int H = kMfmaHeads;
constexpr int D = kMfmaDim;
constexpr int NW = 8;
constexpr int BS = NW * kWave;
constexpr int KG = kSharedGroupKeys;  // keys per scoring workgroup
constexpr int NB = KG / 32;           // 32-key MFMA column blocks
constexpr int kListKeys = kSharedListKeys;
constexpr size_t kScoresLds = (size_t)KG * D * 2 + (size_t)NW * KG * 4 + (size_t)NW * KG * 2;
static_assert(BS == kSelThreads, "the list kernel runs the block selection");
static_assert(KG <= BS && (KG * D / 8) % BS == 0, "staging and the final sum");

__device__ __forceinline__ int swz(int row, int ch) { return row * D + ((ch ^ (row & 15)) << 3); }

template <int DT>
__global__ __launch_bounds__(BS, 1) void shared_scores_kernel(KArgs a, int qchunk) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* kt = reinterpret_cast<uint16_t*>(smem);                          // [KG][D]
  float* part = reinterpret_cast<float*>(smem + (size_t)KG * D * 2);         // [NW][KG]
  uint16_t* mlds = reinterpret_cast<uint16_t*>(part + NW * KG);              // [NW][KG] mask entries
  const int tid = threadIdx.x, wv = tid / kWave, lane = tid & (kWave - 1);
  const int g = lane >> 5, m = lane & 31;
  const int64_t ngroups = (a.n_kv + KG - 1) / KG;
  const int64_t kg = blockIdx.x % ngroups, qc = blockIdx.x / ngroups;
  const int64_t s0 = kg * KG;
  const int64_t t0 = qc * qchunk;
  const int64_t t1 = t0 + qchunk < a.n_tok ? t0 + qchunk : a.n_tok;

  // the key group into LDS; rows past n_kv are zeros (their sums are not kept)
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.k);
#pragma unroll
  for (int i = 0; i < KG * D / 8 / BS; ++i) {
    const int c = i * BS + tid, r = c / (D / 8), ch = c % (D / 8);
    const int64_t s = s0 + r;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (s < a.n_kv) x = *reinterpret_cast<const u32x4*>(kb + s * D + ch * 8);
    *reinterpret_cast<u32x4*>(kt + swz(r, ch)) = x;
  }
  // each wavefront's per-key sums live in its own row of part (lanes 0..31
  // of the wavefront own the 32 keys of a block: no other writer)
  float* prow = part + wv * KG;
  for (int i = lane; i < KG; i += kWave) prow[i] = 0.f;
  __syncthreads();

  using M = MfmaS<DT>;
  using T = typename M::T;
  // q fragments (16 KiB) and the 256 mask entries of a query: loaded one
  // query ahead into the other register set, so the loads of the next query
  // fly while the current one is scored.  The mask row is read through a
  // buffer resource of the key group's entries: past n_kv, or without a
  // mask (an empty buffer), the loads return 0 and read nothing, so they are
  // unconditional.
  T A[2][8], An[2][8];
  uint32_t M4[4], M4n[4];
  uint16_t* mrow = mlds + wv * KG;
  auto load_q = [&](int64_t t, T (&Aq)[2][8], uint32_t (&mq)[4]) {
    const int64_t tc = t < t1 ? t : t0;  // past the chunk: any valid row (not used)
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + tc * H * D;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        Aq[rb][j] = __builtin_bit_cast(T, *reinterpret_cast<const u32x4*>(qrow + (32 * rb + m) * D + 64 * g + 8 * j));
    const int64_t nm = a.n_kv - s0 < KG ? a.n_kv - s0 : KG;
    const __amdgpu_buffer_rsrc_t mr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.mask ? a.mask + tc * a.mask_ld + s0 : reinterpret_cast<const uint16_t*>(a.w)),
        (short)0, a.mask ? (int)(nm * 2) : 0, 0x00020000);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      mq[i] = __builtin_amdgcn_raw_buffer_load_b16(mr, (uint32_t)(lane + kWave * i) * 2u, 0, 0);
  };
  // score query t (its fragments in Aq, mask entries in mq) against the key group
  auto process = [&](int64_t t, const T (&Aq)[2][8], const uint32_t (&mq)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) mrow[lane + kWave * i] = (uint16_t)mq[i];
    __builtin_amdgcn_wave_barrier();
    float wq[2][16];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) wq[rb][jj] = a.w[t * H + 32 * rb + 8 * (jj >> 2) + 4 * g + (jj & 3)];
    int64_t lo = 0, hi = a.n_kv;
    if (a.kv_range) {
      const int64_t l0 = a.kv_range[2 * t], h0 = a.kv_range[2 * t + 1];
      lo = l0 < 0 ? 0 : l0;
      hi = h0 > a.n_kv ? a.n_kv : h0;
    }
#pragma unroll 1
    for (int b = 0; b < NB; ++b) {
      f32x16 acc0, acc1;
#pragma unroll
      for (int e = 0; e < 16; ++e) { acc0[e] = 0.f; acc1[e] = 0.f; }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const T bf = __builtin_bit_cast(T, *reinterpret_cast<const u32x4*>(kt + swz(32 * b + m, 8 * g + j)));
        acc0 = M::run(Aq[0][j], bf, acc0);
        acc1 = M::run(Aq[1][j], bf, acc1);
      }
      // sum_h w_h relu(S[h, key]) over this lane's 32 heads, then the other 32
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p = __builtin_fmaf(wq[0][e], relu(acc0[e]), p);
        p = __builtin_fmaf(wq[1][e], relu(acc1[e]), p);
      }
      const float tot = p + __uint_as_float(xor_lane_u32<32>(__float_as_uint(p)));
      const int64_t s = s0 + 32 * b + m;
      const uint16_t mb = mrow[32 * b + m];
      const float v = (tot + f16_bits_to_f32(mb)) + 0.0f;
      const bool ok = s >= lo && s < hi && v != -__builtin_inff();
      if (g == 0) prow[32 * b + m] += ok ? v : -__builtin_inff();
    }
    __builtin_amdgcn_wave_barrier();  // every lane has read mrow before the next query's entries
  };
  // two register sets, alternating: the next query's loads fly while the
  // current one is scored
  if (t0 + wv < t1) load_q(t0 + wv, A, M4);
  for (int64_t t = t0 + wv; t < t1; t += 2 * NW) {
    load_q(t + NW, An, M4n);
    process(t, A, M4);
    if (t + NW >= t1) break;
    load_q(t + 2 * NW, A, M4);
    process(t + NW, An, M4n);
  }
  __syncthreads();
  if (tid < KG) {
    float u = part[tid];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) u += part[w2 * KG + tid];
    const int64_t s = s0 + tid;
    if (s < a.n_kv) a.scores[qc * a.scores_ld + s] = u;
  }
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

__global__ __launch_bounds__(kMergeThreads) void shared_merge_kernel(KArgs a, int ch) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  merge_lists(a, ch, 0, smem);
}

template <typename F>
hipError_t set_lds_attr(F* f, bool& done) {
  if (done) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(f), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     160 * 1024);
  if (e == hipSuccess) done = true;
  return e;
}

}  // namespace

size_t shared_lists_lds_bytes(int K) {
  return (size_t)kListKeys * 8 + (size_t)next_pow2(K) * 8 + 2 * BS * 8 + sizeof(BlockShared) + (4 * NW + 8) * 4;
}

hipError_t launch_shared_scores(const KArgs& a, int qchunk, int nqc, hipStream_t st) {
  const int64_t ngroups = (a.n_kv + KG - 1) / KG;
  if (ngroups == 0) return hipSuccess;
  dim3 grid((unsigned)(ngroups * nqc));
  hipError_t e;
  if (a.dtype == 2) {
    static bool done = false;
    if ((e = set_lds_attr(&shared_scores_kernel<2>, done)) != hipSuccess) return e;
    hipLaunchKernelGGL(shared_scores_kernel<2>, grid, dim3(BS), kScoresLds, st, a, qchunk);
  } else {
    static bool done = false;
    if ((e = set_lds_attr(&shared_scores_kernel<1>, done)) != hipSuccess) return e;
    hipLaunchKernelGGL(shared_scores_kernel<1>, grid, dim3(BS), kScoresLds, st, a, qchunk);
  }
  return hipGetLastError();
}

size_t shared_merge_lds_bytes(int P, int K, int ch) { return merge_lds_need(P, K, ch); }

hipError_t launch_shared_merge(const KArgs& a, int ch, hipStream_t st) {
  static bool done = false;
  hipError_t e = set_lds_attr(&shared_merge_kernel, done);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(shared_merge_kernel, dim3(1), dim3(kMergeThreads), shared_merge_lds_bytes(a.P, a.K, ch), st, a,
                     ch);
  return hipGetLastError();
}

hipError_t launch_shared_lists(const KArgs& a, int nqc, hipStream_t st) {
  static bool done = false;
  hipError_t e = set_lds_attr(&shared_lists_kernel, done);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(shared_lists_kernel, dim3((unsigned)a.P), dim3(BS), shared_lists_lds_bytes(a.K), st, a, nqc);
  return hipGetLastError();
}

}  // namespace lid
