// k_merge.hip -- reduce the P per-split candidate lists of each query to the
// final top-k row (selection order as in ggml-org llama.cpp issue 25468,
// "Root cause" comment: per-token top-k of the masked score; ties by index).
//
// One workgroup per query.  Each list holds the K best keys of one split,
// sorted descending (empty slots = 0).  Lists are read in rounds of CH entries
// per list: after the first round the workgroup keeps the K best candidates
// seen so far, and their K-th key tau is a lower bound of the final threshold.
// A list whose last entry read is <= tau cannot contribute any more (it is
// sorted), so it drops out; typically every list drops out after a round or
// two, and only a small prefix of each list is ever read.
#include "lid_device.h"
#include "lid_kernels.h"

namespace lid {
namespace {

constexpr int BS = 512;

__global__ __launch_bounds__(BS) void merge_kernel(KArgs a, int ch) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int P = a.P, K = a.K;
  const int n2 = next_pow2(K);
  const int capm = K + P * ch;
  uint64_t* cand = reinterpret_cast<uint64_t*>(smem);          // [capm]
  uint64_t* sel = cand + capm;                                 // [n2]
  uint64_t* tmp = sel + n2;                                    // [2 * BS]
  uint64_t* last = tmp + 2 * BS;                               // [P] last key read per list
  BlockShared* sh = reinterpret_cast<BlockShared*>(last + P);
  int* counters = reinterpret_cast<int*>(sh + 1);             // [2]
  int& s_count = counters[0];
  int& s_active = counters[1];
  uint8_t* done = reinterpret_cast<uint8_t*>(counters + 2);    // [P]
  uint8_t* done_next = done + P;                               // [P]

  const int64_t t = blockIdx.x;
  const uint64_t* lists = a.lists + (size_t)t * P * K;
  for (int i = threadIdx.x; i < P; i += BS) { done[i] = 0; done_next[i] = 0; }
  if (threadIdx.x == 0) s_count = 0;
  __syncthreads();

  uint64_t tau = 0ull;
  const int nrounds = (K + ch - 1) / ch;
  for (int r = 0; r < nrounds; ++r) {
    const int jbase = r * ch;
    for (int it0 = 0; it0 < P * ch; it0 += BS) {
      const int it = it0 + threadIdx.x;
      const int lp = it / ch, e = it - lp * ch;
      const int j = jbase + e;
      const bool act = it < P * ch && !done[lp] && j < K;
      const uint64_t key = act ? lists[(size_t)lp * K + j] : 0ull;
      const bool ins = act && key > tau;
      const uint64_t msk = ballot(ins);
      int base = 0;
      if (msk) {
        const int leader = __ffsll((unsigned long long)msk) - 1;
        if (lane_id() == leader) base = atomicAdd(&s_count, __popcll(msk));
        base = __builtin_amdgcn_readlane(base, leader);
      }
      if (ins) cand[base + mbcnt(msk)] = key;
      // the last entry of this list's chunk decides whether the list goes on
      if (act && (e == ch - 1 || j == K - 1)) {
        last[lp] = key;
        if (key <= tau || j == K - 1) done_next[lp] = 1;
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) s_active = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < P; i += BS) {
      done[i] |= done_next[i];
      if (!done[i]) s_active = 1;
    }
    __syncthreads();
    const int count = s_count;
    const bool more = s_active != 0 && r + 1 < nrounds;
    if (!more) break;
    // keep the K best; their K-th key bounds the final threshold from below,
    // and every list whose last key read is below it is finished
    if (count > K && (r == 0 || count + P * ch > capm)) {
      uint64_t ka, ko;
      block_key_stats(cand, count, &ka, &ko, *sh);
      const uint64_t kap = block_kth_largest(cand, count, K, ka, ko, *sh);
      const int kept = block_compact(cand, count, kap, sel, *sh);
      for (int i = threadIdx.x; i < kept; i += BS) cand[i] = sel[i];
      if (threadIdx.x == 0) s_count = kept;
      tau = kap;
      for (int i = threadIdx.x; i < P; i += BS)
        if (last[i] <= tau) done[i] = 1;
      __syncthreads();
    }
  }
  const int count = s_count;
  __syncthreads();
  if (count == K && tau != 0ull) {
    // the last cut left exactly the K best and no list had more to give
    for (int i = threadIdx.x; i < K; i += BS) sel[i] = cand[i];
    for (int i = K + threadIdx.x; i < n2; i += BS) sel[i] = 0ull;
    __syncthreads();
    block_sort_desc(sel, n2, tmp);
  } else {
    block_select_sorted(cand, count, K, sel, tmp, *sh);
  }
  for (int i = threadIdx.x; i < K; i += BS) {
    a.idx[t * K + i] = key_index(sel[i]);
    if (a.score) a.score[t * K + i] = key_score(sel[i]);
  }
}

}  // namespace

size_t merge_lds_bytes(int P, int K, int ch) {
  size_t capm = (size_t)K + (size_t)P * ch;
  return capm * 8 + (size_t)next_pow2(K) * 8 + 2 * BS * 8 + (size_t)P * 8 + sizeof(BlockShared) +
         2 * sizeof(int) + 2 * (size_t)P;
}

hipError_t launch_merge(const KArgs& a, int ch, hipStream_t st) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&merge_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)a.n_tok), dim3(BS), merge_lds_bytes(a.P, a.K, ch), st, a, ch);
  return hipGetLastError();
}

}  // namespace lid
