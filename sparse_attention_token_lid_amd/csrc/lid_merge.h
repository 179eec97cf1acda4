// lid_merge.h -- reduction of the P per-split candidate lists of one query
// to its final top-k row, by one workgroup of kMergeThreads threads (the
// merge kernel runs one workgroup per query; the decode kernel runs it in the
// last workgroup of a query to finish).
//
// Selection order as in ggml-org llama.cpp issue 25468 ("Root cause"
// comment): per-token top-k of the masked score; ties by index.  Each list
// holds the K best keys of one split, sorted descending (empty slots = 0).
// Lists are read in rounds of ch entries per list: after the first round the
// workgroup keeps the K best candidates seen so far, and their K-th key tau is
// a lower bound of the final threshold.  A list whose last entry read is
// <= tau cannot contribute any more (it is sorted), so it drops out;
// typically every list drops out after a round or two, and only a small
// prefix of each list is ever read.
#pragma once
#include "lid_device.h"
#include "lid_kernels.h"
#include "lid_select.h"

namespace lid {

constexpr int kMergeThreads = 512;

// LDS bytes merge_lists() needs.
__host__ __device__ inline size_t merge_lds_need(int P, int K, int ch) {
  const size_t capm = (size_t)K + (size_t)P * ch;
  return capm * 8 + (size_t)next_pow2(K) * 8 + 2 * kMergeThreads * 8 + (size_t)P * 8 + sizeof(BlockShared) +
         2 * sizeof(int) + 2 * (size_t)P + 16 + kSelHistBytes + kSelRedBytes;
}

__device__ __forceinline__ void merge_lists(const KArgs& a, int ch, int64_t t, unsigned char* smem) {
  const int P = a.P, K = a.K;
  const int n2 = next_pow2(K);
  const int capm = K + P * ch;
  uint64_t* cand = reinterpret_cast<uint64_t*>(smem);          // [capm]
  uint64_t* sel = cand + capm;                                 // [n2]
  uint64_t* tmp = sel + n2;                                    // [2 * kMergeThreads]
  uint64_t* last = tmp + 2 * kMergeThreads;                               // [P] last key read per list
  BlockShared* sh = reinterpret_cast<BlockShared*>(last + P);
  int* counters = reinterpret_cast<int*>(sh + 1);             // [2]
  int& s_count = counters[0];
  int& s_active = counters[1];
  uint8_t* done = reinterpret_cast<uint8_t*>(counters + 2);    // [P]
  uint8_t* done_next = done + P;                               // [P]
  uint32_t* hw = reinterpret_cast<uint32_t*>(                  // selection histograms, 16-byte aligned
      (reinterpret_cast<uintptr_t>(done_next + P) + 15) & ~static_cast<uintptr_t>(15));
  uint32_t* red = hw + kSelHistBytes / 4;
  static_assert(18 * kMergeThreads >= 1024 + 8192, "capm <= K + P ch <= 1024 + 8192");

  const uint64_t* lists = a.lists + (size_t)t * P * K;
  for (int i = threadIdx.x; i < P; i += kMergeThreads) { done[i] = 0; done_next[i] = 0; }
  if (threadIdx.x == 0) { s_count = 0; sh->red_min = ~0ull; }
  __syncthreads();

  uint64_t tau = 0ull;
  const int nrounds = (K + ch - 1) / ch;
  for (int r = 0; r < nrounds; ++r) {
    const int jbase = r * ch;
    for (int it0 = 0; it0 < P * ch; it0 += kMergeThreads) {
      const int it = it0 + threadIdx.x;
      const int lp = it / ch, e = it - lp * ch;
      const int j = jbase + e;
      const bool act = it < P * ch && !done[lp] && j < K;
      // agent-scope loads: the lists may have just been written by other
      // workgroups of the same launch (decode), on other XCDs
      const uint64_t key = act ? __hip_atomic_load(&lists[(size_t)lp * K + j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                               : 0ull;
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
    for (int i = threadIdx.x; i < P; i += kMergeThreads) {
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
      const int kept = block_select_compact_any(cand, count, K, sel, hw, sh, red);
      // kept == K: their minimum is the K-th key
      uint64_t mn = ~0ull;
      for (int i = threadIdx.x; i < kept; i += kMergeThreads) {
        cand[i] = sel[i];
        mn = sel[i] < mn ? sel[i] : mn;
      }
      mn = wave_min_u64(mn);
      if (lane_id() == 0) atomicMin((unsigned long long*)&sh->red_min, mn);
      if (threadIdx.x == 0) s_count = kept;
      __syncthreads();
      const uint64_t kap = sh->red_min;
      __syncthreads();
      if (threadIdx.x == 0) sh->red_min = ~0ull;
      tau = kap;
      for (int i = threadIdx.x; i < P; i += kMergeThreads)
        if (last[i] <= tau) done[i] = 1;
      __syncthreads();
    }
  }
  const int count = s_count;
  __syncthreads();
  if (count == K && tau != 0ull) {
    // the last cut left exactly the K best and no list had more to give
    for (int i = threadIdx.x; i < K; i += kMergeThreads) sel[i] = cand[i];
    for (int i = K + threadIdx.x; i < n2; i += kMergeThreads) sel[i] = 0ull;
    __syncthreads();
    block_sort_desc(sel, n2, tmp);
  } else {
    block_select_sorted_any(cand, count, K, sel, tmp, hw, sh, red);
  }
  for (int i = threadIdx.x; i < K; i += kMergeThreads) {
    a.idx[t * K + i] = key_index(sel[i]);
    if (a.score) a.score[t * K + i] = key_score(sel[i]);
  }
}


}  // namespace lid
