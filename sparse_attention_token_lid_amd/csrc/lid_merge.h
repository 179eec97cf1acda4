// lid_merge.h -- reduction of the P per-split candidate lists of one query
// to its final top-k row, by one workgroup of kMergeThreads threads (the
// merge kernel runs one workgroup per query; the decode kernel runs it in the
// last workgroup of a query to finish).
//
// Selection order as in ggml-org llama.cpp issue 25468 ("Root cause"
// comment): per-token top-k of the masked score; ties by index.  Each list
// holds the K best keys of one split, sorted descending (empty slots = 0),
// and only a short prefix of most lists can reach the final row.  Two ways:
//  * merge_lists_tree (next_pow2(K) == 512): the first 8 entries of every
//    list go through the merge tree of lid_select.h, whose K-th key tau
//    bounds the answer; lists whose last entry read is above tau give as
//    many entries again, for another tree pass, until none is left above tau;
//  * merge_lists: lists are read in rounds of ch entries; after a round the
//    workgroup keeps the K best candidates seen so far, whose K-th key tau is
//    a lower bound of the final threshold, and a list whose last entry read
//    is <= tau drops out (it is sorted).
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

// Fast path for next_pow2(K) == kTreeCap and P kTreePrefix <= 4096: the
// first kTreePrefix entries of every list go through the merge tree
// (block_topk_tree_any), whose K-th key tau bounds the answer from below.  A
// list whose last entry read is above tau may hold more of the answer: each
// such list gives as many further entries as it has given so far, which join
// the current K best for another tree pass.  Returns false (nothing written)
// when that would exceed the tree's 4096 candidates; the caller then runs
// merge_lists.
constexpr int kTreePrefix = 8;
__host__ __device__ inline size_t merge_tree_lds_need(int P) {
  return (size_t)4096 * 8 + (size_t)2048 * 8 + (size_t)kTreeCap * 8 + (size_t)P * 8 + (size_t)P * 16 + 16;
}

__device__ __forceinline__ bool merge_lists_tree(const KArgs& a, int64_t t, unsigned char* smem) {
  const int P = a.P, K = a.K;
  uint64_t* cand = reinterpret_cast<uint64_t*>(smem);    // [4096]
  uint64_t* alt = cand + 4096;                           // [2048]
  uint64_t* best = alt + 2048;                           // [kTreeCap] the tree's result
  uint64_t* last = best + kTreeCap;                      // [P] last entry read per list
  uint32_t* rd = reinterpret_cast<uint32_t*>(last + P);  // [P] entries read per list
  uint32_t* fl = rd + P;                                 // [P][3] flagged: list, offset, count
  int* s_cnt = reinterpret_cast<int*>(fl + 3 * P);       // [0] flagged lists, [1] entries they add
  const uint64_t* lists = a.lists + (size_t)t * P * K;
  const int tid = threadIdx.x;
  // agent-scope loads: the lists may have just been written by other
  // workgroups of the same launch, on other XCDs
  auto ld = [&](int lp, int j) -> uint64_t {
    return __hip_atomic_load(&lists[(size_t)lp * K + j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  for (int i = tid; i < P * kTreePrefix; i += kMergeThreads) {
    const int lp = i / kTreePrefix, j = i % kTreePrefix;
    const uint64_t key = j < K ? ld(lp, j) : 0ull;
    cand[i] = key;
    if (j == kTreePrefix - 1) { last[lp] = key; rd[lp] = kTreePrefix; }
  }
  if (tid == 0) { s_cnt[0] = 0; s_cnt[1] = 0; }
  __syncthreads();
  int m = P * kTreePrefix;
  for (;;) {
    block_topk_tree_any(cand, alt, m, K, nullptr, nullptr, best);
    const uint64_t tau = best[K - 1];
    // lists that may hold more keys above tau (keys are unique: a list whose
    // last entry read is <= tau has nothing further above it)
    for (int lp = tid; lp < P; lp += kMergeThreads) {
      const int r = (int)rd[lp];
      if (r < K && last[lp] > tau) {
        const int n = r < K - r ? r : K - r;
        const int f = atomicAdd(&s_cnt[0], 1);
        fl[3 * f] = (uint32_t)lp;
        fl[3 * f + 1] = (uint32_t)atomicAdd(&s_cnt[1], n);
        fl[3 * f + 2] = (uint32_t)n;
      }
    }
    __syncthreads();
    const int nflag = s_cnt[0], nadd = s_cnt[1];
    if (nflag == 0) break;
    if (K + nadd > 4096) return false;
    for (int f = 0; f < nflag; ++f) {
      const int lp = (int)fl[3 * f], off = (int)fl[3 * f + 1], n = (int)fl[3 * f + 2], r = (int)rd[lp];
      for (int j = tid; j < n; j += kMergeThreads) {
        const uint64_t key = ld(lp, r + j);
        cand[K + off + j] = key;
        if (j == n - 1) last[lp] = key;
      }
    }
    for (int i = tid; i < K; i += kMergeThreads) cand[i] = best[i];
    __syncthreads();  // every rd[] read above precedes its update
    for (int f = tid; f < nflag; f += kMergeThreads) rd[fl[3 * f]] += fl[3 * f + 2];
    if (tid == 0) { s_cnt[0] = 0; s_cnt[1] = 0; }
    m = K + nadd;
    __syncthreads();
  }
  for (int i = tid; i < K; i += kMergeThreads) {
    a.idx[t * K + i] = key_index(best[i]);
    if (a.score) a.score[t * K + i] = key_score(best[i]);
  }
  return true;
}

__device__ __forceinline__ void merge_lists(const KArgs& a, int ch, int64_t t, unsigned char* smem);

// LDS for finish_lists(): the larger of the two paths.
__host__ __device__ inline size_t finish_lds_need(int P, int K, int ch) {
  const size_t a = merge_lds_need(P, K, ch), b = merge_tree_lds_need(P);
  return next_pow2(K) == kTreeCap && P * kTreePrefix <= 4096 && b > a ? b : a;
}

// The final row of query t from its P sorted split lists: the tree fast path
// when it applies and suffices, else the round-based merge.
__device__ __forceinline__ void finish_lists(const KArgs& a, int ch, int64_t t, unsigned char* smem) {
  if (next_pow2(a.K) == kTreeCap && a.P * kTreePrefix <= 4096 && merge_lists_tree(a, t, smem)) return;
  __syncthreads();
  merge_lists(a, ch, t, smem);
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
