// k_merge.hip -- the merge kernel: one workgroup per query reduces the P
// per-split candidate lists to the final top-k row (lid_merge.h).
#include "lid_merge.h"

namespace lid {
namespace {

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(KArgs a, int ch) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  finish_lists(a, ch, blockIdx.x, smem);
}

}  // namespace

size_t merge_lds_bytes(int P, int K, int ch) { return finish_lds_need(P, K, ch); }

hipError_t launch_merge(const KArgs& a, int ch, hipStream_t st) {
  hipError_t e = set_lds_limit(reinterpret_cast<const void*>(&merge_kernel), 160 * 1024);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)a.n_tok), dim3(kMergeThreads), merge_lds_bytes(a.P, a.K, ch), st, a,
                     ch);
  return hipGetLastError();
}

}  // namespace lid
