// k_decode.hip -- the few-query (decode) shape: one or a few query tokens
// against a long key range, H = 64 heads, D = 128.
//
// Scoring is the same fused chain as the prefill kernel (per-head q.k, ReLU,
// head weight, head sum, f16 mask; ggml-org llama.cpp issue 25468, "Root
// cause" comment), but the parallelism comes from the keys: the visible range
// of each query is cut into P contiguous splits, one workgroup per
// (query, split).  Each wavefront streams its own 32-key blocks (8 KiB): the
// loads are fully coalesced (64 lanes x 16 B = 1 KiB of consecutive bytes per
// instruction), land in registers while the previous block is scored, and go
// through a private LDS slot (XOR-swizzled) that turns them into the MFMA
// B-operand layout.  The score of every key the workgroup sees goes to LDS as a
// 64-bit selection key; the workgroup then selects its k_top best (radix
// select + bitonic sort) and writes them as a sorted candidate list, which the
// merge kernel reduces across splits.  Memory per split is bounded by the
// LDS array, never by n_kv.
#include "lid_device.h"
#include "lid_kernels.h"

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

constexpr int H = kMfmaHeads;
constexpr int D = kMfmaDim;
constexpr int NW = 8;     // wavefronts per workgroup
constexpr int KB = 32;    // keys per MFMA column block
constexpr int kBlockBytes = KB * D * 2;          // 8 KiB per wavefront slot
constexpr int kStageBytes = NW * kBlockBytes;    // 64 KiB

__device__ __forceinline__ int swz(int row, int ch) { return row * D + ((ch ^ (row & 15)) << 3); }

template <int DT>
__global__ __launch_bounds__(NW * 64, 1) void decode_kernel(KArgs a, int keys_per_wg) {
  using M = Mfma<DT>;
  using T = typename M::T;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* stage_all = reinterpret_cast<uint16_t*>(smem);           // [NW][KB * D]
  uint64_t* arr = reinterpret_cast<uint64_t*>(smem + kStageBytes);   // [keys_per_wg]
  uint64_t* sel = arr + keys_per_wg;                                 // [next_pow2(K)]
  uint64_t* tmp = sel + next_pow2(a.K);                              // [2 * NW * 64]
  BlockShared* sh = reinterpret_cast<BlockShared*>(tmp + 2 * NW * 64);

  const int wv = threadIdx.x / kWave;
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
  const int64_t last_row = hi - 1;
  uint16_t* stage = stage_all + wv * (KB * D);
  auto load_blk = [&](int64_t b, u32x4 (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int64_t s = lo + b * KB + 4 * i + (lane >> 4);
      s = s < last_row ? s : last_row;
      f[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + s * D + (lane & 15) * 8));
    }
  };
  auto load_mask = [&](int64_t b) -> uint16_t {
    if (!a.mask) return 0;
    int64_t s = lo + b * KB + m;
    s = s < last_row ? s : last_row;
    return __builtin_nontemporal_load(a.mask + t * a.mask_ld + s);
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
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      part = __builtin_fmaf(wr[0][e], relu(acc0[e]), part);
      part = __builtin_fmaf(wr[1][e], relu(acc1[e]), part);
    }
    const float tot = part + __uint_as_float(xor_lane_u32<32>(__float_as_uint(part)));
    const float v = (tot + f16_bits_to_f32(mbits)) + 0.0f;
    if (g == 0) {
      const bool valid = s < hi && v != -__builtin_inff();
      arr[(b - b0) * KB + m] = valid ? make_key(v, (uint32_t)s) : 0ull;
    }
  };

  // ping-pong register sets: the loads of one block fly while the other is scored
  if (hi > lo) {
    u32x4 fa[8], fb[8];
    int64_t b = b0 + wv;
    uint16_t ma = 0, mb = 0;
    if (b < b1) { ma = load_mask(b); load_blk(b, fa); }
    while (b < b1) {
      const int64_t bn = b + NW;
      if (bn < b1) { mb = load_mask(bn); load_blk(bn, fb); }
      score_blk(b, fa, ma);
      if (bn >= b1) break;
      const int64_t bnn = bn + NW;
      if (bnn < b1) { ma = load_mask(bnn); load_blk(bnn, fa); }
      score_blk(bn, fb, mb);
      b = bnn;
    }
  }
  __syncthreads();

  block_select_sorted(arr, nkeys, a.K, sel, tmp, *sh);

  if (P == 1) {
    for (int i = threadIdx.x; i < a.K; i += blockDim.x) {
      a.idx[t * a.K + i] = key_index(sel[i]);
      if (a.score) a.score[t * a.K + i] = key_score(sel[i]);
    }
  } else {
    uint64_t* out = a.lists + ((size_t)t * P + p) * a.K;
    for (int i = threadIdx.x; i < a.K; i += blockDim.x) out[i] = sel[i];
  }
}

template <int DT>
hipError_t launch_one(const KArgs& a, int keys_per_wg, hipStream_t st) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<DT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid((unsigned)(a.n_tok * a.P));
  hipLaunchKernelGGL((decode_kernel<DT>), grid, dim3(NW * 64), decode_lds_bytes(keys_per_wg, a.K), st, a,
                     keys_per_wg);
  return hipGetLastError();
}

}  // namespace

size_t decode_lds_bytes(int keys_per_wg, int K) {
  return (size_t)kStageBytes + (size_t)keys_per_wg * 8 + (size_t)next_pow2(K) * 8 + 2 * NW * 64 * 8 +
         sizeof(BlockShared);
}

hipError_t launch_decode(const KArgs& a, int keys_per_wg, hipStream_t st) {
  return a.dtype == 1 ? launch_one<1>(a, keys_per_wg, st) : launch_one<2>(a, keys_per_wg, st);
}

}  // namespace lid
