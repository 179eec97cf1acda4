// k_attn.hip -- sparse attention over the selected keys, the consumer of the
// top-k: for query t and head h,
//     s_j    = scale * qa[t,h,:] . kv[idx[t,j], :]
//     o[t,h] = sum_j softmax_j(s) kv[idx[t,j], :]
// over the selection entries with 0 <= idx[t,j] < n_kv (a selection without
// one gives o = 0).  Issue 25468, "Root cause" comment: each CSA layer's
// score chain ends in a per-token top-512 selection of the compressed KV
// rows; ggml-org llama.cpp PR 22378, the flash-attention unblock commit:
// V4's MLA latent KV has K width 512 and attention is Q K^T -> softmax -> *V.
// The absorbed-MLA form is read: one latent row serves as key and value.
//
// Two kernels.  For a latent width of 512 (the pages' width) the per-query
// work is a dense contraction shared by all heads -- S = Q_t K_sel^T and O_t =
// softmax(S) K_sel -- and runs on MFMA (sparse_attn_mfma_kernel, below).  Other
// widths run on the vector ALU (sparse_attn_kernel):
//
// One wavefront per (query, head): lane l holds dims 512 c + 8 l .. + 7 of q
// and of the output for the c-th 512-dim chunk of the latent row (L <= 1024).
// The selected rows are read 16 bytes per lane (a 1 KiB row per
// instruction), four rows per group with the next group's loads in flight
// while the current one is scored; the softmax is computed online in f32 (a
// running maximum, the rescaled denominator and accumulator).  An invalid
// index reads row 0 and gets s = -inf (weight 0), so no load is conditional.
#include "lid_device.h"
#include "lid_kernels.h"

namespace lid {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NW = 4;          // wavefronts (heads) per workgroup
constexpr int BS = NW * kWave;
constexpr int G = 4;           // selected rows per load group

template <int DT>
__device__ __forceinline__ void unpack8(const u32x4& x, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = x[i];
    if constexpr (DT == 1) {
      f[2 * i] = f16_bits_to_f32((uint16_t)(w & 0xFFFFu));
      f[2 * i + 1] = f16_bits_to_f32((uint16_t)(w >> 16));
    } else {
      f[2 * i] = __uint_as_float(w << 16);
      f[2 * i + 1] = __uint_as_float(w & 0xFFFF0000u);
    }
  }
}

template <int DT, int NCH>
__global__ __launch_bounds__(BS) void sparse_attn_kernel(const uint16_t* __restrict__ qa, const uint16_t* __restrict__ kv,
                                                         const int32_t* __restrict__ idx, float* __restrict__ out,
                                                         int64_t n_tok, int64_t n_kv, int H, int L, int k_sel,
                                                         float scale) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int hb = (H + NW - 1) / NW;
  const int64_t t = blockIdx.x / hb;
  const int h = (int)(blockIdx.x % hb) * NW + wv;
  if (h >= H) return;  // (no barriers in this kernel)

  float q[NCH][8];
  bool has[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int d0 = 512 * c + 8 * lane;
    has[c] = d0 < L;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (has[c]) x = *reinterpret_cast<const u32x4*>(qa + ((t * H + h) * L + d0));
    unpack8<DT>(x, q[c]);
  }
  // lane offsets of this lane's chunks in a row (chunks past L read dims
  // 0..7 instead and are multiplied by q = 0)
  int coff[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) coff[c] = has[c] ? 512 * c + 8 * lane : 0;

  float acc[NCH][8];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[c][e] = 0.f;
  float mx = -__builtin_inff(), den = 0.f;

  const int32_t* irow = idx + t * (int64_t)k_sel;
  const int ngroups = (k_sel + G - 1) / G;
  u32x4 ra[G][NCH], rb[G][NCH];
  bool va[G], vb[G];
  auto issue = [&](int grp, u32x4 (&r)[G][NCH], bool (&v)[G]) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int j = grp * G + i;
      const int32_t ri = j < k_sel ? irow[j] : -1;  // (uniform: every lane reads the same entry)
      v[i] = ri >= 0 && (int64_t)ri < n_kv;
      const int64_t row = v[i] ? ri : 0;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        r[i][c] = *reinterpret_cast<const u32x4*>(kv + row * L + coff[c]);   // cached: the query's other heads re-read it
    }
  };
  auto consume = [&](const u32x4 (&r)[G][NCH], const bool (&v)[G]) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      float k[NCH][8];
      float part = 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        unpack8<DT>(r[i][c], k[c]);
#pragma unroll
        for (int e = 0; e < 8; ++e) part = __builtin_fmaf(q[c][e], k[c][e], part);
      }
      part += __uint_as_float(xor_lane_u32<1>(__float_as_uint(part)));
      part += __uint_as_float(xor_lane_u32<2>(__float_as_uint(part)));
      part += __uint_as_float(xor_lane_u32<4>(__float_as_uint(part)));
      part += __uint_as_float(xor_lane_u32<8>(__float_as_uint(part)));
      part += __uint_as_float(xor_lane_u32<16>(__float_as_uint(part)));
      part += __uint_as_float(xor_lane_u32<32>(__float_as_uint(part)));
      if (!v[i]) continue;  // uniform
      const float s = scale * part;
      const float m2 = s > mx ? s : mx;
      const float cf = __expf(mx - m2);  // 0 while mx is -inf
      const float p = __expf(s - m2);
      den = den * cf + p;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[c][e] = __builtin_fmaf(p, k[c][e], acc[c][e] * cf);
      mx = m2;
    }
  };
  if (ngroups > 0) issue(0, ra, va);
  for (int grp = 0; grp < ngroups; grp += 2) {
    if (grp + 1 < ngroups) issue(grp + 1, rb, vb);
    consume(ra, va);
    if (grp + 1 >= ngroups) break;
    if (grp + 2 < ngroups) issue(grp + 2, ra, va);
    consume(rb, vb);
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (!has[c]) continue;
    float* o = out + (t * H + h) * (int64_t)L + 512 * c + 8 * lane;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = acc[c][e] * inv;
  }
}

// ------------------------------------------------------------------ MFMA path
//
// One workgroup of 4 wavefronts per (query t, tile of 64 heads); wavefront w
// owns heads 16 w .. 16 w + 15 of the tile.  The selection is walked in
// blocks of 32 entries.  Per block and wavefront, with v_mfma_f32_16x16x32:
//   S^T (32 keys x 16 heads) = K_blk Q^T: A = key rows (16 B per lane, one
//       ds_read_b128) from the block's rows in LDS, B = this wavefront's q
//       rows, held in registers for the whole walk (16 k-steps of 32 dims);
//   online softmax in f32: lane l has head l % 16 and the block's keys
//       4 (l / 16) + i and 16 + 4 (l / 16) + i (i < 4), so a head's maximum
//       and sum are two cross-lane steps; the running maximum is only moved
//       when the block's maximum exceeds it by more than 8 (weights up to e^8
//       stay exact in f32), so the accumulator is rarely rescaled;
//   O^T (512 dims x 16 heads) += K_blk^T P^T: the MFMA's k-slot
//       8 (l / 16) + j is the key the lane already holds (4 (l / 16) + j, then
//       16 + 4 (l / 16) + j - 4), so P^T never leaves the registers (the sum
//       over k is order-free); A (16 dims x those 8 keys) is read from the same
//       row-major rows by two transposing reads (ds_read_b64_tr_b16: in each
//       16-lane group, lane i names 4 dims of key row i / 4 and receives one
//       dim of all 4 rows), so the block is held in LDS once.
// Gathering: the block's 32 rows go straight from global memory to LDS
// (global_load_lds_dwordx4, one 1 KiB row per instruction, 8 per wavefront),
// the row index broadcast from a vector load of the block's entries made one
// block earlier; no register holds a row and no VALU touches one.  Two LDS
// buffers: block b + 1 is gathered while block b is computed, and one barrier
// per block (after the gather's completion wait) hands the buffers over.
// Row j sits at 1 KiB x j and holds its 16-byte chunk c at position
// c ^ (2 (j mod 8) + (j / 8 mod 2)) (the gather applies this by choosing which
// chunk each lane fetches), which leaves the 4-row transposing reads of O^T
// free of bank conflicts; the 16-byte S^T reads of 16 rows at one column
// still conflict two-way (a 16-byte read goes in 8-byte passes of 32 lanes,
// and 1 KiB rows give those 32 reads only 16 chunk positions).  Every LDS
// address a gather writes stays below 64 KiB.  64 KiB of LDS and at most 256 registers
// per lane, so two workgroups share a compute unit and each hides the other's
// barrier and dependency waits.
// The weights enter the O^T product rounded once to the operand type (bf16
// or f16, as flash-attention kernels do), and the denominator sums the
// rounded weights, so the output is an exact convex combination of the rows
// with each weight off by its one rounding.  (Keeping a second 16-bit part,
// p = hi + lo, would keep about 16 bits per weight at the price of a third
// more MFMAs.)  The S^T phase runs at a raised wave priority: its LDS reads
// are the latency the co-resident workgroup's MFMAs hide.
// Invalid entries are gathered as row 0 and given s = -inf.

constexpr int kAL = 512;               // latent width of this path
constexpr int kAKB = 32;               // selection entries per block
constexpr int kARowBytes = 2 * kAL;    // one gathered row
constexpr int kABufBytes = kAKB * kARowBytes;   // one block's rows
constexpr int kANks = kAL / 32;        // k-steps of S^T
constexpr int kANdt = kAL / 16;        // 16-dim tiles of O^T
constexpr float kAMaxSlack = 8.f;

// chunk swizzle of block row j (0 <= j < 32): chunk c of the row is stored at
// chunk position c ^ attn_swz(j); rows j and 16 + j share it
__host__ __device__ constexpr int attn_swz(int j) { return 2 * (j & 7) + ((j >> 3) & 1); }
static_assert(2 * kABufBytes <= 65536, "the gathers' LDS addresses must stay below 64 KiB");

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int DT> struct AMfma;
template <> struct AMfma<1> {
  typedef f16x8 T;
  static __device__ __forceinline__ f32x4 run(T a, T b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  // nearest 16-bit value of a finite f32 (ties to even), and back
  static __device__ __forceinline__ uint32_t to16(float x) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
  }
  static __device__ __forceinline__ float from16(uint32_t b) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
  }
};
template <> struct AMfma<2> {
  typedef bf16x8 T;
  static __device__ __forceinline__ f32x4 run(T a, T b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t to16(float x) {   // hardware conversion, ties to even
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
  }
  static __device__ __forceinline__ float from16(uint32_t b) { return __uint_as_float(b << 16); }
};

template <int DT>
__global__ __launch_bounds__(256, 2) void sparse_attn_mfma_kernel(const uint16_t* __restrict__ qa,
                                                                  const uint16_t* __restrict__ kv,
                                                                  const int32_t* __restrict__ idx,
                                                                  float* __restrict__ out, int64_t n_kv, int H,
                                                                  int k_sel, float scale) {
  typedef AMfma<DT> M;
  typedef typename M::T T;
  __shared__ __align__(1024) unsigned char rows[2 * kABufBytes];   // [buf][row][chunk position]

  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int g = lane >> 4, r = lane & 15;
  const int nht = (H + 63) / 64;
  const int64_t t = blockIdx.x / nht;
  const int h = (int)(blockIdx.x % nht) * 64 + 16 * w + r;  // this lane's head
  const bool hok = h < H;

  // q^T as the B operand of S^T: B[k = dim 32 ks + 8 g + i][n = head r]
  T qf[kANks];
  {
    const uint16_t* qrow = qa + ((t * H + (hok ? h : 0)) * (int64_t)kAL + 8 * g);
#pragma unroll
    for (int ks = 0; ks < kANks; ++ks) {
      u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 32 * ks);
      if (!hok) x = u32x4{0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(T, x);
    }
  }

  const int32_t* irow = idx + t * (int64_t)k_sel;
  const int nb = (k_sel + kAKB - 1) / kAKB;
  // the selection entry 32 b + (lane mod 32) (clamped: k_sel >= 1 whenever a
  // block exists), one vector load per block
  auto load_idx = [&](int b) -> int32_t {
    const int e = b * kAKB + (lane & (kAKB - 1));
    return irow[e < k_sel ? e : k_sel - 1];
  };
  // bit j: entry 32 b + j is in the selection and names a row
  auto valid_mask = [&](int b, int32_t ix) -> uint32_t {
    const int e = b * kAKB + (lane & (kAKB - 1));
    return (uint32_t)__ballot(e < k_sel && ix >= 0 && (int64_t)ix < n_kv);
  };
  // rows 8 w .. 8 w + 7 of a block into LDS buffer `buf` (invalid entries
  // fetch row 0, which exists: a call with no keys walks no blocks)
  const unsigned char* kvb = reinterpret_cast<const unsigned char*>(kv);
  const uint32_t lds0 = (uint32_t)(uintptr_t)rows;
  // (lane l lands at chunk position l, so it fetches chunk l ^ attn_swz(j))
  auto gather = [&](int buf, int32_t ix, uint32_t vm) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = 8 * w + i;
      const int32_t ri = __builtin_amdgcn_readlane(ix, j);
      const int64_t row = ((vm >> j) & 1u) ? ri : 0;
      dma_row4(kvb + row * kARowBytes, (uint32_t)(16 * (lane ^ attn_swz(j))),
               lds0 + (uint32_t)(buf * kABufBytes + j * kARowBytes));
    }
  };

  // S^T reads row r (and 16 + r), chunk 4 ks + g; the transposing reads name
  // row 4 g + r / 4 (and 16 + that), dims 16 d + 4 (r % 4) .. + 3, i.e. chunk
  // 2 d + (r % 4) / 2, bytes 8 (r % 2) ..
  const int s_row = r * kARowBytes, s_swz = attn_swz(r);
  const int t_rowi = 4 * g + (r >> 2);
  const int t_row = t_rowi * kARowBytes + 8 * (r & 1), t_swz = attn_swz(t_rowi), t_c = (r & 3) >> 1;

  f32x4 acc[kANdt];
#pragma unroll
  for (int d = 0; d < kANdt; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -__builtin_inff(), den = 0.f;

  // S^T of a block: lane gets head r and keys 4 g + i (s0), 16 + 4 g + i
  // (s1); even and odd k-steps in separate chains
  auto scores = [&](int buf, f32x4& s0, f32x4& s1) {
    const unsigned char* base = rows + buf * kABufBytes + s_row;
    // (4 ks + g) ^ swz = 16 (ks / 4) + ((4 (ks % 4) + g) ^ swz): four per-lane
    // bases, the rest an immediate offset
    auto at = [&](int ks) { return base + 16 * ((4 * (ks & 3) + g) ^ s_swz) + 256 * (ks >> 2); };
    f32x4 s2 = {0.f, 0.f, 0.f, 0.f}, s3 = s2;
    s0 = s2;
    s1 = s2;
#pragma unroll
    for (int ks = 0; ks < kANks; ks += 2) {
      const T a0 = __builtin_bit_cast(T, *reinterpret_cast<const u32x4*>(at(ks)));
      const T a1 = __builtin_bit_cast(T, *reinterpret_cast<const u32x4*>(at(ks) + 16 * kARowBytes));
      const T a2 = __builtin_bit_cast(T, *reinterpret_cast<const u32x4*>(at(ks + 1)));
      const T a3 = __builtin_bit_cast(T, *reinterpret_cast<const u32x4*>(at(ks + 1) + 16 * kARowBytes));
      s0 = M::run(a0, qf[ks], s0);
      s1 = M::run(a1, qf[ks], s1);
      s2 = M::run(a2, qf[ks + 1], s2);
      s3 = M::run(a3, qf[ks + 1], s3);
    }
    s0 += s2;
    s1 += s3;
  };
  // online softmax of a block's scores: moves the running maximum (rescaling
  // the accumulator and the denominator when it moves), rounds the block's
  // weights to the operand type, adds the rounded weights to the denominator
  // and returns them
  auto softmax = [&](uint32_t vm, const f32x4& s0, const f32x4& s1, T& phi) {
    const uint32_t f0 = vm >> (4 * g), f1 = vm >> (16 + 4 * g);
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = ((f0 >> i) & 1u) ? scale * s0[i] : -__builtin_inff();
      sv[4 + i] = ((f1 >> i) & 1u) ? scale * s1[i] : -__builtin_inff();
    }
    float bm = sv[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) bm = fmaxf(bm, sv[j]);
    bm = fmaxf(bm, __uint_as_float(xor_lane_u32<16>(__float_as_uint(bm))));
    bm = fmaxf(bm, __uint_as_float(xor_lane_u32<32>(__float_as_uint(bm))));
    const float mn = bm > m + kAMaxSlack ? bm : m;   // m = -inf: takes bm
    const float mref = mn == -__builtin_inff() ? 0.f : mn;
    const float cf = __expf(m - mref);              // m = -inf: 0 (nothing accumulated yet)
    uint32_t hi[8];
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      hi[j] = M::to16(__expf(sv[j] - mref));       // invalid: exp(-inf) = 0
      ps += M::from16(hi[j]);
    }
    ps += __uint_as_float(xor_lane_u32<16>(__float_as_uint(ps)));
    ps += __uint_as_float(xor_lane_u32<32>(__float_as_uint(ps)));
    if (__ballot(mn != m)) {   // some head of this wavefront moved its maximum
      den *= cf;
#pragma unroll
      for (int d = 0; d < kANdt; ++d) acc[d] *= cf;
    }
    den += ps;
    m = mn;
    phi = __builtin_bit_cast(T, u32x4{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16),
                                      hi[6] | (hi[7] << 16)});
  };
  // O^T += K_blk^T P^T: A[m = dim 16 d + r][k-slot 8 g + j] from two
  // transposing reads (keys 4 g .. 4 g + 3, then 16 + 4 g .. 16 + 4 g + 3)
  auto weighted_sum = [&](int buf, const T& phi) {
    const unsigned char* base = rows + buf * kABufBytes + t_row;
    auto afrag = [&](int d) {
      // (2 d + c) ^ swz = 16 (d / 8) + ((2 (d % 8) + c) ^ swz): eight per-lane bases
      const unsigned char* p = base + 16 * ((2 * (d & 7) + t_c) ^ t_swz) + 256 * (d >> 3);
      const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
      const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 16 * kARowBytes));
      const uint2 y0 = __builtin_bit_cast(uint2, x0), y1 = __builtin_bit_cast(uint2, x1);
      return __builtin_bit_cast(T, u32x4{y0.x, y0.y, y1.x, y1.y});
    };
#pragma unroll
    for (int d = 0; d < kANdt; ++d) acc[d] = M::run(afrag(d), phi, acc[d]);
  };

  // Block b: gather block b + 1 into the other buffer (its entries were
  // loaded one block earlier) and load block b + 2's entries, then compute
  // block b; the completion wait and the barrier at the end make block b + 1
  // visible and free block b's buffer for block b + 2.
  int32_t ixn = 0;     // entries of the next block to gather
  uint32_t vmc = 0;    // validity bits of the block being computed
  if (nb > 0) {
    const int32_t ix0 = load_idx(0);
    vmc = valid_mask(0, ix0);
    gather(0, ix0, vmc);
    if (nb > 1) ixn = load_idx(1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  auto block = [&](int b, int buf) {
    uint32_t vmn = 0;
    if (b + 1 < nb) {
      vmn = valid_mask(b + 1, ixn);
      gather(buf ^ 1, ixn, vmn);
      if (b + 2 < nb) ixn = load_idx(b + 2);
    }
    f32x4 s0, s1;
    __builtin_amdgcn_s_setprio(2);
    scores(buf, s0, s1);
    __builtin_amdgcn_s_setprio(0);
    T phi;
    softmax(vmc, s0, s1, phi);
    weighted_sum(buf, phi);
    vmc = vmn;
    if (b + 1 < nb) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
  };
  for (int b = 0; b < nb; b += 2) {
    block(b, 0);
    if (b + 1 < nb) block(b + 1, 1);
  }
  // lane: head r, dims 16 d + 4 g .. + 3
  if (hok) {
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    float* o = out + (t * H + h) * (int64_t)kAL + 4 * g;
#pragma unroll
    for (int d = 0; d < kANdt; ++d)
      *reinterpret_cast<f32x4*>(o + 16 * d) = acc[d] * inv;
  }
}
}  // namespace

hipError_t launch_sparse_attn(const void* qa, const void* kv, const int32_t* idx, float* out, int64_t n_tok,
                              int64_t n_kv, int H, int L, int k_sel, int dtype, float scale, hipStream_t st) {
  const int64_t blocks = n_tok * ((H + NW - 1) / NW);
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(BS);
  const uint16_t* q16 = reinterpret_cast<const uint16_t*>(qa);
  const uint16_t* k16 = reinterpret_cast<const uint16_t*>(kv);
  if (L == kAL) {
    const dim3 mgrid((unsigned)(n_tok * ((H + 63) / 64))), mblock(256);
    if (dtype == 2) hipLaunchKernelGGL((sparse_attn_mfma_kernel<2>), mgrid, mblock, 0, st, q16, k16, idx, out, n_kv, H, k_sel, scale);
    else hipLaunchKernelGGL((sparse_attn_mfma_kernel<1>), mgrid, mblock, 0, st, q16, k16, idx, out, n_kv, H, k_sel, scale);
  } else if (L <= 512) {
    if (dtype == 2) hipLaunchKernelGGL((sparse_attn_kernel<2, 1>), grid, block, 0, st, q16, k16, idx, out, n_tok, n_kv, H, L, k_sel, scale);
    else hipLaunchKernelGGL((sparse_attn_kernel<1, 1>), grid, block, 0, st, q16, k16, idx, out, n_tok, n_kv, H, L, k_sel, scale);
  } else {
    if (dtype == 2) hipLaunchKernelGGL((sparse_attn_kernel<2, 2>), grid, block, 0, st, q16, k16, idx, out, n_tok, n_kv, H, L, k_sel, scale);
    else hipLaunchKernelGGL((sparse_attn_kernel<1, 2>), grid, block, 0, st, q16, k16, idx, out, n_tok, n_kv, H, L, k_sel, scale);
  }
  return hipGetLastError();
}

}  // namespace lid
