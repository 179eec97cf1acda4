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
//   S^T (32 keys x 16 heads) = K_blk Q^T: A = key rows (16 B per lane) from
//       a row-major LDS copy of the block, B = this wavefront's q rows, held
//       in registers for the whole walk (16 k-steps of 32 dims);
//   online softmax in f32: lane l has head l % 16 and the block's keys
//       4 (l / 16) + i and 16 + 4 (l / 16) + i (i < 4), so a head's maximum
//       and sum are two cross-lane steps; the running maximum is only moved
//       when the block's maximum exceeds it by more than 8 (weights up to e^8
//       stay exact in f32), so the accumulator is rarely rescaled;
//   O^T (512 dims x 16 heads) += K_blk^T P^T: the MFMA's k-slot
//       8 (l / 16) + j is the key the lane already holds (4 (l / 16) + j, then
//       16 + 4 (l / 16) + j - 4), so P^T never leaves the registers (the sum
//       over k is order-free); A comes from a second, transposed LDS copy of
//       the block whose rows (one per latent dim) list the keys in that
//       order, so each A fragment is one 16-byte read.
// Gathering: wavefront w loads the rows of keys 4 w .. 4 w + 3 and
// 16 + 4 w .. 16 + 4 w + 3 (1 KiB per row per instruction), which are
// exactly the 8 keys of one 16-byte chunk of the transposed rows, into
// registers three blocks ahead (their indices four blocks ahead), and writes
// both LDS copies (double-buffered) two blocks ahead.  The blocks are
// software-pipelined: block b + 1's S^T and softmax run beside block b's
// weighted sum.  The transposed rows (80 B pitch) swizzle their four chunks
// by (dim / 8) mod 4 so that both the writes (lanes 8 dims apart) and the
// reads (16 consecutive dims) spread over the banks.
// The weights are split into two 16-bit parts, p = hi + lo (lo = the
// rounding residual of hi), and both are multiplied in, so the weighted sum
// keeps about 16 bits of each weight instead of the 8 of a single bf16; the
// denominator sums hi + lo, the weights actually applied.
// Invalid entries are gathered as row 0 and given s = -inf.

constexpr int kAL = 512;               // latent width of this path
constexpr int kAKB = 32;               // selection entries per block
constexpr int kAPitch = kAL + 8;       // row-major copy: row pitch in 16-bit elements (1040 B)
constexpr int kATPitch = 40;           // transposed copy: row pitch in 16-bit elements (80 B)
constexpr int kANks = kAL / 32;        // k-steps of S^T
constexpr int kANdt = kAL / 16;        // 16-dim tiles of O^T
constexpr float kAMaxSlack = 8.f;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

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

// block key of k-slot j (0..7) of lane group g (0..3)
__device__ __forceinline__ int attn_key(int g, int j) { return j < 4 ? 4 * g + j : 12 + 4 * g + j; }

template <int DT>
__global__ __launch_bounds__(256, 1) void sparse_attn_mfma_kernel(const uint16_t* __restrict__ qa,
                                                                  const uint16_t* __restrict__ kv,
                                                                  const int32_t* __restrict__ idx,
                                                                  float* __restrict__ out, int64_t n_kv, int H,
                                                                  int k_sel, float scale) {
  typedef AMfma<DT> M;
  typedef typename M::T T;
  __shared__ __align__(16) uint16_t krow[2][kAKB][kAPitch];   // [buf][key][dim]
  __shared__ __align__(16) uint16_t kt[2][kAL][kATPitch];     // [buf][dim][key, in k-slot order, swizzled]
  __shared__ __align__(4) uint8_t vflag[2][kAKB];

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
  // a block's gathered rows in registers: keys attn_key(w, i), dims 8 lane ..
  // 8 lane + 7, and their validity bits
  struct Rows {
    u32x4 st[8];
    uint32_t vm;
  };
  // the selection entries of a block's rows, read one block ahead of the rows
  // themselves by one vector load (lane i < 8 holds entry attn_key(w, i);
  // clamped, so no branch: k_sel >= 1 whenever a block exists) and broadcast
  // with readlane when the rows are fetched, so the row loads never wait on
  // them (a scalar load would be waited for with the LDS reads)
  int32_t ixv = 0;
  auto load_idx = [&](int b) {
    const int e = b * kAKB + attn_key(w, lane & 7);
    ixv = irow[e < k_sel ? e : k_sel - 1];
  };
  auto fetch = [&](int b, Rows& R) {
    uint32_t vm = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = b * kAKB + attn_key(w, i);
      const int32_t ri = __builtin_amdgcn_readlane(ixv, i);
      const bool v = e < k_sel && ri >= 0 && (int64_t)ri < n_kv;
      vm |= (uint32_t)v << i;
      const int64_t row = v ? ri : 0;
      R.st[i] = *reinterpret_cast<const u32x4*>(kv + row * kAL + 8 * lane);
    }
    R.vm = vm;
  };
  auto stage = [&](int buf, const Rows& R) {
    const u32x4* st = R.st;
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(&krow[buf][attn_key(w, i)][8 * lane]) = st[i];
    // transposed: dim 8 lane + c gets the 8 keys of chunk w (swizzled by lane & 3)
    const int chunk = w ^ (lane & 3);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int q = c >> 1;
      uint32_t x[4];
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        const uint32_t a = st[2 * k2][q], b = st[2 * k2 + 1][q];
        x[k2] = (c & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
      }
      *reinterpret_cast<u32x4*>(&kt[buf][8 * lane + c][8 * chunk]) = u32x4{x[0], x[1], x[2], x[3]};
    }
    if (lane < 8) vflag[buf][attn_key(w, lane)] = (uint8_t)((R.vm >> lane) & 1u);
  };

  f32x4 acc[kANdt];
#pragma unroll
  for (int d = 0; d < kANdt; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -__builtin_inff(), den = 0.f;

  // S^T of a staged block: lane gets head r and keys 4 g + i (s0), 16 + 4 g + i
  // (s1); even and odd k-steps in separate chains
  auto scores = [&](int buf, f32x4& s0, f32x4& s1) {
    f32x4 s2 = {0.f, 0.f, 0.f, 0.f}, s3 = s2;
    s0 = s2;
    s1 = s2;
#pragma unroll
    for (int ks = 0; ks < kANks; ks += 2) {
      const T a0 = __builtin_bit_cast(T, *reinterpret_cast<const u32x4*>(&krow[buf][r][32 * ks + 8 * g]));
      const T a1 = __builtin_bit_cast(T, *reinterpret_cast<const u32x4*>(&krow[buf][16 + r][32 * ks + 8 * g]));
      const T a2 = __builtin_bit_cast(T, *reinterpret_cast<const u32x4*>(&krow[buf][r][32 * ks + 32 + 8 * g]));
      const T a3 = __builtin_bit_cast(T, *reinterpret_cast<const u32x4*>(&krow[buf][16 + r][32 * ks + 32 + 8 * g]));
      s0 = M::run(a0, qf[ks], s0);
      s1 = M::run(a1, qf[ks], s1);
      s2 = M::run(a2, qf[ks + 1], s2);
      s3 = M::run(a3, qf[ks + 1], s3);
    }
    s0 += s2;
    s1 += s3;
  };
  // online softmax of a block's scores: moves the running maximum (rescaling
  // the accumulator and the denominator when it moves), adds the block's
  // weights to the denominator and returns them as the two 16-bit parts
  auto softmax = [&](int buf, const f32x4& s0, const f32x4& s1, T& phi, T& plo) {
    const uint32_t f0 = *reinterpret_cast<const uint32_t*>(&vflag[buf][4 * g]);
    const uint32_t f1 = *reinterpret_cast<const uint32_t*>(&vflag[buf][16 + 4 * g]);
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = ((f0 >> (8 * i)) & 1u) ? scale * s0[i] : -__builtin_inff();
      sv[4 + i] = ((f1 >> (8 * i)) & 1u) ? scale * s1[i] : -__builtin_inff();
    }
    float bm = sv[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) bm = fmaxf(bm, sv[j]);
    bm = fmaxf(bm, __uint_as_float(xor_lane_u32<16>(__float_as_uint(bm))));
    bm = fmaxf(bm, __uint_as_float(xor_lane_u32<32>(__float_as_uint(bm))));
    const float mn = bm > m + kAMaxSlack ? bm : m;   // m = -inf: takes bm
    const float mref = mn == -__builtin_inff() ? 0.f : mn;
    const float cf = __expf(m - mref);              // m = -inf: 0 (nothing accumulated yet)
    uint32_t hi[8], lo[8];
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = __expf(sv[j] - mref);         // invalid: exp(-inf) = 0
      hi[j] = M::to16(p);
      const float ph = M::from16(hi[j]);
      lo[j] = M::to16(p - ph);
      ps += ph + M::from16(lo[j]);
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
    plo = __builtin_bit_cast(T, u32x4{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16),
                                      lo[6] | (lo[7] << 16)});
  };
  // O^T += K_blk^T P^T: A[m = dim 16 d + r][k-slot 8 g + j], one 16-byte read;
  // the lo product of tile d - 1 is issued between the hi products of tiles d
  // and d + 1, so no MFMA waits on the one just before it
  auto weighted_sum = [&](int buf, const T& phi, const T& plo) {
    auto afrag = [&](int d) {
      const int dim = 16 * d + r;
      const int chunk = g ^ ((dim >> 3) & 3);
      return __builtin_bit_cast(T, *reinterpret_cast<const u32x4*>(&kt[buf][dim][8 * chunk]));
    };
    T aprev = afrag(0);
    acc[0] = M::run(aprev, phi, acc[0]);
#pragma unroll
    for (int d = 1; d < kANdt; ++d) {
      const T a = afrag(d);
      acc[d] = M::run(a, phi, acc[d]);
      acc[d - 1] = M::run(aprev, plo, acc[d - 1]);
      aprev = a;
    }
    acc[kANdt - 1] = M::run(aprev, plo, acc[kANdt - 1]);
  };

  // Software pipeline over the blocks: iteration b runs block b + 1's scores
  // and softmax beside block b's weighted sum, so the softmax arithmetic and
  // the LDS latencies overlap the MFMAs.  Both LDS buffers hold staged blocks
  // (b and b + 1); block b + 2 is staged into b's buffers once every
  // wavefront is done with them.  Rows are gathered three blocks ahead into
  // two register sets used in turn (block j's rows in set j mod 2; the loop
  // is unrolled by two so that the sets are fixed registers), their indices
  // one block ahead of the rows.
  Rows ra, rb;
  T phi = {}, plo = {};
  if (nb > 0) {
    load_idx(0);
    fetch(0, ra);
    stage(0, ra);
    if (nb > 1) {
      load_idx(1);
      fetch(1, rb);
      stage(1, rb);
    }
    if (nb > 2) {
      load_idx(2);
      fetch(2, ra);
    }
    if (nb > 3) load_idx(3);
    __syncthreads();
    f32x4 s0, s1;
    scores(0, s0, s1);
    softmax(0, s0, s1, phi, plo);
  }
  // rstage holds block b + 2's rows; rfetch (block b + 1's, staged) takes block b + 3's
  auto block = [&](int b, const Rows& rstage, Rows& rfetch) {
    const int buf = b & 1;
    if (b + 3 < nb) fetch(b + 3, rfetch);
    if (b + 4 < nb) load_idx(b + 4);
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
    if (b + 1 < nb) scores(buf ^ 1, s0, s1);
    weighted_sum(buf, phi, plo);
    if (b + 1 < nb) softmax(buf ^ 1, s0, s1, phi, plo);
    if (b + 2 < nb) {
      __syncthreads();   // every wavefront is done with block b's buffers
      stage(buf, rstage);
      __syncthreads();   // block b + 2 is visible
    }
  };
  for (int b = 0; b < nb; b += 2) {
    block(b, ra, rb);
    if (b + 1 < nb) block(b + 1, rb, ra);
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
