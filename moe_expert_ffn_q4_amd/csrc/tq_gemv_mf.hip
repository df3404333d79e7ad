// tq_gemv_mf.hip -- batch-1 Q4_K GEMV with the multiply-adds on the fp16 matrix cores.
//
// Per 256-weight block of a row (d, dmin, sub-block scales sc_j and mins m_j, quants q) the product
// with x is  d * sum_j sc_j sum_{k in j} q_k x_k  -  dmin * sum_j m_j S_j  (S_j = sum of x over
// sub-block j, j = 0..7). The inner sums go to v_mfma_f32_16x16x32_f16:
//   * weight operand (B, 32 k x 16 rows): the nibbles themselves, as fp16 subnormals q * 2^-24
//     (a word masked with 0x000F000F is two of them; with 0x00F000F0, two of 16 q * 2^-24), so
//     building it takes a few AND/shift operations per 8 weights and nothing else;
//   * activation operand (A, 16 operand rows x 32 k): the sub-block's x scaled by a power of two
//     2^e (e per sub-block, bringing its max |x| into [2^14, 2^15)) and split into two fp16 halves,
//     hi = fp16(x 2^e) and lo = fp16(x 2^e - hi); operand row 2 j + h (h = 0 hi, 1 lo) is non-zero
//     only in the k positions that hold sub-block j's weights, so one product per 32 k separates all
//     eight sub-blocks of a block in its output rows and a block's eight products accumulate into
//     one 16x16 fp32 tile.
// Lane l of the wave holds weight row n = l % 16 and group g = l / 16 of every block (quant bytes
// 32 g .. 32 g + 31, i.e. sub-blocks 2 g and 2 g + 1); product t = 0..3 takes dwords 2t, 2t + 1 of
// the group's low nibbles (sub-block 2 g), t = 4..7 the high nibbles (sub-block 2 g + 1). The output
// lane l then holds operand rows 4 g .. 4 g + 3 of row n, i.e. exactly the hi and lo sums of the
// two sub-blocks whose scales and mins sit in the header that lane loaded, and folds them:
//   d * 2^24 * sc_j f_j (C_hi + C_lo) - dmin * m_j S_j     (f_j = 2^-e_j)
// (with a factor 1/16 on the high-nibble sub-block). The products are exact (an fp16 subnormal
// quant times an 11-bit fp16 value), they add in fp32, and x enters with 22 significant bits.
//
// Work split: a workgroup takes whole 16-row tiles and all of k. It first splits x into the
// operand layout in LDS (with the zero bytes the empty operand rows read), then wave w streams
// blocks [w KB, w KB + KB) of its tiles, the next tile's weights loaded while it computes the
// current one, and leaves one partial sum per row in LDS; after one barrier the workgroup adds the
// waves' partial sums in wave order and stores the rows. Nothing is split across workgroups, so a
// row's sum is formed the same way whatever the matrix height, the part it falls in or the launch.
#include <hip/hip_runtime.h>

#include <utility>

#include "tq_device.h"
#include "tq_gemv_core.h"
#include "tq_gemv_mf.h"
#include "tq_launch.h"

namespace tq {

typedef _Float16 mf_h8 __attribute__((ext_vector_type(8)));
typedef float mf_f4 __attribute__((ext_vector_type(4)));

constexpr int kMfZero = 64;         // zero bytes at the start of LDS
constexpr int kMfBlockLds = 1024;   // one block's activation operands: 8 sub-blocks x hi/lo x 4 x 16 B
constexpr int kMfSumLds = 64;       // one block's [group][S_2g, S_2g+1, f_2g, f_2g+1]

// LDS bytes of a workgroup: zeros, operands, sums and scales, the waves' partial sums.
__host__ __device__ inline int mf_lds_bytes(int nblk, int waves, int tiles) {
  return kMfZero + nblk * (kMfBlockLds + kMfSumLds) + tiles * waves * 16 * 4;
}

// One block of one row as the lane loads it: header (d, dmin, packed scales) and its group's 32
// quant bytes.
struct MfBlk {
  u32x4 hdr, qa, qb;
};

// 1. x -> operand layout. Cell c = (block b, sub-block j, quarter u) holds positions 8u .. 8u + 7
// of the sub-block, in the order the weight operand takes them (a masked word holds the nibbles of
// bytes 0 and 2, the word shifted by 8 those of bytes 1 and 3): 0 2 1 3 4 6 5 7. Thread t takes
// cells t, t + blockDim, ... (at most MC); four neighbouring threads take the four quarters of one
// sub-block, and whole quads are in or out of range together. The values are loaded before the
// weights (mf_split_load), so that the split waits only for them.
template <int MC>
struct MfCells {
  float4 v[MC][2];
};
template <int MC>
__device__ __forceinline__ void mf_split_load(const float *__restrict__ x, int nblk, MfCells<MC> &c) {
  const int cells = nblk * 32;
#pragma unroll
  for (int i = 0; i < MC; ++i) {  // unconditional (clamped): the compiler then counts them
    const int ci = min((int)threadIdx.x + i * (int)blockDim.x, cells - 1);
    const float4 *src = reinterpret_cast<const float4 *>(x + 8 * ci);
    c.v[i][0] = src[0];
    c.v[i][1] = src[1];
  }
}
template <int MC>
__device__ __forceinline__ void mf_split(const MfCells<MC> &cv, int nblk, uint8_t *lds) {
  if (threadIdx.x < kMfZero / 16) *reinterpret_cast<u32x4 *>(lds + 16 * threadIdx.x) = u32x4{0, 0, 0, 0};
  const int cells = nblk * 32;
  uint8_t *ops = lds + kMfZero;
  float *sums = reinterpret_cast<float *>(lds + kMfZero + nblk * kMfBlockLds);
#pragma unroll
  for (int i = 0; i < MC; ++i) {
    const int c = threadIdx.x + i * blockDim.x;
    if (c >= cells) break;
    const float4 v0 = cv.v[i][0], v1 = cv.v[i][1];
    float m = fmaxf(fmaxf(fmaxf(fabsf(v0.x), fabsf(v0.y)), fmaxf(fabsf(v0.z), fabsf(v0.w))),
                    fmaxf(fmaxf(fabsf(v1.x), fabsf(v1.y)), fmaxf(fabsf(v1.z), fabsf(v1.w))));
    m = fmaxf(m, xor_recv(m, 1));
    m = fmaxf(m, xor_recv(m, 2));
    int e = 0;
    if (m > 0.f) {
      int ex;
      frexpf(m, &ex);  // m in [2^(ex-1), 2^ex)
      e = min(max(15 - ex, -126), 126);
    }
    const float s = ldexpf(1.f, e);
    // hi: x 2^e with its low 13 significand bits cleared, an fp16 value when |x 2^e| >= 2^-14 (else
    // fp16 keeps fewer bits and the difference, below 2^-24 against a sub-block max of at least
    // 2^14, is dropped); lo = x 2^e - hi exactly, rounded to fp16 (toward zero)
    const float xs[8] = {v0.x * s, v0.z * s, v0.y * s, v0.w * s,
                         v1.x * s, v1.z * s, v1.y * s, v1.w * s};  // order 0 2 1 3 4 6 5 7
    float hf[8], lf[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      hf[k] = __uint_as_float(__float_as_uint(xs[k]) & 0xFFFFE000u);
      lf[k] = xs[k] - hf[k];
    }
    u32x4 hi, lo;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      hi[k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(hf[2 * k], hf[2 * k + 1]));
      lo[k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lf[2 * k], lf[2 * k + 1]));
    }
    const int b = c >> 5, j = (c >> 2) & 7, u = c & 3;
    uint8_t *dst = ops + b * kMfBlockLds + (4 * (2 * j) + u) * 16;
    *reinterpret_cast<u32x4 *>(dst) = hi;
    *reinterpret_cast<u32x4 *>(dst + 64) = lo;
    float sum = ((v0.x + v0.y) + (v0.z + v0.w)) + ((v1.x + v1.y) + (v1.z + v1.w));
    sum += xor_recv(sum, 1);
    sum += xor_recv(sum, 2);
    if (u == 0) {
      float *q = sums + b * 16 + (j >> 1) * 4;
      q[j & 1] = sum;
      q[2 + (j & 1)] = ldexpf(1.f, -e);
    }
  }
}

// 2. the lane's loads of one block of its tile row
__device__ __forceinline__ void mf_load_blk(const uint8_t *p, int g, MfBlk &b) {
  b.hdr = gload(p);
  b.qa = gload(p + 16 + 32 * g);
  b.qb = gload(p + 32 + 32 * g);
}

// The weight operand of product t from the lane's two quant dwords (low or high nibbles).
template <bool HIGH>
__device__ __forceinline__ mf_h8 mf_wop(uint32_t d0, uint32_t d1) {
  constexpr uint32_t M = HIGH ? 0x00F000F0u : 0x000F000Fu;
  const u32x4 v = {d0 & M, (d0 >> 8) & M, d1 & M, (d1 >> 8) & M};
  return __builtin_bit_cast(mf_h8, v);
}

// 3. one block: eight products into one tile, then the fold of the lane's two sub-blocks.
// The lane's activation operands of one block (products 0..3 from its a_lo, 4..7 from its a_hi:
// its own operand row, or the zero bytes) and the block's sums and scales of its group.
struct MfAct {
  mf_h8 A[8];
  mf_f4 sf;
};
__device__ __forceinline__ void mf_act_load(const uint8_t *lds, uint32_t a_lo, uint32_t a_hi,
                                            uint32_t sum_off, MfAct &a) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    a.A[t] = *reinterpret_cast<const mf_h8 *>(lds + a_lo + 16 * t);
    a.A[4 + t] = *reinterpret_cast<const mf_h8 *>(lds + a_hi + 16 * t);
  }
  a.sf = *reinterpret_cast<const mf_f4 *>(lds + sum_off);
}
__device__ __forceinline__ float mf_block(const MfBlk &b, const MfAct &a, const Q4kField &f0,
                                          const Q4kField &f1) {
  const uint32_t qd[8] = {b.qa.x, b.qa.y, b.qa.z, b.qa.w, b.qb.x, b.qb.y, b.qb.z, b.qb.w};
  mf_f4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 4; ++t)
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.A[t], mf_wop<false>(qd[2 * t], qd[2 * t + 1]), c, 0, 0, 0);
#pragma unroll
  for (int t = 0; t < 4; ++t)
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.A[4 + t], mf_wop<true>(qd[2 * t], qd[2 * t + 1]), c, 0, 0, 0);
  const uint32_t h0 = b.hdr.x;
  const float d24 = half_bits_to_float(h0) * 0x1p24f, dmin = half_bits_to_float(h0 >> 16);
  float sc_a, m_a, sc_b, m_b;
  q4k_scale_min_at(b.hdr.y, b.hdr.z, b.hdr.w, f0, sc_a, m_a);
  q4k_scale_min_at(b.hdr.y, b.hdr.z, b.hdr.w, f1, sc_b, m_b);
  const mf_f4 sf = a.sf;
  const float pa = d24 * sc_a * sf[2], pb = d24 * sc_b * 0.0625f * sf[3];
  const float mn = __builtin_fmaf(m_a, sf[0], m_b * sf[1]);
  return __builtin_fmaf(pa, c[0] + c[1], __builtin_fmaf(pb, c[2] + c[3], -dmin * mn));
}

// Every block slot is loaded (past the wave's last block: that block again), so that no load sits
// behind a branch: the compiler then counts the loads in flight and waits for each block's own.
template <int KB>
__device__ __forceinline__ void mf_load_tile(const KlMap &m, int tile, int b0, int nb, int n16,
                                             int g, MfBlk (&buf)[KB]) {
  const uint8_t *rp = m.row(min(tile * 16 + n16, m.total - 1)) + (int64_t)b0 * 144;
#pragma unroll
  for (int b = 0; b < KB; ++b) mf_load_blk(rp + min(b, nb - 1) * 144, g, buf[b]);
}

// The sum of v over lanes l and l ^ 16 (SWAP16) or l and l ^ 32, by a lane swap between rows
// of 16 (or halves of 32) lanes: each lane gets its own value and its partner's, and their sum
// is the same in both lanes.
template <bool SWAP16>
__device__ __forceinline__ float mf_pair_sum(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto sw = SWAP16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                         : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)sw[0]) + __builtin_bit_cast(float, (unsigned)sw[1]);
}

// One tile's blocks of the wave (the activation operands read from LDS per block: holding them
// in registers across tiles measured no faster), then the sum over the lane's four groups.
template <int KB>
__device__ __forceinline__ void mf_tile(const MfBlk (&buf)[KB], int nb, const uint8_t *lds,
                                        uint32_t a_lo, uint32_t a_hi, uint32_t inc_lo,
                                        uint32_t inc_hi, uint32_t sum_off, const Q4kField &f0,
                                        const Q4kField &f1, float *red, int n16, int g,
                                        bool keep) {
  float acc = 0.f;
#pragma unroll
  for (int b = 0; b < KB; ++b)
    if (b < nb) {
      MfAct a;
      mf_act_load(lds, a_lo + b * inc_lo, a_hi + b * inc_hi, sum_off + b * kMfSumLds, a);
      acc += mf_block(buf[b], a, f0, f1);
    }
  acc = mf_pair_sum<true>(acc);   // groups 0 + 1, 2 + 3
  acc = mf_pair_sum<false>(acc);  // (0 + 1) + (2 + 3)
  if (keep && g == 0) red[n16] = acc;
}

template <int N, class F, int... I>
__device__ __forceinline__ void mf_unroll_(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(std::integral_constant<int, i>) for i = 0 .. N-1, in order
template <int N, class F>
__device__ __forceinline__ void mf_unroll(F &&f) {
  mf_unroll_<N>(f, std::make_integer_sequence<int, N>{});
}

// Grid: G workgroups, workgroup w taking the 16-row tiles w, w + G, w + 2G, ... (TPW of them, or
// fewer for the grid's last workgroups): at any time the workgroups stream neighbouring tiles, one
// window of the matrix. blockDim = 64 * ceil(nblk / KB): at most 16 waves (128 VGPRs a lane), at
// most 8 when DEPTH = 2 (256). DEPTH 0 (one buffer): each tile after the first is loaded just
// before its products.
// The tiles' code is straight-line (TPW and the buffer of each tile fixed at compile time), with
// the weights of the next DEPTH tiles in flight while a tile is computed: the compiler then counts
// every load in flight and waits for each tile's own. (In a loop, loads carried across the back
// edge and the joins of the buffers' values make it wait for all loads before the next prefetch.)
// A workgroup with fewer than TPW tiles loads its last tile again for the missing ones and does
// not keep their sums.
template <int KB, int TPW, int DEPTH>
__global__ __launch_bounds__(DEPTH > 1 ? 512 : 1024) void k_gemv_mf(KlMap m, int nblk,
                                                                    const float *__restrict__ x) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = wave_index(), nw = blockDim.x >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const int ntiles = (m.total + 15) >> 4, G = gridDim.x;
  const int nt = min(TPW, (ntiles - (int)blockIdx.x + G - 1) / G);  // >= 1
  const int b0 = wave * KB, nb = min(KB, nblk - b0);
  float *red = reinterpret_cast<float *>(lds + kMfZero + nblk * (kMfBlockLds + kMfSumLds));
  auto tile_of = [&](int i) { return (int)blockIdx.x + min(i, nt - 1) * G; };

  // operand rows 4g, 4g+1 take sub-block 2g (products 0..3), rows 4g+2, 4g+3 sub-block 2g+1
  const Q4kField f0 = q4k_field(2 * g), f1 = q4k_field(2 * g + 1);
  const bool mlo = (n16 >> 1) == 2 * g, mhi = (n16 >> 1) == 2 * g + 1;
  const uint32_t own = kMfZero + (uint32_t)b0 * kMfBlockLds + 64u * n16;
  const uint32_t a_lo = mlo ? own : 0u, a_hi = mhi ? own : 0u;
  const uint32_t inc_lo = mlo ? kMfBlockLds : 0u, inc_hi = mhi ? kMfBlockLds : 0u;
  const uint32_t sum_off = kMfZero + nblk * kMfBlockLds + (uint32_t)b0 * kMfSumLds + 16u * g;
  float *wred = red + wave * 16;
  const int wstride = nw * 16;

  // the activations' loads, the first DEPTH tiles' weights, then the split (waiting for the
  // activations only)
  constexpr int MC = KB >= 2 ? KB / 2 : 1;  // cells per thread: 32 nblk cells, 64 ceil(nblk / KB) threads
  constexpr int NB = DEPTH + 1;             // weight buffers
  constexpr int PRE = DEPTH > 1 ? DEPTH : 1;  // tiles loaded before the split
  MfCells<MC> cv;
  mf_split_load<MC>(x, nblk, cv);
  MfBlk buf[NB][KB];
  mf_unroll<PRE>([&](auto T) {
    constexpr int t = decltype(T)::value;
    if constexpr (t < TPW) mf_load_tile<KB>(m, tile_of(t), b0, nb, n16, g, buf[t % NB]);
  });
  mf_split<MC>(cv, nblk, lds);
  __syncthreads();
  mf_unroll<TPW>([&](auto T) {
    constexpr int t = decltype(T)::value;
    if constexpr (t + DEPTH < TPW && t + DEPTH >= PRE)  // (DEPTH 0: tile t, just before its use)
      mf_load_tile<KB>(m, tile_of(t + DEPTH), b0, nb, n16, g, buf[(t + DEPTH) % NB]);
    mf_tile<KB>(buf[t % NB], nb, lds, a_lo, a_hi, inc_lo, inc_hi, sum_off, f0, f1,
                wred + t * wstride, n16, g, t < nt);
  });
  __syncthreads();

  // 4. the rows: the waves' partial sums in wave order
  const int rows = nt * 16;
  if (m.swiglu) {  // virtual rows (gate r, up r) pairs; tiles start at even rows
    for (int i = 2 * (int)threadIdx.x; i < rows; i += 2 * (int)blockDim.x) {
      const int v = tile_of(i >> 4) * 16 + (i & 15);
      if (v >= m.total) continue;
      const float *r = red + (i >> 4) * wstride + (i & 15);
      float gs = 0.f, us = 0.f;
      for (int w = 0; w < nw; ++w) {
        gs += r[w * 16];
        us += r[w * 16 + 1];
      }
      gstore(m.swiglu_out(v >> 1), silu_mul(gs, us));
    }
  } else {
    for (int i = threadIdx.x; i < rows; i += blockDim.x) {
      const int v = tile_of(i >> 4) * 16 + (i & 15);
      if (v >= m.total) continue;
      const float *r = red + (i >> 4) * wstride + (i & 15);
      float s = 0.f;
      for (int w = 0; w < nw; ++w) s += r[w * 16];
      m.put(v, s);
    }
  }
}

// ---- host side ----------------------------------------------------------------------------------

// Blocks per wave: 1 up to k = 2048, 2 up to k = 8192, else 4 (at most 16 waves, k < 16384).
static int mf_kb(int nblk) {
  const int v = knob(TQ_KNOB_MF_KB, 0);
  int kb = v == 1 || v == 2 || v == 4 ? v : nblk <= 8 ? 1 : nblk <= 32 ? 2 : 4;
  while ((nblk + kb - 1) / kb > 16) kb *= 2;
  return kb;
}

// k < 16384 whose operands fit 64 KB of LDS with one tile per workgroup (k <= 15104)
bool mf_gemv_ok(int64_t k) {
  if (!knob(TQ_KNOB_GEMV_MF, 1) || k % 256 != 0 || k < 256 || k >= 16384) return false;
  const int nblk = (int)(k / 256), kb = mf_kb(nblk);
  return kb <= 4 && mf_lds_bytes(nblk, (nblk + kb - 1) / kb, 1) <= 65536;
}

// Tiles per workgroup that have a kernel (the next one up is taken).
constexpr int kMfTpw[] = {1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 14, 16};

template <int KB, int DEPTH>
static void mf_launch_kb(int tpw, dim3 gd, dim3 bd, int lds, hipStream_t s, const KlMap &m,
                         int nblk, const float *x) {
  switch (tpw) {
#define TQ_MF(T) \
  case T: hipLaunchKernelGGL((k_gemv_mf<KB, T, DEPTH>), gd, bd, lds, s, m, nblk, x); break;
    TQ_MF(1) TQ_MF(2) TQ_MF(3) TQ_MF(4) TQ_MF(5) TQ_MF(6) TQ_MF(7) TQ_MF(8) TQ_MF(10) TQ_MF(12)
    TQ_MF(14) TQ_MF(16)
#undef TQ_MF
  }
}

int launch_gemv_mf(const KlMap &m, int64_t k, const float *x, hipStream_t s) {
  const int nblk = (int)(k / 256);
  const int kb = mf_kb(nblk);
  const int waves = (nblk + kb - 1) / kb;
  const int ntiles = (m.total + 15) / 16;
  const int target = knob(TQ_KNOB_MF_WGS, 256);
  const int want = clampi((ntiles + target - 1) / (target > 0 ? target : 1), 1, 16);
  int ti = 0;
  while (kMfTpw[ti] < want) ++ti;
  while (ti > 0 && mf_lds_bytes(nblk, waves, kMfTpw[ti]) > 65536) --ti;
  const int tpw = kMfTpw[ti];
  const int lds = mf_lds_bytes(nblk, waves, tpw);
  if (lds > 65536) return -2;
  const int grid = (ntiles + tpw - 1) / tpw;
  const dim3 gd(grid), bd(64 * waves);
  // two tiles ahead where the workgroup has several tiles and at most 8 waves (256 VGPRs a lane)
  const bool deep = kb == 2 && waves <= 8 && tpw >= 3 && knob(TQ_KNOB_MF_DEEP, 1);
  if (kb == 1)
    mf_launch_kb<1, 1>(tpw, gd, bd, lds, s, m, nblk, x);
  else if (kb == 2 && deep)
    mf_launch_kb<2, 2>(tpw, gd, bd, lds, s, m, nblk, x);
  else if (kb == 2)
    mf_launch_kb<2, 1>(tpw, gd, bd, lds, s, m, nblk, x);
  else
    mf_launch_kb<4, 0>(tpw, gd, bd, lds, s, m, nblk, x);  // one buffer (128 VGPRs)
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace tq
