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
// a_lo / a_hi: the lane's activation operands of products 0..3 / 4..7 (or the zero bytes),
// sum_off: the block's [group] sums and scales.
__device__ __forceinline__ float mf_block(const MfBlk &b, const uint8_t *lds, uint32_t a_lo,
                                          uint32_t a_hi, uint32_t sum_off, const Q4kField &f0,
                                          const Q4kField &f1) {
  mf_h8 A[8];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    A[t] = *reinterpret_cast<const mf_h8 *>(lds + a_lo + 16 * t);
    A[4 + t] = *reinterpret_cast<const mf_h8 *>(lds + a_hi + 16 * t);
  }
  const mf_f4 sf = *reinterpret_cast<const mf_f4 *>(lds + sum_off);
  const uint32_t qd[8] = {b.qa.x, b.qa.y, b.qa.z, b.qa.w, b.qb.x, b.qb.y, b.qb.z, b.qb.w};
  mf_f4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 4; ++t)
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[t], mf_wop<false>(qd[2 * t], qd[2 * t + 1]), c, 0, 0, 0);
#pragma unroll
  for (int t = 0; t < 4; ++t)
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[4 + t], mf_wop<true>(qd[2 * t], qd[2 * t + 1]), c, 0, 0, 0);
  const uint32_t h0 = b.hdr.x;
  const float d24 = half_bits_to_float(h0) * 0x1p24f, dmin = half_bits_to_float(h0 >> 16);
  float sc_a, m_a, sc_b, m_b;
  q4k_scale_min_at(b.hdr.y, b.hdr.z, b.hdr.w, f0, sc_a, m_a);
  q4k_scale_min_at(b.hdr.y, b.hdr.z, b.hdr.w, f1, sc_b, m_b);
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

template <int KB>
__device__ __forceinline__ void mf_tile(const MfBlk (&buf)[KB], int nb, const uint8_t *lds,
                                        uint32_t a_lo, uint32_t a_hi, uint32_t inc_lo,
                                        uint32_t inc_hi, uint32_t sum_off, const Q4kField &f0,
                                        const Q4kField &f1, float *red, int n16, int g) {
  float acc = 0.f;
#pragma unroll
  for (int b = 0; b < KB; ++b)
    if (b < nb)
      acc += mf_block(buf[b], lds, a_lo + b * inc_lo, a_hi + b * inc_hi, sum_off + b * kMfSumLds,
                      f0, f1);
  acc += xor_recv(acc, 16);
  acc += xor_recv(acc, 32);
  if (g == 0) red[n16] = acc;
}

// Grid: G workgroups, workgroup w taking the 16-row tiles w, w + G, w + 2G, ... (at most
// tiles_per_wg): at any time the workgroups stream neighbouring tiles, one window of the matrix.
// blockDim = 64 * ceil(nblk / KB) (at most 16 waves, so at most 128 VGPRs a lane).
template <int KB>
__global__ __launch_bounds__(1024) void k_gemv_mf(KlMap m, int nblk, int tiles_per_wg,
                                                  const float *__restrict__ x) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = wave_index(), nw = blockDim.x >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const int ntiles = (m.total + 15) >> 4, G = gridDim.x;
  const int nt = min(tiles_per_wg, (ntiles - (int)blockIdx.x + G - 1) / G);  // >= 1
  const int b0 = wave * KB, nb = min(KB, nblk - b0);
  float *red = reinterpret_cast<float *>(lds + kMfZero + nblk * (kMfBlockLds + kMfSumLds));
  auto tile_of = [&](int i) { return (int)blockIdx.x + min(i, nt - 1) * G; };

  // the activations' loads, then the first tile's weights, then the split (which waits for the
  // activations only)
  constexpr int MC = KB >= 2 ? KB / 2 : 1;  // cells per thread: 32 nblk cells, 64 ceil(nblk / KB) threads
  MfCells<MC> cv;
  mf_split_load<MC>(x, nblk, cv);
  MfBlk va[KB];
  mf_load_tile<KB>(m, tile_of(0), b0, nb, n16, g, va);
  mf_split<MC>(cv, nblk, lds);
  __syncthreads();

  // operand rows 4g, 4g+1 take sub-block 2g (products 0..3), rows 4g+2, 4g+3 sub-block 2g+1
  const Q4kField f0 = q4k_field(2 * g), f1 = q4k_field(2 * g + 1);
  const bool mlo = (n16 >> 1) == 2 * g, mhi = (n16 >> 1) == 2 * g + 1;
  const uint32_t own = kMfZero + (uint32_t)b0 * kMfBlockLds + 64u * n16;
  const uint32_t a_lo = mlo ? own : 0u, a_hi = mhi ? own : 0u;
  const uint32_t inc_lo = mlo ? kMfBlockLds : 0u, inc_hi = mhi ? kMfBlockLds : 0u;
  const uint32_t sum_off = kMfZero + nblk * kMfBlockLds + (uint32_t)b0 * kMfSumLds + 16u * g;
  float *wred = red + wave * 16;
  const int wstride = nw * 16;
  if constexpr (KB >= 4) {  // one buffer: such launches take one tile per workgroup
    for (int i = 0; i < nt; ++i) {
      if (i > 0) mf_load_tile<KB>(m, tile_of(i), b0, nb, n16, g, va);  // after this tile's waits
      mf_tile<KB>(va, nb, lds, a_lo, a_hi, inc_lo, inc_hi, sum_off, f0, f1, wred + i * wstride,
                  n16, g);
    }
  } else {  // the next tile's weights in flight while the current one is computed
    // (the loads past the last tile re-read that tile: unconditional, as above)
    MfBlk vb[KB];
    for (int i = 0; i < nt; i += 2) {
      mf_load_tile<KB>(m, tile_of(i + 1), b0, nb, n16, g, vb);
      mf_tile<KB>(va, nb, lds, a_lo, a_hi, inc_lo, inc_hi, sum_off, f0, f1, wred + i * wstride,
                  n16, g);
      if (i + 1 >= nt) break;
      mf_load_tile<KB>(m, tile_of(i + 2), b0, nb, n16, g, va);
      mf_tile<KB>(vb, nb, lds, a_lo, a_hi, inc_lo, inc_hi, sum_off, f0, f1,
                  wred + (i + 1) * wstride, n16, g);
    }
  }
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

int launch_gemv_mf(const KlMap &m, int64_t k, const float *x, hipStream_t s) {
  const int nblk = (int)(k / 256);
  const int kb = mf_kb(nblk);
  const int waves = (nblk + kb - 1) / kb;
  const int ntiles = (m.total + 15) / 16;
  const int target = knob(TQ_KNOB_MF_WGS, 256);
  int tpw = clampi(ntiles / (target > 0 ? target : 1), 1, 16);
  while (tpw > 1 && mf_lds_bytes(nblk, waves, tpw) > 65536) --tpw;
  const int lds = mf_lds_bytes(nblk, waves, tpw);
  if (lds > 65536) return -2;
  const int grid = (ntiles + tpw - 1) / tpw;
  if (kb == 1)
    hipLaunchKernelGGL(k_gemv_mf<1>, dim3(grid), dim3(64 * waves), lds, s, m, nblk, tpw, x);
  else if (kb == 2)
    hipLaunchKernelGGL(k_gemv_mf<2>, dim3(grid), dim3(64 * waves), lds, s, m, nblk, tpw, x);
  else
    hipLaunchKernelGGL(k_gemv_mf<4>, dim3(grid), dim3(64 * waves), lds, s, m, nblk, tpw, x);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace tq
