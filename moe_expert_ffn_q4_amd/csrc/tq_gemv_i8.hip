// tq_gemv_i8.hip -- batch-1 Q4_K GEMV with the multiply-adds on the int8 matrix cores.
//
// Per 256-weight block of a row (d, dmin, sub-block scales sc_j and mins m_j, quants q) the product
// with x is  d * sum_j sc_j sum_{k in j} q_k x_k  -  dmin * sum_j m_j S_j  (S_j = sum of x over
// sub-block j). The inner sums go to v_mfma_i32_32x32x32_i8 with exact integers on both sides:
//   * the quants are the nibbles themselves (a mask of 0x0F0F0F0F yields four int8 operands);
//   * each 256-value block of x is scaled by its own power of two 2^e and rounded to integers x'
//     with |x'| < 2^27, written as four signed 7-bit digits, x' = c0 + 2^7 c1 + 2^14 c2 + 2^21 c3
//     (c0..c2 in [-64, 63]). e is the smaller of the value that brings the block's max|x| into
//     [2^26, 2^27) and the number of fractional bits the block's values need, so blocks of
//     integers (or of values with few significant bits) stay exact.
// One 32-k step of the matrix cores is exactly one sub-block: weight operand = 32 rows x 32 k
// (lane l: row l % 32, k = 16 (l / 32) .. +15 of the sub-block), activation operand = 32 rows of
// (sub-block j', digit d) = 4 j' + d, non-zero only in the rows of the step's own sub-block, so
// the 32x32 int32 accumulator of a block holds sum_{k in j} c_d q_k for all 8 sub-blocks x 4
// digits x 32 rows and is folded once per block: lane l (row l % 32, parity h = l / 32) holds
// sub-blocks 2q + h, q = 0..3, and adds d * sc_j * (its four digit sums recombined) and
// -dmin * m_j * S_j, both times the block's 2^-e. Everything before the fold is exact; the fold
// is fp32.
//
// Work split: one workgroup per 32 rows; its waves take the row tile's blocks in turn (the count
// of waves depends on k only, so a row's sum is formed in the same order whatever the matrix
// height), then add their partial sums in LDS in wave order.
#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_gemv_core.h"
#include "tq_gemv_i8.h"
#include "tq_launch.h"
#include "tq_mfma.h"

namespace tq {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

constexpr int kDigitBlockBytes = 1024;  // one token's digits of one block: 8 sub-blocks x 4 x 32

// Fractional bits v needs: the least e with v * 2^e an integer.
__device__ __forceinline__ int frac_bits(float v) {
  const uint32_t b = __float_as_uint(v) & 0x7FFFFFFFu;
  if (b == 0) return 0;
  const int ef = (int)(b >> 23);
  const uint32_t mant = (b & 0x7FFFFFu) | (ef ? 0x800000u : 0u);
  const int E = ef ? ef - 127 : -126;
  const int f = 23 - E - __builtin_ctz(mant);
  return f > 0 ? f : 0;
}

// ---- activation digits --------------------------------------------------------------------------
// A thread per 16 values, the 16 threads of a 256-value block together. Layout per token row:
// xd [kb][j][d][32 bytes] (the 32 digits d of sub-block j of block kb), S [kb][h][q] fp32 = sum
// of x' over sub-block 2q + h, unscale [kb] = 2^-e of the block.
__global__ __launch_bounds__(256) void k_x_digits(const float *__restrict__ x, int64_t ldx,
                                                  int64_t T, int K, int8_t *__restrict__ xd,
                                                  float *__restrict__ S,
                                                  float *__restrict__ unscale) {
  const int per_row = K / 16;  // a multiple of 16: the threads of a block are active together
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= T * per_row) return;
  const int64_t t = gid / per_row;
  const int gi = (int)(gid - t * per_row);
  const int k0 = 16 * gi, kb = k0 >> 8, j = (k0 >> 5) & 7, hh = (k0 >> 4) & 1;
  const int nblk = K / 256;
  const float4 *x4 = reinterpret_cast<const float4 *>(x + t * ldx + k0);
  float v[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 f = x4[q];
    v[4 * q] = f.x;
    v[4 * q + 1] = f.y;
    v[4 * q + 2] = f.z;
    v[4 * q + 3] = f.w;
  }
  float m = 0.f;
  int fb = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    m = fmaxf(m, fabsf(v[i]));
    fb = max(fb, frac_bits(v[i]));
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) {  // the block's 16 threads
    m = fmaxf(m, __shfl_xor(m, o));
    fb = max(fb, __shfl_xor(fb, o));
  }
  int e = 0;
  if (m > 0.f) {
    int ex;
    frexpf(m, &ex);  // m in [2^(ex-1), 2^ex)
    e = min(min(27 - ex, fb), 126);
  }
  const float s = ldexpf(1.f, e);
  if ((gi & 15) == 0) unscale[t * nblk + kb] = ldexpf(1.f, -e);

  uint32_t dig[4][4];
  long long sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t b[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int r = (int)rintf(v[4 * q + i] * s);
      sum += r;
      const int c0 = ((r + 64) & 127) - 64;
      r = (r - c0) >> 7;
      const int c1 = ((r + 64) & 127) - 64;
      r = (r - c1) >> 7;
      const int c2 = ((r + 64) & 127) - 64;
      const int c3 = (r - c2) >> 7;
      b[0] |= (uint32_t)(c0 & 0xFF) << (8 * i);
      b[1] |= (uint32_t)(c1 & 0xFF) << (8 * i);
      b[2] |= (uint32_t)(c2 & 0xFF) << (8 * i);
      b[3] |= (uint32_t)(c3 & 0xFF) << (8 * i);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) dig[d][q] = b[d];
  }
  int8_t *dst = xd + (t * nblk + kb) * kDigitBlockBytes + j * 128 + 16 * hh;
#pragma unroll
  for (int d = 0; d < 4; ++d)
    *reinterpret_cast<u32x4 *>(dst + 32 * d) = (u32x4){dig[d][0], dig[d][1], dig[d][2], dig[d][3]};
  // the sub-block's other half is the neighbouring thread's
  const int lo = __shfl_xor((int)(sum & 0xFFFFFFFFll), 1);
  const int hi = __shfl_xor((int)(sum >> 32), 1);
  sum += ((long long)hi << 32) | (unsigned)lo;
  if (hh == 0) S[(t * nblk + kb) * 8 + (j & 1) * 4 + (j >> 1)] = (float)sum;
}

// ---- the product --------------------------------------------------------------------------------

template <int NTOK>
__global__ __launch_bounds__(1024) void k_gemv_i8(KlMap m, int nblk, I8Digits dg, int ldy_rows) {
  __shared__ float red[16][NTOK][32];
  const int lane = threadIdx.x & 63, w = wave_index(), W = blockDim.x >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int r0 = blockIdx.x * 32;
  const uint8_t *row = m.row(min(r0 + n, m.total - 1));
  const int my_sub = n >> 2;  // the sub-block whose digit row this lane supplies

  struct Blk {
    u32x4 head, q[4];
    u32x4 xa[NTOK];
    u32x4 S[NTOK];  // fp32 bits
    uint32_t us[NTOK];  // the block's 2^-e, fp32 bits
  };
  auto load = [&](Blk &b, int kb) {
    const uint8_t *p = row + (int64_t)kb * 144;
    b.head = gload(p);
#pragma unroll
    for (int c = 0; c < 4; ++c) b.q[c] = gload(p + 16 + 32 * c + 16 * h);
#pragma unroll
    for (int t = 0; t < NTOK; ++t) {
      const int64_t blk = (int64_t)t * nblk + kb;
      b.xa[t] = gload(dg.xd + blk * kDigitBlockBytes + n * 32 + 16 * h);
      b.S[t] = gload(dg.S + blk * 8 + 4 * h);
      b.us[t] = *(const uint32_t __attribute__((address_space(1))) *)(dg.unscale + blk);
    }
  };
  float acc[NTOK];
#pragma unroll
  for (int t = 0; t < NTOK; ++t) acc[t] = 0.f;
  const i32x16 zero = {};

  auto compute = [&](const Blk &b) {
    i32x16 C[NTOK];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const u32x4 &qw = b.q[j >> 1];
      const u32x4 bq = (j & 1) ? ((qw >> 4u) & 0x0F0F0F0Fu) : (qw & 0x0F0F0F0Fu);
      const bool mine = my_sub == j;
#pragma unroll
      for (int t = 0; t < NTOK; ++t) {
        const u32x4 a = mine ? b.xa[t] : (u32x4){0u, 0u, 0u, 0u};
        C[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                                     __builtin_bit_cast(i32x4, bq),
                                                     j == 0 ? zero : C[t], 0, 0, 0);
      }
    }
    // the lane's sub-blocks 2q + h: scales and mins (bytes 0 and 2 after a shift by 8h)
    const uint32_t h0 = b.head.x, s0 = b.head.y, s1 = b.head.z, s2 = b.head.w;
    const float d = half_bits_to_float(h0), dmin = half_bits_to_float(h0 >> 16);
    const uint32_t sh = 8u * (uint32_t)h;
    const uint32_t sc_lo = (s0 & 0x3F3F3F3Fu) >> sh;
    const uint32_t sc_hi = ((s2 & 0x0F0F0F0Fu) | ((s0 >> 2) & 0x30303030u)) >> sh;
    const uint32_t m_lo = (s1 & 0x3F3F3F3Fu) >> sh;
    const uint32_t m_hi = (((s2 >> 4) & 0x0F0F0F0Fu) | ((s1 >> 2) & 0x30303030u)) >> sh;
    const float sc[4] = {byte_to_float(sc_lo, 0), byte_to_float(sc_lo, 2), byte_to_float(sc_hi, 0),
                         byte_to_float(sc_hi, 2)};
    const float mn[4] = {byte_to_float(m_lo, 0), byte_to_float(m_lo, 2), byte_to_float(m_hi, 0),
                         byte_to_float(m_hi, 2)};
#pragma unroll
    for (int t = 0; t < NTOK; ++t) {
      float bs = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // rows 8q + 4h + digit of the accumulator: sub-block 2q + h, digits 0..3
        const int lo3 = C[t][4 * q] + (C[t][4 * q + 1] << 7) + (C[t][4 * q + 2] << 14);
        const float f = __builtin_fmaf((float)C[t][4 * q + 3], 0x1p21f, (float)lo3);
        bs = __builtin_fmaf(sc[q], f, bs);
      }
      const float sv[4] = {__uint_as_float(b.S[t].x), __uint_as_float(b.S[t].y),
                           __uint_as_float(b.S[t].z), __uint_as_float(b.S[t].w)};
      float ms = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) ms = __builtin_fmaf(mn[q], sv[q], ms);
      const float us = __uint_as_float(b.us[t]);
      acc[t] = __builtin_fmaf(d * us, bs, __builtin_fmaf(-dmin * us, ms, acc[t]));
    }
  };

  // the wave's blocks w, w + W, ..., one block ahead in registers
  Blk b0, b1;
  int kb = w;
  if (kb < nblk) load(b0, kb);
  while (kb < nblk) {
    if (kb + W < nblk) load(b1, kb + W);
    compute(b0);
    kb += W;
    if (kb >= nblk) break;
    if (kb + W < nblk) load(b0, kb + W);
    compute(b1);
    kb += W;
  }

  // rows: the two parities, then the waves in order
#pragma unroll
  for (int t = 0; t < NTOK; ++t) {
    acc[t] += __shfl_xor(acc[t], 32);
    if (h == 0) red[w][t][n] = acc[t];
  }
  __syncthreads();
  if ((int)threadIdx.x < 32 * NTOK) {
    const int t = threadIdx.x >> 5, i = threadIdx.x & 31;
    float s = 0.f;
    for (int q = 0; q < W; ++q) s += red[q][t][i];
    const int v = r0 + i;
    if (m.swiglu) {
      // virtual rows alternate gate, up; the even lane combines its pair
      const float u = __shfl_down(s, 1);
      if ((i & 1) == 0 && v + 1 < m.total) m.y[0][(int64_t)t * ldy_rows + (v >> 1)] = silu_mul(s, u);
    } else if (v < m.total) {
      int p = 0;
#pragma unroll
      for (int k = 1; k < 4; ++k) p += (k < m.nparts && v >= m.cum[k]) ? 1 : 0;
      m.y[p][(int64_t)t * (m.cum[p + 1] - m.cum[p]) + (v - m.cum[p])] = s;
    }
  }
}

// ---- host side ----------------------------------------------------------------------------------

size_t i8_digits_bytes(int64_t tokens, int64_t k) {
  return (size_t)(align256(tokens * 4 * k) + align256(tokens * (k / 8)) +
                  align256(tokens * (k / 64)));
}

I8Digits i8_digits_at(void *base, int64_t tokens, int64_t k) {
  char *p = (char *)base;
  I8Digits d;
  d.xd = (int8_t *)p;
  d.S = (float *)(p + align256(tokens * 4 * k));
  d.unscale = (float *)(p + align256(tokens * 4 * k) + align256(tokens * (k / 8)));
  return d;
}

// Taken from k = 16384 on: below that the lanes-along-k kernel, which reads x as it is, is as fast
// once the digits pass (a launch of its own) is counted; above it that kernel's per-weight VALU
// work and its workgroups of k / 4096 waves hold it to about half the rate of this one.
// TQ_GEMV_I8: 0 never, 2 for every Q4_K batch-1 shape (tests and tuning), else the rule above.
bool i8_gemv_ok(int fmt, int64_t k, int64_t batch) {
  const int mode = env_int("TQ_GEMV_I8", 1);
  if (mode == 0 || fmt != FMT_Q4_K || batch != 1 || k % 256 != 0 || k < 256) return false;
  return mode == 2 || k >= 16384;
}

// Waves per workgroup: about two blocks each, at most 16 (a function of k only).
static int i8_waves(int nblk) { return clampi(nblk / 2, 1, 16); }

int launch_gemv_i8(const KlMap &m, int64_t k, const float *x, void *digits, hipStream_t s) {
  const int nblk = (int)(k / 256);
  const I8Digits dg = i8_digits_at(digits, 1, k);
  const int64_t threads = k / 16;
  hipLaunchKernelGGL(k_x_digits, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, x, k,
                     (int64_t)1, (int)k, dg.xd, dg.S, dg.unscale);
  const int W = i8_waves(nblk);
  const int grid = (m.total + 31) / 32;
  int ldy = m.swiglu ? m.total / 2 : 0;
  hipLaunchKernelGGL(k_gemv_i8<1>, dim3((unsigned)grid), dim3(64 * W), 0, s, m, nblk, dg, ldy);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace tq
