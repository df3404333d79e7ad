// tq_gemv_i8.h -- batch-1 Q4_K and Q8_0 GEMV on the int8 matrix cores (internal to libtq).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_gemv_core.h"

namespace tq {

// ---- the exact int8 activation digits and the per-block fold (shared by the int8 GEMV kernels
// and the persistent decode chain) ----

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

constexpr int kDigitBytes = 1024;  // one block's digits: 8 sub-blocks x 4 digits x 32 int8
constexpr int kLdsBlock = 1088;    // per block in LDS: digits, S [h][q] (8 fp32), 2^-e (fp32), pad
constexpr int kMaxSliceBlocks = 16;
constexpr int kMaxSlices = 8;

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

// Digits of values 16 gi .. 16 gi + 15 of one 256-value block of x (xb), written into the block's
// LDS record (blk): 4 x 16 bytes at [j][d][16 hh], then the sub-block sums and 2^-e. The block's
// 16 threads (16 consecutive lanes of one wave) call this together.
__device__ __forceinline__ void make_digits(const float *__restrict__ xb, int gi, uint8_t *blk) {
  const int j = gi >> 1, hh = gi & 1;  // sub-block j, half hh
  const float4 *x4 = reinterpret_cast<const float4 *>(xb + 16 * gi);
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
#pragma unroll
  for (int d = 0; d < 4; ++d)
    *reinterpret_cast<u32x4 *>(blk + j * 128 + 32 * d + 16 * hh) =
        (u32x4){dig[d][0], dig[d][1], dig[d][2], dig[d][3]};
  // the sub-block's other half is the neighbouring thread's
  const int lo = __shfl_xor((int)(sum & 0xFFFFFFFFll), 1);
  const int hi = __shfl_xor((int)(sum >> 32), 1);
  sum += ((long long)hi << 32) | (unsigned)lo;
  float *sf = reinterpret_cast<float *>(blk + kDigitBytes);
  if (hh == 0) sf[(j & 1) * 4 + (j >> 1)] = (float)sum;
  if (gi == 0) sf[8] = ldexpf(1.f, -e);
}

// One block of 32 rows: the lane's row header and quant half-bytes, its digit piece, its
// sub-blocks' sums and the block's 2^-e -> the block's contribution to the lane's row (lanes l and
// l + 32 hold the two sub-block parities of row l % 32).
__device__ __forceinline__ float i8_block(const u32x4 &head, const u32x4 (&q)[4], const u32x4 &xa,
                                          const u32x4 &S, float us, int my_sub, int h) {
  const i32x16 zero = {};
  i32x16 C;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const u32x4 &qw = q[j >> 1];
    const u32x4 bq = (j & 1) ? ((qw >> 4u) & 0x0F0F0F0Fu) : (qw & 0x0F0F0F0Fu);
    const u32x4 a = my_sub == j ? xa : (u32x4){0u, 0u, 0u, 0u};
    C = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                              __builtin_bit_cast(i32x4, bq), j == 0 ? zero : C,
                                              0, 0, 0);
  }
  // the lane's sub-blocks 2q + h: scales and mins (bytes 0 and 2 after a shift by 8h)
  const uint32_t h0 = head.x, s0 = head.y, s1 = head.z, s2 = head.w;
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
  float bs = 0.f;
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    // rows 8 qq + 4h + digit of the accumulator: sub-block 2 qq + h, digits 0..3
    const int lo3 = C[4 * qq] + (C[4 * qq + 1] << 7) + (C[4 * qq + 2] << 14);
    const float f = __builtin_fmaf((float)C[4 * qq + 3], 0x1p21f, (float)lo3);
    bs = __builtin_fmaf(sc[qq], f, bs);
  }
  const float sv[4] = {__uint_as_float(S.x), __uint_as_float(S.y), __uint_as_float(S.z),
                       __uint_as_float(S.w)};
  float ms = 0.f;
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) ms = __builtin_fmaf(mn[qq], sv[qq], ms);
  return __builtin_fmaf(d * us, bs, -dmin * us * ms);
}

// ---- Q8_0 on the same matrix cores ----
// Eight Q8_0 blocks (fp16 d, 32 int8 quants: 34 bytes each) make one 256-weight unit of 272
// bytes, and one 32-k step of the matrix cores is one block: the quants are int8 operands as they
// are. Lane (row n, half h) needs bytes 34 j + 2 + 16 h .. +15 of the unit for block j: a
// dword-aligned 16-byte load for odd j, and for even j (2 bytes past a dword) the 16 bytes before
// it plus the next dword, realigned in registers. Its fold covers blocks 2 q + h, q = 0..3, whose
// scales come out of the same loads: d of an even block is the first half-word of its first
// load, d of an odd block the last half-word of the extra dword of the block before it (the
// h = 1 lane's).
struct Q8Unit {
  u32x4 p[8];
  uint32_t tail[4];  // the dword after the even blocks' 16 bytes
  static constexpr int kLoads = 12;
};

__device__ __forceinline__ void q8_load_unit(Q8Unit &u, const uint8_t *unit, int h) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j & 1) {
      u.p[j] = *(gu32x4a4)(unit + 34 * j + 2 + 16 * h);
    } else {
      u.p[j] = *(gu32x4a4)(unit + 34 * j + 16 * h);
      u.tail[j >> 1] = *(const __attribute__((address_space(1))) uint32_t *)(unit + 34 * j + 16 * h + 16);
    }
  }
}

// The unit's products: the digits' sums of each block recombined (C0 + 2^7 C1 exactly in int32,
// C2 + 2^7 C3 the same, then one fp32 FMA: |C| <= 32 * 64 * 128), times the block's d, added over
// the lane's four blocks and scaled by the unit's 2^-e.
__device__ __forceinline__ float q8_i8_unit(const Q8Unit &u, const u32x4 &xa, float us,
                                            int my_blk, int h) {
  const i32x16 zero = {};
  i32x16 C;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    u32x4 bq = u.p[j];
    if (!(j & 1)) {
      const uint32_t t = u.tail[j >> 1];
      bq = (u32x4){shift2(u.p[j].x, u.p[j].y), shift2(u.p[j].y, u.p[j].z),
                   shift2(u.p[j].z, u.p[j].w), shift2(u.p[j].w, t)};
    }
    const u32x4 a = my_blk == j ? xa : (u32x4){0u, 0u, 0u, 0u};
    C = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                              __builtin_bit_cast(i32x4, bq), j == 0 ? zero : C,
                                              0, 0, 0);
  }
  float bs = 0.f;
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    // rows 8 qq + 4h + digit of the accumulator: block 2 qq + h, digits 0..3
    const int lo = C[4 * qq] + (C[4 * qq + 1] << 7);
    const int hi = C[4 * qq + 2] + (C[4 * qq + 3] << 7);
    const float f = __builtin_fmaf((float)hi, 0x1p14f, (float)lo);
    const uint32_t dbits = h ? (u.tail[qq] >> 16) : (u.p[2 * qq].x & 0xFFFFu);
    bs = __builtin_fmaf(half_bits_to_float(dbits), f, bs);
  }
  return bs * us;
}

// Shapes the int8 kernel takes: Q4_K, one token, k a multiple of 256, 16384 <= k <= 32768 (all
// k <= 32768 with TQ_KNOB_GEMV_I8 = 2); Q8_0, one token, k a multiple of 256 up to 32768
// (TQ_KNOB_GEMV_I8 = 0: never).
bool i8_gemv_ok(int fmt, int64_t k, int64_t batch);
// Workspace after the completion counters: the k slices' partial sums of `rows` rows (0 when k
// is one slice).
size_t i8_workspace_bytes(int64_t rows, int64_t k);
// The rows of m against x [k] (16-byte aligned). partial: i8_workspace_bytes(m.total, k) bytes;
// counters: one 8-byte word per row group (Arrivals; max_counters of them), any contents.
int launch_gemv_i8(int fmt, const KlMap &m, int64_t k, const float *x, float *partial,
                   unsigned long long *counters, int max_counters, hipStream_t s);

}  // namespace tq
