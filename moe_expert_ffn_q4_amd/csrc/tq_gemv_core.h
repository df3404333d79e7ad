// tq_gemv_core.h -- the streaming core shared by the dense GEMV and the grouped expert GEMV.
//
// Mapping (gfx950, wave64): one lane owns one output row; a wave owns 64 consecutive rows and
// walks a contiguous range of 256-weight "units" of those rows (one Q4_K or Q6_K block, or
// eight Q8_0 blocks). Every lane streams its own row with 16-byte loads while the activation
// values are the same for all 64 lanes, so they come through scalar loads and feed the FMAs as
// SGPR operands: no LDS traffic and no VGPRs for activations in the inner loop. Per weight the
// inner loop costs one FMA per token plus the conversion of the quant to fp32 (one
// v_cvt_f32_ubyte per weight, or for 4-bit quants half a packed fp8 conversion), and a mask per
// 4 weights.
//
// The affine block terms are factored out of the inner loop:
//   sum_i w_i x_i = sum_j d*sc_j * sum_{i in j} q_i x_i  -  sum_j dmin*m_j * S_j     (Q4_K)
//   sum_i w_i x_i = sum_s d*sc_s * (sum_{i in s} q_i x_i - 32 * S_s)                (Q6_K)
//   sum_i w_i x_i = sum_b d_b * (sum_{i in b} (q_i + 128) x_i - 128 * S_b)          (Q8_0)
//   sum_i w_i x_i = sum_j d*sc_j * sum_{i in j} q_i x_i  -  sum_j dmin*m_j * S_j     (Q5_K)
//   sum_i w_i x_i = sum_b d_b * (sum_{i in b} q_i x_i - 8 * S_b)                    (Q4_0)
// where S is the sum of x over the 32- (or 16-) weight group. The group sums of the tile's
// tokens are computed once per workgroup into LDS and read with wave-uniform addresses.
#pragma once

#include "tq_device.h"

namespace tq {

enum { FMT_Q4_K = 1, FMT_Q6_K = 2, FMT_Q8_0 = 3, FMT_Q5_K = 4, FMT_Q4_0 = 5 };

template <int FMT>
struct Fmt;
template <>
struct Fmt<FMT_Q4_K> {
  static constexpr int unit_bytes = 144;  // one block
  static constexpr int group = 32;        // x-sum group (sub-block)
};
template <>
struct Fmt<FMT_Q6_K> {
  static constexpr int unit_bytes = 210;  // one block
  static constexpr int group = 16;        // one int8 scale per 16 weights
};
template <>
struct Fmt<FMT_Q8_0> {
  static constexpr int unit_bytes = 272;  // eight 34-byte blocks
  static constexpr int group = 32;        // one block
};
template <>
struct Fmt<FMT_Q5_K> {
  static constexpr int unit_bytes = 176;  // one block
  static constexpr int group = 32;        // sub-block
};
template <>
struct Fmt<FMT_Q4_0> {
  static constexpr int unit_bytes = 144;  // eight 18-byte blocks
  static constexpr int group = 32;        // one block
};

// Raw bytes of one unit of one row, as loaded.
template <int FMT>
struct Unit;
template <>
struct Unit<FMT_Q4_K> {
  u32x4 v[9];
};
template <>
struct Unit<FMT_Q6_K> {
  uint32_t v[53];  // v[0..51]: block bytes 0..207 (after realignment); v[52]: d in low half
};
template <>
struct Unit<FMT_Q8_0> {
  uint32_t v[68];
};
template <>
struct Unit<FMT_Q5_K> {
  uint32_t v[44];  // header (4 dwords), 32 high-bit bytes (8), 128 low-nibble bytes (32)
};
template <>
struct Unit<FMT_Q4_0> {
  uint32_t v[36];
};

// ---- loads ---------------------------------------------------------------------------------

// Q4_K: the block starts at a multiple of 144 bytes from a 16-byte aligned row start.
__device__ __forceinline__ void load_unit(Unit<FMT_Q4_K> &u, const uint8_t *row, int idx) {
  const gu32x4 p = (gu32x4)(row + (size_t)idx * 144);
#pragma unroll
  for (int i = 0; i < 9; ++i) u.v[i] = *(p + i);
}

// Q6_K: row start is 4-byte aligned; block idx starts at 210*idx, i.e. two bytes past a dword
// boundary for odd idx. The 208 bytes before the fp16 d are loaded as 52 dwords from the dword
// boundary at or below the block start (never before the row start, never past the block end)
// and shifted down by two bytes when needed; d itself is loaded as a 16-bit value.
__device__ __forceinline__ void load_unit(Unit<FMT_Q6_K> &u, const uint8_t *row, int idx) {
  const int off = idx * 210;
  const uint8_t *base = row + (off & ~3);
  const gu32x4a4 p = (gu32x4a4)base;
  uint32_t r[53];
#pragma unroll
  for (int i = 0; i < 13; ++i) {
    u32x4a4 t = *(p + i);
    r[4 * i + 0] = t.x;
    r[4 * i + 1] = t.y;
    r[4 * i + 2] = t.z;
    r[4 * i + 3] = t.w;
  }
  const uint32_t dbits = *(const __attribute__((address_space(1))) uint16_t *)(row + off + 208);
  if (off & 2) {  // wave-uniform: every lane is at the same block index
    r[52] = *(const __attribute__((address_space(1))) uint32_t *)(base + 208);
#pragma unroll
    for (int i = 0; i < 52; ++i) u.v[i] = shift2(r[i], r[i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < 52; ++i) u.v[i] = r[i];
  }
  u.v[52] = dbits;
}

// Q8_0: eight blocks (272 bytes) starting at a multiple of 272 from a 16-byte aligned row
// start (k is a multiple of 256).
__device__ __forceinline__ void load_unit(Unit<FMT_Q8_0> &u, const uint8_t *row, int idx) {
  const gu32x4 p = (gu32x4)(row + (size_t)idx * 272);
#pragma unroll
  for (int i = 0; i < 17; ++i) {
    u32x4 t = *(p + i);
    u.v[4 * i + 0] = t.x;
    u.v[4 * i + 1] = t.y;
    u.v[4 * i + 2] = t.z;
    u.v[4 * i + 3] = t.w;
  }
}

// Q5_K: the block starts at a multiple of 176 bytes from a 16-byte aligned row start.
__device__ __forceinline__ void load_unit(Unit<FMT_Q5_K> &u, const uint8_t *row, int idx) {
  const gu32x4 p = (gu32x4)(row + (size_t)idx * 176);
#pragma unroll
  for (int i = 0; i < 11; ++i) {
    u32x4 t = *(p + i);
    u.v[4 * i + 0] = t.x;
    u.v[4 * i + 1] = t.y;
    u.v[4 * i + 2] = t.z;
    u.v[4 * i + 3] = t.w;
  }
}

// Q4_0: eight blocks (144 bytes) starting at a multiple of 144 from a 16-byte aligned row start
// (k is a multiple of 256).
__device__ __forceinline__ void load_unit(Unit<FMT_Q4_0> &u, const uint8_t *row, int idx) {
  const gu32x4 p = (gu32x4)(row + (size_t)idx * 144);
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    u32x4 t = *(p + i);
    u.v[4 * i + 0] = t.x;
    u.v[4 * i + 1] = t.y;
    u.v[4 * i + 2] = t.z;
    u.v[4 * i + 3] = t.w;
  }
}

// ---- per-unit arithmetic -------------------------------------------------------------------

// `off`, but only known to the compiler once `dep` has been computed: the scalar activation
// loads addressed with it cannot be hoisted far ahead of their use (which would need more
// scalar registers than a wave has).
__device__ __forceinline__ int after(int off, float dep) {
  asm("" : "+s"(off) : "v"(dep));
  return off;
}

__device__ __forceinline__ uint32_t dword_of(const u32x4 &v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// sum_e f[e] * x[e] over 16 / 32 values; x is wave-uniform (scalar loads). Two chains.
__device__ __forceinline__ float dot16(const float (&f)[16], const float *x) {
  float a = 0.f, b = 0.f;
#pragma unroll
  for (int e = 0; e < 16; e += 2) {
    a = __builtin_fmaf(f[e], x[e], a);
    b = __builtin_fmaf(f[e + 1], x[e + 1], b);
  }
  return a + b;
}
__device__ __forceinline__ float dot32(const float (&f)[32], const float *x) {
  float a = 0.f, b = 0.f;
#pragma unroll
  for (int e = 0; e < 32; e += 2) {
    a = __builtin_fmaf(f[e], x[e], a);
    b = __builtin_fmaf(f[e + 1], x[e + 1], b);
  }
  return a + b;
}

// Q6_K: the 6-bit quants of weights l..l+3 of the four 32-weight groups of one half block, from
// the low-bit dwords A (groups 0, 2), B (groups 1, 3) and the high-bit dword QH, one per byte.
__device__ __forceinline__ void q6k_quads(uint32_t A, uint32_t B, uint32_t QH, uint32_t (&q)[4]) {
  q[0] = opaque((A & 0x0F0F0F0Fu) | ((QH << 4) & 0x30303030u));
  q[1] = opaque((B & 0x0F0F0F0Fu) | ((QH << 2) & 0x30303030u));
  q[2] = opaque(((A >> 4) & 0x0F0F0F0Fu) | (QH & 0x30303030u));
  q[3] = opaque(((B >> 4) & 0x0F0F0F0Fu) | ((QH >> 2) & 0x30303030u));
}

// xp[t]: wave-uniform pointer to token t's activations at the unit's first weight.
// gs[t]: wave-uniform LDS pointer to token t's group sums at the unit's first group.

template <int NT>
__device__ __forceinline__ void unit_dot(const Unit<FMT_Q4_K> &u, const float *const (&xp)[NT],
                                         const float *const (&gs)[NT], float (&acc)[NT]) {
  const uint32_t h0 = u.v[0].x, s0 = u.v[0].y, s1 = u.v[0].z, s2 = u.v[0].w;
  const float d = half_bits_to_float(h0), dmin = half_bits_to_float(h0 >> 16);
  float sc[8], mn[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sc[j] = (float)((s0 >> (8 * j)) & 63u);
    mn[j] = (float)((s1 >> (8 * j)) & 63u);
    sc[4 + j] = (float)(((s2 >> (8 * j)) & 15u) | (((s0 >> (8 * j + 6)) & 3u) << 4));
    mn[4 + j] = (float)(((s2 >> (8 * j + 4)) & 15u) | (((s1 >> (8 * j + 6)) & 3u) << 4));
  }
  float bs[NT], ms[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    bs[t] = 0.f;
    ms[t] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ms[t] = __builtin_fmaf(mn[j], gs[t][j], ms[t]);
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    // quant bytes 32c..32c+31: low nibbles are sub-block 2c (weights 64c + 0..31), high
    // nibbles are sub-block 2c+1 (weights 64c + 32..63).
    static_assert(NT == 1, "multi-token Q4_K streams 64-weight groups (stream_q4k_groups)");
    {
      // quants come out of the fp8 converter as q * unit; 1/unit is folded into the scales
      float dl = 0.f, dh = 0.f;
#pragma unroll
      for (int dw = 0; dw < 8; ++dw) {
        const uint32_t w = dword_of(u.v[1 + 2 * c + (dw >> 2)], dw & 3);
        const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
        const int i = 64 * c + 4 * dw;
        float f[4];
        nibbles_to_float<false>(lo, f[0], f[1]);
        nibbles_to_float<true>(lo, f[2], f[3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) dl = __builtin_fmaf(f[e], xp[0][i + e], dl);
        nibbles_to_float<false>(hi, f[0], f[1]);
        nibbles_to_float<true>(hi, f[2], f[3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) dh = __builtin_fmaf(f[e], xp[0][i + 32 + e], dh);
      }
      bs[0] = __builtin_fmaf(sc[2 * c], dl, bs[0]);
      bs[0] = __builtin_fmaf(sc[2 * c + 1], dh, bs[0]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const float dq = d / nibble_fp8_unit();  // exact: a power-of-two rescale
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = __builtin_fmaf(dq, bs[t], __builtin_fmaf(-dmin, ms[t], acc[t]));
}

template <int NT>
__device__ __forceinline__ void unit_dot(const Unit<FMT_Q6_K> &u, const float *const (&xp)[NT],
                                         const float *const (&gs)[NT], float (&acc)[NT]) {
  const float d = half_bits_to_float(u.v[52]);
  float bs[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) bs[t] = 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int lh = 0; lh < 2; ++lh) {
      float dot[4][NT];
      if constexpr (NT == 1) {
#pragma unroll
        for (int g = 0; g < 4; ++g) dot[g][0] = 0.f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = 4 * lh + jj;  // weights l = 4j..4j+3 of each 32-weight group of half h
          uint32_t q[4];
          q6k_quads(u.v[16 * h + j], u.v[16 * h + 8 + j], u.v[32 + 8 * h + j], q);
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              dot[g][0] = __builtin_fmaf(byte_to_float(q[g], e), xp[0][128 * h + 32 * g + 4 * j + e],
                                         dot[g][0]);
        }
      } else {
        float f[4][16];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          uint32_t q[4];
          const int j = 4 * lh + jj;
          q6k_quads(u.v[16 * h + j], u.v[16 * h + 8 + j], u.v[32 + 8 * h + j], q);
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) f[g][4 * jj + e] = byte_to_float(q[g], e);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            dot[g][t] = dot16(f[g], xp[t] + 128 * h + 32 * g + 16 * lh);
            __builtin_amdgcn_sched_barrier(0);
          }
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int s = 8 * h + 2 * g + lh;  // int8 scale index of these 16 weights
        const uint32_t sw = u.v[48 + (s >> 2)];
        const float scf = (float)(int32_t)(int8_t)(uint8_t)(sw >> (8 * (s & 3)));
#pragma unroll
        for (int t = 0; t < NT; ++t)
          bs[t] = __builtin_fmaf(scf, __builtin_fmaf(-32.f, gs[t][s], dot[g][t]), bs[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = __builtin_fmaf(d, bs[t], acc[t]);
}

template <int NT>
__device__ __forceinline__ void unit_dot(const Unit<FMT_Q8_0> &u, const float *const (&xp)[NT],
                                         const float *const (&gs)[NT], float (&acc)[NT]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
#pragma unroll
    for (int odd = 0; odd < 2; ++odd) {
      const int bb = 2 * p + odd;  // block within the unit, bytes 34*bb .. 34*bb+33
      float d;
      uint32_t q[8];
      if (!odd) {  // starts on a dword boundary: d = low half, quants start two bytes in
        d = half_bits_to_float(u.v[17 * p]);
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = shift2(u.v[17 * p + i], u.v[17 * p + i + 1]);
      } else {  // starts two bytes into a dword: d = high half, quants dword-aligned
        d = half_bits_to_float(u.v[17 * p + 8] >> 16);
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = u.v[17 * p + 9 + i];
      }
      float dot[NT];
      if constexpr (NT == 1) {
        dot[0] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t biased = opaque(q[i] ^ 0x80808080u);  // int8 q -> q + 128 as unsigned bytes
#pragma unroll
          for (int e = 0; e < 4; ++e)
            dot[0] = __builtin_fmaf(byte_to_float(biased, e), xp[0][32 * bb + 4 * i + e], dot[0]);
        }
      } else {
        float f[32];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t biased = opaque(q[i] ^ 0x80808080u);
#pragma unroll
          for (int e = 0; e < 4; ++e) f[4 * i + e] = byte_to_float(biased, e);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          dot[t] = dot32(f, xp[t] + 32 * bb);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[t] = __builtin_fmaf(d, __builtin_fmaf(-128.f, gs[t][bb], dot[t]), acc[t]);
    }
  }
}

// Q5_K, one token: quants of sub-block j as bytes (low nibble from the Q4_K-style plane, fifth bit
// from bit j of the high-bit byte of the same position), converted one byte per weight; each
// sub-block's scale and min unpacked where they are used, the min term added last. Batches run
// this once per token: the multi-token forms of it spilled registers to scratch memory.
template <int NT>
__device__ __forceinline__ void unit_dot(const Unit<FMT_Q5_K> &u, const float *const (&xp)[NT],
                                         const float *const (&gs)[NT], float (&acc)[NT]) {
  static_assert(NT == 1, "Q5_K runs one token per pass");
  const uint32_t h0 = u.v[0], s0 = u.v[1], s1 = u.v[2], s2 = u.v[3];
  float bs = 0.f, ms = 0.f;
  float dep = 0.f;  // the previous sub-block's result: its activation loads wait for it
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = j >> 1, sh = 8 * (j & 3);
    const float *xj = xp[0] + after(32 * j, dep);
    const uint32_t scj = j < 4 ? (s0 >> sh) & 63u : ((s2 >> sh) & 15u) | (((s0 >> (sh + 6)) & 3u) << 4);
    const uint32_t mj = j < 4 ? (s1 >> sh) & 63u
                              : ((s2 >> (sh + 4)) & 15u) | (((s1 >> (sh + 6)) & 3u) << 4);
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w = u.v[12 + 8 * c + i];
      const uint32_t hb = u.v[4 + i];
      const uint32_t nib = (j & 1) ? ((w >> 4) & 0x0F0F0F0Fu) : (w & 0x0F0F0F0Fu);
      const uint32_t q = opaque(nib | (((hb >> j) & 0x01010101u) << 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) dot = __builtin_fmaf(byte_to_float(q, e), xj[4 * i + e], dot);
    }
    bs = __builtin_fmaf((float)scj, dot, bs);
    ms = __builtin_fmaf((float)mj, gs[0][j], ms);
    dep = bs;
    __builtin_amdgcn_sched_barrier(0);
  }
  const float d = half_bits_to_float(h0), dmin = half_bits_to_float(h0 >> 16);
  acc[0] = __builtin_fmaf(d, bs, __builtin_fmaf(-dmin, ms, acc[0]));
}

// Q4_0: eight blocks; block 2p starts on a dword boundary (d in the low half, quants two bytes
// in), block 2p + 1 two bytes past one (d in the high half, quants dword-aligned). Nibbles go
// through the fp8 converter (q * unit, the unit folded into d).
template <int NT>
__device__ __forceinline__ void unit_dot(const Unit<FMT_Q4_0> &u, const float *const (&xp)[NT],
                                         const float *const (&gs)[NT], float (&acc)[NT]) {
  const float inv_unit = 1.f / nibble_fp8_unit();  // exact: a power of two
#pragma unroll
  for (int p = 0; p < 4; ++p) {
#pragma unroll
    for (int odd = 0; odd < 2; ++odd) {
      const int bb = 2 * p + odd;
      float d;
      uint32_t q[4];
      if (!odd) {
        d = half_bits_to_float(u.v[9 * p]);
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = shift2(u.v[9 * p + i], u.v[9 * p + i + 1]);
      } else {
        d = half_bits_to_float(u.v[9 * p + 4] >> 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = u.v[9 * p + 5 + i];
      }
      // weights 4i..4i+3 are the low nibbles of quant dword i, weights 16+4i.. the high ones
      float f[32];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = q[i] & 0x0F0F0F0Fu, hi = (q[i] >> 4) & 0x0F0F0F0Fu;
        nibbles_to_float<false>(lo, f[4 * i], f[4 * i + 1]);
        nibbles_to_float<true>(lo, f[4 * i + 2], f[4 * i + 3]);
        nibbles_to_float<false>(hi, f[16 + 4 * i], f[16 + 4 * i + 1]);
        nibbles_to_float<true>(hi, f[16 + 4 * i + 2], f[16 + 4 * i + 3]);
      }
      const float dq = d * inv_unit;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float dot = dot32(f, xp[t] + 32 * bb);
        acc[t] = __builtin_fmaf(dq, dot, __builtin_fmaf(-8.f * d, gs[t][bb], acc[t]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Header and the 32 quant bytes of 64-weight group `it` (= 4 * unit + group) of a Q4_K row.
__device__ __forceinline__ void q4k_group_load(const uint8_t *row, int it, u32x4 (&v)[3]) {
  const gu32x4 p = (gu32x4)(row + (size_t)(it >> 2) * 144);
  v[0] = *(p);
  v[1] = *(p + 1 + 2 * (it & 3));
  v[2] = *(p + 2 + 2 * (it & 3));
}

// Q4_K with several tokens: the lane loads its row's whole 144-byte block at once (nine 16-byte
// loads, the next block's issued before this block's math), so every cache line of the block is
// used while it is in flight; rows of one wave lie far apart, and loading a block in pieces over
// time would let the lines leave L2 between the pieces. The block's four 64-weight groups are
// then processed one after another (a scheduling barrier between them keeps only one group's
// converted quants live).
struct Q4kBlock {
  u32x4 v[9];  // header, then 128 quant bytes
};

__device__ __forceinline__ void q4k_block_load(const uint8_t *row, int u, Q4kBlock &b) {
  const gu32x4 p = (gu32x4)(row + (size_t)u * 144);
#pragma unroll
  for (int i = 0; i < 9; ++i) b.v[i] = p[i];
}

template <int NT>
__device__ __forceinline__ void q4k_block_dot(const Q4kBlock &b, int u,
                                              const float *const (&x)[NT],
                                              const float *const (&gsum)[NT], float (&acc)[NT]) {
  const uint32_t h0 = b.v[0].x, s0 = b.v[0].y, s1 = b.v[0].z, s2 = b.v[0].w;
  const float dq = half_bits_to_float(h0) / nibble_fp8_unit(), dmin = half_bits_to_float(h0 >> 16);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int j0 = 2 * c, j1 = 2 * c + 1;
    uint32_t sc0, m0, sc1, m1;
    if (c < 2) {
      sc0 = (s0 >> (8 * j0)) & 63u;
      m0 = (s1 >> (8 * j0)) & 63u;
      sc1 = (s0 >> (8 * j1)) & 63u;
      m1 = (s1 >> (8 * j1)) & 63u;
    } else {
      const int a = j0 - 4, bb = j1 - 4;
      sc0 = ((s2 >> (8 * a)) & 15u) | (((s0 >> (8 * a + 6)) & 3u) << 4);
      m0 = ((s2 >> (8 * a + 4)) & 15u) | (((s1 >> (8 * a + 6)) & 3u) << 4);
      sc1 = ((s2 >> (8 * bb)) & 15u) | (((s0 >> (8 * bb + 6)) & 3u) << 4);
      m1 = ((s2 >> (8 * bb + 4)) & 15u) | (((s1 >> (8 * bb + 6)) & 3u) << 4);
    }
    const float dsc0 = dq * (float)sc0, dsc1 = dq * (float)sc1;
    const float dm0 = dmin * (float)m0, dm1 = dmin * (float)m1;
    float fl[32], fh[32];
#pragma unroll
    for (int dw = 0; dw < 8; ++dw) {
      const uint32_t w = dword_of(b.v[1 + 2 * c + (dw >> 2)], dw & 3);
      const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
      nibbles_to_float<false>(lo, fl[4 * dw], fl[4 * dw + 1]);
      nibbles_to_float<true>(lo, fl[4 * dw + 2], fl[4 * dw + 3]);
      nibbles_to_float<false>(hi, fh[4 * dw], fh[4 * dw + 1]);
      nibbles_to_float<true>(hi, fh[4 * dw + 2], fh[4 * dw + 3]);
    }
    float prev = fl[0], prev2 = fh[0];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float *xg = x[t] + 256 * u + 64 * c;
      const float dl = dot32(fl, xg + after(0, prev2));
      const float dh = dot32(fh, xg + after(32, prev));
      prev2 = dl;
      prev = dh;
      const float *g = gsum[t] + 8 * u + j0;
      float a = __builtin_fmaf(dsc0, dl, acc[t]);
      a = __builtin_fmaf(dsc1, dh, a);
      a = __builtin_fmaf(-dm0, g[0], a);
      acc[t] = __builtin_fmaf(-dm1, g[1], a);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int NT>
__device__ __forceinline__ void stream_q4k_groups(const uint8_t *row, int u0, int u1,
                                                  const Q4kBlock &first,
                                                  const float *const (&x)[NT],
                                                  const float *const (&gsum)[NT], float (&acc)[NT]) {
  Q4kBlock cur = first, nxt;
#pragma unroll 1
  for (int u = u0; u < u1; ++u) {
    if (u + 1 < u1) q4k_block_load(row, u + 1, nxt);
    q4k_block_dot<NT>(cur, u, x, gsum, acc);
    cur = nxt;
  }
}

// Stream units [u0, u1) of this lane's row, next unit's loads issued before this one's math.
// Stream units [u0, u1) of this lane's row; `cur` already holds unit u0 (loaded by the caller
// so that its latency overlaps other work). The next unit's loads are issued before this unit's
// math.
template <int FMT, int NT>
__device__ __forceinline__ void stream_units(const uint8_t *row, int u0, int u1, Unit<FMT> &cur,
                                             const float *const (&x)[NT],
                                             const float *const (&gsum)[NT], float (&acc)[NT]) {
  constexpr int G = Fmt<FMT>::group;
  Unit<FMT> nxt;
  for (int u = u0; u < u1; ++u) {
    if (u + 1 < u1) load_unit(nxt, row, u + 1);
    const float *xp[NT];
    const float *gs[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      xp[t] = x[t] + 256 * u;
      gs[t] = gsum[t] + (256 / G) * u;
    }
    unit_dot<NT>(cur, xp, gs, acc);
    cur = nxt;
  }
}

// One workgroup's share of a GEMV tile: rows [row0, row0+64) (one per lane, clamped to n-1),
// units [ku0, ku1) split over the waves (upw units each), NT tokens whose activation rows are
// xr[t]. Leaves sum over this workgroup's units of w[row][:] . x[t][:] in lds_out[t*64 + lane]
// (the first NT*64 floats of `lds`), summed over waves in wave order. `lds` must hold
// max(NT * groups of the slice, waves * NT * 64) floats. Ends with a barrier.
template <int FMT, int NT>
__device__ __forceinline__ void gemv_tile(const uint8_t *__restrict__ w, int64_t row_bytes, int n,
                                          int row0, int ku0, int ku1, int upw,
                                          const float *const (&xr)[NT], float *lds) {
  constexpr int G = Fmt<FMT>::group;
  constexpr int GPU_ = 256 / G;  // groups per unit
  const int nw = blockDim.x >> 6;
  const int wave = wave_index();
  const int lane = threadIdx.x & 63;
  const int ngl = (ku1 - ku0) * GPU_;
  const int row = min(row0 + lane, n - 1);  // rows past n repeat the last row; never stored
  const int u0 = ku0 + wave * upw, u1 = min(u0 + upw, ku1);
  const uint8_t *wrow = w + (int64_t)row * row_bytes;
  // the first weights of this wave are requested before the group sums are formed
  constexpr bool kGroups = FMT == FMT_Q4_K && NT > 1;
  Unit<FMT> first;
  Q4kBlock gfirst;
  if constexpr (kGroups) {
    if (u0 < u1) q4k_block_load(wrow, u0, gfirst);
  } else {
    if (u0 < u1) load_unit(first, wrow, u0);
  }
  // group sums of this slice of x, for every token of the tile
  for (int i = threadIdx.x; i < NT * ngl; i += blockDim.x) {
    const int t = i / ngl, gi = i - t * ngl;
    const float *p = xr[t] + (int64_t)(ku0 * GPU_ + gi) * G;
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < G; ++e) s += p[e];
    lds[i] = s;
  }
  __syncthreads();
  const float *gs[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) gs[t] = lds + t * ngl - ku0 * GPU_;  // absolute group numbers
  float acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.f;
  if constexpr (kGroups) {
    if (u0 < u1) stream_q4k_groups<NT>(wrow, u0, u1, gfirst, xr, gs, acc);
  } else {
    if (u0 < u1) stream_units<FMT, NT>(wrow, u0, u1, first, xr, gs, acc);
  }
  __syncthreads();  // every wave is done with the group sums
#pragma unroll
  for (int t = 0; t < NT; ++t) lds[NT * 64 + (wave * NT + t) * 64 + lane] = acc[t];
  __syncthreads();
  for (int i = threadIdx.x; i < NT * 64; i += blockDim.x) {
    const int t = i >> 6, l = i & 63;
    float s = 0.f;
    for (int v = 0; v < nw; ++v) s += lds[NT * 64 + (v * NT + t) * 64 + l];
    lds[i] = s;
  }
  __syncthreads();
}

// LDS floats gemv_tile needs for NT tokens, `upk` units per slice and `waves` waves.
template <int FMT>
__host__ __device__ inline int gemv_tile_lds_floats(int nt, int upk, int waves) {
  const int g = nt * upk * (256 / Fmt<FMT>::group);
  const int r = nt * 64 + waves * nt * 64;
  return g > r ? g : r;
}

}  // namespace tq

namespace tq {

// ---- batch-1 Q4_K GEMV with lanes along k ---------------------------------------------------------
// A wave covers 16 blocks (4096 weights) of k: lane l owns the 64-weight group c = l % 4 of block
// 16w + l / 4, i.e. quant bytes 32c..32c+31 (sub-blocks 2c and 2c+1). Its 64 activations stay in
// VGPRs for all rows, with their two 32-element sums. For each row the lane loads the block
// header and its 32 quant bytes (three 16-byte loads; consecutive lanes read consecutive bytes of
// the row), forms its partial dot product, and partial sums are added across lanes every R rows
// (a butterfly that halves the rows at each step) and across the waves of the workgroup in LDS.
// Nothing is split across workgroups, so there is no cross-workgroup reduction.

// Field positions of the 6-bit scale and min of sub-block j inside the 12 packed bytes, as bit
// offsets / widths used with v_bfe (a field of width 0 reads as 0), so that lanes with j < 4 and
// j >= 4 run the same instructions:
//   sc = bfe(j < 4 ? S0..3 : S8..11, lo_off, lo_w) | bfe(S0..3, hi_off, hi_w) << 4
//   m  = bfe(j < 4 ? S4..7 : S8..11, lo_off + mo, lo_w) | bfe(S4..7, hi_off, hi_w) << 4
struct Q4kField {
  uint32_t lo_off, lo_w, hi_off, hi_w, m_off;
  bool from_s2;
};
__device__ __forceinline__ Q4kField q4k_field(int j) {
  Q4kField f;
  const uint32_t a = 8u * (uint32_t)(j & 3);
  f.from_s2 = j >= 4;
  f.lo_off = a;
  f.lo_w = f.from_s2 ? 4u : 6u;
  f.hi_off = a + 6u;
  f.hi_w = f.from_s2 ? 2u : 0u;
  f.m_off = f.from_s2 ? a + 4u : a;
  return f;
}
__device__ __forceinline__ uint32_t bfe(uint32_t v, uint32_t off, uint32_t w) {
  return __builtin_amdgcn_ubfe(v, off, w);
}
__device__ __forceinline__ void q4k_scale_min_at(uint32_t s0, uint32_t s1, uint32_t s2,
                                                 const Q4kField &f, float &sc, float &m) {
  const uint32_t lsc = f.from_s2 ? s2 : s0, lm = f.from_s2 ? s2 : s1;
  sc = (float)(bfe(lsc, f.lo_off, f.lo_w) | (bfe(s0, f.hi_off, f.hi_w) << 4));
  m = (float)(bfe(lm, f.m_off, f.lo_w) | (bfe(s1, f.hi_off, f.hi_w) << 4));
}

// The rows of one batch-1 launch: up to four matrices that share the activations, their rows
// taken one after another (multi), or a gate and an up matrix taken alternately, row r of gate
// then row r of up (swiglu: the pair is combined into h[r] = silu(gate) * up).
struct KlMap {
  const uint8_t *w[4];
  float *y[4];
  int cum[5];  // multi: cum[p] = first virtual row of matrix p, cum[nparts] = all rows
  int nparts;
  int swiglu;  // 1: w[0] gate, w[1] up, y[0] = h; 2 * n virtual rows
  int total;   // virtual rows
  int64_t row_bytes;

  // Row v's bytes and output. The part is picked with selects among the four pointers held in
  // scalar registers (opaque to the compiler): indexing the argument's arrays with a per-lane part
  // number compiles to a vector load from the argument segment and a wait on every outstanding
  // load, the next rows' prefetch included.
  __device__ __forceinline__ const uint8_t *row(int v) const {
    const uint8_t *p0 = w[0], *p1 = w[1], *p2 = w[2], *p3 = w[3];
    asm("" : "+s"(p0), "+s"(p1), "+s"(p2), "+s"(p3));
    if (swiglu) return ((v & 1) ? p1 : p0) + (int64_t)(v >> 1) * row_bytes;
    const int c1 = nparts > 1 ? cum[1] : 1 << 30, c2 = nparts > 2 ? cum[2] : 1 << 30,
              c3 = nparts > 3 ? cum[3] : 1 << 30;
    const uint8_t *b = v >= c3 ? p3 : v >= c2 ? p2 : v >= c1 ? p1 : p0;
    const int first = v >= c3 ? c3 : v >= c2 ? c2 : v >= c1 ? c1 : 0;
    return b + (int64_t)(v - first) * row_bytes;
  }
  // SwiGLU output j (rows 2j, 2j+1)
  __device__ __forceinline__ float *swiglu_out(int j) const { return y[0] + j; }
  __device__ __forceinline__ void put(int v, float s) const { gstore(out(v), s); }
  __device__ __forceinline__ float *out(int v) const {
    float *p0 = y[0], *p1 = y[1], *p2 = y[2], *p3 = y[3];
    asm("" : "+s"(p0), "+s"(p1), "+s"(p2), "+s"(p3));
    const int c1 = nparts > 1 ? cum[1] : 1 << 30, c2 = nparts > 2 ? cum[2] : 1 << 30,
              c3 = nparts > 3 ? cum[3] : 1 << 30;
    float *b = v >= c3 ? p3 : v >= c2 ? p2 : v >= c1 ? p1 : p0;
    const int first = v >= c3 ? c3 : v >= c2 ? c2 : v >= c1 ? c1 : 0;
    return b + (v - first);
  }
};

// A pointer that is the same in every lane, moved to scalar registers.
__device__ __forceinline__ const uint8_t *uniform_ptr(const uint8_t *p) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u),
                 hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const uint8_t *)(((uint64_t)hi << 32) | lo);
}

// Rows of one expert's matrices for the one-token MoE kernel: two pointers and no arrays (a
// general row map built inside a kernel and indexed at run time is kept in scratch memory).
struct MoeRowMap {
  const uint8_t *w0, *w1;  // gate, up (gate_up) or down, unused
  float *y;
  int swiglu, total;
  int64_t row_bytes;
  int coherent;  // sums stored at device scope (read back in the same launch)
  // The gate / up pick is a select between two scalar registers (opaque to the compiler): left
  // to itself it makes a two-entry table of the pointers per lane in LDS and reads it back before
  // every pass's loads.
  __device__ __forceinline__ const uint8_t *row(int v) const {
    const uint8_t *p0 = uniform_ptr(w0), *p1 = uniform_ptr(w1);
    asm("" : "+s"(p0), "+s"(p1));
    return swiglu ? ((v & 1) ? p1 : p0) + (int64_t)(v >> 1) * row_bytes
                  : p0 + (int64_t)v * row_bytes;
  }
  __device__ __forceinline__ float *swiglu_out(int j) const { return y + j; }
  __device__ __forceinline__ float *out(int v) const { return y + v; }
  __device__ __forceinline__ void put(int v, float s) const {
    if (coherent)
      __hip_atomic_store(y + v, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      gstore(y + v, s);
  }
};

template <int R, class Map>
__device__ __forceinline__ void kl_load_rows(const Map &m, int r0, int boff, int c,
                                             u32x4 (&v)[R][3]) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = min(r0 + r, m.total - 1);
    const uint8_t *p = m.row(row) + boff;
    v[r][0] = gload(p);
    v[r][1] = gload(p + 16 * (1 + 2 * c));
    v[r][2] = gload(p + 16 * (2 + 2 * c));
  }
}

// The value of v in lane (lane ^ d), d a power of two fixed at compile time: DPP for 1, 2 and 8
// (quad permutes, a rotation by 8 within rows of 16), a swizzle for 4 and 16, a lane-half swap for
// 32 -- register moves instead of LDS permutes on the reduction's dependent chain. The same values
// as __shfl_xor, so every sum is formed exactly as before.
__device__ __forceinline__ float xor_recv(float v, int d) {
  const int iv = __builtin_bit_cast(int, v);
  int r;
  if (d == 1) {
    r = __builtin_amdgcn_update_dpp(0, iv, 0xB1, 0xF, 0xF, false);  // quad_perm [1, 0, 3, 2]
  } else if (d == 2) {
    r = __builtin_amdgcn_update_dpp(0, iv, 0x4E, 0xF, 0xF, false);  // quad_perm [2, 3, 0, 1]
  } else if (d == 8) {
    r = __builtin_amdgcn_update_dpp(0, iv, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else if (d == 4) {
    r = __builtin_amdgcn_ds_swizzle(iv, 0x101F);  // bit mode: xor 4 within 32 lanes
  } else if (d == 16) {
    r = __builtin_amdgcn_ds_swizzle(iv, 0x401F);  // bit mode: xor 16 within 32 lanes
  } else {  // 32: lanes 0-31 and 32-63 exchange halves
    const auto sw = __builtin_amdgcn_permlane32_swap((unsigned)iv, (unsigned)iv, false, false);
    r = (int)((threadIdx.x & 32) ? sw[0] : sw[1]);
  }
  return __builtin_bit_cast(float, r);
}

// The scale and min of the group's two sub-blocks applied to its two partial sums: dl = sum over
// the low sub-block of q x (quants as fp16 subnormals, i.e. q * 2^-24), dh the same for the high
// sub-block with the quants scaled by 16 (their nibble sits 4 bits up).
__device__ __forceinline__ float kl_group_finish(const u32x4 &hdr, float dl, float dh, float sx_lo,
                                                 float sx_hi, const Q4kField &f0,
                                                 const Q4kField &f1) {
  const uint32_t h0 = hdr.x, s0 = hdr.y, s1 = hdr.z, s2 = hdr.w;
  const float d = half_bits_to_float(h0) * 0x1p24f, dmin = half_bits_to_float(h0 >> 16);
  float sc_lo, m_lo, sc_hi, m_hi;
  q4k_scale_min_at(s0, s1, s2, f0, sc_lo, m_lo);
  q4k_scale_min_at(s0, s1, s2, f1, sc_hi, m_hi);
  const float pos = __builtin_fmaf(sc_lo, dl, sc_hi * dh * 0.0625f) * d;
  return __builtin_fmaf(-dmin, __builtin_fmaf(m_lo, sx_lo, m_hi * sx_hi), pos);
}

typedef _Float16 kl_h2 __attribute__((ext_vector_type(2)));

// Quant dword dw (0..7) of a row's 32 group bytes against four activations of each sub-block
// (xl: weights 4 dw .. 4 dw + 3 of the low sub-block, xh: the same of the high one), added to
// the running sums in a fixed order. The nibble of bits 0-3 (16-19) of a word read as binary16 is
// exactly q * 2^-24, that of bits 4-7 (20-23) exactly 16 q * 2^-24; the FMAs take the halves as
// fp16 operands (v_fma_mix_f32), so a word yields two weights for one AND.
__device__ __forceinline__ void kl_dword_fma(uint32_t wq, const float *xl, const float *xh,
                                             float &dl, float &dh) {
  const uint32_t w8 = wq >> 8;
  const kl_h2 l02 = __builtin_bit_cast(kl_h2, opaque(wq & 0x000F000Fu));
  const kl_h2 l13 = __builtin_bit_cast(kl_h2, opaque(w8 & 0x000F000Fu));
  const kl_h2 u02 = __builtin_bit_cast(kl_h2, opaque(wq & 0x00F000F0u));
  const kl_h2 u13 = __builtin_bit_cast(kl_h2, opaque(w8 & 0x00F000F0u));
  dl = __builtin_fmaf((float)l02[0], xl[0], dl);
  dl = __builtin_fmaf((float)l13[0], xl[1], dl);
  dl = __builtin_fmaf((float)l02[1], xl[2], dl);
  dl = __builtin_fmaf((float)l13[1], xl[3], dl);
  dh = __builtin_fmaf((float)u02[0], xh[0], dh);
  dh = __builtin_fmaf((float)u13[0], xh[1], dh);
  dh = __builtin_fmaf((float)u02[1], xh[2], dh);
  dh = __builtin_fmaf((float)u13[1], xh[3], dh);
}

// Partial dot product of one row's 64-weight group with this lane's activations; f0 / f1 locate
// the scale and min of the group's two sub-blocks.
__device__ __forceinline__ float kl_group_dot(const u32x4 (&v)[3], const float (&xv)[64],
                                              float sx_lo, float sx_hi, const Q4kField &f0,
                                              const Q4kField &f1) {
  float dl = 0.f, dh = 0.f;
#pragma unroll
  for (int dw = 0; dw < 8; ++dw)
    kl_dword_fma(dword_of(v[1 + (dw >> 2)], dw & 3), xv + 4 * dw, xv + 32 + 4 * dw, dl, dh);
  return kl_group_finish(v[0], dl, dh, sx_lo, sx_hi, f0, f1);
}

}  // namespace tq
