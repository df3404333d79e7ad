// tq_gemv_mf.hip -- batch-1 Q4_K and Q6_K GEMV with the multiply-adds on the fp16 matrix cores.
//
// Q4_K. Per 256-weight block of a row (d, dmin, sub-block scales sc_j and mins m_j, quants q) the
// product with x is  d * sum_j sc_j sum_{k in j} q_k x_k  -  dmin * sum_j m_j S_j  (S_j = sum of x
// over sub-block j, j = 0..7). The inner sums go to v_mfma_f32_16x16x32_f16:
//   * weight operand (B, 32 k x 16 rows): the nibbles themselves, as fp16 subnormals q * 2^-24
//     (a word masked with 0x000F000F is two of them; with 0x00F000F0, two of 16 q * 2^-24), so
//     building it takes a few AND/shift operations per 8 weights and nothing else;
//   * activation operand (A, 16 operand rows x 32 k): the sub-block's x scaled by a power of two
//     2^e (e per sub-block, bringing its max |x| into [2^14, 2^15)) and split into two fp16 halves,
//     hi = fp16(x 2^e) and lo = fp16(x 2^e - hi); operand row 2 j + h (h = 0 hi, 1 lo) is non-zero
//     only in the k positions that hold sub-block j's weights, so one product per 32 k separates all
//     eight sub-blocks of a block in its output rows and a block's eight products accumulate into
//     one 16x16 fp32 tile.
// Lane l of the wave holds weight row n = l % 16 and, with g = l / 16, quant bytes 16 g .. 16 g + 15
// (piece P = 0) and 64 + 16 g .. 64 + 16 g + 15 (P = 1) of every block: the four lanes of a row
// load 64 consecutive bytes per instruction, so each cache line of a block is requested by about
// one load (whole 32-byte groups per lane put every line under all three loads). Piece P of lane g
// holds half g % 2 of the 32-byte group 2 P + g / 2, i.e. positions 16 (g % 2) .. + 15 of
// sub-blocks j = 4 P + 2 (g / 2) (low nibbles) and j + 1 (high nibbles); product (P, t, nibble)
// takes the piece's dwords 2t, 2t + 1. Operand rows 2 j, 2 j + 1 are non-zero at the k positions
// of the lanes holding sub-block j, so the output lane l still holds operand rows 4 g .. 4 g + 3
// of row n, i.e. exactly the hi and lo sums of sub-blocks 2 g and 2 g + 1, whose scales and mins
// sit in the header that lane loaded, and folds them:
//   d * 2^24 * sc_j f_j (C_hi + C_lo) - dmin * m_j S_j     (f_j = 2^-e_j)
// (with a factor 1/16 on the high-nibble sub-block). The products are exact (an fp16 subnormal
// quant times an 11-bit fp16 value), they add in fp32, and x enters with 22 significant bits.
//
// Q6_K. Per block (d, sixteen int8 scales sc_j of 16-weight sub-blocks, quants q = low4 + 16 high2
// in 0..63, weight i = 128 h + 32 r + l: low4 a nibble of ql[64 h + l + 32 (r % 2)], low for r < 2,
// high2 bits 2r, 2r+1 of qh[32 h + l], sub-block j = i / 16) the product with x is
//   d * sum_j sc_j (sum_{k in j} q_k x_k - 32 S_j).
// Lane l (row n = l % 16, quarter g = l / 16) loads, of each 128-weight half h, ql bytes
// 64 h + 16 g .. + 15 and the qh bytes of the same positions l (16 (g % 2) .. + 15): low nibbles of
// r = g / 2 and high nibbles of r = g / 2 + 2. Product t (0..3) of half h takes positions
// 16 (g % 2) + 8 (t % 2) .. + 7 of r = g / 2 + 2 (t / 2), i.e. sub-block 8 h + 4 (t / 2) + g, as two
// products into the half's accumulator: the low nibbles (in place: 1 or 16 times the nibble) and
// the high bits shifted to 16 (or 256) times their value, so both carry the same factor F (1 or
// 16) of their sub-block. Operand rows 2 jj + h' (jj = j - 8 h) separate the half's 8 sub-blocks;
// the output lane holds sub-blocks 2 g, 2 g + 1 of each half (F = 16 for g >= 2) and folds
//   d * sc_j (2^24 / F * f_j (C_hi + C_lo) - 32 S_j).
// Rows start on a dword (k a multiple of 512): an even block starts on a dword, an odd one two bytes
// past one, and its pieces are loaded from the dword below and realigned in registers.
//
// Work split: a workgroup takes whole 16-row tiles and all of k. It first splits x into the
// operand layout in LDS (with the zero bytes the empty operand rows read), then wave w streams
// blocks [w KB, w KB + KB) of its tiles, the next tiles' weights loaded while it computes the
// current one, and leaves one partial sum per row in LDS; after one barrier the workgroup adds the
// waves' partial sums in wave order and stores the rows. Nothing is split across workgroups, so a
// row's sum is formed the same way whatever the matrix height, the part it falls in or the launch.
#include <hip/hip_runtime.h>

#include <utility>

#include "tq_device.h"
#include "tq_gemv_core.h"
#include "tq_gemv_mf.h"
#include "tq_launch.h"
#include "tq_moe.h"

namespace tq {

typedef _Float16 mf_h8 __attribute__((ext_vector_type(8)));
typedef float mf_f4 __attribute__((ext_vector_type(4)));

template <class F, int... I>
__device__ __forceinline__ void static_for_mf_(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(std::integral_constant<int, i>) for i = 0 .. N-1, in order
template <int N, class F>
__device__ __forceinline__ void static_for_mf(F &&f) {
  static_for_mf_(f, std::make_integer_sequence<int, N>{});
}

// LDS starts with zero bytes [0, 96), which the lanes whose operand rows are empty read, and the
// operands start at byte 192. The real rows' reads sit at 0 or 64 bytes past a 128-byte boundary
// (Q4_K) or at 64 + 32 n16 (Q6_K); the empty lanes of the same instruction read the zeros at a
// different 16-byte slot of that boundary (Q4_K at 32, Q6_K at 0 or 64 by the group's parity), so
// they do not land on the banks of the lanes that read data.
constexpr int kMfZero = 192;        // bytes before the operands (zeros in [0, 96))
constexpr uint32_t kMfZeroQ4 = 32;  // the empty Q4_K lanes' reads: [32, 96)
constexpr int kMfBlockLds = 1024;   // one block's activation operands: 256 values x hi/lo x 2 B

// The activation operands and sums of one block in LDS, and the lane's part of a block.
template <int FMT>
struct MfFmt;

__device__ __forceinline__ mf_f4 mf_lds4(const uint8_t *lds, uint32_t off) {
  return *reinterpret_cast<const mf_f4 *>(lds + off);
}
__device__ __forceinline__ mf_h8 mf_lds_op(const uint8_t *lds, uint32_t off) {
  return *reinterpret_cast<const mf_h8 *>(lds + off);
}
__device__ __forceinline__ mf_f4 mf_mfma(mf_h8 a, u32x4 b, mf_f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(mf_h8, b), c, 0, 0, 0);
}

// ---- Q4_K ----
template <>
struct MfFmt<FMT_Q4_K> {
  static constexpr int kBytes = 144;  // block bytes in a row
  static constexpr int kSub = 8;      // sub-blocks of 32 weights
  static constexpr int kSumLds = 64;  // per block: [group g][S_2g, S_2g+1, f_2g, f_2g+1]
  // cell (sub-block j, hi/lo h, quarter u) of a block's operands
  static __device__ int cell_off(int j, int h, int u) { return (8 * j + 4 * h + u) * 16; }
  // header (d, dmin, packed scales) and the group's 32 quant bytes
  struct Blk {
    u32x4 hdr, qa, qb;
  };
  struct Lane {
    Q4kField f0, f1;
    uint32_t a[4], inc[4], sum_off;  // [2 P + nibble]
  };
  // operand row n16 (sub-block n16 / 2, hi or lo) in the products of piece P and a nibble: the
  // row's quarters 2 (g % 2), 2 (g % 2) + 1 where that sub-block is the lane's, the zeros elsewhere
  static __device__ Lane lane(int n16, int g, int b0, int nblk) {
    Lane L;
    L.f0 = q4k_field(2 * g);
    L.f1 = q4k_field(2 * g + 1);
    const uint32_t own = kMfZero + (uint32_t)b0 * kMfBlockLds + 64u * n16 + 32u * (g & 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool m = (n16 >> 1) == 4 * (i >> 1) + 2 * (g >> 1) + (i & 1);
      L.a[i] = m ? own : kMfZeroQ4;
      L.inc[i] = m ? kMfBlockLds : 0u;
    }
    L.sum_off = kMfZero + nblk * kMfBlockLds + (uint32_t)b0 * kSumLds + 16u * g;
    return L;
  }
  // the block slot past the wave's last block re-reads that block
  static __device__ int clamp_block(int b, int nb) { return min(b, nb - 1); }
  template <int B>
  static __device__ void load(const uint8_t *p, int g, Blk &b) {
    b.hdr = gload(p);
    b.qa = gload(p + 16 + 16 * g);
    b.qb = gload(p + 80 + 16 * g);
  }
  // The weight operand from the lane's two quant dwords (low or high nibbles).
  template <bool HIGH>
  static __device__ u32x4 wop(uint32_t d0, uint32_t d1) {
    constexpr uint32_t M = HIGH ? 0x00F000F0u : 0x000F000Fu;
    return u32x4{d0 & M, (d0 >> 8) & M, d1 & M, (d1 >> 8) & M};
  }
  // eight products into one tile, then the fold of the lane's two sub-blocks
  template <int B>
  static __device__ float block(const Blk &b, const uint8_t *lds, const Lane &L) {
    mf_h8 A[8];  // [2 (2 P + nibble) + t]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      A[2 * i] = mf_lds_op(lds, L.a[i] + B * L.inc[i]);
      A[2 * i + 1] = mf_lds_op(lds, L.a[i] + B * L.inc[i] + 16);
    }
    const mf_f4 sf = mf_lds4(lds, L.sum_off + B * kSumLds);
    const uint32_t qd[8] = {b.qa.x, b.qa.y, b.qa.z, b.qa.w, b.qb.x, b.qb.y, b.qb.z, b.qb.w};
    mf_f4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int P = i >> 1;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t d0 = qd[4 * P + 2 * t], d1 = qd[4 * P + 2 * t + 1];
        c = mf_mfma(A[2 * i + t], (i & 1) ? wop<true>(d0, d1) : wop<false>(d0, d1), c);
      }
    }
    const uint32_t h0 = b.hdr.x;
    const float d24 = half_bits_to_float(h0) * 0x1p24f, dmin = half_bits_to_float(h0 >> 16);
    float sc_a, m_a, sc_b, m_b;
    q4k_scale_min_at(b.hdr.y, b.hdr.z, b.hdr.w, L.f0, sc_a, m_a);
    q4k_scale_min_at(b.hdr.y, b.hdr.z, b.hdr.w, L.f1, sc_b, m_b);
    const float pa = d24 * sc_a * sf[2], pb = d24 * sc_b * 0.0625f * sf[3];
    const float mn = __builtin_fmaf(m_a, sf[0], m_b * sf[1]);
    return __builtin_fmaf(pa, c[0] + c[1], __builtin_fmaf(pb, c[2] + c[3], -dmin * mn));
  }
};

// ---- Q6_K ----
template <>
struct MfFmt<FMT_Q6_K> {
  static constexpr int kBytes = 210;
  static constexpr int kSub = 16;      // sub-blocks of 16 weights
  static constexpr int kSumLds = 128;  // per block: [half h][g][S_j, S_j+1, f_j, f_j+1], j = 8h + 2g
  static __device__ int cell_off(int j, int h, int u) { return (4 * j + 2 * h + u) * 16; }
  // pieces: ql of half 0 and 1, qh of half 0 and 1, scales; for an odd block each loaded from two
  // bytes below with the dword after it (e), realigned at use; e[4] also holds d (even: d in its
  // low half, odd: in its high half)
  struct Blk {
    u32x4 c[5];
    uint32_t e[5];
  };
  struct Lane {
    uint32_t a0, a1, incb0, incb1, inch0, inch1, sum_off, sh, shr, sc_bit;
    int sc_hi;       // the scale dword of half h is 2h + sc_hi
    float k24f;      // 2^24 / F
    int g;
  };
  // Operand row i = 2 jj + h' of a half takes sub-block jj: products 0, 1 of the half give quarter g
  // sub-block g, products 2, 3 sub-block 4 + g; lane (i, g) reads its row's cell for the products
  // whose quarter-g sub-block is i / 2, the zero bytes for the others.
  static __device__ Lane lane(int n16, int g, int b0, int nblk) {
    Lane L;
    const bool m0 = (n16 >> 1) == g, m1 = (n16 >> 1) == 4 + g;
    const uint32_t own = kMfZero + (uint32_t)b0 * kMfBlockLds + 32u * n16;
    const uint32_t zero = 64u * (g & 1);  // [0, 32) or [64, 96)
    L.a0 = m0 ? own : zero;
    L.a1 = m1 ? own : zero;
    L.incb0 = m0 ? kMfBlockLds : 0u;
    L.incb1 = m1 ? kMfBlockLds : 0u;
    L.inch0 = m0 ? 512u : 0u;
    L.inch1 = m1 ? 512u : 0u;
    L.sum_off = kMfZero + nblk * kMfBlockLds + (uint32_t)b0 * kSumLds + 16u * g;
    L.sh = (g >> 1) ? 2u : 4u;  // high bits 2r, 2r+1 of r = g/2 (+2) to bits 4, 5 (8, 9)
    L.shr = 8u - L.sh;
    L.sc_bit = 16u * (g & 1);
    L.sc_hi = g >> 1;
    L.k24f = g >= 2 ? 0x1p20f : 0x1p24f;
    L.g = g;
    return L;
  }
  // (the wave's blocks start at an even index and nb is even: the slot keeps its parity)
  static __device__ int clamp_block(int b, int nb) { return b < nb ? b : nb - 2 + (b & 1); }
  static __device__ uint32_t off(int i, int g) {
    return i < 2 ? 64 * i + 16 * g : i < 4 ? 128 + 32 * (i - 2) + 16 * (g & 1) : 192;
  }
  template <int B>
  static __device__ void load(const uint8_t *p, int g, Blk &b) {
    if constexpr ((B & 1) == 0) {
#pragma unroll
      for (int i = 0; i < 5; ++i) b.c[i] = *(gu32x4a4)(p + off(i, g));
      b.e[4] = *(const __attribute__((address_space(1))) uint32_t *)(p + 208);
    } else {
      const uint8_t *q = p - 2;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        b.c[i] = *(gu32x4a4)(q + off(i, g));
        b.e[i] = *(const __attribute__((address_space(1))) uint32_t *)(q + off(i, g) + 16);
      }
    }
  }
  template <int B>
  static __device__ u32x4 piece(const Blk &b, int i) {
    if constexpr ((B & 1) == 0) {
      return b.c[i];
    } else {
      const u32x4 w = b.c[i];
      return u32x4{shift2(w.x, w.y), shift2(w.y, w.z), shift2(w.z, w.w), shift2(w.w, b.e[i])};
    }
  }
  template <int B>
  static __device__ float block(const Blk &b, const uint8_t *lds, const Lane &L) {
    const u32x4 sc = piece<B>(b, 4);
    const float d = half_bits_to_float((B & 1) ? b.e[4] >> 16 : b.e[4]);
    float acc = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 ql = piece<B>(b, h), qh = piece<B>(b, 2 + h);
      const uint32_t a0 = L.a0 + B * L.incb0 + h * L.inch0, a1 = L.a1 + B * L.incb1 + h * L.inch1;
      const mf_f4 sf = mf_lds4(lds, L.sum_off + B * kSumLds + 64 * h);
      mf_f4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t l0 = ql[2 * u], l1 = ql[2 * u + 1], l0s = l0 >> 8, l1s = l1 >> 8;
        const uint32_t hq0 = qh[2 * u], hq1 = qh[2 * u + 1];
        const uint32_t h0l = hq0 << L.sh, h0r = hq0 >> L.shr, h1l = hq1 << L.sh, h1r = hq1 >> L.shr;
#pragma unroll
        for (int ts = 0; ts < 2; ++ts) {  // r = g/2 (low nibbles, high bits x16), r = g/2 + 2 (x16)
          const uint32_t ML = ts ? 0x00F000F0u : 0x000F000Fu, MH = ts ? 0x03000300u : 0x00300030u;
          const mf_h8 A = mf_lds_op(lds, (ts ? a1 : a0) + 16 * u);
          c = mf_mfma(A, u32x4{l0 & ML, l0s & ML, l1 & ML, l1s & ML}, c);
          c = mf_mfma(A, u32x4{h0l & MH, h0r & MH, h1l & MH, h1r & MH}, c);
        }
      }
      // sub-blocks j = 8h + 2g + s (s = 0, 1): scale bytes 2 (g % 2) + s of dword 2h + g / 2
      const uint32_t sd = L.sc_hi ? sc[2 * h + 1] : sc[2 * h];
      // (the builtin's result type is unsigned: the sign-extended field is read back as int)
      const float s0 = (float)(int)__builtin_amdgcn_sbfe(sd, L.sc_bit, 8);
      const float s1 = (float)(int)__builtin_amdgcn_sbfe(sd, L.sc_bit + 8, 8);
      const float t0 = __builtin_fmaf(L.k24f * sf[2], c[0] + c[1], -32.f * sf[0]);
      const float t1 = __builtin_fmaf(L.k24f * sf[3], c[2] + c[3], -32.f * sf[1]);
      acc = __builtin_fmaf(s0, t0, __builtin_fmaf(s1, t1, acc));
    }
    return d * acc;
  }
};

// LDS bytes of a workgroup: zeros, operands, sums and scales, the waves' partial sums.
template <int FMT>
__host__ __device__ inline int mf_lds_bytes(int nblk, int waves, int tiles) {
  return kMfZero + nblk * (kMfBlockLds + MfFmt<FMT>::kSumLds) + tiles * waves * 16 * 4;
}

// 1. x -> operand layout. Cell c = (block b, sub-block j, part u) holds 8 values of the sub-block,
// in the order the weight operand takes them (a masked word holds the nibbles of bytes 0 and 2, the
// word shifted by 8 those of bytes 1 and 3): 0 2 1 3 4 6 5 7. Thread t takes cells t, t + blockDim,
// ... (at most MC); the neighbouring threads of one sub-block (4 for Q4_K, 2 for Q6_K) are in or
// out of range together. The values are loaded before the weights (mf_split_load), so that the
// split waits only for them.
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
template <int FMT, int MC>
__device__ __forceinline__ void mf_split(const MfCells<MC> &cv, int nblk, uint8_t *lds) {
  using F = MfFmt<FMT>;
  constexpr int kCells = 32 / F::kSub;  // cells per sub-block
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
    if constexpr (kCells == 4) m = fmaxf(m, xor_recv(m, 2));
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
    const int b = c >> 5, j = (c & 31) / kCells, u = c % kCells;
    uint8_t *blk = ops + b * kMfBlockLds;
    *reinterpret_cast<u32x4 *>(blk + F::cell_off(j, 0, u)) = hi;
    *reinterpret_cast<u32x4 *>(blk + F::cell_off(j, 1, u)) = lo;
    float sum = ((v0.x + v0.y) + (v0.z + v0.w)) + ((v1.x + v1.y) + (v1.z + v1.w));
    sum += xor_recv(sum, 1);
    if constexpr (kCells == 4) sum += xor_recv(sum, 2);
    if (u == 0) {  // sums [j / 2][S_j, S_j^1, f_j, f_j^1] (pairs of neighbouring sub-blocks)
      float *q = sums + b * (F::kSumLds / 4) + (j >> 1) * 4;
      q[j & 1] = sum;
      q[2 + (j & 1)] = ldexpf(1.f, -e);
    }
  }
}

// 2. the lane's loads of its tile row. Every block slot is loaded (past the wave's last block: a
// block again), so that no load sits behind a branch: the compiler then counts the loads in
// flight and waits for each block's own.
template <int FMT, int KB, class Map>
__device__ __forceinline__ void mf_load_tile(const Map &m, int tile, int b0, int nb, int n16,
                                             int g, typename MfFmt<FMT>::Blk (&buf)[KB]) {
  using F = MfFmt<FMT>;
  const uint8_t *rp = m.row(min(tile * 16 + n16, m.total - 1)) + (int64_t)b0 * F::kBytes;  // b0: block in the row
  static_for_mf<KB>([&](auto B) {
    constexpr int b = decltype(B)::value;
    F::template load<b>(rp + F::clamp_block(b, nb) * F::kBytes, g, buf[b]);
  });
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

// 3. one tile's blocks of the wave (the activation operands read from LDS per block: holding them
// in registers across tiles measured no faster), then the sum over the lane's four groups
template <int FMT, int KB>
__device__ __forceinline__ void mf_tile(const typename MfFmt<FMT>::Blk (&buf)[KB], int nb,
                                        const uint8_t *lds, const typename MfFmt<FMT>::Lane &L,
                                        float *red, int n16, int g, bool keep) {
  float acc = 0.f;
  static_for_mf<KB>([&](auto B) {
    constexpr int b = decltype(B)::value;
    if (b < nb) acc += MfFmt<FMT>::template block<b>(buf[b], lds, L);
  });
  acc = mf_pair_sum<true>(acc);   // groups 0 + 1, 2 + 3
  acc = mf_pair_sum<false>(acc);  // (0 + 1) + (2 + 3)
  if (keep && g == 0) red[n16] = acc;
}

// Grid: G workgroups, workgroup w taking the 16-row tiles w, w + G, w + 2G, ... (TPW of them, or
// fewer for the grid's last workgroups): at any time the workgroups stream neighbouring tiles, one
// window of the matrix. blockDim = 64 * ceil(nblk / KB): at most 16 waves (128 VGPRs a lane), at
// most 8 when BIG (256). DEPTH 0 (one buffer): each tile after the first is loaded just before its
// products.
// The tiles' code is straight-line (TPW and the buffer of each tile fixed at compile time), with
// the weights of the next DEPTH tiles in flight while a tile is computed: the compiler then counts
// every load in flight and waits for each tile's own. (In a loop, loads carried across the back
// edge and the joins of the buffers' values make it wait for all loads before the next prefetch.)
// A workgroup with fewer than TPW tiles loads its last tile again for the missing ones and does
// not keep their sums.
//
// k slices (ksplit > 1, k too long for one workgroup's LDS): workgroup (set gi, slice s) takes
// the tiles of set gi over blocks [s sb, s sb + sb) only (sb blocks in every slice), stores its
// rows' sums device-coherently to `partial` and counts itself on set gi's arrival word; the last
// slice to arrive adds the ksplit sums in slice order and stores the rows.
//
// The body of one workgroup: tile set gi of G, k slice `slice` of ksplit, over rows of any row map
// (a matrix, or one expert's matrices). Returns false where a slice that was not the last to
// arrive has left its sums to another workgroup.
template <int FMT, int KB, int TPW, int DEPTH, class Map>
__device__ __forceinline__ bool mf_body(const Map &m, int gi, int G, int sb, int ksplit, int slice,
                                        const float *__restrict__ xall, float *partial,
                                        const Arrivals &arr, uint8_t *lds) {
  using F = MfFmt<FMT>;
  __shared__ int is_last;
  const int lane = threadIdx.x & 63, wave = wave_index(), nw = blockDim.x >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const int ntiles = (m.total + 15) >> 4;
  const int nt = min(TPW, (ntiles - gi + G - 1) / G);  // >= 1
  const int nblk = sb;                                  // blocks of this slice
  const float *x = xall + (int64_t)slice * sb * 256;
  const int b0 = wave * KB, nb = min(KB, nblk - b0);
  const int rb0 = slice * sb + b0;                      // the wave's first block in the row
  float *red = reinterpret_cast<float *>(lds + kMfZero + nblk * (kMfBlockLds + F::kSumLds));
  auto tile_of = [&](int i) { return gi + min(i, nt - 1) * G; };
  const typename F::Lane L = F::lane(n16, g, b0, nblk);
  float *wred = red + wave * 16;
  const int wstride = nw * 16;

  // the activations' loads, the first DEPTH tiles' weights, then the split (waiting for the
  // activations only)
  constexpr int MC = KB >= 2 ? KB / 2 : 1;  // cells per thread: 32 nblk cells, 64 ceil(nblk / KB) threads
  constexpr int NB = DEPTH + 1;             // weight buffers
  constexpr int PRE = DEPTH > 1 ? DEPTH : 1;  // tiles loaded before the split
  MfCells<MC> cv;
  mf_split_load<MC>(x, nblk, cv);
  typename F::Blk buf[NB][KB];
  static_for_mf<PRE>([&](auto T) {
    constexpr int t = decltype(T)::value;
    if constexpr (t < TPW) mf_load_tile<FMT, KB>(m, tile_of(t), rb0, nb, n16, g, buf[t % NB]);
  });
  mf_split<FMT, MC>(cv, nblk, lds);
  __syncthreads();
  static_for_mf<TPW>([&](auto T) {
    constexpr int t = decltype(T)::value;
    if constexpr (t + DEPTH < TPW && t + DEPTH >= PRE)  // (DEPTH 0: tile t, just before its use)
      mf_load_tile<FMT, KB>(m, tile_of(t + DEPTH), rb0, nb, n16, g, buf[(t + DEPTH) % NB]);
    mf_tile<FMT, KB>(buf[t % NB], nb, lds, L, wred + t * wstride, n16, g, t < nt);
  });
  __syncthreads();

  // 4. the rows: the waves' partial sums in wave order (and, with k slices, the slices' sums in
  // slice order)
  const int rows = nt * 16;
  auto wave_sum = [&](int i) {
    const float *r = red + (i >> 4) * wstride + (i & 15);
    float v = 0.f;
    for (int w = 0; w < nw; ++w) v += r[w * 16];
    return v;
  };
  const float *total = nullptr;  // with slices: the row's slice sums, ksplit apart
  if (ksplit > 1) {
    float *mine = partial + ((int64_t)gi * ksplit + slice) * TPW * 16;
    for (int i = threadIdx.x; i < rows; i += blockDim.x)
      __hip_atomic_store(mine + i, wave_sum(i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's stores have completed
    __syncthreads();
    if (threadIdx.x == 0) is_last = arrive_last(arr, gi, (unsigned)ksplit);
    __syncthreads();
    if (!is_last) return false;
    total = partial + (int64_t)gi * ksplit * TPW * 16;
  }
  auto row_sum = [&](int i) {
    if (!total) return wave_sum(i);
    float v = 0.f;
    for (int q = 0; q < ksplit; ++q)
      v += __hip_atomic_load(total + q * TPW * 16 + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return v;
  };
  if (m.swiglu) {  // virtual rows (gate r, up r) pairs; tiles start at even rows
    for (int i = 2 * (int)threadIdx.x; i < rows; i += 2 * (int)blockDim.x) {
      const int v = tile_of(i >> 4) * 16 + (i & 15);
      if (v >= m.total) continue;
      gstore(m.swiglu_out(v >> 1), silu_mul(row_sum(i), row_sum(i + 1)));
    }
  } else {
    for (int i = threadIdx.x; i < rows; i += blockDim.x) {
      const int v = tile_of(i >> 4) * 16 + (i & 15);
      if (v >= m.total) continue;
      m.put(v, row_sum(i));
    }
  }
  if (total && threadIdx.x == 0) done_arrivals(arr, gi);
  return true;
}

template <int FMT, int KB, int TPW, int DEPTH, bool BIG>
__global__ __launch_bounds__(BIG ? 512 : 1024) void k_gemv_mf(KlMap m, int sb, int ksplit,
                                                              const float *__restrict__ xall,
                                                              float *partial, Arrivals arr) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int slice = (int)blockIdx.x % ksplit, gi = (int)blockIdx.x / ksplit;
  mf_body<FMT, KB, TPW, DEPTH>(m, gi, (int)gridDim.x / ksplit, sb, ksplit, slice, xall, partial,
                               arr, lds);
}

// The same body over the experts of a one-token MoE step: workgroup b takes tile set b % sets of
// active slot slot0 + b / sets (every active expert has that one token); gate/up: the expert's gate
// and up rows interleaved with the SwiGLU in the epilogue, x = the token's activations, h out;
// down: x = h of the slot's position, o out. With the combine fused into the down launch, each
// workgroup then counts itself on its tile set's counter, and the last active slot to arrive adds,
// for each row of the set, the slots in routing order and the shared expert (the combine kernel's
// order). The gate/up launch's first workgroup clears the counters. With route1 (one token, all
// stages in one call) the gate/up launch also makes the top-k selection: every workgroup computes
// it from the router's partial sums before its products (a few microseconds, in place of a launch
// of its own and the gap before the next), and workgroup 0 stores the routing outputs, which the
// down launch reads.
template <int FMT, int KB, int TPW, int DEPTH, bool BIG>
__global__ __launch_bounds__(BIG ? 512 : 1024) void k_moe_mf(MoeKlArgs a, int sets) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int last;
  if (a.nctr > 0 && blockIdx.x == 0)
    for (int i = (int)threadIdx.x; i < a.nctr; i += blockDim.x)
      __hip_atomic_store(a.ctr + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int slot = a.slot0 + (int)blockIdx.x / sets, gi = (int)blockIdx.x % sets;
  int e, p;
  int64_t xrow;
  if (a.route1) {
    // one token, the selection made here: slot r < topk takes the chosen expert of rank r (its
    // position r), slot topk the shared expert (position topk); the token's row is row 0
    e = route_one_token(a.route, a.topk, slot, blockIdx.x == 0);
    p = slot < a.topk ? slot : a.Tk;
    xrow = 0;
  } else {
    if (slot >= *a.n_active) return;
    e = a.act[slot];
    p = a.act[a.act_stride + slot];
    xrow = !a.gate_up ? p : p >= a.Tk ? p - a.Tk : a.pairs[p] / a.topk;
  }
  if ((unsigned)e > (unsigned)a.E) return;  // never past the expert table (id E: shared expert)
  const uint8_t *w[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int mat = a.gate_up ? q : 2;
    if (e == a.E)
      w[q] = (const uint8_t *)a.shared.m[mat];
    else if (a.staging != nullptr)
      w[q] = a.staging + (int64_t)slot * a.stage_stride + a.stage_off[mat];
    else
      w[q] = (const uint8_t *)a.experts[e].m[mat];
  }
  const MoeRowMap m{w[0], w[1], a.out + (int64_t)p * a.ldo, a.gate_up, a.rows, a.row_bytes,
                    a.fuse_y != nullptr};
  mf_body<FMT, KB, TPW, DEPTH>(m, gi, sets, (int)(a.row_bytes / MfFmt<FMT>::kBytes), 1, 0,
                               a.x + xrow * a.ldx, nullptr, Arrivals{}, lds);
  if (a.fuse_y == nullptr) return;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's sums are stored
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(&a.ctr[gi], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           (unsigned)(*a.n_active - 1);
  __syncthreads();
  if (!last) return;
  const int ntiles = (a.rows + 15) >> 4, nt = min(TPW, (ntiles - gi + sets - 1) / sets);
  for (int i = (int)threadIdx.x; i < nt * 16; i += blockDim.x) {
    const int c = (gi + (i >> 4) * sets) * 16 + (i & 15);
    if (c < a.rows) a.fuse_y[c] = moe_combine_value(a, c);
  }
}

// ---- host side ----------------------------------------------------------------------------------

// Blocks per wave. Q4_K: 1 up to k = 2048, 2 up to k = 8192, else 4 (at most 16 waves, k < 16384).
// Q6_K (a block's pieces take 20-25 registers): 2 up to k = 4096, else 4 (at most 8 waves).
static int mf_kb(int fmt, int nblk) {
  const int v = knob(TQ_KNOB_MF_KB, 0);
  if (fmt == FMT_Q6_K) {
    int kb = v == 2 || v == 4 ? v : nblk <= 16 ? 2 : 4;
    while ((nblk + kb - 1) / kb > 8) kb *= 2;
    return kb;
  }
  int kb = v == 1 || v == 2 || v == 4 ? v : nblk <= 8 ? 1 : nblk <= 32 ? 2 : 4;
  while ((nblk + kb - 1) / kb > 16) kb *= 2;
  return kb;
}

static int mf_lds(int fmt, int nblk, int waves, int tiles) {
  return fmt == FMT_Q6_K ? mf_lds_bytes<FMT_Q6_K>(nblk, waves, tiles)
                         : mf_lds_bytes<FMT_Q4_K>(nblk, waves, tiles);
}

// Tiles per workgroup that have a kernel (the next one up is taken).
constexpr int kMfTpw[] = {1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 14, 16};

// The launch of rows x k: blocks per slice sb and slices (a slice takes all of k when its operands
// fit 64 KB of LDS: Q4_K up to k = 14336, Q6_K up to 8192; longer Q6_K rows, k a multiple of 512,
// go in 2..8 equal slices of an even number of blocks, at most 32), blocks per wave, waves, tiles
// per workgroup, grid.
struct MfPlan {
  int sb, ksplit, kb, waves, tpw, sets, lds;
};
// LDS beyond the dynamic part: the kernels' own __shared__ variables (k_moe_mf: the selection's
// logits), kept out of the 64 KB a workgroup may take.
constexpr int kMfStaticLds = 64, kMoeMfStaticLds = 1152;

static bool mf_plan(int fmt, int64_t rows, int64_t k, MfPlan &p, int slots = 1,
                    int static_lds = kMfStaticLds) {
  if (!knob(TQ_KNOB_GEMV_MF, 2) || k % 256 != 0 || k < 256 || rows < 1 || rows >= (1ll << 30))
    return false;
  if (fmt != FMT_Q4_K && fmt != FMT_Q6_K) return false;
  const int nblk = (int)(k / 256);
  p.ksplit = 1;
  p.sb = nblk;
  // longest slice: Q6_K 32 blocks (an even number), Q4_K all of k below 16384, else 32
  const bool q6 = fmt == FMT_Q6_K;
  if (q6 && k % 512 != 0) return false;
  if ((q6 && nblk > 32) || (!q6 && nblk >= 64)) {
    p.ksplit = 0;
    for (int q = 2; q <= 8 && !p.ksplit; ++q)
      if (nblk % q == 0 && (!q6 || (nblk / q) % 2 == 0) && nblk / q <= 32) p.ksplit = q;
    if (!p.ksplit) return false;
    p.sb = nblk / p.ksplit;
  }
  if (const int fk = knob(TQ_KNOB_MF_KSPLIT, 0); fk > 1 && p.ksplit == 1 && nblk % fk == 0 &&
                                                 (!q6 || (nblk / fk) % 2 == 0)) {
    p.ksplit = fk;  // tuning: forced slices
    p.sb = nblk / fk;
  }
  p.kb = mf_kb(fmt, p.sb);
  if (p.kb > 4) return false;
  p.waves = (p.sb + p.kb - 1) / p.kb;
  const int64_t ntiles = (rows + 15) / 16;
  const int target = knob(TQ_KNOB_MF_WGS, 256);
  const int64_t want = (ntiles * p.ksplit * slots + target - 1) / (target > 0 ? target : 1);
  int ti = 0;
  while (ti < 11 && kMfTpw[ti] < want) ++ti;
  const int cap = 65536 - static_lds;
  while (ti > 0 && mf_lds(fmt, p.sb, p.waves, kMfTpw[ti]) > cap) --ti;
  p.tpw = kMfTpw[ti];
  p.lds = mf_lds(fmt, p.sb, p.waves, p.tpw);
  p.sets = (int)((ntiles + p.tpw - 1) / p.tpw);
  return p.lds <= cap;
}

bool mf_gemv_ok(int fmt, int64_t k) {
  MfPlan p;
  return mf_plan(fmt, 16, k, p) && p.ksplit == 1;
}

bool mf_gemv_sliced(int fmt, int64_t k) {
  MfPlan p;
  return mf_plan(fmt, 16, k, p) && p.ksplit > 1;
}

size_t mf_workspace_bytes(int fmt, int64_t rows, int64_t k) {
  MfPlan p;
  if (!mf_plan(fmt, rows, k, p) || p.ksplit == 1) return 0;
  return (size_t)align256((int64_t)p.sets * p.ksplit * p.tpw * 16 * 4);
}

template <int V>
using mf_c = std::integral_constant<int, V>;

// Calls launch(FMT, KB, DEPTH, BIG, TPW) with plan p's kernel variant as compile-time constants.
template <class L>
static void mf_variant(int fmt, const MfPlan &p, L &&launch) {
  auto by_tpw = [&](auto fmt_c, auto kb_c, auto depth_c, auto big_c) {
    switch (p.tpw) {
#define TQ_MF(T)                                \
  case T:                                       \
    launch(fmt_c, kb_c, depth_c, big_c, mf_c<T>{}); \
    break;
      TQ_MF(1) TQ_MF(2) TQ_MF(3) TQ_MF(4) TQ_MF(5) TQ_MF(6) TQ_MF(7) TQ_MF(8) TQ_MF(10) TQ_MF(12)
      TQ_MF(14) TQ_MF(16)
#undef TQ_MF
    }
  };
  if (fmt == FMT_Q6_K) {  // at most 8 waves (256 VGPRs): two buffers (235 VGPRs at 4 blocks a wave)
    if (p.kb == 2)
      by_tpw(mf_c<FMT_Q6_K>{}, mf_c<2>{}, mf_c<1>{}, mf_c<1>{});
    else if (p.tpw >= 2 && knob(TQ_KNOB_MF_DEEP, 1) != 0)
      by_tpw(mf_c<FMT_Q6_K>{}, mf_c<4>{}, mf_c<1>{}, mf_c<1>{});
    else
      by_tpw(mf_c<FMT_Q6_K>{}, mf_c<4>{}, mf_c<0>{}, mf_c<1>{});
    return;
  }
  // two tiles ahead where the workgroup has several tiles and at most 8 waves (256 VGPRs a lane)
  // (three or four tiles ahead measured slower)
  // (one ahead by default: two ahead, with twice the registers and half the waves per SIMD, made
  // the 8B-shaped gate|up launch slower once each load covered a 64-byte run)
  const bool deep = p.kb == 2 && p.waves <= 8 && p.tpw >= 3 && knob(TQ_KNOB_MF_DEEP, 1) == 2;
  if (p.kb == 1)
    by_tpw(mf_c<FMT_Q4_K>{}, mf_c<1>{}, mf_c<1>{}, mf_c<0>{});
  else if (p.kb == 2 && deep)
    by_tpw(mf_c<FMT_Q4_K>{}, mf_c<2>{}, mf_c<2>{}, mf_c<1>{});
  else if (p.kb == 2)
    by_tpw(mf_c<FMT_Q4_K>{}, mf_c<2>{}, mf_c<1>{}, mf_c<0>{});
  else
    by_tpw(mf_c<FMT_Q4_K>{}, mf_c<4>{}, mf_c<0>{}, mf_c<0>{});  // one buffer (128 VGPRs)
}

int launch_gemv_mf(int fmt, const KlMap &m, int64_t k, const float *x, float *partial,
                   unsigned long long *counters, int max_counters, hipStream_t s) {
  MfPlan p;
  if (!mf_plan(fmt, m.total, k, p)) return -2;
  if (p.ksplit > 1 && (!partial || !counters || p.sets > max_counters)) return -2;
  const Arrivals arr{counters, p.ksplit > 1 ? call_tag() : 0ull};
  const dim3 gd(p.sets * p.ksplit), bd(64 * p.waves);
  mf_variant(fmt, p, [&](auto F, auto KB, auto D, auto BIG, auto T) {
    hipLaunchKernelGGL((k_gemv_mf<F(), KB(), T(), D(), (bool)BIG()>), gd, bd, p.lds, s, m, p.sb,
                       p.ksplit, x, partial, arr);
  });
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

bool moe_mf_ok(int fmt, int64_t hidden, int64_t ffn) {
  MfPlan p;
  return fmt == FMT_Q4_K && knob(TQ_KNOB_MOE_MF, 1) &&
         mf_plan(fmt, 16, hidden, p, 1, kMoeMfStaticLds) && p.ksplit == 1 &&
         mf_plan(fmt, 16, ffn, p, 1, kMoeMfStaticLds) && p.ksplit == 1;
}

int launch_moe_mf(const MoeKlArgs &a, int64_t k, int nslots, hipStream_t s) {
  MfPlan p;
  if (!moe_mf_ok(FMT_Q4_K, k, k) || nslots < 1 || a.row_bytes != k / 256 * 144 ||
      ((uintptr_t)a.x & 15) != 0 || a.ldx % 4 != 0 || !mf_plan(FMT_Q4_K, a.rows, k, p, nslots, kMoeMfStaticLds))
    return -2;
  // the fused combine counts on one counter per tile set; the selection is made for slots from 0
  if (a.fuse_y != nullptr && (a.ctr == nullptr || p.sets > a.ctr_cap)) return -2;
  if (a.route1 && (!a.gate_up || a.slot0 != 0 || a.route.E > 256 || nslots > a.topk + 1)) return -2;
  const dim3 gd((unsigned)(nslots * p.sets)), bd(64 * p.waves);
  mf_variant(FMT_Q4_K, p, [&](auto F, auto KB, auto D, auto BIG, auto T) {
    if constexpr (F() == FMT_Q4_K)
      hipLaunchKernelGGL((k_moe_mf<F(), KB(), T(), D(), (bool)BIG()>), gd, bd, p.lds, s, a, p.sets);
  });
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace tq
