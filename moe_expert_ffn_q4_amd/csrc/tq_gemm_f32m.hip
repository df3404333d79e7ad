// tq_gemm_f32m.hip -- Q6_K and Q8_0 products of 2..16 tokens on the fp32 matrix cores.
//
// The products of the block formats whose weights do not fit an exact fp16 operand (Q6_K:
// sc * (q - 32) reaches 4096 with odd values above 2048; Q8_0: one fp16 scale per 32 weights)
// run on v_mfma_f32_16x16x4_f32 with the weights dequantized once per block in registers and the
// tokens' fp32 activations as the other operand, so the arithmetic is the fp32 GEMV's (exact
// dequantized weights, fp32 products and sums) at twice the fp32 vector rate and with one
// dequantization per weight for all the tokens:
//   Q8_0: operand d * q (exact in fp32);
//   Q6_K: operand sc * (q - 32) (an integer below 2^13, exact), the block's d applied to the
//         block's accumulator (d is one value per 256 weights).
// Layout (A = 16 token rows x 4 k, B = 4 k x 16 weight rows, D = 16 x 16): lane l = 16 g + t
// supplies token t's x and weight row t's value at k = 64 g + s in step s = 0..63 of a block, so
// each lane dequantizes one contiguous quarter of a block of its row and reads one contiguous
// 64-value piece of one token row; it receives D[token 4 g + i][row t].
// Up to 4 tokens (T4) the same lanes run v_mfma_f32_4x4x1f32 instead (16 blocks of 4 x 4 x 1, the
// same rate per cycle, none of it spent on padding tokens): lane l = 16 g + t supplies, of block
// b = l / 4, A_b[l % 4] = token (t % 4)'s x and B_b[l % 4] = weight row t's value, both at
// k = 64 g + s, and receives D_b[token i][row t] for i = 0..3: the sum over quarter g of the block's
// k, so the four quarters' sums (lanes t, t + 16, t + 32, t + 48) are added once at the end.
// Work split: a workgroup of 4 waves covers 4 x RT x 16 rows and one k slice (blocks per slice a
// function of k only); with several slices the last workgroup of a row group adds the slices in
// slice order (device-coherent partial stores, agent-scope counter, reset afterwards).
#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_gemm_f32m.h"
#include "tq_launch.h"

namespace tq {

typedef float f32x4m __attribute__((ext_vector_type(4)));

constexpr int kF32mRT = 2;         // 16-row tiles per wave
constexpr int kF32mMaxSlices = 8;  // k slices

// Dwords read through the global address space (row pointers from the row map are generic).
typedef const __attribute__((address_space(1))) uint32_t gu32;

template <int FMT>
struct F32mRaw;

// Q8_0: blocks 2g and 2g+1 of the 256-weight unit (68 bytes, dword aligned).
template <>
struct F32mRaw<FMT_Q8_0> {
  uint32_t v[17];
  __device__ __forceinline__ void load(const uint8_t *row, int kb, int g) {
    const gu32 *p = (const gu32 *)(row + (int64_t)kb * 272 + 68 * g);
#pragma unroll
    for (int i = 0; i < 17; ++i) v[i] = p[i];
  }
};

// Q6_K: of block kb, the 64 low-bit bytes of half h = g / 2, its 32 high-bit bytes, the four int8
// scales of the quarter and d, as loaded: dword runs from the dword boundary at or below each run
// (blocks start 2 bytes past one for odd kb; rows are dword aligned), one dword longer than the
// run. Each dword is realigned (v_alignbyte) where it is used, so the loads stay in flight while
// the previous block is computed and no realigned copy is kept. Every dword read lies inside the
// block: the extra dword of the scale run is read only for odd kb (for even kb it would pass the
// block's end).
template <>
struct F32mRaw<FMT_Q6_K> {
  uint32_t ql[17], qh[9], sc[2];
  uint32_t dbits;
  uint32_t shift;  // 2 for odd kb, else 0 (wave-uniform)
  __device__ __forceinline__ void load(const uint8_t *row, int kb, int g) {
    const int off = kb * 210, h = g >> 1;
    const gu32 *base = (const gu32 *)(row + (off & ~3));
    shift = (uint32_t)(off & 2);
    dbits = *(const __attribute__((address_space(1))) uint16_t *)(row + off + 208);
#pragma unroll
    for (int i = 0; i < 17; ++i) ql[i] = base[16 * h + i];
#pragma unroll
    for (int i = 0; i < 9; ++i) qh[i] = base[32 + 8 * h + i];
    sc[0] = base[48 + g];
    sc[1] = shift ? base[49 + g] : 0u;
  }
};

// The lane's 16 activations of steps 16 j .. 16 j + 15 (its token row's piece in LDS).
__device__ __forceinline__ void f32m_x16(const float *xs, int j, float (&xv)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4m v = *reinterpret_cast<const f32x4m *>(xs + 16 * j + 4 * i);
    xv[4 * i] = v[0];
    xv[4 * i + 1] = v[1];
    xv[4 * i + 2] = v[2];
    xv[4 * i + 3] = v[3];
  }
}

// One step of the matrix cores: 16 tokens x 4 k x 16 rows, or (T4) 16 blocks of 4 x 1 x 4.
template <bool T4>
__device__ __forceinline__ f32x4m f32m_mfma(float x, float w, f32x4m c) {
  if constexpr (T4)
    return __builtin_amdgcn_mfma_f32_4x4x1f32(x, w, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x4f32(x, w, c, 0, 0, 0);
}

// The tile's contribution of one block: 64 steps of the matrix cores; Q6_K folds d at the end.
template <int FMT, bool T4>
__device__ __forceinline__ void f32m_block(const F32mRaw<FMT> (&raw)[kF32mRT], const float *xs,
                                           int g, f32x4m (&acc)[kF32mRT]) {
  const f32x4m zero = {0.f, 0.f, 0.f, 0.f};
  if constexpr (FMT == FMT_Q8_0) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float d[kF32mRT];
#pragma unroll
      for (int r = 0; r < kF32mRT; ++r)
        d[r] = half_bits_to_float(half ? raw[r].v[8] >> 16 : raw[r].v[0] & 0xFFFFu);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float xv[16];
        f32m_x16(xs, 2 * half + j, xv);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int o = 34 * half + 2 + 16 * j + e;  // byte of quant 16 j + e of this half
#pragma unroll
          for (int r = 0; r < kF32mRT; ++r) {
            const int q = __builtin_amdgcn_sbfe(raw[r].v[o >> 2], 8 * (o & 3), 8);
            acc[r] = f32m_mfma<T4>(xv[e], d[r] * (float)q, acc[r]);
          }
        }
      }
    }
  } else {
    // the quarter's nibbles: low ones for even g, high ones for odd g; its two high bits: bits
    // 4 (g & 1) + 2 (s / 32) of the high-bit byte. Four consecutive steps take bytes l..l+3 of
    // one low-bit and one high-bit dword, so their 6-bit quants are assembled as the four bytes of
    // one dword (five integer operations), then each is one byte conversion and one FMA:
    // sc * q - 32 sc, an integer below 2^13 in magnitude, exact in fp32.
    const uint32_t sh = 4u * (uint32_t)(g & 1);
    uint32_t scw[kF32mRT];
#pragma unroll
    for (int r = 0; r < kF32mRT; ++r)
      scw[r] = __builtin_amdgcn_alignbyte(raw[r].sc[1], raw[r].sc[0], raw[r].shift);
    f32x4m D[kF32mRT];
#pragma unroll
    for (int r = 0; r < kF32mRT; ++r) D[r] = zero;
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {  // 16 weights per int8 scale
      float xv[16];
      f32m_x16(xs, grp, xv);
      float scf[kF32mRT], nscf[kF32mRT];
#pragma unroll
      for (int r = 0; r < kF32mRT; ++r) {
        // the signed byte goes through a full register before its conversion: folded into one
        // SDWA conversion, the extract came out as an unsigned conversion of the sign-extended
        // byte (negative scales turned into values near 2^32)
        scf[r] = (float)(int)opaque((uint32_t)__builtin_amdgcn_sbfe(scw[r], 8 * grp, 8));
        nscf[r] = -32.f * scf[r];
      }
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int s0 = 16 * grp + 4 * e4, l = s0 & 31, hi = s0 >> 5;
        const int qb = l + 32 * hi;  // low-bit byte within the half's 64
        uint32_t q4[kF32mRT];
#pragma unroll
        for (int r = 0; r < kF32mRT; ++r) {
          const uint32_t qlw = __builtin_amdgcn_alignbyte(raw[r].ql[(qb >> 2) + 1],
                                                          raw[r].ql[qb >> 2], raw[r].shift);
          const uint32_t qhw = __builtin_amdgcn_alignbyte(raw[r].qh[(l >> 2) + 1],
                                                          raw[r].qh[l >> 2], raw[r].shift);
          const uint32_t lo = (qlw >> sh) & 0x0F0F0F0Fu;
          const uint32_t h2 = (qhw >> (sh + 2 * hi)) & 0x03030303u;
          q4[r] = opaque(lo | (h2 << 4));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
          for (int r = 0; r < kF32mRT; ++r) {
            const float v = __builtin_fmaf(byte_to_float(q4[r], e), scf[r], nscf[r]);
            D[r] = f32m_mfma<T4>(xv[4 * e4 + e], v, D[r]);
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kF32mRT; ++r) {
      const float d = half_bits_to_float(raw[r].dbits);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[r][i] = __builtin_fmaf(d, D[r][i], acc[r][i]);
    }
  }
}

// Lane's four outputs of a 16-row tile whose first row is rb: tokens 4 g + i of row rb + t.
__device__ __forceinline__ void f32m_store(const KlMap &m, int B, int rb, int t, int g,
                                           const f32x4m &v) {
  const int row = rb + t;
  if (m.swiglu) {  // (gate, up) row pairs on neighbouring lanes
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float u = __shfl_down(v[i], 1);
      const int tok = 4 * g + i;
      if ((t & 1) == 0 && row + 1 < m.total && tok < B)
        m.y[0][(int64_t)tok * (m.total >> 1) + (row >> 1)] = silu_mul(v[i], u);
    }
    return;
  }
  if (row >= m.total) return;
  int p = 0;
#pragma unroll
  for (int k = 1; k < 4; ++k) p += (k < m.nparts && row >= m.cum[k]) ? 1 : 0;
  const int np = m.cum[p + 1] - m.cum[p];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tok = 4 * g + i;
    if (tok < B) m.y[p][(int64_t)tok * np + (row - m.cum[p])] = v[i];
  }
}

constexpr int kF32mXRow = 260;  // LDS floats per token row of a block (+4: rows on distinct banks)

template <int FMT, bool T4>
__device__ __forceinline__ void f32m_body(const KlMap &m, const float *__restrict__ x, int B,
                                          int kblocks, int ksplit, int upk,
                                          float *__restrict__ partial, const Arrivals &arr,
                                          float (*xsh)[16 * kF32mXRow], int *is_last_p) {
  int &is_last = *is_last_p;
  constexpr int RT = kF32mRT;
  const int lane = threadIdx.x & 63, w = wave_index();
  const int t = lane & 15, g = lane >> 4;
  // blockIdx -> (row group, slice): XCD x takes the row groups g = x (mod 8) and runs all slices
  // of one group back to back (the cache lines two neighbouring slices of a row share are then
  // fetched once, into that XCD's L2)
  const int xcd = blockIdx.x & 7, bi = blockIdx.x >> 3;
  const int grp = xcd + 8 * (bi / ksplit), ks = bi % ksplit;
  if (grp * (64 * RT) >= m.total) return;  // the whole workgroup: no barrier has been passed
  const int kb0 = ks * upk, nb = min(upk, kblocks - kb0);
  const int rbase = grp * (64 * RT) + w * (16 * RT);
  const uint8_t *wrow[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) wrow[r] = m.row(min(rbase + 16 * r + t, m.total - 1));

  // token rows of a block: 16 (T4: 4) rows x 64 float4, four (one) per thread (rows past the
  // batch repeat the last token; their outputs are never stored)
  const int64_t xld = (int64_t)kblocks * 64;  // float4 per token row
  constexpr int XJ = T4 ? 1 : 4;
  // (a native vector type: HIP's float4 struct kept this array in scratch memory, and every
  // fetch waited for its loads to store them there)
  f32x4m xn[XJ];
  auto fetch_x = [&](int kb) {
#pragma unroll
    for (int j = 0; j < XJ; ++j) {
      const int idx = (int)threadIdx.x + 256 * j, tok = idx >> 6, c4 = idx & 63;
      xn[j] = reinterpret_cast<const f32x4m *>(x)[(int64_t)min(tok, B - 1) * xld + kb * 64 + c4];
    }
  };
  auto put_x = [&](int b) {
#pragma unroll
    for (int j = 0; j < XJ; ++j) {
      const int idx = (int)threadIdx.x + 256 * j, tok = idx >> 6, c4 = idx & 63;
      *reinterpret_cast<f32x4m *>(&xsh[b][tok * kF32mXRow + 4 * c4]) = xn[j];
    }
  };

  f32x4m acc[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) acc[r] = (f32x4m){0.f, 0.f, 0.f, 0.f};
  F32mRaw<FMT> ra[RT], rb[RT];
  auto load = [&](F32mRaw<FMT>(&raw)[RT], int kb) {
#pragma unroll
    for (int r = 0; r < RT; ++r) raw[r].load(wrow[r], kb, g);
  };
  auto compute = [&](const F32mRaw<FMT>(&raw)[RT], int b) {
    f32m_block<FMT, T4>(raw, &xsh[b][(T4 ? (t & 3) : t) * kF32mXRow + 64 * g], g, acc);
  };
  // Weights one block ahead in two register sets used in turn; token rows one block ahead in
  // registers, then in the other LDS buffer. The barrier at the end of block i makes block i+1's
  // rows visible and frees block i's buffer for block i+2.
  load(ra, kb0);
  fetch_x(kb0);
  put_x(0);
  __syncthreads();
  for (int i = 0;;) {
    if (i + 1 < nb) {
      load(rb, kb0 + i + 1);
      fetch_x(kb0 + i + 1);
    }
    compute(ra, i & 1);
    if (i + 1 < nb) put_x((i + 1) & 1);
    __syncthreads();
    if (++i >= nb) break;
    if (i + 1 < nb) {
      load(ra, kb0 + i + 1);
      fetch_x(kb0 + i + 1);
    }
    compute(rb, i & 1);
    if (i + 1 < nb) put_x((i + 1) & 1);
    __syncthreads();
    if (++i >= nb) break;
  }

  if constexpr (T4) {
    // the four k quarters: (g0 + g1) + (g2 + g3), the same bits in every lane of a row; lanes with
    // g = 0 then hold tokens 0..3 of row t, and the others' labels (tokens 4 g + i) are never
    // stored (B <= 4)
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[r][i] += __shfl_xor(acc[r][i], 16);
        acc[r][i] += __shfl_xor(acc[r][i], 32);
      }
  }
  if (ksplit == 1) {
#pragma unroll
    for (int r = 0; r < RT; ++r) f32m_store(m, B, rbase + 16 * r, t, g, acc[r]);
    return;
  }
  // this slice's sums, then the last workgroup of the row group adds the slices in order
  const int tiles = 4 * RT;
  float *mine = partial + ((int64_t)grp * ksplit + ks) * tiles * 256;
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __hip_atomic_store(mine + (w * RT + r) * 256 + 4 * lane + i, acc[r][i], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the partial sums are stored before counting
  __syncthreads();
  if (threadIdx.x == 0) is_last = arrive_last(arr, grp, (unsigned)ksplit);
  __syncthreads();
  if (!is_last) return;
  const float *base = partial + (int64_t)grp * ksplit * tiles * 256;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    f32x4m s = {0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < ksplit; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s[i] += __hip_atomic_load(base + ((int64_t)q * tiles + w * RT + r) * 256 + 4 * lane + i,
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    f32m_store(m, B, rbase + 16 * r, t, g, s);
  }
  if (threadIdx.x == 0) done_arrivals(arr, grp);
}

// Q8_0 fits three waves per SIMD (the compiler then reaches four); Q6_K keeps two (at three its
// two register sets of raw runs spill).
template <bool T4>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_gemm_f32m_q8(
    KlMap m, const float *__restrict__ x, int B, int kblocks, int ksplit, int upk,
    float *__restrict__ partial, Arrivals arr) {
  __shared__ __attribute__((aligned(16))) float xsh[2][16 * kF32mXRow];
  __shared__ int is_last;
  f32m_body<FMT_Q8_0, T4>(m, x, B, kblocks, ksplit, upk, partial, arr, xsh, &is_last);
}

template <bool T4>
__global__ __launch_bounds__(256) void k_gemm_f32m_q6(KlMap m, const float *__restrict__ x, int B,
                                                      int kblocks, int ksplit, int upk,
                                                      float *__restrict__ partial,
                                                      Arrivals arr) {
  __shared__ __attribute__((aligned(16))) float xsh[2][16 * kF32mXRow];
  __shared__ int is_last;
  f32m_body<FMT_Q6_K, T4>(m, x, B, kblocks, ksplit, upk, partial, arr, xsh, &is_last);
}

// ---- host side ----------------------------------------------------------------------------------

// Q8_0 at 2..16 tokens, Q6_K (dword-aligned rows: k a multiple of 512) at 2..16 tokens (4..16
// without the 4-token form), k up to 65536. On the 70B-shaped gate and down matrices Q6_K at 2 / 3
// / 4 tokens takes 207 / 198 / 206 and 91 / 88 / 89 us on the 4-token form against 202 / 266 / 345
// and 101 / 136 / 175 us on the fp32 vector GEMV (and 258-261 / 115-120 us padded to 16 tokens).
// TQ_KNOB_GEMM_F32M = 0 turns the path off, =2 takes every batch of 2..16 (tests).
bool f32m_ok(int fmt, int64_t k, int64_t batch) {
  const int mode = knob(TQ_KNOB_GEMM_F32M, 1);
  if (mode == 0) return false;
  if (batch < 2 || batch > 16 || k <= 0 || k > 65536) return false;
  const bool t4 = batch <= 4 && knob(TQ_KNOB_F32M_T4, 1) != 0;
  if (fmt == FMT_Q6_K) return k % 512 == 0 && (batch >= 4 || t4 || mode == 2);
  return fmt == FMT_Q8_0 && k % 256 == 0;
}

// Blocks per k slice, from k alone: at least TQ_KNOB_F32M_UPK (8), at most 8 slices.
static int f32m_upk(int64_t k) {
  const int nblk = (int)(k / 256);
  const int least = (nblk + kF32mMaxSlices - 1) / kF32mMaxSlices;
  const int v = knob(TQ_KNOB_F32M_UPK, 8);
  return clampi(v > least ? v : least, 1, nblk);
}

static int64_t f32m_groups(int64_t rows) { return (rows + 64 * kF32mRT - 1) / (64 * kF32mRT); }

size_t f32m_workspace_bytes(int64_t rows, int64_t k) {
  const int nblk = (int)(k / 256), upk = f32m_upk(k), ksplit = (nblk + upk - 1) / upk;
  if (ksplit == 1) return 0;
  return (size_t)align256(f32m_groups(rows) * ksplit * 4 * kF32mRT * 256 * 4);
}

int launch_gemm_f32m(int fmt, const KlMap &m, int64_t k, const float *x, int64_t batch,
                     float *partial, unsigned long long *counters, int max_counters,
                     hipStream_t s) {
  const int nblk = (int)(k / 256), upk = f32m_upk(k), ksplit = (nblk + upk - 1) / upk;
  if (ksplit > kF32mMaxSlices) return -2;
  const int64_t groups = f32m_groups(m.total);
  if (ksplit > 1 && groups > max_counters) return -2;
  const dim3 grid((unsigned)((groups + 7) / 8 * 8 * ksplit));
  const Arrivals arr{counters, ksplit > 1 ? call_tag() : 0ull};
  const bool t4 = batch <= 4 && knob(TQ_KNOB_F32M_T4, 1) != 0;
  if (fmt == FMT_Q6_K && t4)
    hipLaunchKernelGGL(k_gemm_f32m_q6<true>, grid, dim3(256), 0, s, m, x, (int)batch, nblk, ksplit,
                       upk, partial, arr);
  else if (fmt == FMT_Q6_K)
    hipLaunchKernelGGL(k_gemm_f32m_q6<false>, grid, dim3(256), 0, s, m, x, (int)batch, nblk,
                       ksplit, upk, partial, arr);
  else if (t4)
    hipLaunchKernelGGL(k_gemm_f32m_q8<true>, grid, dim3(256), 0, s, m, x, (int)batch, nblk, ksplit,
                       upk, partial, arr);
  else
    hipLaunchKernelGGL(k_gemm_f32m_q8<false>, grid, dim3(256), 0, s, m, x, (int)batch, nblk,
                       ksplit, upk, partial, arr);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace tq
