// tq_qmm.hip -- grouped Q4_K expert products for a few tokens per expert on the fp16 matrix cores,
// accurate to fp32 rounding.
//
// Per 256-weight block of a row (scale d, min dmin, sub-block scales sc_j and mins m_j, quants q)
// the product with a token row x is
//     d * sum_k sc_j(k) q_k x_k  -  dmin * sum_j m_j S_j,     S_j = sum of x over sub-block j.
// Every factor enters the matrix cores exactly:
//   * sc_j q_k <= 63 * 15 = 945 and m_j <= 63 are integers below 1024, so their 16-bit patterns
//     are the fp16 subnormals n * 2^-24 (gfx950's fp16 matrix cores keep subnormal inputs);
//   * each token row is scaled by a power of two 2^e that brings its largest magnitude into
//     [2^14, 2^15) and split as hi = fp16(x'), lo = fp16(x' - hi), so x' = hi + lo to within about
//     2^-22 relative; S_j is kept the same way (scaled by a further 2^-6 to stay in range);
//   * the matrix cores form fp16 products exactly and accumulate in fp32.
// So each output is a sum of exact products rounded in fp32, as with the fp32 GEMV: the two
// accumulate in different orders, which is the whole of their difference.
//
// Kernels:
//   k_split_rows     token rows (gate/up) or h rows (down) -> scaled fp16 hi/lo + sub-block sums
//   k_qmm<true>      per (chunk of <= 16 NT positions, 64 ffn columns): gate and up products,
//                    h = silu(gate) * up, fp32 [position][ffn]
//   k_qmm<false>     per (chunk, 128 hidden rows): down product, o fp32 [position][hidden]
//
// Matrix-core layout (v_mfma_f32_16x16x32_f16). A = 16 token rows x 32 k from LDS, B = 32 k x 16
// weight rows built in registers; lane l holds weight row l % 16 and k group g = l / 16, and
// receives D[token 4 g + i][row l % 16]. Lane group g owns quant bytes 32 g .. 32 g + 31 of every
// block (sub-blocks 2g: low nibbles, 2g+1: high nibbles), so k step s (0..7) of a block covers
// k = 64 g + 8 s + 0..7 for g = 0..3 -- four sub-blocks at once, which is why the sub-block scale
// goes into the weight operand rather than into a per-sub-block rescale of the accumulator.
// Within each run of 8 k the operand holds bytes 0,2,1,3,4,6,5,7 (pairs come out of a dword that
// way); the split rows are stored in the same order. The min term is one more product per block,
// v_mfma_f32_16x16x16_f16 of S (hi, lo) against m.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "tq_device.h"
#include "tq_gemv_core.h"
#include "tq_launch.h"
#include "tq_mfma.h"
#include "tq_moe.h"
#include "tq_prefill.h"
#include "tq_qmm.h"

namespace tq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

constexpr int kXBlockBytes = 1024;  // one row's split block: 256 hi halves, then 256 lo halves
constexpr int kAuxBytes = 32;       // one row's sub-block sums of a block: 8 hi, 8 lo halves

// Position i of a run of 8 holds value perm8(i) (an involution: 1 <-> 2, 5 <-> 6).
__device__ __forceinline__ constexpr int perm8(int i) {
  return (i == 1 || i == 5) ? i + 1 : (i == 2 || i == 6) ? i - 1 : i;
}

// ---- split rows ---------------------------------------------------------------------------------
// One workgroup per row: the row's largest magnitude, then per run of 8 values (a thread each)
// the scaled hi/lo halves and, over four neighbouring threads, the sub-block sums.
__global__ __launch_bounds__(256) void k_split_rows(const float *__restrict__ src, int64_t ld, int K,
                                                    uint8_t *__restrict__ xs,
                                                    uint8_t *__restrict__ aux,
                                                    float *__restrict__ unscale) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const float *x = src + row * ld;
  const float4 *x4 = reinterpret_cast<const float4 *>(x);
  float m = 0.f;
  for (int i = threadIdx.x; i < K / 4; i += 256) {
    const float4 v = x4[i];
    m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  int e = 0;
  if (m > 0.f) {
    int ex;
    frexpf(m, &ex);  // m in [2^(ex-1), 2^ex)
    e = 15 - ex;
    if (e > 126) e = 126;
  }
  const float s = ldexpf(1.f, e);
  if (threadIdx.x == 0) unscale[row] = ldexpf(1.f, -e);

  const int kblocks = K / 256;
  uint8_t *xrow = xs + row * (int64_t)kblocks * kXBlockBytes;
  uint8_t *arow = aux + row * (int64_t)kblocks * kAuxBytes;
  for (int gi = threadIdx.x; gi < K / 8; gi += 256) {  // K / 8 is a multiple of 32
    const float4 a = x4[2 * gi], b = x4[2 * gi + 1];
    const float v[8] = {a.x * s, a.y * s, a.z * s, a.w * s, b.x * s, b.y * s, b.z * s, b.w * s};
    _Float16 hi[8], lo[8];
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      hi[i] = (_Float16)v[i];
      lo[i] = (_Float16)(v[i] - (float)hi[i]);
      sum += (float)hi[i] + (float)lo[i];
    }
    half8 h8, l8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      h8[i] = hi[perm8(i)];
      l8[i] = lo[perm8(i)];
    }
    const int kb = gi >> 5, p = gi & 31;
    uint8_t *dst = xrow + (int64_t)kb * kXBlockBytes + 16 * p;
    *reinterpret_cast<half8 *>(dst) = h8;
    *reinterpret_cast<half8 *>(dst + 512) = l8;
    // sub-block j = runs 4j .. 4j+3 of the block: four neighbouring threads, all active together
    sum += __shfl_xor(sum, 1);
    sum += __shfl_xor(sum, 2);
    if ((gi & 3) == 0) {
      const int j = (gi >> 2) & 7;
      const float s6 = sum * 0x1p-6f;
      const _Float16 sh = (_Float16)s6, sl = (_Float16)(s6 - (float)sh);
      _Float16 *ap = reinterpret_cast<_Float16 *>(arow + (int64_t)kb * kAuxBytes);
      ap[perm8(j)] = sh;
      ap[8 + perm8(j)] = sl;
    }
  }
}

// ---- the grouped product ------------------------------------------------------------------------

typedef const u32x2 __attribute__((address_space(1))) *gu32x2;
__device__ __forceinline__ u32x2 gload8(const void *p) { return *(gu32x2)p; }

// One block of the lane's weight row: header (d, dmin, 12 scale bytes) and the lane group's
// 32 quant bytes.
struct QRow {
  u32x4 head, q0, q1;
};

__device__ __forceinline__ void qrow_load(const uint8_t *row, int kb, int g, QRow &r) {
  const uint8_t *b = row + (int64_t)kb * 144;
  r.head = gload(b);
  r.q0 = gload(b + 16 + 32 * g);
  r.q1 = gload(b + 32 + 32 * g);
}

// The lane's per-block factors: d and -dmin with the operand units folded in, sc of sub-blocks
// 2g and 2g+1 (each in both halves of a dword), and the min operand: m of sub-blocks
// 4 (g & 1) + 0, 2, 1, 3 as fp16 subnormals.
struct QScale {
  float d, ndmin;
  uint32_t sc_lo, sc_hi;
  half4 m;
};

__device__ __forceinline__ QScale qscale(const QRow &r, int g) {
  const uint32_t h0 = r.head.x, s0 = r.head.y, s1 = r.head.z, s2 = r.head.w;
  QScale q;
  q.d = half_bits_to_float(h0) * 0x1p24f;              // sc q enters as n * 2^-24
  q.ndmin = -half_bits_to_float(h0 >> 16) * 0x1p30f;   // m as n * 2^-24, sums as S * 2^-6
  auto sc_of = [&](int j) {
    const Q4kField f = q4k_field(j);
    return bfe(f.from_s2 ? s2 : s0, f.lo_off, f.lo_w) | (bfe(s0, f.hi_off, f.hi_w) << 4);
  };
  const uint32_t a = sc_of(2 * g), b = sc_of(2 * g + 1);
  q.sc_lo = a | (a << 16);
  q.sc_hi = b | (b << 16);
  // mins of sub-blocks 0..3: low 6 bits of bytes 4..7; of 4..7: high nibbles of bytes 8..11 with
  // the top two bits of bytes 4..7 above them
  const uint32_t mb =
      (g & 1) ? (((s2 >> 4) & 0x0F0F0F0Fu) | ((s1 >> 2) & 0x30303030u)) : (s1 & 0x3F3F3F3Fu);
  const u32x2 mp = {mb & 0x00FF00FFu, (mb >> 8) & 0x00FF00FFu};
  q.m = __builtin_bit_cast(half4, mp);
  return q;
}

// Weight operand of k step S: sc * q of bytes 8 (S % 4) .. + 7 of the lane's 32 (low nibbles for
// S < 4, high nibbles after), as fp16 subnormals in the order 0,2,1,3,4,6,5,7.
template <int S>
__device__ __forceinline__ half8 qb(const QRow &r, uint32_t sc2) {
  const u32x4 &q = (S & 3) < 2 ? r.q0 : r.q1;
  uint32_t w0 = dword_of(q, (2 * S) & 3), w1 = dword_of(q, (2 * S + 1) & 3);
  if (S >= 4) {
    w0 >>= 4;
    w1 >>= 4;
  }
  const uint32_t mk = 0x000F000Fu;
  const uint32_t p[4] = {w0 & mk, (w0 >> 8) & mk, w1 & mk, (w1 >> 8) & mk};
  const u16x2 sc = __builtin_bit_cast(u16x2, sc2);
  u32x4 v;
  v.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, p[0]) * sc);
  v.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, p[1]) * sc);
  v.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, p[2]) * sc);
  v.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, p[3]) * sc);
  return __builtin_bit_cast(half8, v);
}

// Token staging: a block of one token row (1 KB of hi/lo halves) is one direct global-to-LDS
// wave instruction, lane l bringing the row's 16-byte piece l ^ (t % 16) to LDS piece l, so that
// the 16 token rows of an operand read (same piece, t = 0..15) fall on distinct banks. Wave w's
// instruction i fills token row 4 i + w. Rows past the chunk repeat its last row; they feed only
// outputs that are never stored.
template <bool GU, int NT, int NTMAX>
__device__ __forceinline__ void qmm_tiles(const QmmArgs &a, uint8_t *__restrict__ xbuf,
                                          const int *rowidx, int rows, int p0,
                                          const uint8_t *const (&wrow)[2], int col0) {
  constexpr int kBuf = 16 * NTMAX * kXBlockBytes;
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int t16 = lane & 15, g = lane >> 4;
  const int64_t xrow_bytes = (int64_t)a.kblocks * kXBlockBytes;
  const int64_t arow_bytes = (int64_t)a.kblocks * kAuxBytes;
  const uint8_t *xsrc[4 * NT];
#pragma unroll
  for (int i = 0; i < 4 * NT; ++i) {
    const int t = 4 * i + wave;
    xsrc[i] = a.x.xs + rowidx[min(t, rows - 1)] * xrow_bytes + 16 * (lane ^ (t & 15));
  }
  const uint8_t *asrc[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
    asrc[tt] = a.x.aux + rowidx[min(16 * tt + t16, rows - 1)] * arow_bytes + 8 * g;

  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_address(xbuf));
  // enqueue block kb of the chunk's token rows into buffer buf (asm loads, awaited explicitly)
  auto stage = [&](int buf, int kb) {
#pragma unroll
    for (int i = 0; i < 4 * NT; ++i)
      load_lds16(xsrc[i] + (int64_t)kb * kXBlockBytes,
                 lds0 + buf * kBuf + (4 * i + wave) * kXBlockBytes);
  };
  auto load_w = [&](QRow (&r)[2], u32x2 (&ax)[NT], int kb) {
    qrow_load(wrow[0], kb, g, r[0]);
    qrow_load(wrow[1], kb, g, r[1]);
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) ax[tt] = gload8(asrc[tt] + (int64_t)kb * kAuxBytes);
  };

  f32x4 acc[2][NT];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[r][tt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  const int steps = a.kblocks;
  // weights and sums run two blocks ahead (set j holds the blocks st with st % 3 == j), token
  // rows one block ahead (buffer st % 2)
  QRow raw[3][2];
  u32x2 axr[3][NT];
  stage(0, 0);
  load_w(raw[0], axr[0], 0);
  load_w(raw[1], axr[1], min(1, steps - 1));
  const uint8_t *rd = xbuf + t16 * kXBlockBytes;

  auto step = [&](int st, const QRow (&rc)[2], const u32x2 (&ac)[NT], QRow (&rf)[2],
                  u32x2 (&af)[NT]) {
    // Outstanding, oldest first: weights and sums of st+1, then (from the previous step) the
    // token rows of st... precisely: [W(st) A(st)] [X(st)] [W(st+1) A(st+1)]; every step issues
    // the same loads (past the end they repeat the last block into registers and a buffer nobody
    // reads), so leaving the 6 + NT newest in flight is exact on every path. After the barrier
    // every wave's rows of block st are in LDS and every wave is done reading block st-1's buffer.
    barrier_after_vmem<6 + NT>();
    const uint8_t *buf = rd + (st & 1) * kBuf;
    auto read_a = [&](int tt, int s, half8 &h, half8 &l) {
      const uint8_t *p = buf + tt * 16 * kXBlockBytes + 16 * ((8 * g + s) ^ t16);
      h = *reinterpret_cast<const half8 *>(p);
      l = *reinterpret_cast<const half8 *>(p + 512);
    };
    half8 ah[NT], al[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) read_a(tt, 0, ah[tt], al[tt]);
    __builtin_amdgcn_sched_barrier(0);
    stage((st + 1) & 1, min(st + 1, steps - 1));
    load_w(rf, af, min(st + 2, steps - 1));
    __builtin_amdgcn_sched_barrier(0);

    const QScale qs[2] = {qscale(rc[0], g), qscale(rc[1], g)};
    f32x4 dq[2][NT], dm[2][NT];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
        dm[r][tt] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4, ac[tt]),
                                                          qs[r].m, zero, 0, 0, 0);
    half8 b0 = qb<0>(rc[0], qs[0].sc_lo), b1 = qb<0>(rc[1], qs[1].sc_lo);
    auto kstep = [&](auto S_) {
      constexpr int S = decltype(S_)::value;
      half8 nh[NT], nl[NT], n0, n1;
      if constexpr (S < 7) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) read_a(tt, S + 1, nh[tt], nl[tt]);
        n0 = qb<S + 1>(rc[0], S + 1 < 4 ? qs[0].sc_lo : qs[0].sc_hi);
        n1 = qb<S + 1>(rc[1], S + 1 < 4 ? qs[1].sc_lo : qs[1].sc_hi);
      }
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        dq[0][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[tt], b0, S == 0 ? zero : dq[0][tt],
                                                           0, 0, 0);
        dq[1][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[tt], b1, S == 0 ? zero : dq[1][tt],
                                                           0, 0, 0);
        dq[0][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[tt], b0, dq[0][tt], 0, 0, 0);
        dq[1][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[tt], b1, dq[1][tt], 0, 0, 0);
      }
      if constexpr (S < 7) {
        b0 = n0;
        b1 = n1;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          ah[tt] = nh[tt];
          al[tt] = nl[tt];
        }
      }
    };
    kstep(std::integral_constant<int, 0>{});
    kstep(std::integral_constant<int, 1>{});
    kstep(std::integral_constant<int, 2>{});
    kstep(std::integral_constant<int, 3>{});
    kstep(std::integral_constant<int, 4>{});
    kstep(std::integral_constant<int, 5>{});
    kstep(std::integral_constant<int, 6>{});
    kstep(std::integral_constant<int, 7>{});
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[r][tt][i] = __builtin_fmaf(qs[r].d, dq[r][tt][i],
                                         __builtin_fmaf(qs[r].ndmin, dm[r][tt][i], acc[r][tt][i]));
  };
  int st = 0;
  for (; st + 3 <= steps; st += 3) {
    step(st, raw[0], axr[0], raw[2], axr[2]);
    step(st + 1, raw[1], axr[1], raw[0], axr[0]);
    step(st + 2, raw[2], axr[2], raw[1], axr[1]);
  }
  if (st < steps) step(st, raw[0], axr[0], raw[2], axr[2]);
  if (st + 1 < steps) step(st + 1, raw[1], axr[1], raw[0], axr[0]);
#pragma unroll
  for (int j = 0; j < 3; ++j) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      keep_alive(raw[j][r].head);
      keep_alive(raw[j][r].q0);
      keep_alive(raw[j][r].q1);
    }
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) keep_alive(axr[j][tt]);
  }
  wait_vmem<0>();  // the surplus loads of the last steps land before the workgroup ends

  // lane: tokens 16 tt + 4 g + i, weight row t16 of each tile
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 16 * tt + 4 * g + i;
      if (tok < rows) {
        const float us = a.x.unscale[rowidx[tok]];
        float *o = a.out + (int64_t)(p0 + tok) * a.ldo + col0 + t16;
        if (GU) {
          o[0] = silu_mul(acc[0][tt][i] * us, acc[1][tt][i] * us);
        } else {
          o[0] = acc[0][tt][i] * us;
          o[16] = acc[1][tt][i] * us;
        }
      }
    }
}

template <bool GU, int NTMAX>
__global__ __launch_bounds__(256) void k_qmm(QmmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t xbuf[2 * 16 * NTMAX * kXBlockBytes];
  __shared__ int rowidx[16 * NTMAX];

  // blockIdx -> (chunk, tile) as in the prefill kernels: XCD x takes the chunks c = x (mod 8)
  // and runs all tiles of one chunk back to back, sharing the chunk's token rows in its L2
  const int b = blockIdx.x, xcd = b & 7, i = b >> 3;
  const int chunk = xcd + 8 * (i / a.ntiles), tile = i % a.ntiles;
  if (chunk >= *a.n_chunks) return;
  const int slot = a.chunks[3 * chunk], p0 = a.chunks[3 * chunk + 1], rows = a.chunks[3 * chunk + 2];
  const int e = a.act[slot];
  const uint8_t *mat[3];
  if (e == a.E) {
#pragma unroll
    for (int m = 0; m < 3; ++m) mat[m] = (const uint8_t *)a.shared.m[m];
  } else if (a.staging != nullptr) {
#pragma unroll
    for (int m = 0; m < 3; ++m) mat[m] = a.staging + (int64_t)slot * a.stage_stride + a.stage_off[m];
  } else {
#pragma unroll
    for (int m = 0; m < 3; ++m) mat[m] = (const uint8_t *)a.experts[e].m[m];
  }
  for (int t = threadIdx.x; t < rows; t += 256) {
    const int p = p0 + t;
    int r = p;
    if (a.x_by_token) r = p >= a.Tk ? p - a.Tk : a.pairs[p] / a.topk;
    rowidx[t] = r;
  }
  const int t16 = threadIdx.x & 15, wave = wave_index();
  const uint8_t *wrow[2];
  int col0;  // GU: the wave's first ffn column; down: its first hidden row
  if (GU) {
    col0 = tile * 64 + wave * 16;
    wrow[0] = mat[0] + (int64_t)(col0 + t16) * a.row_bytes;
    wrow[1] = mat[1] + (int64_t)(col0 + t16) * a.row_bytes;
  } else {
    col0 = tile * 128 + wave * 32;
    wrow[0] = mat[2] + (int64_t)(col0 + t16) * a.row_bytes;
    wrow[1] = mat[2] + (int64_t)(col0 + 16 + t16) * a.row_bytes;
  }
  __syncthreads();  // rowidx
  if (NTMAX == 1 || rows <= 16)
    qmm_tiles<GU, 1, NTMAX>(a, xbuf, rowidx, rows, p0, wrow, col0);
  else
    qmm_tiles<GU, (NTMAX > 1 ? 2 : 1), NTMAX>(a, xbuf, rowidx, rows, p0, wrow, col0);
}

// ---- host side ----------------------------------------------------------------------------------

int qmm_chunk_rows(int nt_max) { return 16 * nt_max; }

bool qmm_shape_ok(int64_t hidden, int64_t ffn) {
  return hidden % 256 == 0 && ffn % 256 == 0 && hidden >= 256 && ffn >= 256;
}

size_t split_rows_bytes(int64_t rows, int64_t k) {
  return align256(rows * k * 4) + align256(rows * (k / 8)) + align256(rows * 4);
}

SplitRows split_rows_at(char *base, int64_t rows, int64_t k) {
  SplitRows s;
  s.xs = (uint8_t *)base;
  s.aux = (uint8_t *)(base + align256(rows * k * 4));
  s.unscale = (float *)(base + align256(rows * k * 4) + align256(rows * (k / 8)));
  return s;
}

void launch_split_rows(const float *src, int64_t ld, int64_t rows, int64_t k, SplitRows out,
                       hipStream_t st) {
  if (rows <= 0) return;
  hipLaunchKernelGGL(k_split_rows, dim3((unsigned)rows), dim3(256), 0, st, src, ld, (int)k, out.xs,
                     out.aux, out.unscale);
}

template <int NTMAX>
static void qmm_launch(const QmmArgs &a, int max_chunks, bool gu, hipStream_t st) {
  const int groups = (max_chunks + 7) / 8;
  const dim3 grid((unsigned)(8 * groups * a.ntiles));
  if (gu)
    hipLaunchKernelGGL((k_qmm<true, NTMAX>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_qmm<false, NTMAX>), grid, dim3(256), 0, st, a);
}

int launch_qmm_moe(QmmArgs a, int nt_max, int max_chunks, const float *x, int64_t tokens,
                   int64_t positions, int64_t hidden, int64_t ffn, char *xsplit, char *hsplit,
                   float *h, float *o, hipStream_t st) {
  const SplitRows xr = split_rows_at(xsplit, tokens, hidden);
  const SplitRows hr = split_rows_at(hsplit, positions, ffn);
  launch_split_rows(x, hidden, tokens, hidden, xr, st);
  launch_chunk_table(a.act, a.n_active, a.act_stride, qmm_chunk_rows(nt_max), max_chunks,
                     (int *)a.chunks, (int *)a.n_chunks, st);
  // gate / up
  a.kblocks = (int)(hidden / 256);
  a.row_bytes = hidden / 256 * 144;
  a.x = xr;
  a.x_by_token = 1;
  a.out = h;
  a.ldo = ffn;
  a.ntiles = (int)(ffn / 64);
  if (nt_max == 1) qmm_launch<1>(a, max_chunks, true, st);
  else qmm_launch<2>(a, max_chunks, true, st);
  // down
  launch_split_rows(h, ffn, positions, ffn, hr, st);
  a.kblocks = (int)(ffn / 256);
  a.row_bytes = ffn / 256 * 144;
  a.x = hr;
  a.x_by_token = 0;
  a.out = o;
  a.ldo = hidden;
  a.ntiles = (int)(hidden / 128);
  if (nt_max == 1) qmm_launch<1>(a, max_chunks, false, st);
  else qmm_launch<2>(a, max_chunks, false, st);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace tq
