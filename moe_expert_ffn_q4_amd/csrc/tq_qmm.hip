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
//   k_qmm_dense      dense products of 2..32 tokens on split rows (k slices, the last workgroup
//                    of a row tile adds them)
//   k_qmm_dense2     dense products of 2..16 tokens, the activations split inside the kernel
//                    with one power of two per (token, block)
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
constexpr int kMaxSlices = 8;       // k slices of the dense products

// Position i of a run of 8 holds value perm8(i) (an involution: 1 <-> 2, 5 <-> 6).
__device__ __forceinline__ constexpr int perm8(int i) {
  return (i == 1 || i == 5) ? i + 1 : (i == 2 || i == 6) ? i - 1 : i;
}

// ---- split rows ---------------------------------------------------------------------------------
// One workgroup per row, each thread holding its runs of 8 values in registers (the row is read
// once): the row's largest magnitude, then per run the scaled hi/lo halves and, over four
// neighbouring threads, the sub-block sums. RUNS = runs of 8 per thread (K <= 2048 RUNS).
template <int RUNS>
__global__ __launch_bounds__(256) void k_split_rows(const float *__restrict__ src, int64_t ld, int K,
                                                    uint8_t *__restrict__ xs,
                                                    uint8_t *__restrict__ aux,
                                                    float *__restrict__ unscale) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const float4 *x4 = reinterpret_cast<const float4 *>(src + row * ld);
  const int runs = K / 8;  // a multiple of 32
  float4 v[RUNS][2];
  float m = 0.f;
#pragma unroll
  for (int r = 0; r < RUNS; ++r) {
    const int gi = threadIdx.x + 256 * r;
    if (gi < runs) {
      v[r][0] = x4[2 * gi];
      v[r][1] = x4[2 * gi + 1];
    } else {
      v[r][0] = v[r][1] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v[r][h].x), fabsf(v[r][h].y)),
                         fmaxf(fabsf(v[r][h].z), fabsf(v[r][h].w))));
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
#pragma unroll
  for (int r = 0; r < RUNS; ++r) {
    const int gi = threadIdx.x + 256 * r;
    if (gi >= runs) break;  // whole groups of 32 runs stay active together
    const float vv[8] = {v[r][0].x * s, v[r][0].y * s, v[r][0].z * s, v[r][0].w * s,
                         v[r][1].x * s, v[r][1].y * s, v[r][1].z * s, v[r][1].w * s};
    _Float16 hi[8], lo[8];
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      hi[i] = (_Float16)vv[i];
      lo[i] = (_Float16)(vv[i] - (float)hi[i]);
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
  static constexpr int kLoads = 3;  // qrow_load issues one 16-byte load per field
};
static_assert(sizeof(QRow) == QRow::kLoads * sizeof(u32x4), "one load per field of QRow");

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
// instruction i fills token row 4 i + w. Rows past the chunk are not loaded: whatever their LDS
// rows hold reaches only their own accumulator rows, which are never stored (the vmcnt waits
// count only the newer weight loads, so a varying number of these loads is fine).
// Blocks kb0 .. kb0 + steps - 1 of the lane's two weight rows (wrow: the rows' first block)
// against token rows rowidx[0 .. rows-1] of the split activations; epi(acc) receives the
// accumulators (lane: tokens 16 tt + 4 g + i, weight row t16 of tiles 0 and 1), in units of the
// scaled activations.
template <bool GU, int NT, int NTMAX, class Epi>
__device__ __forceinline__ void qmm_tiles(const SplitRows &x, uint8_t *__restrict__ xbuf,
                                          const int *rowidx, int rows, int xblocks,
                                          const uint8_t *const (&wrow)[2], int kb0, int steps,
                                          const Epi &epi) {
  constexpr int kBuf = 16 * NTMAX * kXBlockBytes;
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int t16 = lane & 15, g = lane >> 4;
  const int64_t xrow_bytes = (int64_t)xblocks * kXBlockBytes;
  const int64_t arow_bytes = (int64_t)xblocks * kAuxBytes;
  const uint8_t *xsrc[4 * NT];
#pragma unroll
  for (int i = 0; i < 4 * NT; ++i) {
    const int t = 4 * i + wave;
    xsrc[i] = x.xs + rowidx[min(t, rows - 1)] * xrow_bytes + (int64_t)kb0 * kXBlockBytes +
              16 * (lane ^ (t & 15));
  }
  const uint8_t *asrc[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
    asrc[tt] = x.aux + rowidx[min(16 * tt + t16, rows - 1)] * arow_bytes +
               (int64_t)kb0 * kAuxBytes + 8 * g;

  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_address(xbuf));
  // enqueue block kb of the chunk's token rows into buffer buf (asm loads, awaited explicitly)
  auto stage = [&](int buf, int kb) {
#pragma unroll
    for (int i = 0; i < 4 * NT; ++i)
      if (4 * i + wave < rows)  // rows past the chunk: their outputs are never stored
        load_lds16(xsrc[i] + (int64_t)kb * kXBlockBytes,
                   lds0 + buf * kBuf + (4 * i + wave) * kXBlockBytes);
  };
  // the vector-memory loads one load_w issues: two weight rows, then one 8-byte load of the
  // sums per token tile; the barrier of each step leaves exactly these (of the next block) in
  // flight, so the count below must follow the loop bounds here
  constexpr int kRows = 2;
  constexpr int kWLoads = kRows * QRow::kLoads + NT;
  auto load_w = [&](QRow (&r)[kRows], u32x2 (&ax)[NT], int kb) {
#pragma unroll
    for (int q = 0; q < kRows; ++q) qrow_load(wrow[q], kb, g, r[q]);
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) ax[tt] = gload8(asrc[tt] + (int64_t)kb * kAuxBytes);
  };

  f32x4 acc[2][NT];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[r][tt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

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
    static_assert(kWLoads == 6 + NT, "two rows of three loads plus one per token tile");
    barrier_after_vmem<kWLoads>();
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
  epi(acc);
}

// Grouped (MoE) epilogue: unscaled sums of the chunk's positions, SwiGLU'd for gate/up.
template <bool GU>
struct MoeEpi {
  const QmmArgs *a;
  const int *rowidx;
  int rows, p0, col0;
  template <int NT>
  __device__ __forceinline__ void operator()(const f32x4 (&acc)[2][NT]) const {
    const int lane = threadIdx.x & 63, t16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 16 * tt + 4 * g + i;
        if (tok < rows) {
          const float us = a->x.unscale[rowidx[tok]];
          float *o = a->out + (int64_t)(p0 + tok) * a->ldo + col0 + t16;
          if (GU) {
            o[0] = silu_mul(acc[0][tt][i] * us, acc[1][tt][i] * us);
          } else {
            o[0] = acc[0][tt][i] * us;
            o[16] = acc[1][tt][i] * us;
          }
        }
      }
  }
};

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
  const MoeEpi<GU> epi{&a, rowidx, rows, p0, col0};
  if (NTMAX == 1 || rows <= 16)
    qmm_tiles<GU, 1, NTMAX>(a.x, xbuf, rowidx, rows, a.kblocks, wrow, 0, a.kblocks, epi);
  else
    qmm_tiles<GU, (NTMAX > 1 ? 2 : 1), NTMAX>(a.x, xbuf, rowidx, rows, a.kblocks, wrow, 0,
                                              a.kblocks, epi);
}

// ---- dense products (2..32 tokens) --------------------------------------------------------------

// Part of virtual row v: its index among the parts' first rows. The part's pointers are then
// picked with selects among scalar registers (opaque to the compiler): a per-lane index into the
// argument's pointer arrays compiles to a vector load of the pointer and a wait on every
// outstanding load.
struct DensePart {
  int p, first, last;
};
__device__ __forceinline__ DensePart dense_part(const QmmDense &m, int v) {
  const int n = m.nparts, total = m.cum[n];
  const int c1 = n > 1 ? m.cum[1] : total, c2 = n > 2 ? m.cum[2] : total,
            c3 = n > 3 ? m.cum[3] : total;
  if (v >= c3) return {3, c3, total};
  if (v >= c2) return {2, c2, c3};
  if (v >= c1) return {1, c1, c2};
  return {0, 0, c1};
}
template <class T>
__device__ __forceinline__ T *pick4(T *p0, T *p1, T *p2, T *p3, int p) {
  asm("" : "+s"(p0), "+s"(p1), "+s"(p2), "+s"(p3));
  return p == 3 ? p3 : p == 2 ? p2 : p == 1 ? p1 : p0;
}

__device__ __forceinline__ const uint8_t *dense_row(const QmmDense &m, int v) {
  const DensePart q = dense_part(m, v);
  return pick4(m.w[0], m.w[1], m.w[2], m.w[3], q.p) + (int64_t)(v - q.first) * m.row_bytes;
}

// Partial sums of one (row tile, k slice) as [token][128]: GU: gate columns 0..63, up 64..127;
// otherwise the tile's 128 rows. With one slice the sums are the results.
template <bool GU>
struct DenseEpi {
  const QmmDense *m;
  const SplitRows *x;
  int B, tile, ks, ksplit;
  float *partial;
  Arrivals arr;
  int *is_last;  // LDS

  // a final value of row rt of the (non-SwiGLU) tile for token tok
  __device__ __forceinline__ void store(int tok, int rt, float v) const {
    const int vrow = tile * 128 + rt;
    if (vrow < m->cum[m->nparts]) {
      const DensePart q = dense_part(*m, vrow);
      gstore(pick4(m->y[0], m->y[1], m->y[2], m->y[3], q.p) + (int64_t)tok * (q.last - q.first) +
                 (vrow - q.first), v);
    }
  }

  template <int NT>
  __device__ __forceinline__ void operator()(const f32x4 (&acc)[2][NT]) const {
    const int lane = threadIdx.x & 63, t16 = lane & 15, g = lane >> 4, wave = wave_index();
    const int n = GU ? m->cum[1] : m->cum[m->nparts];
    auto row_in_tile = [&](int r) { return GU ? r * 64 + 16 * wave + t16 : 32 * wave + 16 * r + t16; };
    if (ksplit == 1) {
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = 16 * tt + 4 * g + i;
          if (tok >= B) continue;
          const float us = x->unscale[tok];
          if (GU) {
            const int col = tile * 64 + 16 * wave + t16;
            if (col < n)
              m->y[0][(int64_t)tok * n + col] = silu_mul(acc[0][tt][i] * us, acc[1][tt][i] * us);
          } else {
            store(tok, row_in_tile(0), acc[0][tt][i] * us);
            store(tok, row_in_tile(1), acc[1][tt][i] * us);
          }
        }
      return;
    }
    // k split: this slice's sums (device-coherent stores, all completed before the arrival is
    // counted); the last workgroup of the tile adds the slices in order and resets the counter
    float *mine = partial + ((int64_t)tile * ksplit + ks) * B * 128;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 16 * tt + 4 * g + i;
        if (tok >= B) continue;
        const float us = x->unscale[tok];
#pragma unroll
        for (int r = 0; r < 2; ++r)
          __hip_atomic_store(mine + tok * 128 + row_in_tile(r), acc[r][tt][i] * us,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (threadIdx.x == 0) *is_last = arrive_last(arr, tile, (unsigned)ksplit);
    __syncthreads();
    if (!*is_last) return;
    const float *base = partial + (int64_t)tile * ksplit * B * 128;
    const int per = GU ? 64 : 128;
    for (int idx = threadIdx.x; idx < B * per; idx += blockDim.x) {
      const int tok = idx / per, rt = idx - tok * per;
      float v0[kMaxSlices], v1[kMaxSlices];
#pragma unroll
      for (int q = 0; q < kMaxSlices; ++q) {  // every slice's value in flight, then the sums
        const float *pq = base + (int64_t)q * B * 128 + tok * 128;
        v0[q] = q < ksplit ? __hip_atomic_load(pq + rt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                           : 0.f;
        v1[q] = GU && q < ksplit
                    ? __hip_atomic_load(pq + 64 + rt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                    : 0.f;
      }
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int q = 0; q < kMaxSlices; ++q)
        if (q < ksplit) {
          s0 += v0[q];
          s1 += v1[q];
        }
      if (GU) {
        const int col = tile * 64 + rt;
        if (col < n) m->y[0][(int64_t)tok * n + col] = silu_mul(s0, s1);
      } else {
        store(tok, rt, s0);
      }
    }
    if (threadIdx.x == 0) done_arrivals(arr, tile);
  }
};

template <bool GU, int NTMAX>
__global__ __launch_bounds__(256) void k_qmm_dense(QmmDense m, SplitRows x, int B, int kblocks,
                                                   int ksplit, int upk, float *partial,
                                                   Arrivals arr) {
  __shared__ __attribute__((aligned(16))) uint8_t xbuf[2 * 16 * NTMAX * kXBlockBytes];
  __shared__ int rowidx[16 * NTMAX];
  __shared__ int is_last;
  // blockIdx -> (tile, slice): XCD x takes the tiles t = x (mod 8) and runs all slices of one
  // tile back to back (the cache lines two neighbouring slices of a row share are then fetched
  // once, into that XCD's L2)
  const int xcd = blockIdx.x & 7, bi = blockIdx.x >> 3;
  const int tile = xcd + 8 * (bi / ksplit), ks = bi % ksplit;
  if (tile * (GU ? 64 : 128) >= (GU ? m.cum[1] : m.cum[m.nparts])) return;
  const int kb0 = ks * upk, steps = min(upk, kblocks - kb0);
  if ((int)threadIdx.x < 16 * NTMAX) rowidx[threadIdx.x] = min((int)threadIdx.x, B - 1);
  const int t16 = threadIdx.x & 15, wave = wave_index();
  const uint8_t *wrow[2];
  if (GU) {
    const int c = min(tile * 64 + wave * 16 + t16, m.cum[1] - 1);
    wrow[0] = m.w[0] + (int64_t)c * m.row_bytes + (int64_t)kb0 * 144;
    wrow[1] = m.w[1] + (int64_t)c * m.row_bytes + (int64_t)kb0 * 144;
  } else {
    const int total = m.cum[m.nparts];
#pragma unroll
    for (int r = 0; r < 2; ++r)
      wrow[r] = dense_row(m, min(tile * 128 + wave * 32 + 16 * r + t16, total - 1)) +
                (int64_t)kb0 * 144;
  }
  __syncthreads();  // rowidx
  const DenseEpi<GU> epi{&m, &x, B, tile, ks, ksplit, partial, arr, &is_last};
  if (NTMAX == 1 || B <= 16)
    qmm_tiles<GU, 1, NTMAX>(x, xbuf, rowidx, B, kblocks, wrow, kb0, steps, epi);
  else
    qmm_tiles<GU, (NTMAX > 1 ? 2 : 1), NTMAX>(x, xbuf, rowidx, B, kblocks, wrow, kb0, steps, epi);
}

// ---- dense products with the activations split in the kernel ------------------------------------
// The same products without a split launch. A workgroup owns one row tile and one k slice of at
// most UPK blocks. It requests the slice's fp32 activations, then all of the slice's weights;
// while the weights are in flight it splits the activations into LDS (each (token, block) scaled
// by its own power of two, which puts the block's largest magnitude into [2^14, 2^15)) and meets
// the other waves at one barrier; the blocks are then multiplied back to back, each block's sums
// folded with its own 2^-e. NR 16-row weight tiles per wave (gate / up: always the pair). RB LDS
// token rows per block: 8 (up to 8 tokens; operand rows 8..15 repeat rows 0..7 and their outputs
// are never stored) or 16.
// Largest value over each 32-lane half of the wave (every lane of the half gets it): quad
// exchanges and row rotations by 4 and 8 give the maximum over a row of 16 lanes, a swap of
// neighbouring rows the maximum over two. Register moves only, no LDS.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}
__device__ __forceinline__ float half_wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  v = fmaxf(v, dpp_f<0x124>(v));  // row_ror:4
  v = fmaxf(v, dpp_f<0x128>(v));  // row_ror:8
  const auto sw = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v),
                                                   __builtin_bit_cast(unsigned, v), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)sw[0]), __builtin_bit_cast(float, (unsigned)sw[1]));
}

// Splits one (block, token) pair of activations into LDS. A half wave holds the pair's 256
// fp32 values, lane q of the half values 8q .. 8q+7 (run q of the block). The pair's power of
// two 2^e puts its largest magnitude (a half-wave maximum) into [2^14, 2^15); the scaled values
// go to xr, the pair's 1 KB row (hi halves, then lo halves at +512, each run of 8 in the order
// 0,2,1,3,4,6,5,7, run q stored at 16-byte piece q ^ swz); 2^-6 times each sub-block's sum of
// the scaled values (a quad's sum of its fp32 values, times 2^e) to ar (hi halves, then lo,
// sub-blocks in the same order); and 2^-e to *us.
__device__ __forceinline__ void split_pair_half(float4 v0, float4 v1, int swz, uint8_t *xr,
                                                uint8_t *ar, float *us) {
  const int q = threadIdx.x & 31;
  const float mx = half_wave_max(fmaxf(fmaxf(fmaxf(fabsf(v0.x), fabsf(v0.y)),
                                             fmaxf(fabsf(v0.z), fabsf(v0.w))),
                                       fmaxf(fmaxf(fabsf(v1.x), fabsf(v1.y)),
                                             fmaxf(fabsf(v1.z), fabsf(v1.w)))));
  int e = 0;
  if (mx > 0.f) {
    int ex;
    frexpf(mx, &ex);  // mx in [2^(ex-1), 2^ex)
    e = 15 - ex;
    if (e > 126) e = 126;
  }
  const float s = ldexpf(1.f, e);
  const float a[8] = {v0.x * s, v0.y * s, v0.z * s, v0.w * s, v1.x * s, v1.y * s, v1.z * s, v1.w * s};
  half8 h8, l8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const _Float16 hi = (_Float16)a[perm8(i)];
    h8[i] = hi;
    l8[i] = (_Float16)(a[perm8(i)] - (float)hi);
  }
  uint8_t *p = xr + 16 * (q ^ swz);
  *reinterpret_cast<half8 *>(p) = h8;
  *reinterpret_cast<half8 *>(p + 512) = l8;
  // sub-block j = runs 4j .. 4j+3: a quad
  float sum = ((v0.x + v0.y) + (v0.z + v0.w)) + ((v1.x + v1.y) + (v1.z + v1.w));
  sum += dpp_f<0xB1>(sum);
  sum += dpp_f<0x4E>(sum);
  if ((q & 3) == 0) {
    const int j = q >> 2;
    const float s6 = sum * s * 0x1p-6f;
    const _Float16 sh = (_Float16)s6, sl = (_Float16)(s6 - (float)sh);
    _Float16 *ap = reinterpret_cast<_Float16 *>(ar);
    ap[perm8(j)] = sh;
    ap[8 + perm8(j)] = sl;
  }
  if (q == 0) *us = ldexpf(1.f, -e);
}

template <int RB, int UPK>
struct DenseLds {
  static constexpr int kX = UPK * RB * kXBlockBytes;  // split blocks [block][row][1 KB]
  static constexpr int kAux = UPK * RB * kAuxBytes;   // sub-block sums [block][row][32 B]
  static constexpr int kUs = UPK * RB * 4;            // 2^-e [block][row]
  static constexpr int kBytes = kX + kAux + kUs;
};
constexpr int kMaxSlicesInline = 32;

// Loops f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>).
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(const F &f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// Sums of one (row tile, k slice), [token][kPer]: gate columns 0..63 and up 64..127, or the
// tile's 64 NR rows. With one slice the sums are the results.
template <bool GU, int NR>
struct Dense2Tile {
  static constexpr int kRows = GU ? 64 : 64 * NR;  // outputs (columns) per tile
  static constexpr int kPer = GU ? 128 : 64 * NR;  // partial sums per token
  static __device__ __forceinline__ int pos(int r, int wave, int t16) {
    return GU ? r * 64 + 16 * wave + t16 : 16 * NR * wave + 16 * r + t16;
  }
};

template <bool GU, int NR, int RB, int UPK>
__global__ __launch_bounds__(256) void k_qmm_dense2(QmmDense m, const float *__restrict__ x, int B,
                                                    int kblocks, int ksplit, int tiles,
                                                    float *partial, Arrivals arr) {
  static_assert(!GU || NR == 2, "a gate/up tile holds the gate and the up rows");
  static_assert(RB == 8 || RB == 16, "token rows per block");
  using L = DenseLds<RB, UPK>;
  using T = Dense2Tile<GU, NR>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[L::kBytes];
  __shared__ int is_last;
  // blockIdx -> (tile, slice): XCD x (workgroups are dealt to the 8 XCDs round-robin) takes the
  // tiles t = x (mod 8) and runs all slices of one tile back to back, so the cache lines that two
  // neighbouring slices of a row share are fetched once, into that XCD's L2
  const int xcd = blockIdx.x & 7, bi = blockIdx.x >> 3;
  const int tile = xcd + 8 * (bi / ksplit), ks = bi % ksplit;
  if (tile >= tiles) return;
  const int kb0 = ks * UPK, steps = min(UPK, kblocks - kb0);
  const int lane = threadIdx.x & 63, t16 = lane & 15, g = lane >> 4, wave = wave_index();
  const int64_t ldx = (int64_t)kblocks * 256;

  // 1. the slice's activations: pair p = b B + t (block b, token t) goes to half wave p % 8,
  // lane q of the half taking values 8q .. 8q+7 of it (1 KB per pair, coalesced); (b, t) are
  // stepped by 8 pairs without a division
  constexpr int kIt = RB * UPK / 8;
  const int hw = 2 * wave + (lane >> 5), q32 = lane & 31;
  const int step_b = 8 / B, step_t = 8 - step_b * B;
  int pb = hw / B, pt = hw - (hw / B) * B;
  float4 xv[kIt][2];
#pragma unroll
  for (int j = 0; j < kIt; ++j) {
    if (pb < steps) {
      const float *src = x + pt * ldx + (int64_t)(kb0 + pb) * 256 + 8 * q32;
      xv[j][0] = *reinterpret_cast<const float4 *>(src);
      xv[j][1] = *reinterpret_cast<const float4 *>(src + 4);
    } else {
      xv[j][0] = xv[j][1] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    pt += step_t;
    pb += step_b;
    if (pt >= B) {
      pt -= B;
      ++pb;
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. every block of the slice for the lane's weight rows (past the slice's end: its last
  // block again, never used)
  const uint8_t *wrow[NR];
  if (GU) {
    const int c = min(tile * 64 + wave * 16 + t16, m.cum[1] - 1);
    wrow[0] = m.w[0] + (int64_t)c * m.row_bytes + (int64_t)kb0 * 144;
    if constexpr (NR > 1) wrow[NR - 1] = m.w[1] + (int64_t)c * m.row_bytes + (int64_t)kb0 * 144;
  } else {
    const int total = m.cum[m.nparts];
#pragma unroll
    for (int r = 0; r < NR; ++r)
      wrow[r] = dense_row(m, min(tile * T::kRows + wave * 16 * NR + 16 * r + t16, total - 1)) +
                (int64_t)kb0 * 144;
  }
  QRow w[UPK][NR];
#pragma unroll
  for (int b = 0; b < UPK; ++b)
#pragma unroll
    for (int r = 0; r < NR; ++r) qrow_load(wrow[r], min(b, steps - 1), g, w[b][r]);
  __builtin_amdgcn_sched_barrier(0);

  // 3. split into LDS (waits for the activations only), then one barrier
  pb = hw / B;
  pt = hw - pb * B;
#pragma unroll
  for (int j = 0; j < kIt; ++j) {
    if (pb < steps) {
      const int row = pb * RB + pt;
      split_pair_half(xv[j][0], xv[j][1], pt, lds + row * kXBlockBytes,
                      lds + L::kX + row * kAuxBytes,
                      reinterpret_cast<float *>(lds + L::kX + L::kAux) + row);
    }
    pt += step_t;
    pb += step_b;
    if (pt >= B) {
      pt -= B;
      ++pb;
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");

  // 4. the blocks; operand row = t16 % RB. With up to 8 tokens (RB = 8) the hi and lo halves of
  // the activations share one operand: rows 0..7 hi of tokens 0..7, rows 8..15 their lo, one
  // product per k step; the lanes holding rows 8..15 (g = 2, 3) carry no min term and add their
  // sums to the lanes holding rows 0..7 at the end.
  constexpr bool kPack = RB == 8;
  const int row = t16 & (RB - 1);
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const bool min_lane = !kPack || g < 2;
  f32x4 acc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = zero;
#pragma unroll
  for (int b = 0; b < UPK; ++b) {
    if (b >= steps) break;
    const uint8_t *xb = lds + (b * RB + row) * kXBlockBytes + (kPack ? 512 * (t16 >> 3) : 0);
    const half4 am = *reinterpret_cast<const half4 *>(lds + L::kX + (b * RB + row) * kAuxBytes + 8 * g);
    const f32x4 us = *reinterpret_cast<const f32x4 *>(lds + L::kX + L::kAux +
                                                      (b * RB + ((4 * g) & (RB - 1))) * 4);
    QScale qs[NR];
    f32x4 dm[NR], dq[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      qs[r] = qscale(w[b][r], g);
      dm[r] = __builtin_amdgcn_mfma_f32_16x16x16f16(am, qs[r].m, zero, 0, 0, 0);
    }
    static_for<8>([&](auto S_) {
      constexpr int S = decltype(S_)::value;
      const uint8_t *p = xb + 16 * ((8 * g + S) ^ row);
      const half8 ah = *reinterpret_cast<const half8 *>(p);
      half8 al;
      if constexpr (!kPack) al = *reinterpret_cast<const half8 *>(p + 512);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const half8 bq = qb<S>(w[b][r], S < 4 ? qs[r].sc_lo : qs[r].sc_hi);
        dq[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bq, S == 0 ? zero : dq[r], 0, 0, 0);
        if constexpr (!kPack) dq[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bq, dq[r], 0, 0, 0);
      }
    });
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[r][i] = __builtin_fmaf(
            us[i], __builtin_fmaf(qs[r].d, dq[r][i], min_lane ? qs[r].ndmin * dm[r][i] : 0.f),
            acc[r][i]);
  }
  if constexpr (kPack) {  // the lo halves' sums (lanes 32..63) onto the hi halves' (lanes 0..31)
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[r][i] += xor_recv(acc[r][i], 32);
  }

  // 5. results (one slice) or this slice's sums and, for the tile's last workgroup, the total
  const int n = GU ? m.cum[1] : m.cum[m.nparts];
  auto store = [&](int tok, int vrow, float v) {
    if (vrow < n) {
      const DensePart q = dense_part(m, vrow);
      gstore(pick4(m.y[0], m.y[1], m.y[2], m.y[3], q.p) + (int64_t)tok * (q.last - q.first) +
                 (vrow - q.first), v);
    }
  };
  if (ksplit == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 4 * g + i;
      if (tok >= B) continue;
      if (GU) {
        const int col = tile * 64 + 16 * wave + t16;
        if (col < n) m.y[0][(int64_t)tok * n + col] = silu_mul(acc[0][i], acc[NR - 1][i]);
      } else {
#pragma unroll
        for (int r = 0; r < NR; ++r) store(tok, tile * T::kRows + T::pos(r, wave, t16), acc[r][i]);
      }
    }
    return;
  }
  float *mine = partial + ((int64_t)tile * ksplit + ks) * B * T::kPer;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tok = 4 * g + i;
    if (tok >= B) continue;
#pragma unroll
    for (int r = 0; r < NR; ++r)
      __hip_atomic_store(mine + tok * T::kPer + T::pos(r, wave, t16), acc[r][i], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  if (threadIdx.x == 0) is_last = arrive_last(arr, tile, (unsigned)ksplit);
  __syncthreads();
  if (!is_last) return;
  const float *base = partial + (int64_t)tile * ksplit * B * T::kPer;
  const int64_t sstride = (int64_t)B * T::kPer;
  for (int idx = threadIdx.x; idx < B * T::kRows; idx += blockDim.x) {
    const int tok = idx / T::kRows, rt = idx - tok * T::kRows;
    const float *pt = base + tok * T::kPer + rt;
    float s0 = 0.f, s1 = 0.f;
    for (int q0 = 0; q0 < ksplit; q0 += 8) {  // eight slices' values in flight, added in order
      float v0[8], v1[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool in = q0 + q < ksplit;
        v0[q] = in ? __hip_atomic_load(pt + (q0 + q) * sstride, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT)
                   : 0.f;
        v1[q] = GU && in ? __hip_atomic_load(pt + (q0 + q) * sstride + 64, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT)
                         : 0.f;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q0 + q < ksplit) {
          s0 += v0[q];
          s1 += v1[q];
        }
    }
    if (GU) {
      const int col = tile * 64 + rt;
      if (col < n) m.y[0][(int64_t)tok * n + col] = silu_mul(s0, s1);
    } else {
      store(tok, tile * T::kRows + rt, s0);
    }
  }
  if (threadIdx.x == 0) done_arrivals(arr, tile);
}

// ---- host side ----------------------------------------------------------------------------------

int qmm_chunk_rows(int nt_max) { return 16 * nt_max; }

// The row split keeps a row in registers: k <= 32768.
bool qmm_shape_ok(int64_t hidden, int64_t ffn) {
  return hidden % 256 == 0 && ffn % 256 == 0 && hidden >= 256 && ffn >= 256 && hidden <= 32768 &&
         ffn <= 32768;
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

template <int RUNS>
static void split_rows_launch(const float *src, int64_t ld, int64_t rows, int64_t k,
                              SplitRows out, hipStream_t st) {
  hipLaunchKernelGGL(k_split_rows<RUNS>, dim3((unsigned)rows), dim3(256), 0, st, src, ld, (int)k,
                     out.xs, out.aux, out.unscale);
}

void launch_split_rows(const float *src, int64_t ld, int64_t rows, int64_t k, SplitRows out,
                       hipStream_t st) {
  if (rows <= 0) return;
  const int64_t runs = (k / 8 + 255) / 256;  // runs of 8 per thread
  if (runs <= 2) split_rows_launch<2>(src, ld, rows, k, out, st);
  else if (runs <= 4) split_rows_launch<4>(src, ld, rows, k, out, st);
  else if (runs <= 8) split_rows_launch<8>(src, ld, rows, k, out, st);
  else split_rows_launch<16>(src, ld, rows, k, out, st);  // k <= 32768
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

// ---- dense host side ----------------------------------------------------------------------------

bool qmm_dense_ok(int fmt, int64_t k, int64_t batch) {
  const int mode = knob(TQ_KNOB_GEMV_QMM, 1);
  return mode && fmt == FMT_Q4_K && batch >= 2 && batch <= 32 && k % 256 == 0 && k >= 256 &&
         k <= 32768;
}

// Blocks per k slice: a function of k only -- at least four (measured at batch 8 on the
// Llama-3-8B shapes: 2, 3, 4, 6, 8 blocks give 3.55, 3.46, 3.19, 3.31, 3.24 ms per step), and at
// most 8 slices (the last workgroup of a tile reads every slice's sums, all at once).
static int dense_upk(int64_t k) {
  const int nblk = (int)(k / 256);
  const int v = knob(TQ_KNOB_QMM_UPK, 4);
  const int least = (nblk + kMaxSlices - 1) / kMaxSlices;
  return clampi(v > least ? v : least, 1, nblk);
}

static int64_t dense_tiles(int64_t rows, bool swiglu) { return swiglu ? (rows + 63) / 64 : (rows + 127) / 128; }

// The in-kernel split: blocks per k slice, a function of k only (so that one-launch multi and
// SwiGLU calls stay bitwise equal to single products), and the weight tiles per wave.
struct Dense2Plan {
  int upk, nr, rb, ksplit;
  int64_t tiles;
};
static Dense2Plan dense2_plan(int64_t rows, int64_t k, int64_t batch, bool swiglu, int nr_force) {
  const int nblk = (int)(k / 256);
  Dense2Plan p;
  p.upk = knob(TQ_KNOB_QMM_INLINE_UPK, 0);
  if (p.upk != 2 && p.upk != 4) p.upk = nblk <= 16 ? 2 : 4;
  p.ksplit = (nblk + p.upk - 1) / p.upk;
  p.rb = batch <= 8 ? 8 : 16;
  p.nr = swiglu ? 2 : nr_force ? nr_force : knob(TQ_KNOB_QMM_INLINE_NR, 0);
  if (p.nr != 1 && p.nr != 2) p.nr = 1;  // measured on the 8B shapes at batch 8: 2.34 against 2.55 ms per step for 2
  p.tiles = swiglu ? (rows + 63) / 64 : (rows + 64 * p.nr - 1) / (64 * p.nr);
  return p;
}
static size_t dense2_partial_bytes(const Dense2Plan &p, int64_t batch, bool swiglu) {
  if (p.ksplit == 1) return 0;
  const int64_t per = swiglu ? 128 : 64 * p.nr;
  return (size_t)align256(p.tiles * p.ksplit * batch * per * 4);
}
// Up to 16 tokens, 16-byte aligned activations and at most kMaxSlicesInline slices.
static bool dense2_ok(int64_t k, const float *x, int64_t batch) {
  if (!knob(TQ_KNOB_QMM_INLINE, 1) || batch > 16 || ((uintptr_t)x & 15) != 0) return false;
  return dense2_plan(256, k, batch, false, 1).ksplit <= kMaxSlicesInline;
}

size_t qmm_dense_bytes(int64_t rows, int64_t k, int64_t batch, bool swiglu) {
  const int64_t nblk = k / 256, upk = dense_upk(k), ksplit = (nblk + upk - 1) / upk;
  const int64_t tiles = dense_tiles(rows, swiglu);
  size_t need = split_rows_bytes(batch, k) +
                (ksplit > 1 ? (size_t)align256(tiles * ksplit * batch * 128 * 4) : 0);
  if (batch <= 16)  // either launch shape of the in-kernel split, whichever the knobs pick
    for (int nr = 1; nr <= 2; ++nr) {
      const size_t b = dense2_partial_bytes(dense2_plan(rows, k, batch, swiglu, nr), batch, swiglu);
      need = b > need ? b : need;
    }
  return need;
}

template <bool GU, int NR, int RB, int UPK>
static void dense2_launch(const QmmDense &m, const float *x, int B, int nblk, const Dense2Plan &p,
                          float *partial, Arrivals arr, hipStream_t st) {
  hipLaunchKernelGGL((k_qmm_dense2<GU, NR, RB, UPK>),
                     dim3((unsigned)((p.tiles + 7) / 8 * 8 * p.ksplit)), dim3(256), 0, st, m, x, B,
                     nblk, p.ksplit, (int)p.tiles, partial, arr);
}
template <bool GU, int NR>
static void dense2_launch_nr(const QmmDense &m, const float *x, int B, int nblk,
                             const Dense2Plan &p, float *partial, Arrivals arr, hipStream_t st) {
  if (p.rb == 8 && p.upk == 2) dense2_launch<GU, NR, 8, 2>(m, x, B, nblk, p, partial, arr, st);
  else if (p.rb == 8) dense2_launch<GU, NR, 8, 4>(m, x, B, nblk, p, partial, arr, st);
  else if (p.upk == 2) dense2_launch<GU, NR, 16, 2>(m, x, B, nblk, p, partial, arr, st);
  else dense2_launch<GU, NR, 16, 4>(m, x, B, nblk, p, partial, arr, st);
}

static int launch_qmm_dense2(const QmmDense &m, int64_t k, const float *x, int64_t batch, char *ws,
                             unsigned long long *counters, int max_counters, hipStream_t st) {
  const bool gu = m.swiglu != 0;
  const int64_t rows = gu ? m.cum[1] : m.cum[m.nparts];
  const Dense2Plan p = dense2_plan(rows, k, batch, gu, 0);
  if ((p.ksplit > 1 && p.tiles > max_counters) || p.ksplit > kMaxSlicesInline) return -2;
  const Arrivals arr{counters, p.ksplit > 1 ? call_tag() : 0ull};
  float *partial = (float *)ws;
  const int B = (int)batch, nblk = (int)(k / 256);
  if (gu) dense2_launch_nr<true, 2>(m, x, B, nblk, p, partial, arr, st);
  else if (p.nr == 2) dense2_launch_nr<false, 2>(m, x, B, nblk, p, partial, arr, st);
  else dense2_launch_nr<false, 1>(m, x, B, nblk, p, partial, arr, st);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_qmm_dense(const QmmDense &m, int64_t k, const float *x, int64_t batch, char *ws,
                     unsigned long long *counters, int max_counters, hipStream_t st) {
  if (dense2_ok(k, x, batch)) return launch_qmm_dense2(m, k, x, batch, ws, counters, max_counters, st);
  const int64_t rows = m.swiglu ? m.cum[1] : m.cum[m.nparts];
  const int nblk = (int)(k / 256), upk = dense_upk(k), ksplit = (nblk + upk - 1) / upk;
  const int64_t tiles = dense_tiles(rows, m.swiglu != 0);
  if ((ksplit > 1 && tiles > max_counters) || ksplit > kMaxSlices) return -2;
  const SplitRows xr = split_rows_at(ws, batch, k);
  float *partial = (float *)(ws + split_rows_bytes(batch, k));
  launch_split_rows(x, k, batch, k, xr, st);
  const dim3 grid((unsigned)((tiles + 7) / 8 * 8 * ksplit));
  const int B = (int)batch;
  const Arrivals counters_arr{counters, ksplit > 1 ? call_tag() : 0ull};
  if (m.swiglu) {
    if (B <= 16)
      hipLaunchKernelGGL((k_qmm_dense<true, 1>), grid, dim3(256), 0, st, m, xr, B, nblk, ksplit, upk, partial, counters_arr);
    else
      hipLaunchKernelGGL((k_qmm_dense<true, 2>), grid, dim3(256), 0, st, m, xr, B, nblk, ksplit, upk, partial, counters_arr);
  } else {
    if (B <= 16)
      hipLaunchKernelGGL((k_qmm_dense<false, 1>), grid, dim3(256), 0, st, m, xr, B, nblk, ksplit, upk, partial, counters_arr);
    else
      hipLaunchKernelGGL((k_qmm_dense<false, 2>), grid, dim3(256), 0, st, m, xr, B, nblk, ksplit, upk, partial, counters_arr);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace tq
