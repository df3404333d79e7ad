// tq_prefill.hip -- grouped expert products for prompt-sized batches on the bf16 matrix cores.
//
// When an expert receives many tokens its three products are small dense GEMMs, so they run on
// v_mfma_f32_32x32x16_bf16 instead of the fp32 GEMV (the routing, grouping and combine are the
// decode path's kernels):
//   k_to_bf16         x [T][hidden] fp32 -> bf16 (round to nearest even)
//   k_chunk_table     the active experts' position ranges cut into chunks of at most kChunk rows
//   k_prefill<true>   per (chunk, 128 ffn columns): gate and up products of the chunk's tokens,
//                     h = silu(gate) * up stored as bf16 [position][ffn]
//   k_prefill<false>  per (chunk, 256 hidden rows): down product, o fp32 [position][hidden]
//
// Matrix-core layout. A = weights (32 rows x 16 k), B = token rows (16 k x 32 tokens). Lane l
// owns weight row l % 32 and k-half kg = l / 32 of every 16-wide k step; D[row][token] lands in
// lane l as rows 8*(i/4) + 4*kg + i%4 (i = 0..15) of token column l % 32.
//
// Q4_K block -> k order. One workgroup step covers 128 weights of every row (half a 256-weight
// block); lane kg of that step owns the 64 weights of group c = 2*half + kg (bytes
// qs[32c .. 32c+31]: low nibbles are sub-block 2c, high nibbles sub-block 2c+1), and its 16-wide
// k step s (0..7) holds the 8 consecutive weights 64c + 8s .. 64c + 8s + 7 (in k order, so the
// token operand is 8 consecutive activations).
//
// Each weight is dequantized once per chunk (fp32 fma of d*sc and -dmin*m, then bf16), directly
// into the lane's A registers; the chunk's token rows stream into a 3-deep LDS ring with direct
// global-to-LDS loads, two steps ahead of the matrix cores.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "tq_device.h"
#include "tq_gemv_core.h"
#include "tq_mfma.h"
#include "tq_moe.h"
#include "tq_prefill.h"

namespace tq {

constexpr int kChunk = 160;           // token rows per chunk (5 tiles of 32)
constexpr int kRowStride = 256;       // LDS bytes per token row: 128 bf16 of one step
constexpr int kBufBytes = kChunk * kRowStride;

// ---- x -> bf16 ----------------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_to_bf16(const float *__restrict__ x, int64_t n,
                                                 uint32_t *__restrict__ xb) {
  const int64_t pairs = n / 2, stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < pairs; i += stride) {
    const float2 v = reinterpret_cast<const float2 *>(x)[i];
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 b = {(__bf16)v.x, (__bf16)v.y};
    xb[i] = __builtin_bit_cast(uint32_t, b);
  }
}

// ---- chunk table --------------------------------------------------------------------------------
// chunks[3c .. 3c+2] = (active slot, first position, rows); an expert with cnt rows is cut into
// ceil(cnt / chunk_rows) chunks of near-equal size, chunks in slot order. One workgroup of 256
// threads, a thread per slot, an LDS prefix sum over each batch of 256 slots.
__global__ __launch_bounds__(256) void k_chunk_table(const int *__restrict__ act,
                                                     const int *__restrict__ n_active, int act_stride,
                                                     int chunk_rows, int max_chunks,
                                                     int *__restrict__ chunks,
                                                     int *__restrict__ n_chunks) {
  __shared__ int scan[256];
  const int na = *n_active;
  int base = 0;  // chunks of the earlier batches
  for (int s0 = 0; s0 < na; s0 += 256) {
    const int s = s0 + (int)threadIdx.x;
    int cnt = 0, p0 = 0, parts = 0;
    if (s < na) {
      p0 = act[act_stride + s];
      cnt = act[2 * act_stride + s];
      parts = (cnt + chunk_rows - 1) / chunk_rows;
    }
    scan[threadIdx.x] = parts;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {  // inclusive scan
      const int v = threadIdx.x >= (unsigned)d ? scan[threadIdx.x - d] : 0;
      __syncthreads();
      scan[threadIdx.x] += v;
      __syncthreads();
    }
    int nc = base + scan[threadIdx.x] - parts;
    if (parts) {
      const int rows0 = cnt / parts, extra = cnt - rows0 * parts;
      int p = p0;
      for (int q = 0; q < parts && nc < max_chunks; ++q) {
        const int rows = rows0 + (q < extra ? 1 : 0);
        chunks[3 * nc] = s;
        chunks[3 * nc + 1] = p;
        chunks[3 * nc + 2] = rows;
        p += rows;
        ++nc;
      }
    }
    base += scan[255];
    __syncthreads();
  }
  if (threadIdx.x == 0) *n_chunks = base < max_chunks ? base : max_chunks;
}

// ---- the grouped product ------------------------------------------------------------------------

// Raw bytes of one Q4_K row for one step: the block header (d, dmin, 12 scale bytes) and the
// lane's 32 quant bytes.
struct RawRow {
  u32x4 head, q0, q1;
  static constexpr int kLoads = 3;  // load_raw issues one 16-byte load per field
};
static_assert(sizeof(RawRow) == RawRow::kLoads * sizeof(u32x4), "one load per field of RawRow");

__device__ __forceinline__ void load_raw(const uint8_t *row, int kb, int c, RawRow &r) {
  const uint8_t *b = row + (int64_t)kb * 144;
  r.head = gload(b);
  r.q0 = gload(b + 16 + 32 * c);
  r.q1 = gload(b + 32 + 32 * c);
}

// Scale and offset of the lane's two sub-blocks (2c: low nibbles, 2c+1: high nibbles) of the
// block in r: weight = a * f + b with f = nibble * 2^-9 from the fp8 converter.
struct GroupScale {
  float al, bl, ah, bh;
};

__device__ __forceinline__ GroupScale group_scale(const RawRow &r, int c, float unit_inv) {
  const uint32_t h0 = r.head.x, s0 = r.head.y, s1 = r.head.z, s2 = r.head.w;
  const float d = half_bits_to_float(h0) * unit_inv, dmin = half_bits_to_float(h0 >> 16);
  float sc_lo, m_lo, sc_hi, m_hi;
  q4k_scale_min_at(s0, s1, s2, q4k_field(2 * c), sc_lo, m_lo);
  q4k_scale_min_at(s0, s1, s2, q4k_field(2 * c + 1), sc_hi, m_hi);
  return GroupScale{d * sc_lo, -(dmin * m_lo), d * sc_hi, -(dmin * m_hi)};
}

// The 8 weights of k step s as one bf16x8 A operand: k = 64c + 8s + 0..7 of the lane's group c,
// the low nibbles of quant bytes 8s .. 8s+7 for s < 4 (sub-block 2c), the high nibbles of
// bytes 8(s-4) .. for s >= 4 (sub-block 2c+1).
template <int S>
__device__ __forceinline__ bf16x8 dequant_step(const RawRow &r, const GroupScale &g) {
  const u32x4 &q = (S & 3) < 2 ? r.q0 : r.q1;
  uint32_t w0 = dword_of(q, (2 * S) & 3), w1 = dword_of(q, (2 * S + 1) & 3);
  if (S >= 4) {
    w0 >>= 4;
    w1 >>= 4;
  }
  w0 &= 0x0F0F0F0Fu;
  w1 &= 0x0F0F0F0Fu;
  float f[8];
  nibbles_to_float<false>(w0, f[0], f[1]);
  nibbles_to_float<true>(w0, f[2], f[3]);
  nibbles_to_float<false>(w1, f[4], f[5]);
  nibbles_to_float<true>(w1, f[6], f[7]);
  const float a = S < 4 ? g.al : g.ah, b = S < 4 ? g.bl : g.bh;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = __builtin_fmaf(a, f[e], b);
  u32x4 v;
  v.x = pack_bf16(f[0], f[1]);
  v.y = pack_bf16(f[2], f[3]);
  v.z = pack_bf16(f[4], f[5]);
  v.w = pack_bf16(f[6], f[7]);
  return __builtin_bit_cast(bf16x8, v);
}

// Token staging. A step's token tile (rows of 128 bf16: 16 pieces of 8 k) goes straight from
// global memory to LDS (global_load_lds, 16 bytes per lane: lane l of a wave instruction writes
// bytes 16 l of a 1 KB run = 4 rows). Piece pc of row t is stored at position pc ^ (t % 16) of the
// row, so the 32 lanes of a B-operand read (32 rows, one piece) spread over all banks. Wave w's
// instruction i fills rows 16 i + 4 w .. +3; rows past the chunk are filled from its last row and
// only feed token columns that are never stored.
template <bool GU, int NT>
__device__ __forceinline__ void prefill_tiles(const PrefillArgs &a, uint8_t *__restrict__ tok0,
                                              uint8_t *__restrict__ tok1,
                                              uint8_t *__restrict__ tok2, const int64_t *rowoff,
                                              int rows, int p0, const uint8_t *const (&wrow)[2],
                                              int col0) {
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int lrow = lane & 31, kg = lane >> 5;
  const uint16_t *src[2 * NT];
#pragma unroll
  for (int i = 0; i < 2 * NT; ++i) {
    const int t = 16 * i + 4 * wave + (lane >> 4);
    const int pc = (lane & 15) ^ (t & 15);
    src[i] = a.xsrc + rowoff[min(t, rows - 1)] + 8 * pc;
  }
  // enqueue the token tile of step st into tok. The loads are written as asm so that the
  // compiler does not track them: it cannot tell the three token buffers apart and would
  // otherwise wait for these loads before every LDS read. Their completion is awaited
  // explicitly (barrier_after_vmem) before the step that reads them.
  // the vector-memory loads of one step: the weights of two rows (load_w) and 2 NT token pieces
  // (stage), issued unconditionally; each step's barrier leaves exactly one step's worth (the
  // next step's) in flight, so the count must follow the loop bounds of both lambdas
  constexpr int kRows = 2, kStageLoads = 2 * NT;
  constexpr int kStepLoads = kRows * RawRow::kLoads + kStageLoads;
  auto stage = [&](uint8_t *tok, int st) {
    const uint32_t b = __builtin_amdgcn_readfirstlane(lds_address(tok + 4 * wave * kRowStride));
#pragma unroll
    for (int i = 0; i < kStageLoads; ++i)
      load_lds16(src[i] + 128 * st, b + 16 * i * kRowStride);
  };

  const float unit_inv = 1.f / nibble_fp8_unit();
  f32x16 acc[NT][2];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[t][r][j] = 0.f;

  const int steps = 2 * a.kblocks;
  // Weights and tokens both run two steps ahead: raw[j] holds the weights of the steps st with
  // st % 3 == j, tok_j their tokens.
  RawRow raw[3][2];
  auto load_w = [&](RawRow (&r)[kRows], int st) {
#pragma unroll
    for (int q = 0; q < kRows; ++q) load_raw(wrow[q], st >> 1, 2 * (st & 1) + kg, r[q]);
  };
  load_w(raw[0], 0);
  stage(tok0, 0);
  load_w(raw[1], min(1, steps - 1));
  stage(tok1, min(1, steps - 1));
  // B-operand read of tile t, step s: row 32 t + lrow, piece 8 kg + s
  const int rd = lrow * kRowStride;
  const int sw = lrow & 15;

  // one step: weights of st in `rc`, tokens in `cur_buf`; those of st+2 go to `rf` and `fill`
  auto step = [&](int st, const uint8_t *cur_buf, uint8_t *fill, const RawRow (&rc)[2],
                  RawRow (&rf)[2]) {
    // Outstanding, oldest first: weights and tokens of st, then of st+1. Every step issues the
    // same loads (past the last step they repeat the last block / tile into registers and a
    // buffer nobody reads), so this count is exact on every path.
    // Then a plain barrier (__syncthreads would add a release fence, i.e. a wait for every load
    // in flight, the two steps ahead included): after it every wave's tokens of step st are in
    // LDS and every wave has finished reading `fill` (its tiles of step st-1).
    static_assert(kStepLoads == 6 + 2 * NT, "two rows of three loads plus two per token tile");
    barrier_after_vmem<kStepLoads>();
    const int c = 2 * (st & 1) + kg;  // the lane's group in block st/2
    const RawRow (&cur)[2] = rc;
    const GroupScale gs[2] = {group_scale(cur[0], c, unit_inv), group_scale(cur[1], c, unit_inv)};
    const uint8_t *buf = cur_buf + rd;
    // Software pipeline over the 8 k steps: while the matrix cores work on step s, the lanes
    // dequantize the A operands of step s+1 and read its B operands from LDS.
    bf16x8 bv[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
      bv[t] = *reinterpret_cast<const bf16x8 *>(buf + 32 * t * kRowStride + 16 * ((8 * kg) ^ sw));
    __builtin_amdgcn_sched_barrier(0);
    // The loads of step st+2, issued after the first LDS reads of this step: where the compiler
    // cannot tell the token buffers apart it waits for all earlier loads before those reads,
    // and this way that wait never covers the loads just issued.
    load_w(rf, min(st + 2, steps - 1));
    stage(fill, min(st + 2, steps - 1));
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 a0 = dequant_step<0>(cur[0], gs[0]), a1 = dequant_step<0>(cur[1], gs[1]);
    auto kstep = [&](auto S_) {
      constexpr int S = decltype(S_)::value;
      bf16x8 n0, n1, nb[NT];
      if constexpr (S < 7) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
          nb[t] = *reinterpret_cast<const bf16x8 *>(buf + 32 * t * kRowStride +
                                                    16 * ((8 * kg + S + 1) ^ sw));
        n0 = dequant_step<S + 1>(cur[0], gs[0]);
        n1 = dequant_step<S + 1>(cur[1], gs[1]);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        acc[t][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bv[t], acc[t][0], 0, 0, 0);
        acc[t][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bv[t], acc[t][1], 0, 0, 0);
      }
      if constexpr (S < 7) {
        // issue order: the LDS reads, then each MFMA followed by a share of the VALU work
        __builtin_amdgcn_sched_group_barrier(0x100, NT, 0);
#pragma unroll
        for (int t = 0; t < 2 * NT; ++t) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 40 / (2 * NT) + 1, 0);
        }
        a0 = n0;
        a1 = n1;
#pragma unroll
        for (int t = 0; t < NT; ++t) bv[t] = nb[t];
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
  };
  // three steps per trip so that each step's buffers are distinct LDS objects: the compiler then
  // knows the reads of step st do not touch the tiles still landing for st+1 and st+2
  // (whole trips in the loop, the 0..2 remaining steps after it: every path into a step then
  // has the same loads in flight, which keeps the compiler's own wait counts exact)
  int st = 0;
  for (; st + 3 <= steps; st += 3) {
    step(st, tok0, tok2, raw[0], raw[2]);
    step(st + 1, tok1, tok0, raw[1], raw[0]);
    step(st + 2, tok2, tok1, raw[2], raw[1]);
  }
  if (st < steps) step(st, tok0, tok2, raw[0], raw[2]);
  if (st + 1 < steps) step(st + 1, tok1, tok0, raw[1], raw[0]);
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      keep_alive(raw[j][q].head);
      keep_alive(raw[j][q].q0);
      keep_alive(raw[j][q].q1);
    }
  wait_vmem<0>();  // the surplus loads of the last steps land before the workgroup ends

  // epilogue: lane holds rows 8*(i/4) + 4*kg + i%4 of token column lrow of each tile
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tr = 32 * t + lrow;
    if (tr < rows) {
      const int64_t p = p0 + tr;
      if (GU) {
        uint16_t *h = (uint16_t *)a.out + p * a.ldo + col0;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float hv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) hv[q] = silu_mul(acc[t][0][4 * g + q], acc[t][1][4 * g + q]);
          *reinterpret_cast<u32x2 *>(h + 8 * g + 4 * kg) =
              (u32x2){pack_bf16(hv[0], hv[1]), pack_bf16(hv[2], hv[3])};
        }
      } else {
        float *o = (float *)a.out + p * a.ldo + col0;
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<float4 *>(o + 32 * r + 8 * g + 4 * kg) =
                make_float4(acc[t][r][4 * g], acc[t][r][4 * g + 1], acc[t][r][4 * g + 2],
                            acc[t][r][4 * g + 3]);
      }
    }
  }
}

template <bool GU>
__global__ __launch_bounds__(256) void k_prefill(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t tok0[kBufBytes];
  __shared__ __attribute__((aligned(16))) uint8_t tok1[kBufBytes];
  __shared__ __attribute__((aligned(16))) uint8_t tok2[kBufBytes];
  __shared__ int64_t rowoff[kChunk];

  // blockIdx -> (chunk, tile): workgroups are dealt to the 8 XCDs round-robin; XCD x takes the
  // chunks c = x (mod 8) and runs all tiles of one chunk back to back, so the chunk's token rows
  // are shared through that XCD's L2.
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
    int64_t r = p;
    if (a.x_by_token) r = p >= a.Tk ? p - a.Tk : a.pairs[p] / a.topk;
    rowoff[t] = r * a.ldx;
  }

  const int lrow = threadIdx.x & 31, wave = wave_index();
  // the lane's two weight rows (row-block 0 and 1)
  const uint8_t *wrow[2];
  int col0;  // GU: first ffn column of the wave; down: first hidden row of the wave
  if (GU) {
    col0 = tile * 128 + wave * 32;
    wrow[0] = mat[0] + (int64_t)(col0 + lrow) * a.row_bytes;
    wrow[1] = mat[1] + (int64_t)(col0 + lrow) * a.row_bytes;
  } else {
    col0 = tile * 256 + wave * 64;
    wrow[0] = mat[2] + (int64_t)(col0 + lrow) * a.row_bytes;
    wrow[1] = mat[2] + (int64_t)(col0 + 32 + lrow) * a.row_bytes;
  }
  __syncthreads();  // rowoff
  switch ((rows + 31) >> 5) {
    case 1: prefill_tiles<GU, 1>(a, tok0, tok1, tok2, rowoff, rows, p0, wrow, col0); break;
    case 2: prefill_tiles<GU, 2>(a, tok0, tok1, tok2, rowoff, rows, p0, wrow, col0); break;
    case 3: prefill_tiles<GU, 3>(a, tok0, tok1, tok2, rowoff, rows, p0, wrow, col0); break;
    case 4: prefill_tiles<GU, 4>(a, tok0, tok1, tok2, rowoff, rows, p0, wrow, col0); break;
    default: prefill_tiles<GU, 5>(a, tok0, tok1, tok2, rowoff, rows, p0, wrow, col0); break;
  }
}

// ---- host side ----------------------------------------------------------------------------------

int max_chunks_for(int64_t positions, int max_active, int chunk_rows) {
  return (int)((positions + (int64_t)(chunk_rows - 1) * max_active) / chunk_rows + 1);
}

int prefill_max_chunks(int64_t positions, int max_active) {
  return max_chunks_for(positions, max_active, kChunk);
}

void launch_chunk_table(const int *act, const int *n_active, int act_stride, int chunk_rows,
                        int max_chunks, int *chunks, int *n_chunks, hipStream_t st) {
  hipLaunchKernelGGL(k_chunk_table, dim3(1), dim3(256), 0, st, act, n_active, act_stride,
                     chunk_rows, max_chunks, chunks, n_chunks);
}

int launch_prefill(int max_chunks, PrefillArgs a, const float *x, int64_t tokens, int64_t hidden,
                   int64_t ffn, uint16_t *xb, uint16_t *h, float *o, hipStream_t st) {
  {
    const int64_t n = tokens * hidden;
    int64_t blocks = (n / 2 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(k_to_bf16, dim3((unsigned)blocks), dim3(256), 0, st, x, n, (uint32_t *)xb);
  }
  launch_chunk_table(a.act, a.n_active, a.act_stride, kChunk, max_chunks, (int *)a.chunks,
                     (int *)a.n_chunks, st);
  const int groups = (max_chunks + 7) / 8;
  // gate / up
  a.kblocks = (int)(hidden / 256);
  a.row_bytes = hidden / 256 * 144;
  a.xsrc = xb;
  a.ldx = hidden;
  a.x_by_token = 1;
  a.out = h;
  a.ldo = ffn;
  a.ntiles = (int)(ffn / 128);
  hipLaunchKernelGGL(k_prefill<true>, dim3((unsigned)(8 * groups * a.ntiles)), dim3(256), 0, st, a);
  // down
  a.kblocks = (int)(ffn / 256);
  a.row_bytes = ffn / 256 * 144;
  a.xsrc = h;
  a.ldx = ffn;
  a.x_by_token = 0;
  a.out = o;
  a.ldo = hidden;
  a.ntiles = (int)(hidden / 256);
  hipLaunchKernelGGL(k_prefill<false>, dim3((unsigned)(8 * groups * a.ntiles)), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace tq
