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
// qs[32c .. 32c+31]: low nibbles are sub-block 2c, high nibbles sub-block 2c+1). Its 16-wide k
// step s (0..7) uses the dword qs[32c + 4s ..]: the four low-nibble weights first, then the four
// high-nibble ones. The token tile in LDS is stored in the same order, so a product over a step
// is a plain dot product over one permutation of k.
//
// Each weight is dequantized once per chunk (fp32 fma of d*sc and -dmin*m, then bf16), directly
// into the lane's A registers; the chunk's token rows are staged through LDS, double-buffered.
#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_gemv_core.h"
#include "tq_moe.h"
#include "tq_prefill.h"

namespace tq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChunk = 160;           // token rows per chunk (5 tiles of 32)
constexpr int kRowStride = 272;       // LDS bytes per token row: 128 bf16 + 16 bytes of padding
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
// ceil(cnt / kChunk) chunks of near-equal size, chunks in slot order. One workgroup of 256
// threads, a thread per slot, an LDS prefix sum over each batch of 256 slots.
__global__ __launch_bounds__(256) void k_chunk_table(const int *__restrict__ act,
                                                     const int *__restrict__ n_active, int E,
                                                     int max_chunks, int *__restrict__ chunks,
                                                     int *__restrict__ n_chunks) {
  __shared__ int scan[256];
  const int na = *n_active;
  int base = 0;  // chunks of the earlier batches
  for (int s0 = 0; s0 < na; s0 += 256) {
    const int s = s0 + (int)threadIdx.x;
    int cnt = 0, p0 = 0, parts = 0;
    if (s < na) {
      p0 = act[(E + 1) + s];
      cnt = act[2 * (E + 1) + s];
      parts = (cnt + kChunk - 1) / kChunk;
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

// Loads through the global address space (the blob pointers come from a device table, so the
// compiler would otherwise issue generic loads, which it cannot count precisely).
typedef const u32x4 __attribute__((address_space(1))) *gu32x4;

__device__ __forceinline__ u32x4 gload(const void *p) { return *(gu32x4)p; }

// Raw bytes of one Q4_K row for one step: the block header (d, dmin, 12 scale bytes) and the
// lane's 32 quant bytes.
struct RawRow {
  u32x4 head, q0, q1;
};

__device__ __forceinline__ void load_raw(const uint8_t *row, int kb, int c, RawRow &r) {
  const uint8_t *b = row + (int64_t)kb * 144;
  r.head = gload(b);
  r.q0 = gload(b + 16 + 32 * c);
  r.q1 = gload(b + 32 + 32 * c);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
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

// The 8 weights of k step s (quant dword s of the lane's group) as one bf16x8 A operand.
__device__ __forceinline__ bf16x8 dequant_step(const RawRow &r, const GroupScale &g, int s) {
  const uint32_t wq = dword_of(s < 4 ? r.q0 : r.q1, s & 3);
  const uint32_t lo = wq & 0x0F0F0F0Fu, hi = (wq >> 4) & 0x0F0F0F0Fu;
  float f[8];
  nibbles_to_float<false>(lo, f[0], f[1]);
  nibbles_to_float<true>(lo, f[2], f[3]);
  nibbles_to_float<false>(hi, f[4], f[5]);
  nibbles_to_float<true>(hi, f[6], f[7]);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = __builtin_fmaf(g.al, f[e], g.bl);
    f[4 + e] = __builtin_fmaf(g.ah, f[4 + e], g.bh);
  }
  u32x4 v;
  v.x = pack_bf16(f[0], f[1]);
  v.y = pack_bf16(f[2], f[3]);
  v.z = pack_bf16(f[4], f[5]);
  v.w = pack_bf16(f[6], f[7]);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g * u / (1.f + expf(-g)); }

// Token staging. Thread tid copies the 16 bytes at k offset 8*(tid % 16) of the step's 128 k
// for rows tid/16 + 16 i (i < 2 NT), clamped to the chunk's last row: rows past the chunk only
// feed token columns that are never stored. In LDS the 8 k of that piece go to two entries:
// k-half kg = pc/8, steps s and s+1 (s = 2 (pc % 4)), low-nibble half (bytes 0..7 of the
// 16-byte entry) for pc % 8 < 4, else the high half.
template <bool GU, int NT>
__device__ __forceinline__ void prefill_tiles(const PrefillArgs &a, uint8_t (*tok)[kBufBytes],
                                              const int64_t *rowoff, int rows, int p0,
                                              const uint8_t *const (&wrow)[2], int col0) {
  const int lane = threadIdx.x & 63;
  const int lrow = lane & 31, kg = lane >> 5;
  const int pc = threadIdx.x & 15, trow = threadIdx.x >> 4;
  const uint16_t *src[2 * NT];
#pragma unroll
  for (int i = 0; i < 2 * NT; ++i)
    src[i] = a.xsrc + rowoff[min(trow + 16 * i, rows - 1)] + 8 * pc;
  const int dst = (trow * kRowStride) + ((pc >> 3) * 8 + 2 * (pc & 3)) * 16 + 8 * ((pc >> 2) & 1);
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

  const float unit_inv = 1.f / nibble_fp8_unit();
  f32x16 acc[NT][2];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[t][r][j] = 0.f;

  const int steps = 2 * a.kblocks;
  RawRow raw[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) load_raw(wrow[r], 0, kg, raw[r]);
  u32x4 tv[2 * NT];
#pragma unroll
  for (int i = 0; i < 2 * NT; ++i) tv[i] = gload(src[i]);
#pragma unroll
  for (int i = 0; i < 2 * NT; ++i) {
    uint8_t *d = tok[0] + dst + 16 * i * kRowStride;
    *reinterpret_cast<u32x2 *>(d) = (u32x2){tv[i].x, tv[i].y};
    *reinterpret_cast<u32x2 *>(d + 16) = (u32x2){tv[i].z, tv[i].w};
  }
  __syncthreads();

  for (int st = 0; st < steps; ++st) {
    const int c = 2 * (st & 1) + kg;  // the lane's group in block st/2
    const RawRow cur[2] = {raw[0], raw[1]};
    const bool more = st + 1 < steps;
    if (more) {
      const int nst = st + 1;
#pragma unroll
      for (int r = 0; r < 2; ++r) load_raw(wrow[r], nst >> 1, 2 * (nst & 1) + kg, raw[r]);
#pragma unroll
      for (int i = 0; i < 2 * NT; ++i) tv[i] = gload(src[i] + 128 * nst);
    }
    const GroupScale gs[2] = {group_scale(cur[0], c, unit_inv), group_scale(cur[1], c, unit_inv)};
    const uint8_t *buf = tok[st & 1] + lrow * kRowStride + kg * 128;
    // Software pipeline over the 8 k steps: while the matrix cores work on step s, the lanes
    // dequantize the A operands of step s+1 and read its B operands from LDS.
    bf16x8 a0 = dequant_step(cur[0], gs[0], 0), a1 = dequant_step(cur[1], gs[1], 0);
    bf16x8 bv[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
      bv[t] = *reinterpret_cast<const bf16x8 *>(buf + 32 * t * kRowStride);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x8 n0, n1, nb[NT];
      if (s < 7) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
          nb[t] = *reinterpret_cast<const bf16x8 *>(buf + 32 * t * kRowStride + 16 * (s + 1));
        n0 = dequant_step(cur[0], gs[0], s + 1);
        n1 = dequant_step(cur[1], gs[1], s + 1);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        acc[t][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bv[t], acc[t][0], 0, 0, 0);
        acc[t][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bv[t], acc[t][1], 0, 0, 0);
      }
      if (s < 7) {
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
    }
    if (more) {
      uint8_t *nb = tok[(st + 1) & 1] + dst;
#pragma unroll
      for (int i = 0; i < 2 * NT; ++i) {
        uint8_t *d = nb + 16 * i * kRowStride;
        *reinterpret_cast<u32x2 *>(d) = (u32x2){tv[i].x, tv[i].y};
        *reinterpret_cast<u32x2 *>(d + 16) = (u32x2){tv[i].z, tv[i].w};
      }
    }
    __syncthreads();
  }

  // epilogue: lane holds rows 8*(i/4) + 4*kg + i%4 of token column lrow of each tile
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
  __shared__ __attribute__((aligned(16))) uint8_t tok[2][kBufBytes];
  __shared__ int64_t rowoff[kChunk];

  // blockIdx -> (chunk, tile): workgroups are dealt to the 8 XCDs round-robin; XCD x takes the
  // chunks c = x (mod 8) and runs all tiles of one chunk back to back, so the chunk's token rows
  // are shared through that XCD's L2.
  const int b = blockIdx.x, xcd = b & 7, i = b >> 3;
  const int chunk = xcd + 8 * (i / a.ntiles), tile = i % a.ntiles;
  if (chunk >= *a.n_chunks) return;
  const int slot = a.chunks[3 * chunk], p0 = a.chunks[3 * chunk + 1], rows = a.chunks[3 * chunk + 2];
  const int e = a.act[slot];
  const MoeExpertPtrs &ex = e == a.E ? a.shared : a.experts[e];

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
    wrow[0] = (const uint8_t *)ex.m[0] + (int64_t)(col0 + lrow) * a.row_bytes;
    wrow[1] = (const uint8_t *)ex.m[1] + (int64_t)(col0 + lrow) * a.row_bytes;
  } else {
    col0 = tile * 256 + wave * 64;
    wrow[0] = (const uint8_t *)ex.m[2] + (int64_t)(col0 + lrow) * a.row_bytes;
    wrow[1] = (const uint8_t *)ex.m[2] + (int64_t)(col0 + 32 + lrow) * a.row_bytes;
  }
  __syncthreads();  // rowoff
  switch ((rows + 31) >> 5) {
    case 1: prefill_tiles<GU, 1>(a, tok, rowoff, rows, p0, wrow, col0); break;
    case 2: prefill_tiles<GU, 2>(a, tok, rowoff, rows, p0, wrow, col0); break;
    case 3: prefill_tiles<GU, 3>(a, tok, rowoff, rows, p0, wrow, col0); break;
    case 4: prefill_tiles<GU, 4>(a, tok, rowoff, rows, p0, wrow, col0); break;
    default: prefill_tiles<GU, 5>(a, tok, rowoff, rows, p0, wrow, col0); break;
  }
}

// ---- host side ----------------------------------------------------------------------------------

int prefill_max_chunks(int64_t positions, int max_active) {
  return (int)((positions + (int64_t)(kChunk - 1) * max_active) / kChunk + 1);
}

int launch_prefill(int max_chunks, PrefillArgs a, const float *x, int64_t tokens, int64_t hidden,
                   int64_t ffn, uint16_t *xb, uint16_t *h, float *o, hipStream_t st) {
  {
    const int64_t n = tokens * hidden;
    int64_t blocks = (n / 2 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(k_to_bf16, dim3((unsigned)blocks), dim3(256), 0, st, x, n, (uint32_t *)xb);
  }
  hipLaunchKernelGGL(k_chunk_table, dim3(1), dim3(256), 0, st, a.act, a.n_active, a.E,
                     max_chunks, (int *)a.chunks, (int *)a.n_chunks);
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
