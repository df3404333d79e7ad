// tq_dense.hip -- dequantization, dense GEMV and SwiGLU kernels with their host launchers.
#include "tq_gemv_core.h"
#include "tq_gemm_f32m.h"
#include "tq_gemv_i8.h"
#include "tq_gemv_mf.h"
#include "tq_qmm.h"
#include "tq_launch.h"
#include "tq_moe.h"

#include <stdlib.h>

namespace tq {

// ---- per-weight decode (dequant kernels and the generic GEMV) --------------------------------
// Weight i of a block. Reads single bytes, so any block alignment works.

__device__ __forceinline__ uint32_t rd16(const uint8_t *p) { return (uint32_t)p[0] | ((uint32_t)p[1] << 8); }

// Q4_K scale and min of sub-block j from the 12 packed bytes S.
__device__ __forceinline__ void q4k_sm(const uint8_t *S, int j, uint32_t &sc, uint32_t &m) {
  if (j < 4) {
    sc = S[j] & 63u;
    m = S[j + 4] & 63u;
  } else {
    sc = (S[j + 4] & 15u) | ((uint32_t)(S[j - 4] >> 6) << 4);
    m = (uint32_t)(S[j + 4] >> 4) | ((uint32_t)(S[j] >> 6) << 4);
  }
}

// Exact products: d*sc (<= 17 bits) times q (4 bits) and dmin*m (<= 17 bits) are exact in fp32,
// so the single subtraction is the only rounding, whatever the association or contraction.
__device__ __forceinline__ float q4k_value(float d, float dmin, uint32_t sc, uint32_t m, uint32_t q) {
  return (d * (float)sc) * (float)q - dmin * (float)m;
}

__device__ float weight_at(int fmt, const uint8_t *row, int64_t i) {
  if (fmt == FMT_Q4_K) {
    const uint8_t *b = row + (i >> 8) * 144;
    const int r = (int)(i & 255), j = r >> 5, c = r >> 6, o = r & 63;
    uint32_t sc, m;
    q4k_sm(b + 4, j, sc, m);
    const uint32_t q = o < 32 ? (b[16 + 32 * c + o] & 15u) : (uint32_t)(b[16 + 32 * c + o - 32] >> 4);
    return q4k_value(half_bits_to_float(rd16(b)), half_bits_to_float(rd16(b + 2)), sc, m, q);
  }
  if (fmt == FMT_Q6_K) {
    const uint8_t *b = row + (i >> 8) * 210;
    const int r = (int)(i & 255), h = r >> 7, g = (r >> 5) & 3, l = r & 31;
    const uint8_t qlb = b[64 * h + l + 32 * (g & 1)];
    const uint32_t lo = g < 2 ? (qlb & 15u) : (uint32_t)(qlb >> 4);
    const uint32_t hi = (b[128 + 32 * h + l] >> (2 * g)) & 3u;
    const int q = (int)(lo | (hi << 4)) - 32;
    const float sc = (float)(int8_t)b[192 + (r >> 4)];
    return (half_bits_to_float(rd16(b + 208)) * sc) * (float)q;
  }
  if (fmt == FMT_Q5_K) {
    const uint8_t *b = row + (i >> 8) * 176;
    const int r = (int)(i & 255), j = r >> 5, c = r >> 6, o = r & 63, l = r & 31;
    uint32_t sc, m;
    q4k_sm(b + 4, j, sc, m);
    const uint32_t lo = o < 32 ? (b[48 + 32 * c + o] & 15u) : (uint32_t)(b[48 + 32 * c + o - 32] >> 4);
    const uint32_t q = lo | (((uint32_t)(b[16 + l] >> j) & 1u) << 4);
    // d*sc*q (<= 17 + 5 bits) and dmin*m are exact in fp32: one rounding, in the subtraction
    return (half_bits_to_float(rd16(b)) * (float)sc) * (float)q -
           half_bits_to_float(rd16(b + 2)) * (float)m;
  }
  if (fmt == FMT_Q4_0) {
    const uint8_t *b = row + (i >> 5) * 18;
    const int r = (int)(i & 31);
    const uint32_t q = r < 16 ? (b[2 + r] & 15u) : (uint32_t)(b[2 + r - 16] >> 4);
    return half_bits_to_float(rd16(b)) * (float)((int)q - 8);
  }
  const uint8_t *b = row + (i >> 5) * 34;
  return half_bits_to_float(rd16(b)) * (float)(int8_t)b[2 + (i & 31)];
}

// ---- dequantization ----------------------------------------------------------------------------
// One thread per 32 consecutive weights of a row: k/32 threads per row.

template <bool BF16>
__global__ __launch_bounds__(256) void k_dequant(int fmt, const uint8_t *__restrict__ w,
                                                 int64_t row_bytes, int64_t n, int64_t k,
                                                 void *__restrict__ out) {
  const int64_t per_row = k >> 5;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n * per_row) return;
  const int64_t row = gid / per_row, seg = gid - row * per_row;
  const uint8_t *rp = w + row * row_bytes;
  float v[32];
  if (fmt == FMT_Q4_K) {
    // the whole segment is one sub-block: decode its scale/min once
    const uint8_t *b = rp + (seg >> 3) * 144;
    const int j = (int)(seg & 7), c = j >> 1;
    uint32_t sc, m;
    q4k_sm(b + 4, j, sc, m);
    const float d = half_bits_to_float(rd16(b)), dmin = half_bits_to_float(rd16(b + 2));
    const u32x4 *qp = reinterpret_cast<const u32x4 *>(b + 16 + 32 * c);
    const u32x4 q0 = qp[0], q1 = qp[1];
    const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    const int shift = (j & 1) ? 4 : 0;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const uint32_t q = (qw[e >> 2] >> (8 * (e & 3) + shift)) & 15u;
      v[e] = q4k_value(d, dmin, sc, m, q);
    }
  } else {
#pragma unroll 4
    for (int e = 0; e < 32; ++e) v[e] = weight_at(fmt, rp, seg * 32 + e);
  }
  if (BF16) {
    uint32_t *o = reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(out) + row * k + seg * 32);
#pragma unroll
    for (int e = 0; e < 16; ++e)
      o[e] = (uint32_t)float_to_bf16_rne(v[2 * e]) | ((uint32_t)float_to_bf16_rne(v[2 * e + 1]) << 16);
  } else {
    float *o = static_cast<float *>(out) + row * k + seg * 32;
#pragma unroll
    for (int e = 0; e < 32; ++e) o[e] = v[e];
  }
}

int launch_dequant(int fmt, const void *w, int64_t n, int64_t k, int out_type, void *out,
                   hipStream_t s) {
  const int64_t threads = n * (k >> 5);
  if (threads == 0) return 0;
  const int64_t rb = k / fmt_block_weights(fmt) * fmt_block_bytes(fmt);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (out_type == 1)
    hipLaunchKernelGGL(k_dequant<true>, grid, block, 0, s, fmt, (const uint8_t *)w, rb, n, k, out);
  else
    hipLaunchKernelGGL(k_dequant<false>, grid, block, 0, s, fmt, (const uint8_t *)w, rb, n, k, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ---- dense GEMV --------------------------------------------------------------------------------
// Work decomposition: the rows are cut into groups of 64 (one lane per row) and the k range into
// `ksplit` slices of `upk` units; one workgroup per (row group, slice). Inside a workgroup the
// waves split the slice further and combine their partial sums through LDS in wave order. When
// ksplit > 1 each workgroup stores its partial sums to the workspace; the last workgroup of a row
// group to arrive (counted with a device-scope atomic) adds the slices in slice order. Which
// workgroup does the adding does not change the order of the additions, so the result is
// deterministic. The counters (Arrivals: tagged with the launch's token, so the workspace may hold
// anything beforehand) live in the first kCounterBytes of the workspace, apart from the partial
// sums.

struct GemvPlan {
  int rowgroups, ksplit, upk, waves, upw;
};

GemvPlan plan_gemv(int64_t n, int64_t k, bool split_allowed) {
  const int target_wg = knob(TQ_KNOB_GEMV_TARGET_WG, 1024);
  const int max_waves = knob(TQ_KNOB_GEMV_MAX_WAVES, 4);
  GemvPlan p;
  const int units = (int)(k / 256);
  p.rowgroups = (int)((n + 63) / 64);
  int ks = split_allowed ? (target_wg + p.rowgroups - 1) / p.rowgroups : 1;
  ks = ks < 1 ? 1 : ks > units ? units : ks;
  p.upk = (units + ks - 1) / ks;
  p.ksplit = (units + p.upk - 1) / p.upk;
  int w = p.upk < max_waves ? p.upk : max_waves;
  w = w < 1 ? 1 : w > 8 ? 8 : w;
  p.upw = (p.upk + w - 1) / w;
  p.waves = (p.upk + p.upw - 1) / p.upw;
  return p;
}

static constexpr size_t kCounterBytes = 65536;  // one 8-byte counter per row group

// Workspace of the int8 matrix-core path: counters, then the k slices' partial sums.
static size_t i8_ws_bytes(int fmt, int64_t rows, int64_t k, int64_t batch) {
  return i8_gemv_ok(fmt, k, batch) ? kCounterBytes + i8_workspace_bytes(rows, k) : 0;
}

// The int8 path runs when its workspace is there and x is 16-byte aligned.
static bool use_i8(int fmt, int64_t rows, int64_t k, const float *x, int64_t batch,
                   const void *ws, size_t ws_bytes) {
  const size_t need = i8_ws_bytes(fmt, rows, k, batch);
  return need && ws != nullptr && ws_bytes >= need && ((uintptr_t)x & 15) == 0 &&
         rows < (1ll << 30);
}

// Batch-1 Q6_K shapes that the fp16 matrix-core kernel takes (rows of whole pairs of blocks) in
// one k slice, and single products of longer rows in k slices (with the workspace).
static bool mf6_ok(int fmt, int64_t k, const float *x, int64_t batch) {
  return fmt == FMT_Q6_K && batch == 1 && ((uintptr_t)x & 15) == 0 && mf_gemv_ok(FMT_Q6_K, k);
}
// (Q4_K rows of 16384 and more: in k slices unless TQ_KNOB_GEMV_MF is 1, then the int8 kernel)
static size_t mf6s_ws_bytes(int fmt, int64_t rows, int64_t k, int64_t batch) {
  const bool q4 = fmt == FMT_Q4_K && knob(TQ_KNOB_GEMV_MF, 2) == 2;
  if ((fmt != FMT_Q6_K && !q4) || batch != 1 || !mf_gemv_sliced(fmt, k)) return 0;
  return kCounterBytes + mf_workspace_bytes(fmt, rows, k);
}
static bool use_mf6s(int fmt, int64_t rows, int64_t k, const float *x, int64_t batch,
                     const void *ws, size_t ws_bytes) {
  const size_t need = mf6s_ws_bytes(fmt, rows, k, batch);
  return need && ws != nullptr && ws_bytes >= need && ((uintptr_t)x & 15) == 0;
}

// Q6_K / Q8_0 batches on the fp32 matrix cores: workspace (counters, slice sums) when k is sliced.
static size_t f32m_ws_bytes(int fmt, int64_t rows, int64_t k, int64_t batch) {
  if (!f32m_ok(fmt, k, batch)) return 0;
  const size_t p = f32m_workspace_bytes(rows, k);
  return p ? kCounterBytes + p : 0;
}

static bool use_f32m(int fmt, int64_t rows, int64_t k, const float *x, int64_t batch,
                     const void *ws, size_t ws_bytes) {
  if (!f32m_ok(fmt, k, batch) || ((uintptr_t)x & 15) != 0 || rows >= (1ll << 30)) return false;
  const size_t need = f32m_ws_bytes(fmt, rows, k, batch);
  return need == 0 || (ws != nullptr && ws_bytes >= need);
}

static int launch_f32m(int fmt, const KlMap &m, int64_t k, const float *x, int64_t batch,
                       void *ws, hipStream_t s) {
  return launch_gemm_f32m(fmt, m, k, x, batch, ws ? (float *)((char *)ws + kCounterBytes) : nullptr,
                          (unsigned long long *)ws, (int)(kCounterBytes / 8), s);
}


static int launch_i8(int fmt, const KlMap &m, int64_t k, const float *x, void *ws, hipStream_t s) {
  return launch_gemv_i8(fmt, m, k, x, (float *)((char *)ws + kCounterBytes), (unsigned long long *)ws,
                        (int)(kCounterBytes / 8), s);
}

// Workspace of the fp16 matrix-core path for 2..32 tokens: counters, split x, slice sums.
static size_t qmm_workspace_bytes(int fmt, int64_t rows, int64_t k, int64_t batch, bool swiglu) {
  return qmm_dense_ok(fmt, k, batch) ? kCounterBytes + qmm_dense_bytes(rows, k, batch, swiglu) : 0;
}

static bool use_qmm(int fmt, int64_t rows, int64_t k, const float *x, int64_t batch,
                    const void *ws, size_t ws_bytes, bool swiglu) {
  const size_t need = qmm_workspace_bytes(fmt, rows, k, batch, swiglu);
  return need && ws != nullptr && ws_bytes >= need && ((uintptr_t)x & 15) == 0 &&
         rows < (1ll << 30);
}

// Counters and partial sums of the split-k GEMV (0 when it does not split).
static size_t split_workspace_bytes(int fmt, int64_t n, int64_t k) {
  if (!gemv_fast_shape(fmt, k)) return 0;
  const GemvPlan p = plan_gemv(n, k, true);
  if (p.ksplit == 1 || (size_t)p.rowgroups * 8 > kCounterBytes) return 0;
  // counters, then partial sums for up to 8 tokens
  return kCounterBytes + (size_t)p.rowgroups * p.ksplit * 8 * 64 * 4;
}

static size_t max3(size_t a, size_t b, size_t c) { return a > b ? (a > c ? a : c) : (b > c ? b : c); }

size_t gemv_workspace_bytes(int fmt, int64_t n, int64_t k, int64_t batch) {
  const size_t a = max3(split_workspace_bytes(fmt, n, k), i8_ws_bytes(fmt, n, k, batch),
                        qmm_workspace_bytes(fmt, n, k, batch, false));
  const size_t b = f32m_ws_bytes(fmt, n, k, batch), c = mf6s_ws_bytes(fmt, n, k, batch);
  return max3(a, b, c);
}

static QmmDense dense_map(int nparts, const void *const *w, const int64_t *n, float *const *y,
                          int64_t rb) {
  QmmDense m{};
  for (int p = 0; p < nparts; ++p) {
    m.w[p] = (const uint8_t *)w[p];
    m.y[p] = y[p];
    m.cum[p + 1] = m.cum[p] + (int)n[p];
  }
  m.nparts = nparts;
  m.row_bytes = rb;
  return m;
}

template <int FMT, int NT>
__global__ __launch_bounds__(512) void k_gemv(const uint8_t *__restrict__ w, int64_t row_bytes,
                                              int n, int units, int ksplit, int upk, int upw,
                                              const float *__restrict__ x, int64_t ldx,
                                              float *__restrict__ y, int64_t ldy,
                                              float *__restrict__ partial, Arrivals arr) {
  extern __shared__ float lds[];
  __shared__ int is_last;
  // blockIdx -> (row group, slice): XCD x takes the row groups r = x (mod 8) and runs all slices
  // of one group back to back (the cache lines two neighbouring slices of a row share are then
  // fetched once, into that XCD's L2)
  const int xcd = blockIdx.x & 7, bi = blockIdx.x >> 3;
  const int rg = xcd + 8 * (bi / ksplit), ks = bi % ksplit;
  if (rg * 64 >= n) return;
  const int row0 = rg * 64;
  const int ku0 = ks * upk, ku1 = min(ku0 + upk, units);
  const float *xr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) xr[t] = x + t * ldx;
  gemv_tile<FMT, NT>(w, row_bytes, n, row0, ku0, ku1, upw, xr, lds);
  if (ksplit == 1) {
    for (int i = threadIdx.x; i < NT * 64; i += blockDim.x) {
      const int t = i >> 6, l = i & 63;
      if (row0 + l < n) y[t * ldy + row0 + l] = lds[i];
    }
    return;
  }
  // k split: store this slice's sums; the last workgroup of the row group to finish adds all
  // slices in slice order and zeroes the row group's counter. The partial sums are written and read with device-coherent (sc1)
  // accesses, and every store has completed (s_waitcnt vmcnt(0)) before the workgroup's arrival
  // is counted, so the last workgroup sees all of them; no cache writeback or invalidation is
  // needed.
  float *mine = partial + ((int64_t)rg * ksplit + ks) * NT * 64;
  for (int i = threadIdx.x; i < NT * 64; i += blockDim.x)
    __hip_atomic_store(mine + i, lds[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's stores have completed
  __syncthreads();
  if (threadIdx.x == 0) is_last = arrive_last(arr, rg, (unsigned)ksplit);
  __syncthreads();
  if (!is_last) return;
  const float *base = partial + (int64_t)rg * ksplit * NT * 64;
  for (int i = threadIdx.x; i < NT * 64; i += blockDim.x) {
    const int t = i >> 6, l = i & 63;
    float s = 0.f;
    for (int q0 = 0; q0 < ksplit; q0 += 8) {  // up to 8 loads in flight, added in slice order
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[j] = q0 + j < ksplit ? __hip_atomic_load(base + (q0 + j) * NT * 64 + i, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)
                               : 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (q0 + j < ksplit) s += v[j];
    }
    if (row0 + l < n) y[t * ldy + row0 + l] = s;
  }
  if (threadIdx.x == 0) done_arrivals(arr, rg);
}

// Batch-1 Q4_K GEMV, lanes along k (see tq_gemv_core.h). A lane group of 64 / G lanes covers all
// of k (G > 1 only when k fits in 16 / G blocks, so that short rows leave no lane idle); group g of
// a pass over rows r0.. computes rows r0 + g R .. r0 + g R + R - 1.

template <int R, int G, class Map>
__device__ __forceinline__ void kl_rows(const u32x4 (&v)[R][3], const float (&xv)[64], float sx_lo,
                                        float sx_hi, const Q4kField &f0, const Q4kField &f1,
                                        int r0, int re, float (*red)[G * R],
                                        const Map &m) {
  constexpr int L = 64 / G;  // lanes per group
  static_assert(L >= R, "a group needs at least one lane per row");
  const int lane = threadIdx.x & 63, wave = wave_index(), nw = blockDim.x >> 6;
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = kl_group_dot(v[r], xv, sx_lo, sx_hi, f0, f1);
  // across the group's lanes: each step halves the rows a lane keeps and adds its partner's half
  int cnt = R;
#pragma unroll
  for (int d = L / 2; d >= 1; d >>= 1) {
    if (cnt > 1) {
      const bool upper = (lane & d) != 0;
      const int h = cnt >> 1;
#pragma unroll
      for (int i = 0; i < R / 2; ++i)
        if (i < h) {
          const float send = upper ? acc[i] : acc[i + h];
          const float keep = upper ? acc[i + h] : acc[i];
          acc[i] = keep + xor_recv(send, d);
        }
      cnt = h;
    } else {
      acc[0] += xor_recv(acc[0], d);
    }
  }
  // lane l of group g now holds row g R + sum_s bit(l, log2(L) - 1 - s) * R / 2^(s+1); lanes with
  // zero low bits store it
  int row = (lane / L) * R;
#pragma unroll
  for (int sidx = 0, half = R >> 1; half >= 1; ++sidx, half >>= 1)
    if (lane & ((L / 2) >> sidx)) row += half;
  const bool holder = (lane & (L / R - 1)) == 0;
  if (nw == 1) {  // one wave: its sums are the rows' totals, stored by the lanes that hold them
    if (m.swiglu) {  // the up row (row + 1) sits L / R lanes away (the butterfly's last halving)
      const float u = xor_recv(acc[0], L / R);
      if (holder && (row & 1) == 0 && r0 + row < re)
        gstore(m.swiglu_out((r0 + row) >> 1), silu_mul(acc[0], u));
    } else if (holder && r0 + row < re) {
      m.put(r0 + row, acc[0]);
    }
    return;
  }
  if (holder) red[wave][row] = acc[0];
  __syncthreads();
  if (m.swiglu) {  // rows (gate r, up r) pairs; r0 and re are even
    const int i = 2 * (int)threadIdx.x;
    if (i < G * R && r0 + i < re) {
      float g = 0.f, u = 0.f;
      for (int q = 0; q < nw; ++q) {
        g += red[q][i];
        u += red[q][i + 1];
      }
      gstore(m.swiglu_out((r0 + i) >> 1), silu_mul(g, u));
    }
  } else if (threadIdx.x < G * R && r0 + (int)threadIdx.x < re) {
    float s = 0.f;
    for (int q = 0; q < nw; ++q) s += red[q][threadIdx.x];
    m.put(r0 + threadIdx.x, s);
  }
  __syncthreads();
}

// Rows [rb, re) of the workgroup, G R per pass, loading the next pass's rows while it computes the
// current ones (two register buffers used in turn).
template <int R, int G, class Map>
__device__ __forceinline__ void kl_body(const Map &m, int nblk, int rb, int re,
                                        const float *__restrict__ x, float (*red)[G * R]) {
  constexpr int L = 64 / G, P = G * R;
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int b = (L / 4) * wave + ((lane & (L - 1)) >> 2), c = lane & 3, g = lane / L;
  const bool valid = b < nblk;
  const int bb = valid ? b : nblk - 1;
  const int boff = bb * 144;
  u32x4 va[R][3], vb[R][3];
  // the first rows' weights are requested before the activations
  if (rb < re) kl_load_rows<R, Map>(m, rb + g * R, boff, c, va);
  float xv[64];
  {
    const float4 *xp = reinterpret_cast<const float4 *>(x + 256 * bb + 64 * c);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 t = xp[i];
      xv[4 * i] = valid ? t.x : 0.f;
      xv[4 * i + 1] = valid ? t.y : 0.f;
      xv[4 * i + 2] = valid ? t.z : 0.f;
      xv[4 * i + 3] = valid ? t.w : 0.f;
    }
  }
  float sx_lo = 0.f, sx_hi = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    sx_lo += xv[i];
    sx_hi += xv[32 + i];
  }
  const Q4kField f0 = q4k_field(2 * c), f1 = q4k_field(2 * c + 1);
  for (int r0 = rb; r0 < re; r0 += 2 * P) {
    if (r0 + P < re) kl_load_rows<R, Map>(m, r0 + P + g * R, boff, c, vb);
    kl_rows<R, G, Map>(va, xv, sx_lo, sx_hi, f0, f1, r0, re, red, m);
    if (r0 + P >= re) break;
    if (r0 + 2 * P < re) kl_load_rows<R, Map>(m, r0 + 2 * P + g * R, boff, c, va);
    kl_rows<R, G, Map>(vb, xv, sx_lo, sx_hi, f0, f1, r0 + P, re, red, m);
  }
}

// Batch-1 Q4_K GEMV, lanes along k (see tq_gemv_core.h). Workgroup = ceil(nblk / 16) waves
// covering all of k; it computes rows [blockIdx.x * rows_per_wg, ...) R at a time, loading the
// next R rows while it computes the current ones (two register buffers used in turn).
template <int R, int G>
__global__ __launch_bounds__(512) void k_gemv_kl(KlMap m, int nblk, int rows_per_wg,
                                                 const float *__restrict__ x) {
  __shared__ float red[8][G * R];
  const int rb = blockIdx.x * rows_per_wg, re = min(rb + rows_per_wg, m.total);
  kl_body<R, G, KlMap>(m, nblk, rb, re, x, red);
}

// The combine of a one-token layer inside the down launch: each workgroup counts itself on its
// row range's counter once its sums are stored (device-scope stores, awaited before counting);
// the last of the active slots to arrive adds, for each of the range's rows, the slots in order
// and then the shared expert, exactly as the combine kernel does. Counters start at zero (the
// gate/up launch of the same call clears them); nothing waits on another workgroup.
__device__ __forceinline__ void moe_kl_combine(const MoeKlArgs &a, int rb, int re, int rr) {
  __shared__ int last;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this workgroup's sums are stored
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(&a.ctr[rr], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           (unsigned)(*a.n_active - 1);
  __syncthreads();
  if (!last) return;
  for (int c = rb + (int)threadIdx.x; c < re; c += blockDim.x) a.fuse_y[c] = moe_combine_value(a, c);
}

// The same kernel over the experts of a one-token MoE step: workgroup b works on active slot
// slot0 + b / wgs_per_slot (every active expert has that one token). gate/up: the expert's
// gate and up rows interleaved with the SwiGLU in the epilogue, x = the token's activations,
// h[position][ffn] out; down: x = h[position], o[position][hidden] out.
template <int R, int G>
__global__ __launch_bounds__(512) void k_moe_kl(MoeKlArgs a, int nblk, int rows_per_wg,
                                                int wgs_per_slot) {
  __shared__ float red[8][G * R];
  if (a.nctr > 0 && blockIdx.x == 0)  // gate/up of a fused one-token call: clear the counters
    for (int i = (int)threadIdx.x; i < a.nctr; i += blockDim.x)
      __hip_atomic_store(a.ctr + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int slot = a.slot0 + (int)blockIdx.x / wgs_per_slot;
  if (slot >= *a.n_active) return;
  const int e = a.act[slot], p = a.act[a.act_stride + slot];
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
  int64_t xrow = p;
  if (a.gate_up) xrow = p >= a.Tk ? p - a.Tk : a.pairs[p] / a.topk;
  const int rb = ((int)blockIdx.x % wgs_per_slot) * rows_per_wg;
  const int re = min(rb + rows_per_wg, a.rows);
  kl_body<R, G, MoeRowMap>(m, nblk, rb, re, a.x + xrow * a.ldx, red);
  if (a.fuse_y != nullptr) moe_kl_combine(a, rb, re, (int)blockIdx.x % wgs_per_slot);
}

// Fallback for shapes whose rows are not dword aligned (Q6_K with k % 512 != 0, Q8_0 with
// k % 256 != 0): one thread per (row, token), weights decoded one by one.
__global__ __launch_bounds__(256) void k_gemv_generic(int fmt, const uint8_t *__restrict__ w,
                                                      int64_t row_bytes, int n, int64_t k,
                                                      const float *__restrict__ x, int batch,
                                                      float *__restrict__ y) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)n * batch) return;
  const int t = (int)(gid / n), r = (int)(gid - (int64_t)t * n);
  const uint8_t *rp = w + (int64_t)r * row_bytes;
  const float *xt = x + (int64_t)t * k;
  float s = 0.f;
  for (int64_t i = 0; i < k; ++i) s = __builtin_fmaf(weight_at(fmt, rp, i), xt[i], s);
  y[(int64_t)t * n + r] = s;
}

template <int FMT, int NT>
static void launch_gemv_nt(const uint8_t *w, int64_t rb, int n, int units, const GemvPlan &p,
                           const float *x, int64_t ldx, float *y, int64_t ldy, float *partial,
                           unsigned long long *counters, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((k_gemv<FMT, NT>), dim3((unsigned)((p.rowgroups + 7) / 8 * 8 * p.ksplit)),
                     dim3(64 * p.waves),
                     lds, s, w, rb, n, units, p.ksplit, p.upk, p.upw, x, ldx, y, ldy, partial,
                     Arrivals{counters, counters ? call_tag() : 0ull});
}

template <int FMT>
static int launch_gemv_fmt(const uint8_t *w, int64_t rb, int n, int64_t k, const float *x,
                           int batch, float *y, void *ws, size_t ws_bytes, hipStream_t s) {
  const int units = (int)(k / 256);
  const size_t need = split_workspace_bytes(FMT, n, k);
  const bool split = ws != nullptr && need > 0 && ws_bytes >= need;
  const GemvPlan p = plan_gemv(n, k, split);
  unsigned long long *counters = p.ksplit > 1 ? static_cast<unsigned long long *>(ws) : nullptr;
  float *partial =
      p.ksplit > 1 ? reinterpret_cast<float *>(static_cast<char *>(ws) + kCounterBytes) : nullptr;
  const int max_floats = 65536 / 4;
  for (int t0 = 0; t0 < batch;) {
    int nt = batch - t0 < 8 ? batch - t0 : 8;
    while (nt > 1 && gemv_tile_lds_floats<FMT>(nt, p.upk, p.waves) > max_floats) --nt;
    if (gemv_tile_lds_floats<FMT>(nt, p.upk, p.waves) > max_floats) return -2;
    const size_t lds = (size_t)4 * gemv_tile_lds_floats<FMT>(nt, p.upk, p.waves);
    const float *xt = x + (int64_t)t0 * k;
    float *yt = y + (int64_t)t0 * n;
    if constexpr (FMT == FMT_Q5_K) {  // one token per pass (see unit_dot for Q5_K)
      nt = 1;
      launch_gemv_nt<FMT, 1>(w, rb, n, units, p, xt, k, yt, n, partial, counters,
                             (size_t)4 * gemv_tile_lds_floats<FMT>(1, p.upk, p.waves), s);
    } else {
      switch (nt) {
#define TQ_CASE(NTV) \
  case NTV: launch_gemv_nt<FMT, NTV>(w, rb, n, units, p, xt, k, yt, n, partial, counters, lds, s); break;
        TQ_CASE(1) TQ_CASE(2) TQ_CASE(3) TQ_CASE(4) TQ_CASE(5) TQ_CASE(6) TQ_CASE(7) TQ_CASE(8)
#undef TQ_CASE
      }
    }
    if (hipGetLastError() != hipSuccess) return -1;
    t0 += nt;
  }
  return 0;
}

// Batch-1 Q4_K shapes that the lanes-along-k kernel takes.
static bool klane_ok(int fmt, int64_t k, const float *x, int64_t batch) {
  const int kl_mode = knob(TQ_KNOB_GEMV_KLANE, 1);
  return fmt == FMT_Q4_K && batch == 1 && kl_mode && ((uintptr_t)x & 15) == 0 && k % 256 == 0 &&
         k <= 8 * 4096;
}


// Lane groups per wave: 4 for k <= 1024, 2 for k <= 2048, else 1 (TQ_KNOB_KL_GROUPS = 1 turns them off).
static int kl_groups(int nblk) {
  const int allow = knob(TQ_KNOB_KL_GROUPS, 4);
  const int g = nblk <= 4 ? 4 : nblk <= 8 ? 2 : 1;
  return g < allow ? g : allow >= 4 ? 4 : allow >= 2 ? 2 : 1;
}

// Workgroup rows: whole passes of G R rows, as many as bring the launch near `target` waves.
static int kl_rows_per_wg(int64_t rows, int waves, int pass, int target) {
  int64_t chunks = (rows * waves + (int64_t)pass * target - 1) / ((int64_t)pass * target);
  return pass * (int)(chunks < 1 ? 1 : chunks);  // even: SwiGLU pairs never straddle two workgroups
}

template <int R, int G>
static void launch_kl_rg(const KlMap &m, int nblk, int waves, int target, const float *x,
                         hipStream_t s) {
  const int rows_per_wg = kl_rows_per_wg(m.total, waves, G * R, target);
  const int grid = (m.total + rows_per_wg - 1) / rows_per_wg;
  hipLaunchKernelGGL((k_gemv_kl<R, G>), dim3((unsigned)grid), dim3(64 * waves), 0, s, m, nblk,
                     rows_per_wg, x);
}

static int launch_kl(const KlMap &m, int64_t k, const float *x, hipStream_t s) {
  if (mf_gemv_ok(FMT_Q4_K, k)) return launch_gemv_mf(FMT_Q4_K, m, k, x, nullptr, nullptr, 0, s);
  const int nblk = (int)(k / 256);
  const int waves = (nblk + 15) / 16;
  const int kl_rows_env = knob(TQ_KNOB_KL_ROWS, 4);
  const int target = knob(TQ_KNOB_KL_TARGET_WAVES, 2048);
  const int G = kl_groups(nblk);
  if (kl_rows_env == 2)
    launch_kl_rg<2, 1>(m, nblk, waves, target, x, s);
  else if (kl_rows_env == 8)
    launch_kl_rg<8, 1>(m, nblk, waves, target, x, s);
  else if (G == 4)
    launch_kl_rg<4, 4>(m, nblk, waves, target, x, s);
  else if (G == 2)
    launch_kl_rg<4, 2>(m, nblk, waves, target, x, s);
  else
    launch_kl_rg<4, 1>(m, nblk, waves, target, x, s);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

bool moe_klane_ok(int fmt, int64_t hidden, int64_t ffn, int64_t tokens) {
  const int kl_mode = knob(TQ_KNOB_GEMV_KLANE, 1);
  return fmt == FMT_Q4_K && tokens == 1 && kl_mode && hidden % 256 == 0 && ffn % 256 == 0 &&
         hidden <= 8 * 4096 && ffn <= 8 * 4096;
}

template <int G>
static void launch_moe_kl_g(const MoeKlArgs &a, int nblk, int waves, int nslots, int target,
                            hipStream_t s) {
  const int rows_per_wg = kl_rows_per_wg((int64_t)a.rows * nslots, waves, G * 4, target);
  const int wgs_per_slot = (a.rows + rows_per_wg - 1) / rows_per_wg;
  hipLaunchKernelGGL((k_moe_kl<4, G>), dim3((unsigned)(nslots * wgs_per_slot)), dim3(64 * waves), 0,
                     s, a, nblk, rows_per_wg, wgs_per_slot);
}

int launch_moe_kl(const MoeKlArgs &a, int64_t k, int nslots, hipStream_t s) {
  const int nblk = (int)(k / 256);
  const int waves = (nblk + 15) / 16;
  const int target = knob(TQ_KNOB_KL_TARGET_WAVES, 2048);
  const int G = kl_groups(nblk);
  if (G == 4)
    launch_moe_kl_g<4>(a, nblk, waves, nslots, target, s);
  else if (G == 2)
    launch_moe_kl_g<2>(a, nblk, waves, nslots, target, s);
  else
    launch_moe_kl_g<1>(a, nblk, waves, nslots, target, s);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

bool gemv_fast_shape(int fmt, int64_t k) {
  if (fmt == FMT_Q6_K) return k % 512 == 0;  // 210 * (k/256) bytes per row is dword aligned
  // Q4_K, Q5_K: whole blocks; Q8_0, Q4_0: whole 8-block units; rows 16-byte aligned
  return k % 256 == 0;
}

int launch_gemv(int fmt, const void *w, int64_t n, int64_t k, const float *x, int64_t batch,
                float *y, void *ws, size_t ws_bytes, hipStream_t s) {
  const int64_t rb = k / fmt_block_weights(fmt) * fmt_block_bytes(fmt);
  const uint8_t *wb = (const uint8_t *)w;
  if (!gemv_fast_shape(fmt, k)) {
    const int64_t threads = n * batch;
    hipLaunchKernelGGL(k_gemv_generic, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                       fmt, wb, rb, (int)n, k, x, (int)batch, y);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  if (use_qmm(fmt, n, k, x, batch, ws, ws_bytes, false)) {
    const void *wp[1] = {w};
    float *yp[1] = {y};
    const QmmDense m = dense_map(1, wp, &n, yp, rb);
    return launch_qmm_dense(m, k, x, batch, (char *)ws + kCounterBytes,
                            (unsigned long long *)ws, (int)(kCounterBytes / 8), s);
  }
  if (use_f32m(fmt, n, k, x, batch, ws, ws_bytes)) {
    KlMap m{};
    m.w[0] = wb;
    m.y[0] = y;
    m.cum[1] = (int)n;
    m.nparts = 1;
    m.total = (int)n;
    m.row_bytes = rb;
    return launch_f32m(fmt, m, k, x, batch, ws, s);
  }
  const bool mf6s = use_mf6s(fmt, n, k, x, batch, ws, ws_bytes) && n < (1ll << 30);
  const bool i8 = !mf6s && use_i8(fmt, n, k, x, batch, ws, ws_bytes);
  const bool mf6 = mf6_ok(fmt, k, x, batch) && n < (1ll << 30);
  if (i8 || klane_ok(fmt, k, x, batch) || mf6 || mf6s) {
    KlMap m{};
    m.w[0] = wb;
    m.y[0] = y;
    m.cum[1] = (int)n;
    m.nparts = 1;
    m.total = (int)n;
    m.row_bytes = rb;
    if (i8) return launch_i8(fmt, m, k, x, ws, s);
    if (mf6) return launch_gemv_mf(FMT_Q6_K, m, k, x, nullptr, nullptr, 0, s);
    if (mf6s)
      return launch_gemv_mf(fmt, m, k, x, (float *)((char *)ws + kCounterBytes),
                            (unsigned long long *)ws, (int)(kCounterBytes / 8), s);
    return launch_kl(m, k, x, s);
  }
  switch (fmt) {
    case FMT_Q4_K: return launch_gemv_fmt<FMT_Q4_K>(wb, rb, (int)n, k, x, (int)batch, y, ws, ws_bytes, s);
    case FMT_Q6_K: return launch_gemv_fmt<FMT_Q6_K>(wb, rb, (int)n, k, x, (int)batch, y, ws, ws_bytes, s);
    case FMT_Q5_K: return launch_gemv_fmt<FMT_Q5_K>(wb, rb, (int)n, k, x, (int)batch, y, ws, ws_bytes, s);
    case FMT_Q4_0: return launch_gemv_fmt<FMT_Q4_0>(wb, rb, (int)n, k, x, (int)batch, y, ws, ws_bytes, s);
    default: return launch_gemv_fmt<FMT_Q8_0>(wb, rb, (int)n, k, x, (int)batch, y, ws, ws_bytes, s);
  }
}

size_t gemv_multi_workspace_bytes(int fmt, int nparts, const int64_t *n, int64_t k,
                                  int64_t batch) {
  size_t b = 0;
  int64_t total = 0;
  for (int p = 0; p < nparts; ++p) {
    const size_t q = gemv_workspace_bytes(fmt, n[p], k, batch);
    b = q > b ? q : b;
    total += n[p];
  }
  const size_t fused = qmm_workspace_bytes(fmt, total, k, batch, false);
  const size_t i8 = i8_ws_bytes(fmt, total, k, batch);
  const size_t f32m = f32m_ws_bytes(fmt, total, k, batch);
  const size_t r = max3(b, fused, i8);
  return r > f32m ? r : f32m;
}

int launch_gemv_multi(int fmt, int nparts, const void *const *w, const int64_t *n, float *const *y,
                      int64_t k, const float *x, int64_t batch, void *ws, size_t ws_bytes,
                      hipStream_t s) {
  int64_t total = 0;
  for (int p = 0; p < nparts; ++p) total += n[p];
  if (nparts <= 4 && use_qmm(fmt, total, k, x, batch, ws, ws_bytes, false)) {
    const QmmDense m = dense_map(nparts, w, n, y, k / fmt_block_weights(fmt) * fmt_block_bytes(fmt));
    return launch_qmm_dense(m, k, x, batch, (char *)ws + kCounterBytes,
                            (unsigned long long *)ws, (int)(kCounterBytes / 8), s);
  }
  const bool f32m = use_f32m(fmt, total, k, x, batch, ws, ws_bytes);
  const bool i8 = !f32m && use_i8(fmt, total, k, x, batch, ws, ws_bytes);
  const bool mf6 = !f32m && mf6_ok(fmt, k, x, batch);
  if ((f32m || i8 || klane_ok(fmt, k, x, batch) || mf6) && nparts <= 4 && total < (1ll << 30)) {
    KlMap m{};
    for (int p = 0; p < nparts; ++p) {
      m.w[p] = (const uint8_t *)w[p];
      m.y[p] = y[p];
      m.cum[p + 1] = m.cum[p] + (int)n[p];
    }
    m.nparts = nparts;
    m.total = (int)total;
    m.row_bytes = k / fmt_block_weights(fmt) * fmt_block_bytes(fmt);
    if (f32m) return launch_f32m(fmt, m, k, x, batch, ws, s);
    if (i8) return launch_i8(fmt, m, k, x, ws, s);
    if (mf6) return launch_gemv_mf(FMT_Q6_K, m, k, x, nullptr, nullptr, 0, s);
    return launch_kl(m, k, x, s);
  }
  for (int p = 0; p < nparts; ++p) {  // one launch per matrix, in order on the stream
    const int rc = launch_gemv(fmt, w[p], n[p], k, x, batch, y[p], ws, ws_bytes, s);
    if (rc) return rc;
  }
  return 0;
}

// Workspace of tq_gemv_swiglu: none on the fused path; otherwise that of one GEMV followed by the
// gate and up outputs [batch][n] each.
static int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Two-launch path: the split-k GEMV's workspace, then the gate and up outputs.
static size_t swiglu_two_launch_bytes(int fmt, int64_t n, int64_t k, int64_t batch) {
  return (size_t)align_up((int64_t)split_workspace_bytes(fmt, n, k), 256) +
         (size_t)align_up(4 * batch * n, 256) * 2;
}

size_t gemv_swiglu_workspace_bytes(int fmt, int64_t n, int64_t k, int64_t batch, bool fused) {
  const size_t qmm = qmm_workspace_bytes(fmt, n, k, batch, true);
  if (fused) return i8_ws_bytes(fmt, 2 * n, k, batch);
  const size_t two = swiglu_two_launch_bytes(fmt, n, k, batch);
  const size_t f32m = f32m_ws_bytes(fmt, 2 * n, k, batch);
  return max3(qmm, two, f32m);
}

size_t gemv_swiglu_min_workspace_bytes(int fmt, int64_t n, int64_t k, int64_t batch, bool fused) {
  return fused ? 0 : swiglu_two_launch_bytes(fmt, n, k, batch);
}

int launch_gemv_swiglu(int fmt, const void *wg, const void *wu, int64_t n, int64_t k,
                       const float *x, int64_t batch, float *h, void *ws, size_t ws_bytes,
                       hipStream_t s) {
  const int64_t rb = k / fmt_block_weights(fmt) * fmt_block_bytes(fmt);
  if (use_f32m(fmt, 2 * n, k, x, batch, ws, ws_bytes) && n < (1ll << 29)) {
    KlMap m{};
    m.w[0] = (const uint8_t *)wg;
    m.w[1] = (const uint8_t *)wu;
    m.y[0] = h;
    m.nparts = 1;
    m.swiglu = 1;
    m.total = (int)(2 * n);
    m.cum[1] = m.total;
    m.row_bytes = rb;
    return launch_f32m(fmt, m, k, x, batch, ws, s);
  }
  const bool i8 = use_i8(fmt, 2 * n, k, x, batch, ws, ws_bytes);
  const bool mf6 = mf6_ok(fmt, k, x, batch);
  if ((i8 || klane_ok(fmt, k, x, batch) || mf6) && n < (1ll << 29)) {
    KlMap m{};
    m.w[0] = (const uint8_t *)wg;
    m.w[1] = (const uint8_t *)wu;
    m.y[0] = h;
    m.nparts = 1;
    m.swiglu = 1;
    m.total = (int)(2 * n);
    m.cum[1] = m.total;
    m.row_bytes = rb;
    if (i8) return launch_i8(fmt, m, k, x, ws, s);
    if (mf6) return launch_gemv_mf(FMT_Q6_K, m, k, x, nullptr, nullptr, 0, s);
    return launch_kl(m, k, x, s);
  }
  if (use_qmm(fmt, n, k, x, batch, ws, ws_bytes, true)) {
    QmmDense m{};
    m.w[0] = (const uint8_t *)wg;
    m.w[1] = (const uint8_t *)wu;
    m.y[0] = h;
    m.cum[1] = (int)n;
    m.nparts = 1;
    m.swiglu = 1;
    m.row_bytes = rb;
    return launch_qmm_dense(m, k, x, batch, (char *)ws + kCounterBytes,
                            (unsigned long long *)ws, (int)(kCounterBytes / 8), s);
  }
  // two launches through the workspace: its head is the split GEMV's, then gate and up
  const size_t gws = (size_t)align_up((int64_t)split_workspace_bytes(fmt, n, k), 256);
  float *g = (float *)((char *)ws + gws);
  float *u = (float *)((char *)g + align_up(4 * batch * n, 256));
  int rc = launch_gemv(fmt, wg, n, k, x, batch, g, ws, gws, s);
  if (rc) return rc;
  rc = launch_gemv(fmt, wu, n, k, x, batch, u, ws, gws, s);
  if (rc) return rc;
  return launch_swiglu(g, u, batch * n, h, s);
}

bool gemv_swiglu_fused(int fmt, int64_t k, const float *x, int64_t batch) {
  return klane_ok(fmt, k, x, batch) || mf6_ok(fmt, k, x, batch);
}

// ---- SwiGLU ------------------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_swiglu(const float *g, const float *u, int64_t count,
                                                float *h) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
    h[i] = silu_mul(g[i], u[i]);
}

int launch_swiglu(const float *g, const float *u, int64_t count, float *h, hipStream_t s) {
  if (count == 0) return 0;
  int64_t blocks = (count + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_swiglu, dim3((unsigned)blocks), dim3(256), 0, s, g, u, count, h);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace tq
