// tq_dense.hip -- dequantization, dense GEMV and SwiGLU kernels with their host launchers.
#include "tq_gemv_core.h"
#include "tq_launch.h"

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
// ksplit > 1 each workgroup stores its partial sums to the workspace and a second kernel adds the
// slices in slice order, so the result is deterministic (no atomics, nothing to reset between
// calls).

struct GemvPlan {
  int rowgroups, ksplit, upk, waves, upw;
};

static int env_int(const char *name, int dflt) {
  const char *v = getenv(name);
  return v && *v ? atoi(v) : dflt;
}

GemvPlan plan_gemv(int64_t n, int64_t k, bool split_allowed) {
  static const int target_wg = env_int("TQ_GEMV_TARGET_WG", 1024);
  static const int max_waves = env_int("TQ_GEMV_MAX_WAVES", 4);
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

size_t gemv_workspace_bytes(int fmt, int64_t n, int64_t k, int64_t batch) {
  (void)batch;
  if (!gemv_fast_shape(fmt, k)) return 0;
  const GemvPlan p = plan_gemv(n, k, true);
  if (p.ksplit == 1) return 0;
  // partial sums for up to 8 tokens
  return (size_t)p.rowgroups * p.ksplit * 8 * 64 * 4;
}

template <int FMT, int NT>
__global__ __launch_bounds__(512) void k_gemv(const uint8_t *__restrict__ w, int64_t row_bytes,
                                              int n, int units, int ksplit, int upk, int upw,
                                              const float *__restrict__ x, int64_t ldx,
                                              float *__restrict__ y, int64_t ldy,
                                              float *__restrict__ partial) {
  extern __shared__ float lds[];
  const int rg = blockIdx.x / ksplit, ks = blockIdx.x - rg * ksplit;
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
  } else {
    float *mine = partial + ((int64_t)rg * ksplit + ks) * NT * 64;
    for (int i = threadIdx.x; i < NT * 64; i += blockDim.x) mine[i] = lds[i];
  }
}

// Adds the k slices of every row group in slice order: y[t][r] = sum_q partial[rg][q][t][r%64].
__global__ __launch_bounds__(256) void k_gemv_reduce(const float *__restrict__ partial, int n,
                                                     int ksplit, int nt, float *__restrict__ y,
                                                     int64_t ldy) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)nt * n) return;
  const int t = (int)(gid / n), r = (int)(gid - (int64_t)t * n);
  const int rg = r >> 6, l = r & 63;
  const float *p = partial + (int64_t)rg * ksplit * nt * 64 + t * 64 + l;
  float s = 0.f;
  for (int q = 0; q < ksplit; ++q) s += p[(int64_t)q * nt * 64];
  y[t * ldy + r] = s;
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
                           size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((k_gemv<FMT, NT>), dim3((unsigned)(p.rowgroups * p.ksplit)), dim3(64 * p.waves),
                     lds, s, w, rb, n, units, p.ksplit, p.upk, p.upw, x, ldx, y, ldy, partial);
}

template <int FMT>
static int launch_gemv_fmt(const uint8_t *w, int64_t rb, int n, int64_t k, const float *x,
                           int batch, float *y, void *ws, size_t ws_bytes, hipStream_t s) {
  const int units = (int)(k / 256);
  const bool split = ws != nullptr && ws_bytes >= gemv_workspace_bytes(FMT, n, k, batch);
  const GemvPlan p = plan_gemv(n, k, split);
  float *partial = p.ksplit > 1 ? static_cast<float *>(ws) : nullptr;
  const int max_floats = 65536 / 4;
  for (int t0 = 0; t0 < batch;) {
    int nt = batch - t0 < 8 ? batch - t0 : 8;
    while (nt > 1 && gemv_tile_lds_floats<FMT>(nt, p.upk, p.waves) > max_floats) --nt;
    if (gemv_tile_lds_floats<FMT>(nt, p.upk, p.waves) > max_floats) return -2;
    const size_t lds = (size_t)4 * gemv_tile_lds_floats<FMT>(nt, p.upk, p.waves);
    const float *xt = x + (int64_t)t0 * k;
    float *yt = y + (int64_t)t0 * n;
    switch (nt) {
#define TQ_CASE(NTV) \
  case NTV: launch_gemv_nt<FMT, NTV>(w, rb, n, units, p, xt, k, yt, n, partial, lds, s); break;
      TQ_CASE(1) TQ_CASE(2) TQ_CASE(3) TQ_CASE(4) TQ_CASE(5) TQ_CASE(6) TQ_CASE(7) TQ_CASE(8)
#undef TQ_CASE
    }
    if (p.ksplit > 1) {
      const int64_t threads = (int64_t)nt * n;
      hipLaunchKernelGGL(k_gemv_reduce, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                         partial, n, p.ksplit, nt, yt, (int64_t)n);
    }
    if (hipGetLastError() != hipSuccess) return -1;
    t0 += nt;
  }
  return 0;
}

bool gemv_fast_shape(int fmt, int64_t k) {
  if (fmt == FMT_Q4_K) return k % 256 == 0;
  if (fmt == FMT_Q6_K) return k % 512 == 0;  // 210 * (k/256) bytes per row is dword aligned
  return k % 256 == 0;                       // Q8_0: whole 8-block units, 16-byte aligned rows
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
  switch (fmt) {
    case FMT_Q4_K: return launch_gemv_fmt<FMT_Q4_K>(wb, rb, (int)n, k, x, (int)batch, y, ws, ws_bytes, s);
    case FMT_Q6_K: return launch_gemv_fmt<FMT_Q6_K>(wb, rb, (int)n, k, x, (int)batch, y, ws, ws_bytes, s);
    default: return launch_gemv_fmt<FMT_Q8_0>(wb, rb, (int)n, k, x, (int)batch, y, ws, ws_bytes, s);
  }
}

// ---- SwiGLU ------------------------------------------------------------------------------------

__device__ __forceinline__ float silu_mul(float g, float u) { return g * u / (1.f + expf(-g)); }

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
