// tq_gemv_i8.hip -- batch-1 Q4_K and Q8_0 GEMV with the multiply-adds on the int8 matrix cores
// (Q8_0: see the unit functions in tq_gemv_i8.h).
//
// Per 256-weight block of a row (d, dmin, sub-block scales sc_j and mins m_j, quants q) the product
// with x is  d * sum_j sc_j sum_{k in j} q_k x_k  -  dmin * sum_j m_j S_j  (S_j = sum of x over
// sub-block j). The inner sums go to v_mfma_i32_32x32x32_i8 with exact integers on both sides:
//   * the quants are the nibbles themselves (a mask of 0x0F0F0F0F yields four int8 operands);
//   * each 256-value block of x is scaled by its own power of two 2^e and rounded to integers x'
//     with |x'| < 2^27, written as four signed 7-bit digits, x' = c0 + 2^7 c1 + 2^14 c2 + 2^21 c3
//     (c0..c2 in [-64, 63]). e is the smaller of the value that brings the block's max|x| into
//     [2^26, 2^27) and the number of fractional bits the block's values need, so blocks of
//     integers (or of values with few significant bits) stay exact.
// One 32-k step of the matrix cores is exactly one sub-block: weight operand = 32 rows x 32 k
// (lane l: row l % 32, k = 16 (l / 32) .. +15 of the sub-block), activation operand = 32 rows of
// (sub-block j', digit d) = 4 j' + d, non-zero only in the rows of the step's own sub-block, so
// the 32x32 int32 accumulator of a block holds sum_{k in j} c_d q_k for all 8 sub-blocks x 4
// digits x 32 rows and is folded once per block: lane l (row l % 32, parity h = l / 32) holds
// sub-blocks 2q + h, q = 0..3, and adds d * sc_j * (its four digit sums recombined) and
// -dmin * m_j * S_j, both times the block's 2^-e. Everything before the fold is exact; the fold
// is fp32.
//
// Work split: a workgroup takes one k slice (a number of blocks set by k alone) of 32 W rows, one
// 32-row tile per wave. It first turns the slice of x into digits in LDS (16 threads per block),
// then each wave streams its rows' blocks of the slice, the next block's loads in flight. With
// more than one slice, the last workgroup of a row group to finish adds the slices' sums in slice
// order. A row's sum is thus formed the same way whatever the matrix height or the launch.
#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_gemv_core.h"
#include "tq_gemv_i8.h"
#include "tq_launch.h"
#include "tq_mfma.h"

namespace tq {

// Output of virtual row v (multi: the part it falls in).
__device__ __forceinline__ void i8_store(const KlMap &m, int v, float s) { *m.out(v) = s; }

// The 256-weight unit of each format: its bytes in a row, the lane's loads and its products.
template <int FMT>
struct I8Fmt;
template <>
struct I8Fmt<FMT_Q4_K> {
  static constexpr int kUnitBytes = 144;
  struct Blk {
    u32x4 head, q[4];
  };
  static __device__ __forceinline__ void load(Blk &b, const uint8_t *p, int h) {
    b.head = gload(p);
#pragma unroll
    for (int c = 0; c < 4; ++c) b.q[c] = gload(p + 16 + 32 * c + 16 * h);
  }
  static __device__ __forceinline__ float compute(const Blk &b, const uint8_t *l, int n, int h) {
    const u32x4 xa = *reinterpret_cast<const u32x4 *>(l + n * 32 + 16 * h);
    const u32x4 S = *reinterpret_cast<const u32x4 *>(l + kDigitBytes + 16 * h);
    const float us = *reinterpret_cast<const float *>(l + kDigitBytes + 32);
    return i8_block(b.head, b.q, xa, S, us, n >> 2, h);
  }
};
template <>
struct I8Fmt<FMT_Q8_0> {
  static constexpr int kUnitBytes = 272;
  using Blk = Q8Unit;
  static __device__ __forceinline__ void load(Blk &b, const uint8_t *p, int h) {
    q8_load_unit(b, p, h);
  }
  static __device__ __forceinline__ float compute(const Blk &b, const uint8_t *l, int n, int h) {
    const u32x4 xa = *reinterpret_cast<const u32x4 *>(l + n * 32 + 16 * h);
    const float us = *reinterpret_cast<const float *>(l + kDigitBytes + 32);
    return q8_i8_unit(b, xa, us, n >> 2, h);
  }
};

template <int FMT>
__global__ __launch_bounds__(256) void k_gemv_i8(KlMap m, const float *__restrict__ x, int nblk,
                                                 int upk, int ksplit, int groups,
                                                 float *__restrict__ partial, Arrivals arr) {
  using F = I8Fmt<FMT>;
  __shared__ __attribute__((aligned(16))) uint8_t xl[kMaxSliceBlocks * kLdsBlock];
  __shared__ float red[4][32];
  __shared__ int is_last;
  const int W = blockDim.x >> 6;  // row tiles of this workgroup
  // blockIdx -> (row group, slice): XCD x takes the row groups g = x (mod 8) and runs all slices
  // of one group back to back, so the cache lines that neighbouring slices of a row share are
  // fetched once, into that XCD's L2
  const int xcd = blockIdx.x & 7, bi = blockIdx.x >> 3;
  const int grp = xcd + 8 * (bi / ksplit), ks = bi % ksplit;
  if (grp >= groups) return;
  const int kb0 = ks * upk, nb = min(upk, nblk - kb0);
  const int lane = threadIdx.x & 63, w = wave_index();
  const int n = lane & 31, h = lane >> 5;
  const int r0 = grp * 32 * W + 32 * w;
  const uint8_t *row = m.row(min(r0 + n, m.total - 1)) + (int64_t)kb0 * F::kUnitBytes;
  using Blk = typename F::Blk;
  auto load = [&](Blk &b, int kb) { F::load(b, row + (int64_t)kb * F::kUnitBytes, h); };
  auto compute = [&](const Blk &b, int kb) { return F::compute(b, xl + kb * kLdsBlock, n, h); };
  // the first two blocks' weights are requested before the digits are made, so both latencies
  // overlap; then two blocks stay in flight ahead of the one being computed
  Blk b0, b1;
  load(b0, 0);
  if (nb > 1) load(b1, 1);
  // the slice of x as digits (16 threads per block; groups of 16 stay active together)
  for (int i = threadIdx.x; i < 16 * nb; i += blockDim.x)
    make_digits(x + (int64_t)(kb0 + (i >> 4)) * 256, i & 15, xl + (i >> 4) * kLdsBlock);
  __syncthreads();
  float acc = 0.f;
  for (int kb = 0;;) {
    acc += compute(b0, kb);
    if (++kb >= nb) break;
    if (kb + 1 < nb) load(b0, kb + 1);
    acc += compute(b1, kb);
    if (++kb >= nb) break;
    if (kb + 1 < nb) load(b1, kb + 1);
  }
  acc += __shfl_xor(acc, 32);  // the two sub-block parities of the row

  if (ksplit == 1) {
    const float u = __shfl_down(acc, 1);
    const int v = r0 + n;
    if (h == 0) {
      if (m.swiglu) {
        if ((n & 1) == 0 && v + 1 < m.total) m.y[0][v >> 1] = silu_mul(acc, u);
      } else if (v < m.total) {
        i8_store(m, v, acc);
      }
    }
    return;
  }
  // k slices: this slice's sums (device-coherent stores, completed before the arrival is
  // counted); the last workgroup of the row group adds them in slice order, zeroes the counter
  const int rows = 32 * W;
  float *mine = partial + ((int64_t)grp * ksplit + ks) * rows;
  if (h == 0)
    __hip_atomic_store(mine + 32 * w + n, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  if (threadIdx.x == 0) is_last = arrive_last(arr, grp, (unsigned)ksplit);
  __syncthreads();
  if (!is_last) return;
  const float *base = partial + (int64_t)grp * ksplit * rows;
  for (int i = threadIdx.x; i < rows; i += blockDim.x) {
    float vals[kMaxSlices];
#pragma unroll
    for (int q = 0; q < kMaxSlices; ++q)  // every slice's value in flight, then the sum
      vals[q] = q < ksplit ? __hip_atomic_load(base + (int64_t)q * rows + i, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)
                           : 0.f;
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < kMaxSlices; ++q)
      if (q < ksplit) s += vals[q];
    red[i >> 5][i & 31] = s;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < rows; i += blockDim.x) {
    const int v = grp * rows + i;
    const float s = red[i >> 5][i & 31];
    if (m.swiglu) {
      if ((i & 1) == 0 && v + 1 < m.total) m.y[0][v >> 1] = silu_mul(s, red[i >> 5][(i & 31) + 1]);
    } else if (v < m.total) {
      i8_store(m, v, s);
    }
  }
  if (threadIdx.x == 0) done_arrivals(arr, grp);
}

// ---- host side ----------------------------------------------------------------------------------

// Q4_K, one token, k a multiple of 256 up to 32768; by default from k = 16384 on. Below that the
// lanes-along-k kernel is as fast on the measured shapes (inside a graph, the 8B-shaped step
// 1.60 ms against 1.86 ms with this kernel everywhere), above it this one is about twice as fast
// (8192 x 28672: 26 us against 58 us) -- that kernel's workgroups of k / 4096 waves and its VALU
// work per weight hold it back there. TQ_KNOB_GEMV_I8: 0 never, 2 every such shape (tests, tuning).
bool i8_gemv_ok(int fmt, int64_t k, int64_t batch) {
  const int mode = knob(TQ_KNOB_GEMV_I8, 1);
  if (mode == 0 || (fmt != FMT_Q4_K && fmt != FMT_Q8_0) || batch != 1 || k % 256 != 0 ||
      k < 256 || k > 256 * kMaxSliceBlocks * kMaxSlices)
    return false;
  return fmt == FMT_Q8_0 || mode == 2 || k >= 16384;
}

// Blocks per k slice, a function of k only: at least four, at most 8 slices.
static int i8_upk(int64_t k) {
  const int nblk = (int)(k / 256);
  const int least = (nblk + kMaxSlices - 1) / kMaxSlices;
  const int v = knob(TQ_KNOB_I8_UPK, 4);
  return clampi(v > least ? v : least, 1, nblk);
}

// Row tiles per workgroup: 4 (128 rows) while that gives 512 workgroups, else fewer.
static int i8_tiles_per_wg(int64_t rows, int ksplit) {
  for (int W = 4; W > 1; W >>= 1)
    if (((rows + 32 * W - 1) / (32 * W)) * ksplit >= 512) return W;
  return 1;
}

size_t i8_workspace_bytes(int64_t rows, int64_t k) {
  const int nblk = (int)(k / 256), upk = i8_upk(k), ksplit = (nblk + upk - 1) / upk;
  if (ksplit == 1) return 0;
  const int W = i8_tiles_per_wg(rows, ksplit);
  const int64_t groups = (rows + 32 * W - 1) / (32 * W);
  return (size_t)align256(groups * ksplit * 32 * W * 4);
}

int launch_gemv_i8(int fmt, const KlMap &m, int64_t k, const float *x, float *partial,
                   unsigned long long *counters, int max_counters, hipStream_t s) {
  const int nblk = (int)(k / 256), upk = i8_upk(k), ksplit = (nblk + upk - 1) / upk;
  if (upk > kMaxSliceBlocks || ksplit > kMaxSlices) return -2;
  const int W = i8_tiles_per_wg(m.total, ksplit);
  const int groups = (m.total + 32 * W - 1) / (32 * W);
  if (ksplit > 1 && groups > max_counters) return -2;
  const Arrivals arr{counters, ksplit > 1 ? call_tag() : 0ull};
  const dim3 grid((unsigned)((groups + 7) / 8 * 8 * ksplit));
  if (fmt == FMT_Q8_0)
    hipLaunchKernelGGL(k_gemv_i8<FMT_Q8_0>, grid, dim3(64 * W), 0, s, m, x, nblk, upk, ksplit,
                       groups, partial, arr);
  else
    hipLaunchKernelGGL(k_gemv_i8<FMT_Q4_K>, grid, dim3(64 * W), 0, s, m, x, nblk, upk, ksplit,
                       groups, partial, arr);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace tq
