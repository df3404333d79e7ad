// tq_read_ref.hip -- a plain streaming read of a device buffer: the measurement reference that the
// GEMV kernels' times are compared with (a launch that only moves the same bytes from HBM). Built
// as its own library, libtq_readref.so; not part of libtq.
//
// Every 16-byte unit of the buffer is loaded once with a coalesced 16-byte load: a workgroup of
// 256 threads covers 256 * kUnits consecutive units, thread t loading units t, t + 256, ... so
// that each of its kUnits loads is issued before any result is used. The XOR of everything a wave
// read is stored to sink[] (one word per wave), so no load can be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kUnits = 4;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void k_read_ref(const u32x4 *__restrict__ p, int64_t n16,
                                                       uint32_t *__restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * kThreads * kUnits + threadIdx.x;
  u32x4 v[kUnits];
#pragma unroll
  for (int u = 0; u < kUnits; ++u) {
    const int64_t i = base + (int64_t)u * kThreads;
    v[u] = i < n16 ? p[i] : (u32x4){0u, 0u, 0u, 0u};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < kUnits; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) sink[(int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = acc;
}

}  // namespace

extern "C" {

// Words of sink a read of `bytes` needs (one per wave).
int64_t tq_read_ref_sink_words(int64_t bytes) {
  const int64_t n16 = bytes / 16;
  return (n16 + kThreads * kUnits - 1) / (kThreads * kUnits) * (kThreads / 64);
}

// Reads the first bytes (a multiple of 16) of p (16-byte aligned). 0, or -1 on a bad argument or
// a launch failure.
int tq_read_ref(const void *p, int64_t bytes, uint32_t *sink, void *stream) {
  if (!p || !sink || bytes <= 0 || bytes % 16 || ((uintptr_t)p & 15)) return -1;
  const int64_t n16 = bytes / 16;
  const int64_t grid = (n16 + kThreads * kUnits - 1) / (kThreads * kUnits);
  if (grid > 0x7FFFFFFF) return -1;
  hipLaunchKernelGGL(k_read_ref, dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)stream,
                     (const u32x4 *)p, n16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
