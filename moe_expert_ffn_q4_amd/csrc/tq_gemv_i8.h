// tq_gemv_i8.h -- batch-1 Q4_K GEMV on the int8 matrix cores (internal to libtq).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_gemv_core.h"

namespace tq {

// Shapes the int8 kernel takes: Q4_K, one token, k a multiple of 256, 16384 <= k <= 32768 (all
// k <= 32768 with TQ_GEMV_I8=2).
bool i8_gemv_ok(int fmt, int64_t k, int64_t batch);
// Workspace after the completion counters: the k slices' partial sums of `rows` rows (0 when k
// is one slice).
size_t i8_workspace_bytes(int64_t rows, int64_t k);
// The rows of m against x [k] (16-byte aligned). partial: i8_workspace_bytes(m.total, k) bytes;
// counters: zero, one per row group (max_counters of them), left zero.
int launch_gemv_i8(const KlMap &m, int64_t k, const float *x, float *partial,
                   unsigned *counters, int max_counters, hipStream_t s);

// Streaming form (no workspace; opt-in with TQ_GEMV_I8S=1): Q4_K, one token, k a multiple of 256
// up to 16384; all of x is made
// into digits in each workgroup's LDS and the k parts of a row tile are added inside the workgroup.
bool i8s_gemv_ok(int fmt, int64_t k, int64_t batch);
int launch_gemv_i8s(const KlMap &m, int64_t k, const float *x, hipStream_t s);

}  // namespace tq
