// tq_gemm_f32m.h -- Q6_K / Q8_0 products of 2..16 tokens on the fp32 matrix cores (internal to
// libtq).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_gemv_core.h"

namespace tq {

// Q8_0 with k a multiple of 256 and 2 <= batch <= 16; Q6_K with k a multiple of 512 and
// 4 <= batch <= 16 (2..16 with TQ_KNOB_GEMM_F32M = 2).
bool f32m_ok(int fmt, int64_t k, int64_t batch);
// Partial sums of the k slices after the counters (0 when k is one slice).
size_t f32m_workspace_bytes(int64_t rows, int64_t k);
// The rows of m (y[p] is [batch][n_p]; SwiGLU: y[0] = h [batch][total / 2]) against x
// [batch][k] (16-byte aligned). counters: one 8-byte word per row group (Arrivals), any contents.
int launch_gemm_f32m(int fmt, const KlMap &m, int64_t k, const float *x, int64_t batch,
                     float *partial, unsigned long long *counters, int max_counters,
                     hipStream_t s);

}  // namespace tq
