// tq_gemv_mf.h -- batch-1 Q4_K and Q6_K GEMV on the fp16 matrix cores (internal to libtq).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_gemv_core.h"

namespace tq {

// Format and row length k that the kernel takes (the activation operands of all of k sit in one
// workgroup's LDS: Q4_K k a multiple of 256 up to 14336, Q6_K a multiple of 512 up to 8192) and its
// knob.
bool mf_gemv_ok(int fmt, int64_t k);
// All rows of m (single, multi or SwiGLU pairs) against x (16-byte aligned). 0, -1 (launch error)
// or -2 (LDS).
int launch_gemv_mf(int fmt, const KlMap &m, int64_t k, const float *x, hipStream_t s);

}  // namespace tq
