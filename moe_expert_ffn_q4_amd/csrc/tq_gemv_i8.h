// tq_gemv_i8.h -- batch-1 Q4_K GEMV on the int8 matrix cores (internal to libtq).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_gemv_core.h"

namespace tq {

// Activation digits of `tokens` rows of k values (see tq_gemv_i8.hip for the layout).
struct I8Digits {
  int8_t *xd;
  float *S;
  float *unscale;
};
size_t i8_digits_bytes(int64_t tokens, int64_t k);
I8Digits i8_digits_at(void *base, int64_t tokens, int64_t k);

// Shapes the int8 kernel takes: Q4_K, one token, k a multiple of 256 (by default k >= 16384).
bool i8_gemv_ok(int fmt, int64_t k, int64_t batch);
// x [k] -> digits (in `digits`, i8_digits_bytes(1, k) bytes), then the rows of m.
int launch_gemv_i8(const KlMap &m, int64_t k, const float *x, void *digits, hipStream_t s);

}  // namespace tq
