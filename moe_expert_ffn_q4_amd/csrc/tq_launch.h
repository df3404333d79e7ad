// tq_launch.h -- host-side launchers behind the C ABI (internal to libtq).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "tq.h"

namespace tq {

// The value of tuning knob `id` (TQ_KNOB_*): its override (tq_tuning_set), else `dflt`. Read on
// every call.
int knob(int id, int dflt);
void g_knobs_store(int id, int value);  // value < 0: back to the default
int g_knobs_load(int id);               // the override, or -1
// Tag of one launch's completion counters (Arrivals::tag): a 48-bit token, never zero and distinct
// for every launch of the process (a counter starting from a value drawn at load time), shifted
// past 16 count bits.
unsigned long long call_tag();

inline int clampi(int v, int lo, int hi) { return v < lo ? lo : v > hi ? hi : v; }
inline int64_t align256(int64_t v) { return (v + 255) & ~(int64_t)255; }
// Q4_K, Q6_K, Q8_0, Q5_K, Q4_0
inline int64_t fmt_block_weights(int fmt) {
  return fmt == 1 || fmt == 2 || fmt == 4 ? 256 : fmt == 3 || fmt == 5 ? 32 : 0;
}
inline int64_t fmt_block_bytes(int fmt) {
  return fmt == 1 ? 144 : fmt == 2 ? 210 : fmt == 3 ? 34 : fmt == 4 ? 176 : fmt == 5 ? 18 : 0;
}

// Each returns 0 when everything was enqueued, -1 on a HIP launch error, -2 when the shape needs
// more LDS than one workgroup may use.
int launch_dequant(int fmt, const void *w, int64_t n, int64_t k, int out_type, void *out,
                   hipStream_t s);
bool gemv_fast_shape(int fmt, int64_t k);
size_t gemv_workspace_bytes(int fmt, int64_t n, int64_t k, int64_t batch);
int launch_gemv(int fmt, const void *w, int64_t n, int64_t k, const float *x, int64_t batch,
                float *y, void *ws, size_t ws_bytes, hipStream_t s);
int launch_swiglu(const float *g, const float *u, int64_t count, float *h, hipStream_t s);
size_t gemv_multi_workspace_bytes(int fmt, int nparts, const int64_t *n, int64_t k, int64_t batch);
int launch_gemv_multi(int fmt, int nparts, const void *const *w, const int64_t *n, float *const *y,
                      int64_t k, const float *x, int64_t batch, void *ws, size_t ws_bytes,
                      hipStream_t s);
bool gemv_swiglu_fused(int fmt, int64_t k, const float *x, int64_t batch);
// The least workspace the call accepts (the one-launch paths run without one).
size_t gemv_swiglu_min_workspace_bytes(int fmt, int64_t n, int64_t k, int64_t batch, bool fused);
size_t gemv_swiglu_workspace_bytes(int fmt, int64_t n, int64_t k, int64_t batch, bool fused);
int launch_gemv_swiglu(int fmt, const void *wg, const void *wu, int64_t n, int64_t k,
                       const float *x, int64_t batch, float *h, void *ws, size_t ws_bytes,
                       hipStream_t s);

}  // namespace tq
