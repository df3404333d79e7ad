// tq_api.hip -- the extern "C" entry points of libtq: argument checks, then the launchers.
#include <stdarg.h>
#include <stdio.h>

#include "../../include/tq.h"
#include "tq_launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool known_type(int t) { return t == TQ_Q4_K || t == TQ_Q6_K || t == TQ_Q8_0; }

int launched(int rc, const char *what) {
  if (rc == 0) return TQ_OK;
  if (rc == -2) return fail(TQ_EUNSUPPORTED, "%s: shape needs more LDS than a workgroup has", what);
  return fail(TQ_EDEVICE, "%s: kernel launch failed: %s", what, hipGetErrorString(hipGetLastError()));
}

}  // namespace

extern "C" {

int64_t tq_block_weights(int type) { return known_type(type) ? tq::fmt_block_weights(type) : 0; }
int64_t tq_block_bytes(int type) { return known_type(type) ? tq::fmt_block_bytes(type) : 0; }

int64_t tq_row_bytes(int type, int64_t k) {
  if (!known_type(type) || k < 0 || k % tq::fmt_block_weights(type)) return -1;
  return k / tq::fmt_block_weights(type) * tq::fmt_block_bytes(type);
}

const char *tq_last_error(void) { return g_err; }

int tq_dequant(int type, const void *w, int64_t n, int64_t k, int out_type, void *out,
               void *stream) {
  if (!known_type(type)) return fail(TQ_EINVAL, "tq_dequant: unknown block type %d", type);
  if (out_type != TQ_F32 && out_type != TQ_BF16)
    return fail(TQ_EINVAL, "tq_dequant: unknown output type %d", out_type);
  if (n < 0 || k < 0 || k % tq::fmt_block_weights(type))
    return fail(TQ_ESHAPE, "tq_dequant: n=%lld k=%lld (k must be a multiple of %lld)", (long long)n,
                (long long)k, (long long)tq::fmt_block_weights(type));
  if (n * k > ((int64_t)1 << 40)) return fail(TQ_ESHAPE, "tq_dequant: n*k too large");
  if (n == 0 || k == 0) return TQ_OK;
  if (!w || !out) return fail(TQ_EINVAL, "tq_dequant: null pointer");
  if (!aligned(w, 16) || !aligned(out, 4))
    return fail(TQ_EALIGN, "tq_dequant: w must be 16-byte and out 4-byte aligned");
  return launched(tq::launch_dequant(type, w, n, k, out_type, out, (hipStream_t)stream), "tq_dequant");
}

size_t tq_gemv_workspace_bytes(int type, int64_t n, int64_t k, int64_t batch) {
  if (!known_type(type) || n < 1 || k < 1 || k % tq::fmt_block_weights(type) || batch < 1) return 0;
  return tq::gemv_workspace_bytes(type, n, k, batch);
}

int tq_gemv(int type, const void *w, int64_t n, int64_t k, const float *x, int64_t batch,
            float *y, void *workspace, size_t ws_bytes, void *stream) {
  if (!known_type(type)) return fail(TQ_EINVAL, "tq_gemv: unknown block type %d", type);
  if (!w || !x || !y) return fail(TQ_EINVAL, "tq_gemv: null pointer");
  const int64_t bw = tq::fmt_block_weights(type);
  if (n < 1 || n > (1 << 30) || k < bw || k % bw || k > (1 << 24))
    return fail(TQ_ESHAPE, "tq_gemv: n=%lld k=%lld (need n >= 1, k a positive multiple of %lld)",
                (long long)n, (long long)k, (long long)bw);
  if (batch < 1 || batch > 4096) return fail(TQ_ESHAPE, "tq_gemv: batch=%lld not in 1..4096", (long long)batch);
  if (!aligned(w, 16) || !aligned(x, 4) || !aligned(y, 4) || !aligned(workspace, 256))
    return fail(TQ_EALIGN, "tq_gemv: w must be 16-byte aligned, x and y 4-byte aligned, "
                           "workspace 256-byte aligned");
  return launched(tq::launch_gemv(type, w, n, k, x, batch, y, workspace, ws_bytes, (hipStream_t)stream),
                  "tq_gemv");
}

int tq_swiglu(const float *g, const float *u, int64_t count, float *h, void *stream) {
  if (count < 0) return fail(TQ_ESHAPE, "tq_swiglu: negative count");
  if (count == 0) return TQ_OK;
  if (!g || !u || !h) return fail(TQ_EINVAL, "tq_swiglu: null pointer");
  if (!aligned(g, 4) || !aligned(u, 4) || !aligned(h, 4))
    return fail(TQ_EALIGN, "tq_swiglu: pointers must be 4-byte aligned");
  return launched(tq::launch_swiglu(g, u, count, h, (hipStream_t)stream), "tq_swiglu");
}

}  // extern "C"
