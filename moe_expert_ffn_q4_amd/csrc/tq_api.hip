// tq_api.hip -- the extern "C" entry points of libtq: argument checks, then the launchers.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdint>
#include <mutex>
#include <utility>
#include <vector>

#include "tq.h"
#include "tq_chain.h"
#include "tq_launch.h"
#include "tq_moe.h"

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

bool known_type(int t) {
  return t == TQ_Q4_K || t == TQ_Q6_K || t == TQ_Q8_0 || t == TQ_Q5_K || t == TQ_Q4_0;
}

int launched(int rc, const char *what) {
  if (rc == 0) return TQ_OK;
  if (rc == -2) return fail(TQ_EUNSUPPORTED, "%s: shape needs more LDS than a workgroup has", what);
  return fail(TQ_EDEVICE, "%s: kernel launch failed: %s", what, hipGetErrorString(hipGetLastError()));
}

}  // namespace

namespace tq {

namespace {
std::atomic<int> g_knobs[TQ_KNOB_COUNT] = {};  // value + 1: 0 means no override
}  // namespace

int knob(int id, int dflt) {
  const int v = g_knobs[id].load(std::memory_order_relaxed);
  return v > 0 ? v - 1 : dflt;
}

void g_knobs_store(int id, int value) {
  g_knobs[id].store(value < 0 ? 0 : value + 1, std::memory_order_relaxed);
}

int g_knobs_load(int id) { return g_knobs[id].load(std::memory_order_relaxed) - 1; }

unsigned long long call_tag() {
  // splitmix64 of the load time and an address: where the token sequence starts
  static std::atomic<unsigned long long> next{[] {
    unsigned long long z = (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count() ^
                           (unsigned long long)(uintptr_t)&g_err;
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }()};
  // 47 bits of the sequence plus a set top bit: never zero, the value a finished launch leaves
  return ((next.fetch_add(1, std::memory_order_relaxed) & 0x7FFFFFFFFFFFull) | 0x800000000000ull) << 16;
}

}  // namespace tq

extern "C" {

int tq_tuning_set(int knob, int value) {
  if (knob < 0 || knob >= TQ_KNOB_COUNT) return fail(TQ_EINVAL, "tq_tuning_set: unknown knob %d", knob);
  if (value >= 0x7FFFFFFF) return fail(TQ_EINVAL, "tq_tuning_set: value %d too large", value);
  tq::g_knobs_store(knob, value);
  return TQ_OK;
}

int tq_tuning_get(int knob) {
  if (knob < 0 || knob >= TQ_KNOB_COUNT) return -1;
  return tq::g_knobs_load(knob);
}

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

}  // extern "C"

namespace {

// Scratch of tq_gemv_noalloc. Each GPU the library runs on holds its own copy until the process
// ends; in host code this name is only a stand-in, so every host use goes through the device
// address that noalloc_scratch() looked up for the current device.
static __device__ __align__(256) unsigned char scratch[TQ_GEMV_NOALLOC_MAX_BYTES];

constexpr int kMaxDevices = 64;

// The current device's address of `scratch`, looked up once per device.
int noalloc_scratch(void **out) {
  static std::mutex mu;
  static void *addr[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(TQ_EDEVICE, "tq_gemv_noalloc: no current HIP device (or more than %d)", kMaxDevices);
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(TQ_EDEVICE, "tq_gemv_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    addr[dev] = p;
  }
  *out = addr[dev];
  return TQ_OK;
}

}  // namespace

extern "C" {

int tq_gemv_noalloc(int type, const void *w, int64_t n, int64_t k, const float *x, int64_t batch,
                    float *y, void *stream) {
  if (!known_type(type)) return fail(TQ_EINVAL, "tq_gemv_noalloc: unknown block type %d", type);
  if (!w || !x || !y) return fail(TQ_EINVAL, "tq_gemv_noalloc: null pointer");
  const int64_t bw = tq::fmt_block_weights(type);
  if (n < 1 || n > (1 << 30) || k < bw || k % bw || k > (1 << 24) || batch < 1 || batch > 4096)
    return fail(TQ_ESHAPE, "tq_gemv_noalloc: n=%lld k=%lld batch=%lld out of range",
                (long long)n, (long long)k, (long long)batch);
  if (!aligned(w, 16) || !aligned(x, 4) || !aligned(y, 4))
    return fail(TQ_EALIGN, "tq_gemv_noalloc: w must be 16-byte aligned, x and y 4-byte aligned");
  const size_t need = tq::gemv_workspace_bytes(type, n, k, batch);
  if (need > TQ_GEMV_NOALLOC_MAX_BYTES)
    return fail(TQ_ENOSPC, "tq_gemv_noalloc: n=%lld k=%lld batch=%lld needs %zu bytes of scratch, "
                "more than the %u this entry point has", (long long)n, (long long)k,
                (long long)batch, need, (unsigned)TQ_GEMV_NOALLOC_MAX_BYTES);
  void *ws = nullptr;
  if (need > 0) {
    const int rc = noalloc_scratch(&ws);
    if (rc != TQ_OK) return rc;
  }
  return tq_gemv(type, w, n, k, x, batch, y, ws, need, stream);
}

size_t tq_gemv_multi_workspace_bytes(int type, int nparts, const int64_t *n, int64_t k,
                                     int64_t batch) {
  if (!known_type(type) || nparts < 1 || nparts > 4 || !n || k < 1 ||
      k % tq::fmt_block_weights(type) || batch < 1)
    return 0;
  for (int p = 0; p < nparts; ++p)
    if (n[p] < 1) return 0;
  return tq::gemv_multi_workspace_bytes(type, nparts, n, k, batch);
}

int tq_gemv_multi(int type, int nparts, const void *const *w, const int64_t *n, float *const *y,
                  int64_t k, const float *x, int64_t batch, void *workspace, size_t ws_bytes,
                  void *stream) {
  if (!known_type(type)) return fail(TQ_EINVAL, "tq_gemv_multi: unknown block type %d", type);
  if (nparts < 1 || nparts > 4 || !w || !n || !y)
    return fail(TQ_EINVAL, "tq_gemv_multi: need 1..4 parts and the w, n, y arrays");
  if (!x) return fail(TQ_EINVAL, "tq_gemv_multi: null x");
  const int64_t bw = tq::fmt_block_weights(type);
  if (k < bw || k % bw || k > (1 << 24) || batch < 1 || batch > 4096)
    return fail(TQ_ESHAPE, "tq_gemv_multi: k=%lld batch=%lld", (long long)k, (long long)batch);
  int64_t total = 0;
  for (int p = 0; p < nparts; ++p) {
    if (!w[p] || !y[p]) return fail(TQ_EINVAL, "tq_gemv_multi: null w or y of part %d", p);
    if (n[p] < 1 || n[p] > (1 << 28))
      return fail(TQ_ESHAPE, "tq_gemv_multi: n of part %d is %lld", p, (long long)n[p]);
    if (!aligned(w[p], 16) || !aligned(y[p], 4))
      return fail(TQ_EALIGN, "tq_gemv_multi: w 16-byte, y 4-byte alignment needed");
    total += n[p];
  }
  if (!aligned(x, 16) || !aligned(workspace, 256))
    return fail(TQ_EALIGN, "tq_gemv_multi: x 16-byte, workspace 256-byte alignment needed");
  return launched(tq::launch_gemv_multi(type, nparts, w, n, y, k, x, batch, workspace, ws_bytes,
                                        (hipStream_t)stream),
                  "tq_gemv_multi");
}

size_t tq_gemv_swiglu_workspace_bytes(int type, int64_t n, int64_t k, int64_t batch) {
  if (!known_type(type) || n < 1 || k < 1 || k % tq::fmt_block_weights(type) || batch < 1) return 0;
  static const float probe[4] __attribute__((aligned(16))) = {0, 0, 0, 0};
  return tq::gemv_swiglu_workspace_bytes(type, n, k, batch,
                                         tq::gemv_swiglu_fused(type, k, probe, batch));
}

int tq_gemv_swiglu(int type, const void *w_gate, const void *w_up, int64_t n, int64_t k,
                   const float *x, int64_t batch, float *h, void *workspace, size_t ws_bytes,
                   void *stream) {
  if (!known_type(type)) return fail(TQ_EINVAL, "tq_gemv_swiglu: unknown block type %d", type);
  if (!w_gate || !w_up || !x || !h) return fail(TQ_EINVAL, "tq_gemv_swiglu: null pointer");
  const int64_t bw = tq::fmt_block_weights(type);
  if (n < 1 || n > (1 << 28) || k < bw || k % bw || k > (1 << 24) || batch < 1 || batch > 4096)
    return fail(TQ_ESHAPE, "tq_gemv_swiglu: n=%lld k=%lld batch=%lld", (long long)n, (long long)k,
                (long long)batch);
  if (!aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(x, 16) || !aligned(h, 4) ||
      !aligned(workspace, 256))
    return fail(TQ_EALIGN, "tq_gemv_swiglu: w and x 16-byte, h 4-byte, workspace 256-byte "
                           "alignment needed");
  // the one-launch path runs without a workspace too (the int8 kernel then gives way to the
  // lanes-along-k one); the two-launch path keeps gate and up in it
  const bool fused = tq::gemv_swiglu_fused(type, k, x, batch);
  if (!fused && (ws_bytes < tq::gemv_swiglu_min_workspace_bytes(type, n, k, batch, false) ||
                 !workspace))
    return fail(TQ_ENOSPC, "tq_gemv_swiglu: workspace of %zu bytes too small", ws_bytes);
  return launched(tq::launch_gemv_swiglu(type, w_gate, w_up, n, k, x, batch, h, workspace,
                                         ws_bytes, (hipStream_t)stream),
                  "tq_gemv_swiglu");
}

int tq_swiglu(const float *g, const float *u, int64_t count, float *h, void *stream) {
  if (count < 0) return fail(TQ_ESHAPE, "tq_swiglu: negative count");
  if (count == 0) return TQ_OK;
  if (!g || !u || !h) return fail(TQ_EINVAL, "tq_swiglu: null pointer");
  if (!aligned(g, 4) || !aligned(u, 4) || !aligned(h, 4))
    return fail(TQ_EALIGN, "tq_swiglu: pointers must be 4-byte aligned");
  return launched(tq::launch_swiglu(g, u, count, h, (hipStream_t)stream), "tq_swiglu");
}

// Average routed tokens per expert from which TQ_PATH_AUTO takes the matrix-core path.
constexpr int64_t kMfmaTokens = 64;

static int moe_check(const tq_moe_desc *d, int64_t tokens, tq::MoeShape *out) {
  if (!d) return fail(TQ_EINVAL, "tq_moe_ffn: null descriptor");
  if (!known_type(d->type)) return fail(TQ_EINVAL, "tq_moe_ffn: unknown block type %d", d->type);
  if (d->hidden < 256 || d->ffn < 256 || d->hidden % 256 || d->ffn % 256)
    return fail(TQ_ESHAPE, "tq_moe_ffn: hidden and ffn must be positive multiples of 256");
  if (!tq::gemv_fast_shape(d->type, d->hidden) || !tq::gemv_fast_shape(d->type, d->ffn))
    return fail(TQ_EUNSUPPORTED, "tq_moe_ffn: this block type needs hidden and ffn to be multiples of 512");
  if (d->n_experts < 1 || d->n_experts > 1024 || d->top_k < 1 || d->top_k > 32 || d->top_k > d->n_experts)
    return fail(TQ_ESHAPE, "tq_moe_ffn: n_experts=%lld top_k=%lld out of range",
                (long long)d->n_experts, (long long)d->top_k);
  if (tokens < 1 || tokens > 8192) return fail(TQ_ESHAPE, "tq_moe_ffn: tokens=%lld not in 1..8192", (long long)tokens);
  if (tq::group_lds_bytes(tokens, d->n_experts) > 160 * 1024)
    return fail(TQ_EUNSUPPORTED, "tq_moe_ffn: tokens x experts too large for the grouping kernel");
  if (!d->router_w || !aligned(d->router_w, 16)) return fail(TQ_EINVAL, "tq_moe_ffn: router_w null or not 16-byte aligned");
  if (d->experts_on_host ? !d->experts_host : !d->experts)
    return fail(TQ_EINVAL, "tq_moe_ffn: missing expert table");
  if (d->shared.gate && (!d->shared.up || !d->shared.down))
    return fail(TQ_EINVAL, "tq_moe_ffn: shared expert needs gate, up and down");
  if (d->path != TQ_PATH_AUTO && d->path != TQ_PATH_F32 && d->path != TQ_PATH_BF16_MFMA)
    return fail(TQ_EINVAL, "tq_moe_ffn: unknown path %d", d->path);
  tq::MoeShape s{};
  s.type = d->type;
  s.hidden = d->hidden;
  s.ffn = d->ffn;
  s.n_experts = d->n_experts;
  s.top_k = d->top_k;
  s.tokens = tokens;
  s.has_shared = d->shared.gate != nullptr;
  s.renormalize = d->renormalize != 0;
  s.experts_on_host = d->experts_on_host != 0;
  s.gate_bytes = d->ffn * tq_row_bytes(d->type, d->hidden);
  s.expert_bytes = 2 * s.gate_bytes + d->hidden * tq_row_bytes(d->type, d->ffn);
  // matrix cores once the experts average kMfmaTokens routed tokens or more
  if (d->path == TQ_PATH_BF16_MFMA) {
    if (d->type != TQ_Q4_K)
      return fail(TQ_EUNSUPPORTED, "tq_moe_ffn: the bf16 matrix-core path takes Q4_K experts only");
    s.mfma = 1;
  } else if (d->path == TQ_PATH_AUTO) {
    s.mfma = d->type == TQ_Q4_K && tokens * d->top_k >= kMfmaTokens * d->n_experts;
  }
  *out = s;
  return TQ_OK;
}

size_t tq_moe_workspace_bytes(const tq_moe_desc *desc, int64_t tokens) {
  tq::MoeShape s;
  if (moe_check(desc, tokens, &s) != TQ_OK) return 0;
  return (size_t)tq::plan_moe(s).bytes;
}

static bool host_experts_ok(const tq_moe_desc *d) {
  for (int64_t e = 0; e < d->n_experts; ++e) {
    const tq_expert &x = d->experts_host[e];
    if (!x.gate || !x.up || !x.down) return false;
  }
  return true;
}

// Per-thread resources of the host-resident path: a pinned buffer for the active-expert list and
// events (one per staged expert, one for "the compute stream is done with the staging area").
struct HostPathState {
  int device = -1;
  int *list = nullptr;  // the active-expert list, then (cache only) the call's expert table
  size_t list_ints = 0;
  std::vector<hipEvent_t> copied;
  hipEvent_t ready = nullptr;
};

static int host_path_state(int64_t list_ints, int n_events, HostPathState *&out) {
  static thread_local HostPathState hs;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(TQ_EDEVICE, "tq_moe_ffn: no current device");
  if (hs.device != dev) {  // resources belong to one device; start over on another
    for (hipEvent_t e : hs.copied) (void)hipEventDestroy(e);
    hs.copied.clear();
    if (hs.ready) (void)hipEventDestroy(hs.ready);
    hs.ready = nullptr;
    if (hs.list) (void)hipHostFree(hs.list);
    hs.list = nullptr;
    hs.list_ints = 0;
    hs.device = dev;
  }
  if (hs.list_ints < (size_t)list_ints) {
    if (hs.list) (void)hipHostFree(hs.list);
    hs.list = nullptr;
    hs.list_ints = 0;
    if (hipHostMalloc((void **)&hs.list, (size_t)list_ints * 4, hipHostMallocDefault) != hipSuccess)
      return fail(TQ_EDEVICE, "tq_moe_ffn: pinned host allocation failed");
    hs.list_ints = (size_t)list_ints;
  }
  if (!hs.ready && hipEventCreateWithFlags(&hs.ready, hipEventDisableTiming) != hipSuccess)
    return fail(TQ_EDEVICE, "tq_moe_ffn: event creation failed");
  while ((int)hs.copied.size() < n_events) {
    hipEvent_t e;
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess)
      return fail(TQ_EDEVICE, "tq_moe_ffn: event creation failed");
    hs.copied.push_back(e);
  }
  out = &hs;
  return TQ_OK;
}

// ---- expert residency cache (state in caller memory) ----------------------------------------------

constexpr uint64_t kCacheMagic = 0x5451455843414348ull;  // "TQEXCACH"

struct CacheHeader {
  uint64_t magic;
  int device, type;
  int64_t hidden, ffn, n_experts, expert_bytes, gate_bytes;
  int64_t slots, prefetch, stride;
  uint8_t *mem;
  int64_t clock;
  tq_expert_cache_stats stats;
};

// The arrays that follow the header, each 64-byte aligned.
struct CacheView {
  CacheHeader *h;
  int32_t *slot_expert;  // [slots] expert held, -1: empty
  int64_t *slot_used;    // [slots] clock of the last call that read or filled it
  hipEvent_t *slot_ready;  // [slots] recorded after the slot's latest copy
  uint8_t *slot_pref;    // [slots] 1: filled by a prefetch and not read since
  int32_t *expert_slot;  // [n_experts] slot holding the expert, -1: none
  float *score;          // [n_experts]
};

static size_t cache_layout(int64_t slots, int64_t E, size_t off[6]) {
  auto up = [](size_t v) { return (v + 63) & ~(size_t)63; };
  size_t o = up(sizeof(CacheHeader));
  off[0] = o; o = up(o + 4 * (size_t)slots);
  off[1] = o; o = up(o + 8 * (size_t)slots);
  off[2] = o; o = up(o + sizeof(hipEvent_t) * (size_t)slots);
  off[3] = o; o = up(o + (size_t)slots);
  off[4] = o; o = up(o + 4 * (size_t)E);
  off[5] = o; o = up(o + 4 * (size_t)E);
  return o;
}

static CacheView cache_view(void *state) {
  CacheView v{};
  v.h = (CacheHeader *)state;
  size_t off[6];
  cache_layout(v.h->slots, v.h->n_experts, off);
  char *b = (char *)state;
  v.slot_expert = (int32_t *)(b + off[0]);
  v.slot_used = (int64_t *)(b + off[1]);
  v.slot_ready = (hipEvent_t *)(b + off[2]);
  v.slot_pref = (uint8_t *)(b + off[3]);
  v.expert_slot = (int32_t *)(b + off[4]);
  v.score = (float *)(b + off[5]);
  return v;
}

// The state belongs to this descriptor's expert shape and to the current device.
static int cache_check(const tq_moe_desc *d, const tq::MoeShape &s, CacheView &v) {
  const CacheHeader *h = (const CacheHeader *)d->expert_cache;
  if (h->magic != kCacheMagic) return fail(TQ_EINVAL, "tq_moe_ffn: expert_cache is not an initialized cache state");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(TQ_EDEVICE, "tq_moe_ffn: no current device");
  if (h->device != dev || h->type != s.type || h->hidden != s.hidden || h->ffn != s.ffn ||
      h->n_experts != s.n_experts || h->expert_bytes != s.expert_bytes)
    return fail(TQ_EINVAL, "tq_moe_ffn: expert_cache was set up for another layer shape or device");
  v = cache_view(d->expert_cache);
  return TQ_OK;
}

// Expert products with the routed experts in pinned host memory. The active-expert list is read
// back (one synchronisation of `st`); each selected expert is then copied into its staging slot
// on the copy stream, followed by an event. On the fp32 path the shared expert (resident) runs
// first and every routed expert's kernels wait only for their own copy, so copies and compute
// overlap; the matrix-core path waits for all copies and runs one grouped launch.
static int host_resident_experts(const tq_moe_desc *d, const tq::MoePlan &p,
                                 const tq::MoeExpertPtrs &shared, const float *x, char *ws,
                                 hipStream_t st) {
  const tq::MoeShape &s = p.s;
  const int E = (int)s.n_experts;
  const int S = p.act_stride;
  CacheView cv{};
  const bool cached = d->expert_cache != nullptr;
  if (cached) {
    const int rc = cache_check(d, s, cv);
    if (rc != TQ_OK) return rc;
  }
  // pinned host memory: the active-expert list, then (with a cache) the call's expert table
  const int64_t list_ints = (3 * (int64_t)S + 1 + 1) & ~(int64_t)1;
  const int64_t table_ints = cached ? E * (int64_t)(sizeof(tq::MoeExpertPtrs) / 4) : 0;
  HostPathState *hs = nullptr;
  int rc = host_path_state(list_ints + table_ints, p.max_active, hs);
  if (rc != TQ_OK) return rc;
  int *act = hs->list, *n_active = hs->list + 3 * S;
  if (hipMemcpyAsync(act, ws + p.off_act, (size_t)(3 * S) * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipMemcpyAsync(n_active, ws + p.off_nact, 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return fail(TQ_EDEVICE, "tq_moe_ffn: reading the active-expert list back failed");
  const int na = *n_active;
  if (na < 0 || na > p.max_active) return fail(TQ_EDEVICE, "tq_moe_ffn: corrupt active-expert list");
  for (int a = 0; a < na; ++a)
    if (act[a] < 0 || act[a] > E)
      return fail(TQ_EDEVICE, "tq_moe_ffn: active-expert list holds id %d (of %d experts)", act[a], E);
  hipStream_t cs = d->copy_stream ? (hipStream_t)d->copy_stream : st;
  uint8_t *staging = (uint8_t *)(ws + p.off_stage);
  // copies may overwrite the staging area and the cache slots once the compute stream's earlier
  // work (the calls before this one) is done
  if (hipEventRecord(hs->ready, st) != hipSuccess || hipStreamWaitEvent(cs, hs->ready, 0) != hipSuccess)
    return fail(TQ_EDEVICE, "tq_moe_ffn: event record / wait failed");
  const int64_t bytes[3] = {s.gate_bytes, s.gate_bytes, s.expert_bytes - 2 * s.gate_bytes};
  const int64_t off[3] = {0, s.gate_bytes, 2 * s.gate_bytes};
  auto copy_expert = [&](int e, uint8_t *dst, hipEvent_t done) -> int {
    const tq_expert &hx = d->experts_host[e];
    const void *src[3] = {hx.gate, hx.up, hx.down};
    for (int m = 0; m < 3; ++m)
      if (hipMemcpyAsync(dst + off[m], src[m], (size_t)bytes[m], hipMemcpyHostToDevice, cs) != hipSuccess)
        return fail(TQ_EDEVICE, "tq_moe_ffn: expert copy failed");
    if (hipEventRecord(done, cs) != hipSuccess) return fail(TQ_EDEVICE, "tq_moe_ffn: event record failed");
    return TQ_OK;
  };
  std::vector<hipEvent_t> wait_ev((size_t)na, nullptr);  // what slot a's kernels wait for
  const tq::MoeExpertPtrs *dev_table = reinterpret_cast<const tq::MoeExpertPtrs *>(d->experts);
  const uint8_t *stage_arg = staging;
  if (!cached) {
    for (int a = 0; a < na; ++a) {
      if (act[a] == E) continue;  // the shared expert stays on the device
      rc = copy_expert(act[a], staging + (int64_t)a * p.stage_stride, hs->copied[a]);
      if (rc != TQ_OK) return rc;
      wait_ev[a] = hs->copied[a];
    }
  } else {
    CacheHeader &h = *cv.h;
    h.clock += 1;
    h.stats.calls += 1;
    for (int e = 0; e < E; ++e) cv.score[e] *= 0.875f;
    for (int a = 0; a < na; ++a)
      if (act[a] != E) cv.score[act[a]] += 1.f;
    std::vector<char> used((size_t)h.slots, 0);
    for (int a = 0; a < na; ++a)  // slots this call reads are not victims
      if (act[a] != E && cv.expert_slot[act[a]] >= 0) used[cv.expert_slot[act[a]]] = 1;
    auto *table = reinterpret_cast<tq::MoeExpertPtrs *>(hs->list + list_ints);
    for (int e = 0; e < E; ++e) table[e] = tq::MoeExpertPtrs{{nullptr, nullptr, nullptr}};
    for (int a = 0; a < na; ++a) {
      const int e = act[a];
      if (e == E) continue;
      uint8_t *dst;
      const int sl = cv.expert_slot[e];
      if (sl >= 0) {  // hit
        h.stats.hits += 1;
        if (cv.slot_pref[sl]) {
          h.stats.prefetch_hits += 1;
          cv.slot_pref[sl] = 0;
        }
        cv.slot_used[sl] = h.clock;
        dst = h.mem + (int64_t)sl * h.stride;
        wait_ev[a] = cv.slot_ready[sl];
      } else {
        int victim = -1;
        int64_t oldest = INT64_MAX;
        for (int64_t q = 0; q < h.slots; ++q) {
          if (used[q]) continue;
          if (cv.slot_expert[q] < 0) {
            victim = (int)q;
            break;
          }
          if (cv.slot_used[q] < oldest) {
            oldest = cv.slot_used[q];
            victim = (int)q;
          }
        }
        if (victim < 0) {  // every slot is read by this call: stage it as without a cache
          dst = staging + (int64_t)a * p.stage_stride;
          rc = copy_expert(e, dst, hs->copied[a]);
          wait_ev[a] = hs->copied[a];
          h.stats.fallbacks += 1;
        } else {
          if (cv.slot_expert[victim] >= 0) cv.expert_slot[cv.slot_expert[victim]] = -1;
          cv.slot_expert[victim] = e;
          cv.expert_slot[e] = victim;
          cv.slot_pref[victim] = 0;
          cv.slot_used[victim] = h.clock;
          used[victim] = 1;
          dst = h.mem + (int64_t)victim * h.stride;
          rc = copy_expert(e, dst, cv.slot_ready[victim]);
          wait_ev[a] = cv.slot_ready[victim];
          h.stats.misses += 1;
        }
        if (rc != TQ_OK) return rc;
        h.stats.bytes_copied += s.expert_bytes;
      }
      table[e] = tq::MoeExpertPtrs{{dst + off[0], dst + off[1], dst + off[2]}};
    }
    // prefetch: the highest-scored experts not resident, into slots this call does not read,
    // each over the lowest-scored resident expert, never over a higher score
    if (h.prefetch > 0) {
      std::vector<std::pair<float, int>> cand;
      for (int e = 0; e < E; ++e)
        if (cv.expert_slot[e] < 0 && cv.score[e] > 0.f) cand.push_back({cv.score[e], e});
      const size_t want = std::min(cand.size(), (size_t)h.prefetch);
      std::partial_sort(cand.begin(), cand.begin() + want, cand.end(),
                        [](const std::pair<float, int> &a, const std::pair<float, int> &b) {
                          return a.first > b.first || (a.first == b.first && a.second < b.second);
                        });
      for (size_t i = 0; i < want; ++i) {
        int victim = -1;
        float low = 0.f;
        for (int64_t q = 0; q < h.slots; ++q) {
          if (used[q]) continue;
          if (cv.slot_expert[q] < 0) {
            victim = (int)q;
            low = -1.f;
            break;
          }
          const float sc = cv.score[cv.slot_expert[q]];
          if (victim < 0 || sc < low) {
            victim = (int)q;
            low = sc;
          }
        }
        if (victim < 0 || low >= cand[i].first) break;
        const int e = cand[i].second;
        if (cv.slot_expert[victim] >= 0) cv.expert_slot[cv.slot_expert[victim]] = -1;
        cv.slot_expert[victim] = e;
        cv.expert_slot[e] = victim;
        cv.slot_pref[victim] = 1;
        cv.slot_used[victim] = h.clock;
        used[victim] = 1;
        rc = copy_expert(e, h.mem + (int64_t)victim * h.stride, cv.slot_ready[victim]);
        if (rc != TQ_OK) return rc;
        h.stats.prefetched += 1;
        h.stats.bytes_copied += s.expert_bytes;
      }
    }
    // the call's expert table, on the compute stream ahead of the kernels that read it
    if (hipMemcpyAsync(ws + p.off_table, table, (size_t)E * sizeof(tq::MoeExpertPtrs),
                       hipMemcpyHostToDevice, st) != hipSuccess)
      return fail(TQ_EDEVICE, "tq_moe_ffn: expert table copy failed");
    dev_table = reinterpret_cast<const tq::MoeExpertPtrs *>(ws + p.off_table);
    stage_arg = nullptr;
  }
  if (s.mfma || p.qmm) {  // one grouped launch once every copy it reads has landed
    for (int a = 0; a < na; ++a)
      if (wait_ev[a] && hipStreamWaitEvent(st, wait_ev[a], 0) != hipSuccess)
        return fail(TQ_EDEVICE, "tq_moe_ffn: event wait failed");
    return launched(tq::launch_moe_experts(p, dev_table, shared, stage_arg, x, ws, st),
                    "tq_moe_ffn experts");
  }
  auto slot_range = [&](int a) {
    return tq::SlotRange{a, 1, act[S + a], act[2 * S + a]};
  };
  for (int a = 0; a < na; ++a)  // the shared expert first: it needs no copy
    if (act[a] == E) {
      const tq::SlotRange r = slot_range(a);
      rc = tq::launch_moe_experts(p, dev_table, shared, stage_arg, x, ws, st, &r);
      if (rc) return launched(rc, "tq_moe_ffn experts");
    }
  for (int a = 0; a < na; ++a) {
    if (act[a] == E) continue;
    if (hipStreamWaitEvent(st, wait_ev[a], 0) != hipSuccess)
      return fail(TQ_EDEVICE, "tq_moe_ffn: event wait failed");
    const tq::SlotRange r = slot_range(a);
    rc = tq::launch_moe_experts(p, dev_table, shared, stage_arg, x, ws, st, &r);
    if (rc) return launched(rc, "tq_moe_ffn experts");
  }
  return TQ_OK;
}

size_t tq_expert_cache_slot_bytes(const tq_moe_desc *desc) {
  tq::MoeShape s;
  if (moe_check(desc, 1, &s) != TQ_OK) return 0;
  return (size_t)tq::align256(s.expert_bytes);
}

size_t tq_expert_cache_state_bytes(const tq_moe_desc *desc, int64_t slots) {
  tq::MoeShape s;
  if (slots < 1 || slots > 4096 || moe_check(desc, 1, &s) != TQ_OK) return 0;
  size_t off[6];
  return cache_layout(slots, s.n_experts, off);
}

int tq_expert_cache_init(void *state, size_t state_bytes, const tq_moe_desc *desc, int64_t slots,
                         int64_t prefetch, void *slot_mem, size_t slot_mem_bytes) {
  tq::MoeShape s;
  int rc = moe_check(desc, 1, &s);
  if (rc != TQ_OK) return rc;
  if (!state || !slot_mem) return fail(TQ_EINVAL, "tq_expert_cache_init: null state or slot memory");
  if (slots < 1 || slots > 4096 || prefetch < 0 || prefetch > slots)
    return fail(TQ_ESHAPE, "tq_expert_cache_init: slots=%lld prefetch=%lld (need 1..4096, 0..slots)",
                (long long)slots, (long long)prefetch);
  if (!aligned(state, 64) || !aligned(slot_mem, 256))
    return fail(TQ_EALIGN, "tq_expert_cache_init: state 64-byte and slot memory 256-byte alignment needed");
  size_t off[6];
  if (state_bytes < cache_layout(slots, s.n_experts, off))
    return fail(TQ_ENOSPC, "tq_expert_cache_init: state of %zu bytes too small", state_bytes);
  const int64_t stride = tq::align256(s.expert_bytes);
  if (slot_mem_bytes < (size_t)(slots * stride))
    return fail(TQ_ENOSPC, "tq_expert_cache_init: slot memory of %zu bytes, %lld needed", slot_mem_bytes,
                (long long)(slots * stride));
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(TQ_EDEVICE, "tq_expert_cache_init: no current device");
  CacheHeader *h = (CacheHeader *)state;
  *h = CacheHeader{};
  h->device = dev;
  h->type = (int)s.type;
  h->hidden = s.hidden;
  h->ffn = s.ffn;
  h->n_experts = s.n_experts;
  h->expert_bytes = s.expert_bytes;
  h->gate_bytes = s.gate_bytes;
  h->slots = slots;
  h->prefetch = prefetch;
  h->stride = stride;
  h->mem = (uint8_t *)slot_mem;
  CacheView v = cache_view(state);
  for (int64_t q = 0; q < slots; ++q) {
    v.slot_expert[q] = -1;
    v.slot_used[q] = 0;
    v.slot_pref[q] = 0;
    v.slot_ready[q] = nullptr;
  }
  for (int64_t e = 0; e < s.n_experts; ++e) {
    v.expert_slot[e] = -1;
    v.score[e] = 0.f;
  }
  for (int64_t q = 0; q < slots; ++q)
    if (hipEventCreateWithFlags(&v.slot_ready[q], hipEventDisableTiming) != hipSuccess) {
      for (int64_t r = 0; r < q; ++r) (void)hipEventDestroy(v.slot_ready[r]);
      return fail(TQ_EDEVICE, "tq_expert_cache_init: event creation failed");
    }
  h->magic = kCacheMagic;
  return TQ_OK;
}

int tq_expert_cache_stats_get(const void *state, tq_expert_cache_stats *out) {
  if (!state || !out) return fail(TQ_EINVAL, "tq_expert_cache_stats_get: null argument");
  const CacheHeader *h = (const CacheHeader *)state;
  if (h->magic != kCacheMagic) return fail(TQ_EINVAL, "tq_expert_cache_stats_get: not a cache state");
  *out = h->stats;
  return TQ_OK;
}

int tq_expert_cache_destroy(void *state) {
  if (!state) return fail(TQ_EINVAL, "tq_expert_cache_destroy: null state");
  CacheHeader *h = (CacheHeader *)state;
  if (h->magic != kCacheMagic) return fail(TQ_EINVAL, "tq_expert_cache_destroy: not a cache state");
  CacheView v = cache_view(state);
  for (int64_t q = 0; q < h->slots; ++q) (void)hipEventDestroy(v.slot_ready[q]);
  h->magic = 0;
  return TQ_OK;
}

int tq_moe_ffn_stages(const tq_moe_desc *d, const float *x, int64_t tokens, float *y,
                      void *workspace, size_t ws_bytes, tq_moe_routing *routing_out, int stages,
                      void *stream) {
  tq::MoeShape s;
  int rc = moe_check(d, tokens, &s);
  if (rc != TQ_OK) return rc;
  if (stages <= 0 || (stages & ~TQ_MOE_ALL))
    return fail(TQ_EINVAL, "tq_moe_ffn: stage mask %d not a non-empty subset of TQ_MOE_ALL", stages);
  if (!x || !workspace || ((stages & TQ_MOE_COMBINE) && !y))
    return fail(TQ_EINVAL, "tq_moe_ffn: null x, y or workspace");
  if (!aligned(x, 16) || !aligned(y, 4) || !aligned(workspace, 256))
    return fail(TQ_EALIGN, "tq_moe_ffn: x 16-byte, y 4-byte, workspace 256-byte alignment needed");
  const tq::MoePlan p = tq::plan_moe(s);
  if (ws_bytes < (size_t)p.bytes)
    return fail(TQ_ENOSPC, "tq_moe_ffn: workspace of %zu bytes, %lld needed", ws_bytes, (long long)p.bytes);
  if (s.experts_on_host && (stages & TQ_MOE_EXPERTS) && !host_experts_ok(d))
    return fail(TQ_EINVAL, "tq_moe_ffn: experts_host entries must all be non-null");
  if (d->expert_cache && !s.experts_on_host)
    return fail(TQ_EINVAL, "tq_moe_ffn: expert_cache is for host-resident experts only");
  if (d->expert_cache && ((const CacheHeader *)d->expert_cache)->magic != kCacheMagic)
    return fail(TQ_EINVAL, "tq_moe_ffn: expert_cache is not an initialized cache state");
  hipStream_t st = (hipStream_t)stream;
  char *ws = (char *)workspace;
  // one token, every stage in this call: the combine runs inside the down launch, and (matrix-core
  // experts) the top-k selection inside the gate/up launch
  const bool fuse = stages == TQ_MOE_ALL && !s.experts_on_host && tq::moe_fuse_combine_ok(p);
  const bool route1 = fuse && p.route1;
  auto copy_routing = [&]() -> int {
    if (!routing_out) return TQ_OK;
    const int64_t T = tokens, E = s.n_experts, k = s.top_k;
    struct { void *dst; int64_t off, bytes; } cp[] = {
        {routing_out->topk_ids, p.off_ids, T * k * 4}, {routing_out->topk_w, p.off_wts, T * k * 4},
        {routing_out->logits, p.off_logits, T * E * 4}, {routing_out->counts, p.off_counts, E * 4},
        {routing_out->offsets, p.off_offsets, (E + 1) * 4}, {routing_out->pairs, p.off_pairs, T * k * 4}};
    for (auto &c : cp)
      if (c.dst && hipMemcpyAsync(c.dst, ws + c.off, (size_t)c.bytes, hipMemcpyDeviceToDevice, st) != hipSuccess)
        return fail(TQ_EDEVICE, "tq_moe_ffn: routing copy failed");
    return TQ_OK;
  };
  if (stages & TQ_MOE_ROUTE) {
    if (tq::launch_moe_routing(p, d->router_w, x, ws, st, route1))
      return launched(-1, "tq_moe_ffn routing");
    if (!route1 && (rc = copy_routing()) != TQ_OK) return rc;
  }
  if (stages & TQ_MOE_EXPERTS) {
    tq::MoeExpertPtrs shared{{d->shared.gate, d->shared.up, d->shared.down}};
    if (s.experts_on_host) {
      rc = host_resident_experts(d, p, shared, x, ws, st);
      if (rc != TQ_OK) return rc;
    } else {
      rc = tq::launch_moe_experts(p, reinterpret_cast<const tq::MoeExpertPtrs *>(d->experts),
                                  shared, nullptr, x, ws, st, nullptr, fuse ? y : nullptr, route1);
      if (rc) return launched(rc, "tq_moe_ffn experts");
      if (route1 && (rc = copy_routing()) != TQ_OK) return rc;
    }
  }
  if ((stages & TQ_MOE_COMBINE) && !fuse) {
    if (tq::launch_moe_combine(p, ws, y, st)) return launched(-1, "tq_moe_ffn combine");
  }
  return TQ_OK;
}

int tq_moe_ffn(const tq_moe_desc *d, const float *x, int64_t tokens, float *y, void *workspace,
               size_t ws_bytes, tq_moe_routing *routing_out, void *stream) {
  if (!y) return fail(TQ_EINVAL, "tq_moe_ffn: null x, y or workspace");
  return tq_moe_ffn_stages(d, x, tokens, y, workspace, ws_bytes, routing_out, TQ_MOE_ALL, stream);
}

size_t tq_chain_plan_bytes(int nops) {
  if (nops < 1 || nops > tq::kChainMaxOps) return 0;
  return tq::chain_plan_bytes(nops);
}

int tq_chain_prepare(int type, const tq_chain_op *ops, int nops, void *plan, size_t plan_bytes) {
  if (type != TQ_Q4_K) {
    if (!known_type(type)) return fail(TQ_EINVAL, "tq_chain_prepare: unknown block type %d", type);
    return fail(TQ_EUNSUPPORTED, "tq_chain_prepare: chains take Q4_K products only");
  }
  if (!ops || !plan) return fail(TQ_EINVAL, "tq_chain_prepare: null ops or plan");
  if (nops < 1 || nops > tq::kChainMaxOps)
    return fail(TQ_ESHAPE, "tq_chain_prepare: nops=%d not in 1..%d", nops, tq::kChainMaxOps);
  if (plan_bytes < tq::chain_plan_bytes(nops))
    return fail(TQ_ENOSPC, "tq_chain_prepare: plan has %zu bytes, needs %zu", plan_bytes,
                tq::chain_plan_bytes(nops));
  if (!aligned(plan, 256)) return fail(TQ_EALIGN, "tq_chain_prepare: plan must be 256-byte aligned");
  std::vector<tq::ChainOpDesc> d((size_t)nops);
  for (int i = 0; i < nops; ++i) {
    const tq_chain_op &o = ops[i];
    if (o.swiglu != 0 && o.swiglu != 1)
      return fail(TQ_EINVAL, "tq_chain_prepare: op %d: swiglu must be 0 or 1", i);
    const int np = o.swiglu ? 2 : o.nparts;
    if (np < 1 || np > 4 || (o.swiglu && o.nparts != 2))
      return fail(TQ_EINVAL, "tq_chain_prepare: op %d: nparts=%d (1..4, 2 with swiglu)", i, o.nparts);
    if (o.k < 256 || o.k > 16384 || o.k % 256)
      return fail(TQ_ESHAPE, "tq_chain_prepare: op %d: k=%lld (a multiple of 256 in 256..16384)", i,
                  (long long)o.k);
    if (!o.x) return fail(TQ_EINVAL, "tq_chain_prepare: op %d: null x", i);
    if (!aligned(o.x, 16)) return fail(TQ_EALIGN, "tq_chain_prepare: op %d: x must be 16-byte aligned", i);
    int64_t rows = 0;
    for (int p = 0; p < np; ++p) {
      if (!o.w[p] || (!o.y[p] && !(o.swiglu && p == 1)))
        return fail(TQ_EINVAL, "tq_chain_prepare: op %d: null w or y of matrix %d", i, p);
      if (o.n[p] < 1 || o.n[p] > (1 << 26))
        return fail(TQ_ESHAPE, "tq_chain_prepare: op %d: n[%d]=%lld", i, p, (long long)o.n[p]);
      if (!aligned(o.w[p], 16) || (o.y[p] && !aligned(o.y[p], 4)))
        return fail(TQ_EALIGN, "tq_chain_prepare: op %d: w 16-byte, y 4-byte alignment needed", i);
      rows += o.n[p];
    }
    if (o.swiglu && o.n[0] != o.n[1])
      return fail(TQ_ESHAPE, "tq_chain_prepare: op %d: gate and up rows differ", i);
    if (rows > (1 << 27)) return fail(TQ_ESHAPE, "tq_chain_prepare: op %d: too many rows", i);
    d[i].nparts = np;
    d[i].swiglu = o.swiglu;
    for (int p = 0; p < 4; ++p) {
      d[i].w[p] = p < np ? o.w[p] : o.w[0];
      d[i].n[p] = p < np ? o.n[p] : 0;
      d[i].y[p] = p < np ? o.y[p] : o.y[0];
    }
    d[i].k = o.k;
    d[i].x = o.x;
  }
  std::vector<char> buf;
  if (tq::chain_build(d.data(), nops, buf)) return fail(TQ_ESHAPE, "tq_chain_prepare: too many items");
  if (hipMemcpy(plan, buf.data(), buf.size(), hipMemcpyHostToDevice) != hipSuccess)
    return fail(TQ_EDEVICE, "tq_chain_prepare: copy of the plan failed: %s",
                hipGetErrorString(hipGetLastError()));
  return TQ_OK;
}

int tq_chain_run(void *plan, void *stream) {
  if (!plan) return fail(TQ_EINVAL, "tq_chain_run: null plan");
  if (!aligned(plan, 256)) return fail(TQ_EALIGN, "tq_chain_run: plan must be 256-byte aligned");
  (void)stream;
  // Switched off: the persistent kernel's device-side waits assume that every workgroup of the
  // grid is resident at once, which an ordinary launch does not guarantee; one run of it left
  // the device hung. It stays off until the launch guarantees residency (or the work is dealt
  // by in-order tickets, which needs no residency) and the waits are bounded in time.
  return fail(TQ_EUNSUPPORTED, "tq_chain_run: the persistent chain is switched off in this build "
                               "(its waits need every workgroup resident, which a plain launch "
                               "does not guarantee)");
}

int tq_chain_status(void *plan, void *stream) {
  if (!plan) return fail(TQ_EINVAL, "tq_chain_status: null plan");
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
    return fail(TQ_EDEVICE, "tq_chain_status: stream synchronisation failed: %s",
                hipGetErrorString(hipGetLastError()));
  unsigned word = 0;
  char *err = (char *)plan + tq::kChainErrorOffset;
  if (hipMemcpy(&word, err, sizeof word, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(TQ_EDEVICE, "tq_chain_status: reading the error word failed");
  if (word == 0) return TQ_OK;
  const unsigned zero = 0;
  if (hipMemcpy(err, &zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess)
    return fail(TQ_EDEVICE, "tq_chain_status: clearing the error word failed");
  static const char *const kinds[] = {"?", "for the op before it to complete",
                                      "for its input to be staged", "for room in the sums ring",
                                      "for the slice sums of an item"};
  const unsigned kind = word >> 24;
  return fail(TQ_EDEVICE, "tq_chain_status: a run gave up waiting %s at op %u (the chain's "
                          "workgroups were not all resident, or the device stalled); its outputs "
                          "are undefined", kinds[kind < 5 ? kind : 0], word & 0xFFFFFFu);
}

}  // extern "C"
