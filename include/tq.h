/*
 * tq.h -- C ABI of libtq: block-quantized decode products and top-k MoE expert FFNs on gfx950.
 *
 * The operations follow the problem the pages state for decoding large quantized models: a
 * block-quantized weight blob plus activations in, projected activations (or the routed MoE
 * output) out ("Titan Engine" page (zingnex.cn), sections "Aggressive quantization" and "MoE
 * expert streaming"; KTransformers page (news.fishai.com.cn), the part on quantized GPU
 * matmul kernels and MoE expert handling; "Show HN: Llama 3.1 70B on a single RTX 3090 via
 * NVMe-to-GPU bypassing the CPU" page (hn.213312.xyz), "Quantization support").
 *
 * Block formats (GGUF block layouts, little-endian; the pages name the formats, not the bits):
 *   TQ_Q4_K  256 weights / 144 bytes: d fp16, dmin fp16, 12 bytes of packed 6-bit scales and
 *            mins, 128 bytes of 4-bit quants; w = d*sc*q - dmin*m.
 *   TQ_Q6_K  256 weights / 210 bytes: 128 bytes low 4 bits, 64 bytes high 2 bits, 16 int8
 *            scales, d fp16; w = d*sc*(q - 32).
 *   TQ_Q8_0  32 weights / 34 bytes: d fp16, 32 int8 quants; w = d*q.
 *   TQ_Q5_K  256 weights / 176 bytes: d fp16, dmin fp16, the 12 scale/min bytes of Q4_K, 32 bytes
 *            of fifth bits (bit j of byte l: position l of sub-block j), 128 bytes of low 4 bits
 *            laid out as Q4_K's; w = d*sc*q - dmin*m with q in 0..31.
 *   TQ_Q4_0  32 weights / 18 bytes: d fp16, 16 bytes of nibbles (weight i < 16 the low nibble of
 *            byte i, weight i >= 16 the high nibble of byte i-16); w = d*(q - 8).
 *            (Q5_K and Q4_0: the "Show HN" page's "Quantization support" list.)
 * A weight matrix is n rows ("out") by k columns ("in"), stored row-major as n rows of k/B
 * consecutive blocks (B = weights per block), i.e. n * tq_row_bytes(type, k) bytes.
 *
 * Conventions for every call below:
 *   - Pointers are device pointers (memory the caller allocated on the current HIP device)
 *     unless stated otherwise. The caller owns every buffer; the library allocates no device
 *     memory. One exception on the host: the host-resident MoE variant (experts_on_host) keeps,
 *     per calling thread and device, a small pinned host buffer (the active-expert list and the
 *     call's expert-pointer table) and HIP events, made on first use and kept until the thread
 *     ends.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Every call only
 *     enqueues work on it and returns; results are ready when the stream is synchronized.
 *   - Arguments are checked before anything is enqueued. On a non-TQ_OK status nothing was
 *     enqueued and no output was touched; tq_last_error() returns a description (thread-local).
 *   - A device fault inside a kernel surfaces at the caller's next synchronization (HIP rules).
 *   - Activations and outputs are fp32, token-major: x[t][k], y[t][n].
 *   - Calls on one stream are deterministic: the same inputs give bitwise-identical outputs.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { TQ_Q4_K = 1, TQ_Q6_K = 2, TQ_Q8_0 = 3, TQ_Q5_K = 4, TQ_Q4_0 = 5 }; /* block formats */
enum { TQ_F32 = 0, TQ_BF16 = 1 };                                /* dequant output types */
enum {                                                           /* status codes */
  TQ_OK = 0,
  TQ_EINVAL = 1,       /* null pointer, unknown enum value, negative count */
  TQ_ESHAPE = 2,       /* k not a multiple of the block size, n/batch/tokens out of range */
  TQ_EALIGN = 3,       /* a pointer is not aligned as required */
  TQ_ENOSPC = 4,       /* workspace smaller than tq_moe_workspace_bytes() */
  TQ_EUNSUPPORTED = 5, /* valid request this build does not handle */
  TQ_EDEVICE = 6       /* a HIP runtime call failed (launch, copy, event) */
};
enum { TQ_PATH_AUTO = 0, TQ_PATH_F32 = 1, TQ_PATH_BF16_MFMA = 2 }; /* MoE expert-product path */

/* Weights per block (Q4_K, Q6_K, Q8_0, Q5_K, Q4_0: 256, 256, 32, 256, 32) and bytes per block
 * (144, 210, 34, 176, 18); 0 for an unknown type. */
int64_t tq_block_weights(int type);
int64_t tq_block_bytes(int type);
/* Bytes of one row of k weights; -1 if type is unknown or k is not a multiple of the block. */
int64_t tq_row_bytes(int type, int64_t k);

/*
 * tq_dequant -- expand a blob to dense values (the block decode of the formats above).
 *   w     [n rows of tq_row_bytes(type,k)] blob, 16-byte aligned.
 *   out   [n][k] of out_type: TQ_F32 holds each weight's exact value rounded once to nearest
 *         even (bitwise equal to the exact value for Q6_K, Q8_0 and Q4_0); TQ_BF16 holds the
 *         nearest-even bf16 rounding of that fp32 value, as uint16 bit patterns. 4-byte aligned.
 *   n >= 0, k >= 0 with k % tq_block_weights(type) == 0; n*k == 0 enqueues nothing.
 */
int tq_dequant(int type, const void *w, int64_t n, int64_t k, int out_type, void *out,
               void *stream);

/*
 * tq_gemv -- y[t][r] = sum_c w[r][c] * x[t][c] for t < batch, r < n (decode-time GEMV and
 * small-batch GEMM over quantized weights), fp32 multiply-adds.
 *   w          blob of n x k weights, 16-byte aligned.
 *   x          [batch][k] fp32, 4-byte aligned; y [batch][n] fp32, 4-byte aligned; y must not
 *              overlap w or x.
 *   workspace  device scratch of at least tq_gemv_workspace_bytes(type, n, k, batch) bytes,
 *              256-byte aligned, any contents (its completion counters carry a token that
 *              differs for every call, so bytes left by other work are never taken for a count;
 *              nothing needs clearing before or after). It lets the k dimension be split across
 *              workgroups (the partial sums are added in a fixed order, so results stay
 *              deterministic), also for the int8 matrix-core kernel that takes Q4_K at batch 1
 *              for k >= 16384 (its k-slice sums after the first 64 KiB). NULL or too small: no
 *              split and no matrix-core kernel (slower; results still within the fp32 bar,
 *              though not bitwise those of a call with the workspace). Calls that run
 *              concurrently must not share a workspace.
 *   n >= 1, k >= block size with k % block == 0, 1 <= batch <= 4096. Weights are streamed once
 *   per group of up to 8 tokens; for Q4_K with 2..32 tokens (given the workspace) once for all of
 *   them, on the fp16 matrix cores with exact operands (each activation row scaled by a power of
 *   two and split into fp16 hi + lo, sc * q and the mins as exact fp16 integers), fp32
 *   accumulation. Q8_0 at 2..16 tokens and Q6_K (k % 512 == 0) at 4..16 tokens stream them once
 *   on the fp32 matrix cores, with the exactly dequantized weights as operands (x 16-byte
 *   aligned; the workspace when k spans more than one slice of 8 blocks). Q5_K and Q4_0 take the
 *   lane-per-row fp32 kernel (k % 256 == 0; other Q4_0 k: a per-weight kernel).
 */
size_t tq_gemv_workspace_bytes(int type, int64_t n, int64_t k, int64_t batch);
int tq_gemv(int type, const void *w, int64_t n, int64_t k, const float *x, int64_t batch,
            float *y, void *workspace, size_t ws_bytes, void *stream);

/*
 * tq_gemv_noalloc -- tq_gemv for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc). Same arguments and result as
 * tq_gemv given a workspace of tq_gemv_workspace_bytes(type, n, k, batch) bytes (bitwise), minus
 * the workspace: it uses a scratch array that the library holds on each device (statically, in
 * its code object, until the process ends). Allocates nothing, clears nothing (the scratch may
 * hold anything, as tq_gemv's workspace may).
 *   Returns TQ_ENOSPC when that workspace size exceeds TQ_GEMV_NOALLOC_MAX_BYTES (16 MiB: every
 *   8B- and 70B-shaped projection up to batch 16), TQ_EDEVICE when the scratch's device address
 *   cannot be found.
 *   All calls on one device share its scratch: calls that can overlap on one device (other
 *   streams, other threads) race and must be serialized by the caller.
 */
#define TQ_GEMV_NOALLOC_MAX_BYTES (16u << 20)
int tq_gemv_noalloc(int type, const void *w, int64_t n, int64_t k, const float *x, int64_t batch,
                    float *y, void *stream);

/*
 * tq_gemv_multi -- y_p = W_p x for nparts (1..4) matrices of one block type and the same k that
 * share the activations x (the q, k and v projections of a decode step read the same x), in one
 * launch for Q4_K at batch 1..32 (given the workspace; at batch 1 also without) and for the
 * Q6_K / Q8_0 batches that tq_gemv takes on the fp32 matrix cores, else one launch per matrix.
 *   w, n, y   host arrays of nparts entries: device blob w[p] ([n[p]][k], 16-byte aligned),
 *             rows n[p], device output y[p] ([batch][n[p]] fp32)
 *   x         device [batch][k] fp32, 16-byte aligned
 *   workspace as for tq_gemv: tq_gemv_multi_workspace_bytes(...) bytes, or NULL / smaller
 *             (slower kernels).
 * Each y[p] is bitwise what tq_gemv(type, w[p], n[p], k, x, ...) gives with a workspace of the
 * size each call asks for.
 */
size_t tq_gemv_multi_workspace_bytes(int type, int nparts, const int64_t *n, int64_t k,
                                     int64_t batch);
int tq_gemv_multi(int type, int nparts, const void *const *w, const int64_t *n, float *const *y,
                  int64_t k, const float *x, int64_t batch, void *workspace, size_t ws_bytes,
                  void *stream);

/*
 * tq_gemv_swiglu -- h[t][r] = silu(g) * u with g = (W_gate x_t)[r], u = (W_up x_t)[r] and
 * silu(z) = z / (1 + exp(-z)): the gate and up projections of a SwiGLU FFN and the gating
 * between them (the Llama-family feed-forward; the pages name the models, not the formula), in
 * one launch for Q4_K at batch 1 (gate and up rows interleaved inside the kernel), at batch
 * 2..32 given the workspace (gate and up tiles side by side), and for the Q6_K / Q8_0 batches
 * that tq_gemv takes on the fp32 matrix cores (rows interleaved); otherwise two tq_gemv launches and
 * tq_swiglu through the workspace. w_gate, w_up [n][k]; x [batch][k] (16-byte aligned); h
 * [batch][n] fp32. workspace: tq_gemv_swiglu_workspace_bytes(type, n, k, batch) bytes, 256-byte
 * aligned; on the one-launch path it holds the k-slice sums of the int8 matrix-core kernel
 * (k >= 16384) and may be NULL or smaller (the lanes-along-k kernel runs instead). Bitwise
 * equal to tq_gemv + tq_gemv + tq_swiglu when each call gets the workspace it asks for.
 */
size_t tq_gemv_swiglu_workspace_bytes(int type, int64_t n, int64_t k, int64_t batch);
int tq_gemv_swiglu(int type, const void *w_gate, const void *w_up, int64_t n, int64_t k,
                   const float *x, int64_t batch, float *h, void *workspace, size_t ws_bytes,
                   void *stream);

/*
 * tq_swiglu -- h[i] = silu(g[i]) * u[i], silu(z) = z / (1 + exp(-z)), for i < count (the
 * gated activation between a SwiGLU FFN's gate/up and down projections). fp32, 4-byte
 * aligned; h may alias g or u. count >= 0.
 */
int tq_swiglu(const float *g, const float *u, int64_t count, float *h, void *stream);

/* ---- top-k routed MoE expert FFN ------------------------------------------------------------
 * The layer the pages describe for mixture-of-experts models: a router scores every expert per
 * token, only the top k experts run (e.g. 2 of 8, so three quarters of the expert weights are not
 * touched: "Titan Engine" page, "MoE expert streaming"), each expert is a SwiGLU FFN over
 * block-quantized weights, and an always-on shared expert may be added (DeepSeek-V3-shaped
 * layers; KTransformers page, MoE on the 671B model).
 *
 *   logits[t][e] = sum_h x[t][h] * router_w[e][h]                                  (fp32)
 *   ids[t][0..k-1]  = the k largest logits, ties to the lower expert index; slot j holds the j-th
 *   w[t][j]         = exp(l_j - l_0) / sum_{i < k} exp(l_i - l_0)       (renormalize = 1), or
 *                     exp(l_j - l_0) / sum_{e < E} exp(l_e - l_0)       (renormalize = 0)
 *   y[t] = sum_j w[t][j] * down_e . silu(gate_e . x_t) * (up_e . x_t)   (e = ids[t][j], j in order)
 *        + down_s . silu(gate_s . x_t) * (up_s . x_t)                   (shared expert, if any)
 * silu(z) = z / (1 + exp(-z)). Expert matrices: gate, up [ffn][hidden]; down [hidden][ffn].
 */
typedef struct {
  const void *gate, *up, *down; /* blobs of one expert, 16-byte aligned */
} tq_expert;

typedef struct {
  int type;                      /* block format of every expert matrix (any of the five on the
                                    fp32 path; Q4_K only on TQ_PATH_BF16_MFMA) */
  int64_t hidden, ffn;           /* multiples of 256 */
  int64_t n_experts, top_k;      /* 1 <= top_k <= min(n_experts, 32), n_experts <= 1024 */
  const float *router_w;         /* device [n_experts][hidden] fp32, 16-byte aligned */
  const tq_expert *experts;      /* device array [n_experts] of device blob pointers */
  const tq_expert *experts_host; /* host array [n_experts] of pinned host blob pointers; used
                                    instead of `experts` (which may then be NULL) when
                                    experts_on_host is set */
  tq_expert shared;              /* device blobs of the shared expert; gate == NULL: none */
  int renormalize;               /* 1: weights renormalised over the selected experts */
  int experts_on_host;           /* 1: routed experts live in pinned host memory and are copied
                                    to the workspace on every call (see tq_moe_ffn) */
  void *copy_stream;             /* hipStream_t for those copies (experts_on_host only) */
  int path;                      /* TQ_PATH_AUTO / TQ_PATH_F32 / TQ_PATH_BF16_MFMA */
  void *expert_cache;            /* NULL, or a residency cache set up by tq_expert_cache_init
                                    for this descriptor (experts_on_host only) */
} tq_moe_desc;

typedef struct {                 /* optional copies of the routing, device pointers or NULL */
  int32_t *topk_ids;             /* [T][k] */
  float *topk_w;                 /* [T][k] */
  float *logits;                 /* [T][n_experts], the fp32 values the selection used */
  int32_t *counts;               /* [n_experts] tokens routed to each expert */
  int32_t *offsets;              /* [n_experts + 1] exclusive prefix sum of counts */
  int32_t *pairs;                /* [T*k] t*k + j, sorted by (expert, t) */
} tq_moe_routing;

/*
 * Expert residency cache for the host-resident variant: device slots that keep routed experts
 * between calls, so that an expert used again is not copied again, plus prefetch of the experts
 * most likely to be routed next (the pages' expert streaming: "Titan Engine" page, "MoE expert
 * streaming" -- an LRU expert cache in VRAM, smart prefetch, asynchronous loading; "Show HN" page,
 * "Technical highlights" -- double-buffered streaming that overlaps transfers with compute).
 *
 * The caller owns both pieces of memory: `state` (host, tq_expert_cache_state_bytes) and
 * `slot_mem` (device, slots * tq_expert_cache_slot_bytes, 256-byte aligned). Setting
 * desc->expert_cache = state makes every tq_moe_ffn call with experts_on_host use it:
 *   - a routed expert held by a slot is read there (a hit: no copy);
 *   - otherwise it is copied into the least recently used slot that this call does not use (a
 *     miss), or, when every slot is taken by the call, into the workspace's staging area as
 *     without a cache (a fallback);
 *   - then up to `prefetch` experts that are not resident are copied, highest score first (every
 *     call multiplies each expert's score by 7/8 and adds 1 for each expert it routes to), each
 *     into an empty slot or over the lowest-scored expert in a slot this call does not read, and
 *     never over an expert with the same or a higher score. Prefetches run on the copy stream
 *     behind this call's demand copies, so they overlap with this call's compute.
 * Each slot has an event: the call's kernels wait for the copies of the slots they read, and a
 * slot is overwritten only after the compute stream has finished the calls before the current
 * one. Results are bitwise those of the call without a cache. One state per descriptor and per
 * device; calls that use one state must not overlap (they share its slots and bookkeeping).
 */
typedef struct {
  int64_t calls;         /* tq_moe_ffn calls that used the cache */
  int64_t hits;          /* routed experts found in a slot */
  int64_t misses;        /* routed experts copied into a slot when routed */
  int64_t fallbacks;     /* routed experts staged in the workspace (no free slot this call) */
  int64_t prefetched;    /* experts copied ahead of their use */
  int64_t prefetch_hits; /* hits on a prefetched slot before any other use of it */
  int64_t bytes_copied;  /* host-to-device bytes of all the copies above */
} tq_expert_cache_stats;

/* Device bytes of one slot (one routed expert's three blobs, 256-byte aligned); 0 if invalid. */
size_t tq_expert_cache_slot_bytes(const tq_moe_desc *desc);
/* Host bytes of the cache state for `slots` slots (1..4096); 0 if invalid. */
size_t tq_expert_cache_state_bytes(const tq_moe_desc *desc, int64_t slots);
/* Set up `state` (empty slots, zero statistics) on the current device; creates one HIP event per
 * slot. prefetch: 0..slots experts copied ahead per call. */
int tq_expert_cache_init(void *state, size_t state_bytes, const tq_moe_desc *desc, int64_t slots,
                         int64_t prefetch, void *slot_mem, size_t slot_mem_bytes);
/* Counters since tq_expert_cache_init. */
int tq_expert_cache_stats_get(const void *state, tq_expert_cache_stats *out);
/* Releases the state's events (the caller then frees both pieces of memory). */
int tq_expert_cache_destroy(void *state);

/* Workspace bytes tq_moe_ffn needs for `tokens` tokens (0 if the descriptor is invalid). */
size_t tq_moe_workspace_bytes(const tq_moe_desc *desc, int64_t tokens);

/*
 * tq_moe_ffn -- y = MoE(x) as above for x [tokens][hidden] fp32 (device, 16-byte aligned), y
 * [tokens][hidden] fp32 (device). workspace: device scratch of at least
 * tq_moe_workspace_bytes(desc, tokens) bytes, 256-byte aligned, contents irrelevant; one call at a
 * time per workspace. routing_out: NULL or copies of the routing (each field may be NULL).
 * 1 <= tokens <= 8192. Everything is enqueued on `stream` without host synchronisation, except
 * with experts_on_host (routed experts kept in host memory, the pages' offload setting): the
 * active-expert list is then copied to the host (one synchronisation of `stream`, so such calls
 * cannot be captured into a graph) and each selected expert is copied from pinned host memory
 * into the workspace with hipMemcpyAsync on copy_stream (NULL: on `stream`), each followed by an
 * event. The shared expert (always on the device) runs first; where each expert has kernels of
 * its own (one token, or Q6_K / Q8_0) they wait only for their own copy; on the matrix-core paths
 * (bf16 prefill; Q4_K with 2+ tokens) one grouped launch waits for all copies. Host blobs must
 * stay valid until the call's work has completed; they must be pinned (hipHostMalloc) for the
 * copies to be asynchronous. The output is bitwise identical to the device-resident call's.
 * A one-token Q4_K call with the experts on the device adds the slots inside its down launch
 * (the last workgroup of each row range, counted on counters the same call clears first); the
 * output is bitwise what the separate combine stage gives.
 * Deterministic: the same inputs give bitwise-identical outputs and routing.
 */
int tq_moe_ffn(const tq_moe_desc *desc, const float *x, int64_t tokens, float *y,
               void *workspace, size_t ws_bytes, tq_moe_routing *routing_out, void *stream);

/* Stages of tq_moe_ffn, for tq_moe_ffn_stages. */
enum { TQ_MOE_ROUTE = 1, TQ_MOE_EXPERTS = 2, TQ_MOE_COMBINE = 4, TQ_MOE_ALL = 7 };

/*
 * tq_moe_ffn_stages -- the stages of tq_moe_ffn selected by the bit mask `stages`, enqueued in
 * the order route, experts, combine:
 *   TQ_MOE_ROUTE    logits, top-k selection and the grouping of the (token, slot) pairs per
 *                   expert (the selection step of the MoE layer above); fills routing_out;
 *   TQ_MOE_EXPERTS  every selected expert's SwiGLU FFN on its grouped tokens, and the shared
 *                   expert's on all tokens, into per-pair outputs kept in the workspace;
 *   TQ_MOE_COMBINE  y[t] = the routing-weighted sum of token t's pair outputs (slot order),
 *                   plus the shared expert's.
 * Arguments as for tq_moe_ffn (y may be NULL without TQ_MOE_COMBINE). The workspace carries the
 * state between stages: a call without TQ_MOE_ROUTE relies on an earlier call, on the same
 * stream, with the same desc, tokens, x and workspace, that ran the stages before it. The result
 * equals tq_moe_ffn's. Lets a caller time the stages or place work between them.
 */
int tq_moe_ffn_stages(const tq_moe_desc *desc, const float *x, int64_t tokens, float *y,
                      void *workspace, size_t ws_bytes, tq_moe_routing *routing_out, int stages,
                      void *stream);

/* ---- a decode step as one launch ------------------------------------------------------------
 * A decode step is a chain of products in which every product's input derives from the output of
 * the product before it: q|k|v, then (attention) o, then (residual and norm) gate|up with the
 * SwiGLU, then down, then (residual and norm) the next layer. KTransformers replays each decode
 * step as one CUDA graph (KTransformers page (news.fishai.com.cn), "KTransformers 的技术原理",
 * "CUDA Graph 优化"); here the whole chain of batch-1 Q4_K products runs as one persistent
 * launch that fetches every product's weights before the product's input is ready.
 *
 * Each op is a tq_gemv_multi (nparts matrices sharing x, batch 1) or, with swiglu set, a
 * tq_gemv_swiglu (w[0] gate, w[1] up, h in y[0]), and each output is bitwise what that call gives.
 * Op i reads its x only after op i-1 has stored all of its outputs, so an op may read (or
 * overwrite) any buffer that an earlier op wrote or read. Weights must not be written by the chain.
 */
typedef struct {
  int nparts;          /* 1..4 matrices sharing x, rows taken one after another (2 with swiglu) */
  int swiglu;          /* 0, or 1: y[0][r] = silu((w[0] x)[r]) * (w[1] x)[r], n[0] == n[1] */
  const void *w[4];    /* device Q4_K blobs [n[p]][k], 16-byte aligned (entries past nparts unused) */
  int64_t n[4];        /* rows of each matrix, >= 1 */
  float *y[4];         /* device outputs [n[p]] fp32, 4-byte aligned (swiglu: y[0] only, [n[0]]) */
  int64_t k;           /* a multiple of 256, 256 <= k <= 16384 */
  const float *x;      /* device [k] fp32, 16-byte aligned */
} tq_chain_op;

/* Bytes of the plan of a chain of nops ops (1..4096); 0 if nops is out of range. */
size_t tq_chain_plan_bytes(int nops);

/*
 * tq_chain_prepare -- check the ops (type must be TQ_Q4_K) and write the chain's plan into plan
 * (device memory of tq_chain_plan_bytes(nops) bytes, 256-byte aligned, contents irrelevant).
 * Synchronous (it copies the plan to the device and waits); the ops array may be freed when it
 * returns. The plan holds the device pointers of the ops, which must stay valid while it is run.
 */
int tq_chain_prepare(int type, const tq_chain_op *ops, int nops, void *plan, size_t plan_bytes);

/*
 * tq_chain_run -- SWITCHED OFF in this build: returns TQ_EUNSUPPORTED and enqueues nothing (the
 * persistent kernel's waits need every workgroup of its grid resident at once, which a plain
 * launch does not guarantee). When enabled it enqueues one run of a prepared chain on `stream`:
 * a small kernel that clears the
 * plan's completion counters, then the persistent kernel (its workgroups must all be resident at
 * once; the grid is sized from the device's occupancy for it). No host synchronisation; the pair
 * may be captured into a graph and replayed. A plan is one run at a time: runs of the same plan
 * on different streams race. Every device-side wait is bounded: if the device does not make
 * progress for about a second (e.g. other work holds the compute units the grid needs), the
 * waiting workgroups give up, the outputs are undefined and the plan's error word is set, which
 * tq_chain_status reports; the launch still ends normally.
 */
int tq_chain_run(void *plan, void *stream);

/*
 * tq_chain_status -- wait for `stream`, then TQ_OK if no run of the plan has given up a wait since
 * the last call, else TQ_EDEVICE (and the error word is cleared).
 */
int tq_chain_status(void *plan, void *stream);

/* Text of the last non-TQ_OK status returned on this thread ("" if none). */
const char *tq_last_error(void);

/*
 * Tuning knobs -- for tests and tuning sweeps only. Every knob's default is the production choice
 * (the kernel selection and launch shapes measured to be fastest on gfx950); an override changes
 * which kernel or launch shape a call takes, and so possibly the result bits, never the contract
 * (every path meets the same error bars). The knobs are process-wide and read on every call;
 * set them while no call runs. Nothing else (no environment variable) changes what a call does.
 *   tq_tuning_set(knob, value): value >= 0 overrides, value < 0 restores the default; TQ_EINVAL for
 *   an unknown knob. tq_tuning_get(knob): the override, or -1 (default in effect or unknown knob).
 */
enum {
  TQ_KNOB_GEMV_TARGET_WG = 0, /* lane-per-row GEMV: workgroups the k split aims for (1024) */
  TQ_KNOB_GEMV_MAX_WAVES = 1, /* lane-per-row GEMV: most waves per workgroup (4) */
  TQ_KNOB_GEMV_KLANE = 2, /* batch-1 Q4_K on the lanes-along-k kernel: 1 on (default), 0 off */
  TQ_KNOB_KL_GROUPS = 3, /* lanes-along-k kernel: most lane groups per wave for short rows (4; 1 turns them off) */
  TQ_KNOB_KL_ROWS = 4, /* lanes-along-k kernel: rows per pass, 2, 4 (default) or 8 */
  TQ_KNOB_KL_TARGET_WAVES = 5, /* lanes-along-k kernel: waves the launch aims for (2048) */
  TQ_KNOB_GEMM_F32M = 6, /* Q6_K / Q8_0 batches on the fp32 matrix cores: 1 default shapes, 0 never, 2 every batch */
  TQ_KNOB_F32M_UPK = 7, /* fp32 matrix-core kernel: blocks per k slice (8) */
  TQ_KNOB_GEMV_I8 = 8, /* int8 matrix-core batch-1 GEMV: 1 Q4_K from k = 16384 and Q8_0 always (default), 0 never, 2 Q4_K always too */
  TQ_KNOB_I8_UPK = 9, /* int8 matrix-core kernel: blocks per k slice (4) */
  TQ_KNOB_MOE_QMM = 10, /* MoE steps of 2+ tokens on the fp16 matrix cores: 1 on (default), 0 grouped fp32 GEMV */
  TQ_KNOB_QMM_NT = 11, /* fp16 matrix-core MoE kernel: chunks of 16 (1) or 32 (2) positions (0: chosen from the mean tokens per expert) */
  TQ_KNOB_MOE_NT = 12, /* grouped fp32 MoE GEMV: token tile 1, 2, 4 or 8 (0: chosen from the mean tokens per expert) */
  TQ_KNOB_ROUTER_KL = 13, /* router for up to 8 tokens with lanes along the hidden dimension: 1 on (default), 0 off */
  TQ_KNOB_ROUTER_STEPS = 14, /* that router: 256-value steps per hidden slice (1) */
  TQ_KNOB_ROUTER_MF = 15, /* router for more than 8 tokens and 64+ experts on the fp32 matrix cores: 1 on (default), 0 off */
  TQ_KNOB_GROUP1 = 16, /* one token: grouping written by the top-k kernel: 1 on (default), 0 the grouping kernel */
  TQ_KNOB_COMBINE4 = 17, /* combine by 16-byte column runs: 1 on (default), 0 element-wise */
  TQ_KNOB_FUSE_COMBINE = 18, /* one token: combine inside the down launch: 1 on (default), 0 a combine launch */
  TQ_KNOB_GEMV_QMM = 19, /* Q4_K GEMV of 2..32 tokens on the fp16 matrix cores: 1 on (default), 0 off */
  TQ_KNOB_QMM_UPK = 20, /* fp16 matrix-core dense kernel with a split launch: blocks per k slice (4) */
  TQ_KNOB_QMM_INLINE = 21, /* Q4_K GEMV of 2..16 tokens: activations split inside the product kernel: 1 on (default), 0 a split launch first */
  TQ_KNOB_QMM_INLINE_UPK = 22, /* that kernel: blocks per k slice, 2 or 4 (0: 2 for k <= 4096, else 4) */
  TQ_KNOB_QMM_INLINE_NR = 23, /* that kernel: 16-row weight tiles per wave of a product without SwiGLU, 1 (default) or 2 */
  TQ_KNOB_GEMV_MF = 24, /* batch-1 Q4_K and Q6_K GEMV on the fp16 matrix cores: 2 (default) also single Q4_K products from k = 16384 in k slices (given the workspace), 1 only Q4_K k < 16384 (longer rows on the int8 kernel), 0 off */
  TQ_KNOB_MF_WGS = 25, /* that kernel: workgroups the launch aims for (256: one per CU, several tiles each) */
  TQ_KNOB_MF_KB = 26, /* that kernel: blocks per wave, 1, 2 or 4 (0: from k) */
  TQ_KNOB_MF_DEEP = 27, /* that kernel: more tiles in flight: 1 (default) Q6_K one ahead at 4 blocks a wave, 2 also Q4_K two ahead where a workgroup has 3+ tiles and at most 8 waves, 0 neither */
  TQ_KNOB_MOE_MF = 28, /* one-token Q4_K MoE step: the experts' products on the fp16 matrix cores, 1 (default) or 0 (lanes along k) */
  TQ_KNOB_MOE_ROUTE1 = 29, /* one-token MoE step on the matrix-core kernel: the top-k selection inside the gate/up launch, 1 (default) or 0 (its own launch) */
  TQ_KNOB_F32M_T4 = 30, /* fp32 matrix-core kernel: 2..4 tokens on the 4x4x1 form (1, default) or padded to 16 tokens (0) */
  TQ_KNOB_MF_KSPLIT = 31, /* fp16 matrix-core GEMV: k slices forced on single launches (0 = from k) */
  TQ_KNOB_COUNT = 32
};
int tq_tuning_set(int knob, int value);
int tq_tuning_get(int knob);

#ifdef __cplusplus
}
#endif
#endif
