/*
 * tq_oracle.h -- CPU oracle for block-quantized decode products and top-k MoE expert FFNs.
 *
 * TEST INFRASTRUCTURE. This is the plain, slow, fp64 reference that the GPU library is checked
 * against. Only the test suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or constant with the GPU library, and the GPU library never
 * links or calls it.
 *
 * What it computes, and where that comes from:
 *   - The pages name the block formats (Q4_K, Q6_K, Q8_0) and the GGUF container they live in:
 *     "Titan Engine" page (zingnex.cn), sections "Aggressive quantization" and "Model format
 *     support"; "Show HN: Llama 3.1 70B on a single RTX 3090 via NVMe-to-GPU bypassing the CPU"
 *     page (hn.213312.xyz), section "Quantization support" and the "Core performance" table.
 *     The pages give no bit layout; the oracle reads the formats as the public GGUF k-quant block
 *     layouts (a reading, stated in full in tq_oracle.c next to each decoder).
 *   - The product is the decode-time matrix-vector (or small-batch) product over those weights:
 *     Titan page, "MoE expert streaming" and "Performance" table; KTransformers page
 *     (news.fishai.com.cn), the part on GPU quantized-matmul kernels and CPU expert offload.
 *   - Top-k routing activates a few experts per token (Titan page, "MoE expert streaming": e.g.
 *     2 of 8 experts per forward pass).
 *
 * Conventions: every pointer is host memory owned by the caller. Weight blobs are row-major,
 * rows = outputs ("out x in"), blocks run along the input dimension k. Activations are
 * token-major: x[b][k], y[b][n]. All sums are fp64, taken in ascending index order.
 */
#ifndef TQ_ORACLE_H
#define TQ_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Threads the oracle's parallel loops use (OpenMP). */
int orc_num_threads(void);
/* Threads of the parallel loops from now on (n >= 1; the OpenMP default otherwise). */
void orc_set_num_threads(int n);

/* Block format codes used by the oracle. */
enum { ORC_Q4_K = 1, ORC_Q6_K = 2, ORC_Q8_0 = 3, ORC_Q5_K = 4, ORC_Q4_0 = 5 };

/* Weights per block and bytes per block for a format code; 0 for an unknown code. */
int64_t orc_block_weights(int type);
int64_t orc_block_bytes(int type);

/* IEEE binary16 bit pattern -> exact binary64 value (subnormals kept, inf/NaN preserved). */
double orc_half_to_double(uint16_t h);

/* Exact value of weight i (0 <= i < block_weights) of one block. */
double orc_block_weight(int type, const uint8_t *block, int i);

/* Decoded scale fields of one block (for tests). For Q4_K: d, dmin, sc[8], m[8], q[256].
 * For Q6_K: d, sc[16] (signed), q[256] (0..63). For Q8_0: d, q[32] (signed). Unused outputs
 * may be NULL. Returns 0 on success, -1 for an unknown type. */
int orc_block_fields(int type, const uint8_t *block, double *d, double *dmin, int32_t *sc,
                     int32_t *m, int32_t *q);

/* Dequantize a blob [n][k] to exact fp64 values. */
int orc_dequant_f64(int type, const uint8_t *w, int64_t n, int64_t k, double *out);
/* Dequantize to fp32: each exact value rounded once, to nearest even. */
int orc_dequant_f32(int type, const uint8_t *w, int64_t n, int64_t k, float *out);
/* Dequantize to bf16 bit patterns: round-to-nearest-even of the fp32 value above. */
int orc_dequant_bf16(int type, const uint8_t *w, int64_t n, int64_t k, uint16_t *out);
/* fp32 -> bf16 bit pattern, round to nearest even (NaN stays NaN). */
uint16_t orc_f32_to_bf16(float f);

/* y[b][n] = sum_k w[n][k] * x[b][k] (fp64, ascending k), mag[b][n] = sum_k |w[n][k] * x[b][k]|.
 * Only rows listed in `rows` (n_rows of them) are computed when rows != NULL; the outputs are
 * then packed [b][n_rows]. mag may be NULL. x is fp32 [batch][k]. */
int orc_gemv(int type, const uint8_t *w, int64_t n, int64_t k, const float *x, int64_t batch,
             const int64_t *rows, int64_t n_rows, double *y, double *mag);
/* Same product with fp64 activations (used to chain the oracle's own fp64 intermediates). */
int orc_gemv_f64x(int type, const uint8_t *w, int64_t n, int64_t k, const double *x,
                  int64_t batch, const int64_t *rows, int64_t n_rows, double *y, double *mag);

/* SwiGLU: h = silu(g) * u with silu(z) = z / (1 + exp(-z)), fp64. Inputs fp32 or fp64. */
void orc_swiglu_f32(const float *g, const float *u, int64_t n, double *h);
void orc_swiglu_f64(const double *g, const double *u, int64_t n, double *h);

/* Router logits[t][e] = sum_h x[t][h] * wr[e][h] (fp64, ascending h); x [T][H], wr [E][H]. */
void orc_router_logits(const float *x, int64_t T, const float *wr, int64_t E, int64_t H,
                       double *logits);

/* Top-k selection on a given logits tensor [T][E] (fp32 as used by the caller, or fp64).
 * Slot j of token t holds the j-th largest logit; equal logits go to the lower expert index.
 * weights[t][j] = exp(l_j - l_max) / sum over the selected experts (renormalize = 1) or over
 * all E experts (renormalize = 0), fp64. Returns -1 if k < 1 or k > E. */
int orc_topk_f32(const float *logits, int64_t T, int64_t E, int64_t k, int renormalize,
                 int32_t *ids, double *weights);
int orc_topk_f64(const double *logits, int64_t T, int64_t E, int64_t k, int renormalize,
                 int32_t *ids, double *weights);

/* Expert grouping of the routed pairs. counts[e] = number of (t, j) with ids[t][j] == e;
 * offsets[E+1] is the exclusive prefix sum (offsets[E] == T*k); pairs[offsets[e] + r] = t*k + j
 * of the r-th pair routed to e in ascending t. Returns -1 on an id outside [0, E). */
int orc_group(const int32_t *ids, int64_t T, int64_t k, int64_t E, int32_t *counts,
              int32_t *offsets, int32_t *pairs);

/* One expert of a SwiGLU FFN: gate [ffn][hidden], up [ffn][hidden], down [hidden][ffn]. */
typedef struct {
  const uint8_t *gate, *up, *down;
} orc_expert;

/* MoE FFN output for the given routing:
 *   y[t] = sum_j weights[t][j] * down_e . swiglu(gate_e . x_t, up_e . x_t)   (e = ids[t][j])
 *        + (shared != NULL ? down_s . swiglu(gate_s . x_t, up_s . x_t) : 0)
 * fp64, slot order j = 0..k-1, shared term last. mag[t][i] is the matching sum of absolute
 * products used by the tolerance. Only the tokens listed in `tokens` (n_tok of them) are
 * computed when tokens != NULL; outputs are packed [n_tok][hidden]. mag may be NULL. */
int orc_moe(int type, int64_t hidden, int64_t ffn, const orc_expert *experts, int64_t n_experts,
            const orc_expert *shared, const float *x, int64_t T, int64_t k, const int32_t *ids,
            const double *weights, const int64_t *tokens, int64_t n_tok, double *y, double *mag);

/* orc_moe's result, bitwise, with the work grouped by expert (each expert's rows decoded once for
 * all the tokens routed to it; every output from the same expressions in the same order). */
int orc_moe_grouped(int type, int64_t hidden, int64_t ffn, const orc_expert *experts,
                    int64_t n_experts, const orc_expert *shared, const float *x, int64_t T,
                    int64_t k, const int32_t *ids, const double *weights, const int64_t *tokens,
                    int64_t n_tok, double *y, double *mag);

/* The same MoE output with bf16 operands, the arithmetic of the matrix-core path: x, every
 * weight (the bf16 rounding of its fp32 value) and h = swiglu(g, u) (rounded to fp32, then to
 * bf16) are rounded to nearest even; products and sums stay fp64; mag from the rounded operands.
 * Routing weights and the combine are as in orc_moe. */
int orc_moe_bf16(int type, int64_t hidden, int64_t ffn, const orc_expert *experts,
                 int64_t n_experts, const orc_expert *shared, const float *x, int64_t T,
                 int64_t k, const int32_t *ids, const double *weights, const int64_t *tokens,
                 int64_t n_tok, double *y, double *mag);

/* Reference quantizers (round to nearest, half to even), used only for round-trip tests.
 * orc_requant_*: re-derive the quants of a blob from target values w [n][k] keeping the blob's
 * own scale fields; writes the result to out (same size as w_blob).
 * orc_quantize_*: quantize fp32 data [n][k] from scratch. */
int orc_requant(int type, const uint8_t *w_blob, const double *w, int64_t n, int64_t k,
                uint8_t *out);
int orc_quantize(int type, const float *w, int64_t n, int64_t k, uint8_t *out);

#ifdef __cplusplus
}
#endif
#endif
