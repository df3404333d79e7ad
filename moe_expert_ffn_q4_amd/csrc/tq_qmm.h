// tq_qmm.h -- Q4_K products of a few tokens per expert on the fp16 matrix cores, accurate to
// fp32 rounding (internal to libtq).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_moe.h"

namespace tq {

// Split activation rows: row r of K values is scaled by a power of two 2^e_r that brings its
// largest magnitude into [2^14, 2^15) and stored as fp16 hi/lo pairs, with the per-sub-block sums
// the min term needs. Layout per row, per 256-value block kb:
//   xs  [row][kb][1024 B]: 256 hi halves, then 256 lo halves; within each run of 8 the values are
//                           in the order 0,2,1,3,4,6,5,7 (the order the weight operand is built in)
//   aux [row][kb][32 B]  : 2^-6 * (sum of the 32 scaled values of sub-block j) as fp16 hi (8),
//                           then lo (8), sub-blocks in the same 0,2,1,3,4,6,5,7 order
//   unscale[row]         : 2^-e_r
struct SplitRows {
  uint8_t *xs, *aux;
  float *unscale;
};
size_t split_rows_bytes(int64_t rows, int64_t k);  // xs + aux + unscale, each 256-byte aligned
SplitRows split_rows_at(char *base, int64_t rows, int64_t k);
void launch_split_rows(const float *src, int64_t ld, int64_t rows, int64_t k, SplitRows out,
                       hipStream_t st);

struct QmmArgs {
  const MoeExpertPtrs *experts;  // device table [E]
  MoeExpertPtrs shared;          // by value (id E)
  const uint8_t *staging;        // non-null: routed expert of slot a at staging + a * stage_stride
  int64_t stage_stride;
  int64_t stage_off[3];
  const int *act, *n_active;     // active expert list of the grouping kernel
  int act_stride;
  const int *chunks, *n_chunks;  // chunk table (slot, first position, rows)
  const int *pairs;
  int E, topk, Tk;
  int kblocks;                   // 256-weight blocks along k
  int64_t row_bytes;
  SplitRows x;                   // split activation rows: by token (gate/up) or by position (down)
  int x_by_token;
  float *out;                    // fp32 h [P][ffn] (gate/up, SwiGLU applied) or o [P][hidden]
  int64_t ldo;
  int ntiles;                    // workgroup tiles per chunk
};

// Token rows per chunk of the fp16 matrix-core path: 16 * nt_max (nt_max = 1 or 2).
int qmm_chunk_rows(int nt_max);
// Row tiles: gate/up per 64 ffn columns, down per 128 hidden rows.
bool qmm_shape_ok(int64_t hidden, int64_t ffn);
// x split, chunk table, gate/up with SwiGLU into h (fp32), h split, down into o.
int launch_qmm_moe(QmmArgs a, int nt_max, int max_chunks, const float *x, int64_t tokens,
                   int64_t positions, int64_t hidden, int64_t ffn, char *xsplit, char *hsplit,
                   float *h, float *o, hipStream_t st);

// Dense products of 2..32 tokens: the rows of up to four matrices that share x, one after another
// (multi), or a gate and an up matrix with the SwiGLU applied (swiglu: n = cum[1] columns).
struct QmmDense {
  const uint8_t *w[4];
  float *y[4];  // [batch][n_p]; SwiGLU: y[0] = h [batch][n]
  int cum[5];
  int nparts;
  int swiglu;
  int64_t row_bytes;
};
bool qmm_dense_ok(int fmt, int64_t k, int64_t batch);
// Workspace after the completion counters: the k-slice partial sums (and, for the kernel that
// reads split rows, the split activations), enough for any launch shape the knobs can pick.
size_t qmm_dense_bytes(int64_t rows, int64_t k, int64_t batch, bool swiglu);
// The k dimension is cut into slices of a fixed number of blocks (a function of k only, so every
// row is summed in the same order whatever the launch); the last workgroup of a row tile to finish
// adds the slices in order. counters: one 8-byte word per row tile (Arrivals), any contents.
int launch_qmm_dense(const QmmDense &m, int64_t k, const float *x, int64_t batch, char *ws,
                     unsigned long long *counters, int max_counters, hipStream_t st);

}  // namespace tq
