// tq_prefill.h -- grouped expert products on the bf16 matrix cores (internal to libtq).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_moe.h"

namespace tq {

struct PrefillArgs {
  const MoeExpertPtrs *experts;  // device table [E]
  MoeExpertPtrs shared;          // by value (id E)
  const uint8_t *staging;        // non-null: routed expert of slot a at staging + a * stage_stride
  int64_t stage_stride;
  int64_t stage_off[3];          // offsets of gate / up / down inside one staged expert
  const int *act, *n_active;     // active expert list of the grouping kernel
  int act_stride;
  const int *chunks, *n_chunks;  // chunk table (slot, first position, rows)
  const int *pairs;
  int E, topk, Tk;
  int kblocks;                   // 256-weight blocks along k
  int64_t row_bytes;
  const uint16_t *xsrc;          // bf16 rows: by token (gate/up) or by position (down)
  int64_t ldx;
  int x_by_token;
  void *out;                     // bf16 h [P][ffn] (gate/up) or fp32 o [P][hidden] (down)
  int64_t ldo;
  int ntiles;                    // workgroup tiles per chunk
};

// Upper bound of the chunk count for P positions over at most max_active experts, cut into chunks
// of at most chunk_rows (prefill_max_chunks: the matrix-core prefill's chunk size).
int max_chunks_for(int64_t positions, int max_active, int chunk_rows);
int prefill_max_chunks(int64_t positions, int max_active);

// The active experts' position ranges cut into chunks of at most chunk_rows rows, near-equal in
// size: chunks[3c .. 3c+2] = (active slot, first position, rows), *n_chunks = their count.
void launch_chunk_table(const int *act, const int *n_active, int act_stride, int chunk_rows,
                        int max_chunks, int *chunks, int *n_chunks, hipStream_t st);

// x -> bf16, chunk table, gate/up with SwiGLU into h, down into o (P rows each).
int launch_prefill(int max_chunks, PrefillArgs a, const float *x, int64_t tokens, int64_t hidden,
                   int64_t ffn, uint16_t *xb, uint16_t *h, float *o, hipStream_t st);

}  // namespace tq
