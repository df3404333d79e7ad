// tq_gemv_mf.h -- batch-1 Q4_K and Q6_K GEMV on the fp16 matrix cores (internal to libtq).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_gemv_core.h"

namespace tq {

// Format and row length k that the kernel takes in one slice (the activation operands of all of
// k sit in one workgroup's LDS: Q4_K k a multiple of 256 up to 14336, Q6_K a multiple of 512 up to
// 8192), and longer rows that it takes in k slices (cut into 2..8 equal slices of at most 8192,
// Q6_K slices of an even number of blocks, whose sums meet through the workspace). Both honour
// the knob.
bool mf_gemv_ok(int fmt, int64_t k);
bool mf_gemv_sliced(int fmt, int64_t k);
// Workspace bytes (after the counters) of a sliced launch of `rows` rows; 0 when not sliced.
size_t mf_workspace_bytes(int fmt, int64_t rows, int64_t k);
// All rows of m (single, multi or SwiGLU pairs) against x (16-byte aligned). Sliced launches need
// partial (mf_workspace_bytes) and one counter per tile set. 0, -1 (launch error) or -2 (shape,
// LDS or workspace).
int launch_gemv_mf(int fmt, const KlMap &m, int64_t k, const float *x, float *partial,
                   unsigned long long *counters, int max_counters, hipStream_t s);

struct MoeKlArgs;
// One-token MoE step on the same kernel (Q4_K, hidden and ffn each taken in one slice; honours
// the knob), and the launch over nslots active slots (gate/up or down as MoeKlArgs says; with the
// combine fused, a.ctr holds at least a.ctr_cap >= one counter per tile set). 0, -1 or -2 (shape).
bool moe_mf_ok(int fmt, int64_t hidden, int64_t ffn);
int launch_moe_mf(const MoeKlArgs &a, int64_t k, int nslots, hipStream_t s);

}  // namespace tq
