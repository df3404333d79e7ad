// tq_moe.h -- host-side plan of one MoE layer call (internal to libtq).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_route.h"

namespace tq {

struct MoeExpertPtrs {
  const void *m[3];  // gate [ffn][hidden], up [ffn][hidden], down [hidden][ffn] blobs
};

struct MoeShape {
  int type;
  int64_t hidden, ffn, n_experts, top_k, tokens;
  int has_shared, renormalize, experts_on_host;
  int mfma;              // expert products on the bf16 matrix cores (Q4_K only)
  int64_t gate_bytes;    // bytes of one gate (= up) blob
  int64_t expert_bytes;  // gate + up + down
};

struct MoePlan {
  MoeShape s;
  int64_t P;       // positions: T*k routed pairs, then T shared-expert rows
  int max_active;  // upper bound of active experts (including the shared one)
  int nt;          // token rows per tile of the grouped fp32 GEMV (1, 2, 4 or 8)
  int klane;       // one-token Q4_K step: the lanes-along-k kernels (SwiGLU fused)
  int qmm;         // Q4_K, 2+ tokens: the fp32-accurate fp16 matrix-core kernels
  int qmm_nt;      // their token tiles of 16 per chunk (1 or 2)
  int shared_piece;  // positions per active-list entry of the shared expert
  int act_stride;    // stride of the three arrays of the active-expert list
  int rtiles, hsplit, hpk;
  int router_kl;   // T <= 8: the lanes-along-hidden router (slices of whole 256-value steps)
  int router_mf;   // T > 8, E >= 64: the fp32 matrix-core router (slices of 16-value steps)
  int nctr;        // T = 1: arrival counters of the fused combine (0: none)
  int route1;      // T = 1, E <= 256, matrix-core experts: the gate/up launch can make the
                   // selection itself (no top-k launch) when a call runs every stage
  int gu_rg, gu_ks, gu_upk, gu_waves, gu_upw;
  int d_rg, d_ks, d_upk, d_waves, d_upw;
  int64_t off_rpart, off_logits, off_ids, off_wts, off_counts, off_offsets, off_pairs, off_inv,
      off_act, off_nact, off_gu, off_h, off_o, off_stage, off_ctr, off_table;
  int64_t off_xb, off_hb, off_chunks, off_nchunks;  // matrix-core paths only
  int64_t off_xsplit, off_hsplit;                    // fp16 split rows (qmm)
  int max_chunks;
  int64_t stage_stride;
  int64_t bytes;
};

MoePlan plan_moe(const MoeShape &s);
size_t group_lds_bytes(int64_t T, int64_t E);
// route1: the router's partial sums only (the gate/up launch makes the selection).
int launch_moe_routing(const MoePlan &p, const float *router_w, const float *x, char *ws,
                       hipStream_t st, bool route1 = false);
// Arguments of the lanes-along-k kernel over the experts of a one-token step (Q4_K).
struct MoeKlArgs {
  const MoeExpertPtrs *experts;
  MoeExpertPtrs shared;
  const uint8_t *staging;
  int64_t stage_stride;
  int64_t stage_off[3];
  const int *act, *n_active, *pairs;
  int slot0, act_stride, E, topk, Tk;
  int gate_up;        // 1: gate/up rows interleaved, SwiGLU epilogue; 0: down
  int rows;           // virtual rows per slot: 2 * ffn (gate/up) or hidden (down)
  int64_t row_bytes;
  const float *x;     // token rows (gate/up) or h rows by position (down)
  int64_t ldx;
  float *out;         // h [P][ffn] or o [P][hidden]
  int64_t ldo;
  // One token with the combine fused into the down launch (all null / 0 otherwise):
  unsigned *ctr;      // arrival counters, one per row range of the down launch
  int nctr;           // gate/up: its first workgroup zeroes ctr[0 .. nctr)
  int ctr_cap;        // counters at ctr
  float *fuse_y;      // down: y [hidden], written by the last workgroup of each row range
  const float *wts;   // the token's routing weights [topk]
  const int *inv;     // the positions of the token's slots [topk]
  int has_shared;     // the shared expert's output sits at position Tk
  // One token, gate/up launch: every workgroup makes the selection from the router's partial sums
  // (workgroup 0 stores the routing outputs); act, n_active and pairs are not read.
  int route1;
  Route1Args route;
};

// Output value c of a fused one-token combine: the token's routed slots in routing order, each
// times its weight, then the shared expert's row; the sums are read at device scope (they were
// stored by other workgroups of the same launch).
__device__ __forceinline__ float moe_combine_value(const MoeKlArgs &a, int c) {
  float acc = 0.f;
  for (int j = 0; j < a.topk; ++j) {
    const float v = __hip_atomic_load(a.out + (int64_t)a.inv[j] * a.ldo + c, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
    acc = __builtin_fmaf(a.wts[j], 0.f + v, acc);
  }
  if (a.has_shared)
    acc += 0.f + __hip_atomic_load(a.out + (int64_t)a.Tk * a.ldo + c, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
  return acc;
}

bool moe_klane_ok(int fmt, int64_t hidden, int64_t ffn, int64_t tokens);
int launch_moe_kl(const MoeKlArgs &a, int64_t k, int nslots, hipStream_t s);

// A subset of the active-expert list: slots slot0 .. slot0+nslots-1, whose pairs occupy positions
// pos0 .. pos0+npos-1 (the host knows both once it has read the list back).
struct SlotRange {
  int slot0, nslots;
  int64_t pos0, npos;
};

// Expert products of the routed pairs into the per-position outputs in the workspace: every
// active expert (range == nullptr) or the slots of `range`. staging != nullptr: routed expert
// blobs are read from the workspace's staging area, slot a at staging + a * stage_stride.
int launch_moe_experts(const MoePlan &p, const MoeExpertPtrs *experts_dev,
                       const MoeExpertPtrs &shared, const uint8_t *staging, const float *x,
                       char *ws, hipStream_t st, const SlotRange *range = nullptr,
                       float *fuse_y = nullptr, bool route1 = false);
// One-token layers on the lanes-along-k kernels: the combine can run inside the down launch
// (launch_moe_experts with fuse_y = y; then no launch_moe_combine).
bool moe_fuse_combine_ok(const MoePlan &p);
// y[t] = the routing-weighted sum of the per-position outputs (plus the shared expert's).
int launch_moe_combine(const MoePlan &p, char *ws, float *y, hipStream_t st);

}  // namespace tq
