// tq_route.h -- the top-k selection of the MoE router's logits, shared by the top-k kernel and
// the one-token expert launch that makes the selection itself (internal to libtq).
//
// Top-k and softmax weights (the routing of a mixture-of-experts layer): the k largest logits of
// a token, ties to the lower expert index, and the softmax over the chosen ones (or over all, not
// renormalized). One wave per token; lane l holds the logits of experts l, l + 64, ...
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace tq {

constexpr int kMaxHSplit = 32;  // hidden slices of the router's partial sums

__device__ __forceinline__ bool better(float va, int ea, float vb, int eb) {
  return va > vb || (va == vb && ea < eb);
}

// Keep the better of (v, e) and the pair DPP control CTRL brings from another lane of the row.
template <int CTRL>
__device__ __forceinline__ void argmax_dpp(float &v, int &e) {
  const float ov = __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
  const int oe = __builtin_amdgcn_update_dpp(0, e, CTRL, 0xF, 0xF, false);
  if (better(ov, oe, v, e)) {
    v = ov;
    e = oe;
  }
}

// The wave's best (value, index) pair, in every lane. (value, index) with distinct indices is a
// total order, so the result does not depend on the order of the comparisons. Within each row of
// 16 lanes by DPP (swaps within quads, then the half-row and row mirrors), then the four rows'
// results through readlane.
__device__ __forceinline__ void wave_argmax(float &v, int &e) {
  argmax_dpp<0xB1>(v, e);   // quad_perm [1, 0, 3, 2]
  argmax_dpp<0x4E>(v, e);   // quad_perm [2, 3, 0, 1]
  argmax_dpp<0x141>(v, e);  // row_half_mirror: lane i <-> 7 - i within 8
  argmax_dpp<0x140>(v, e);  // row_mirror: lane i <-> 15 - i within 16
  float bv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  int be = __builtin_amdgcn_readlane(e, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float rv =
        __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16 * r));
    const int re = __builtin_amdgcn_readlane(e, 16 * r);
    if (better(rv, re, bv, be)) {
      bv = rv;
      be = re;
    }
  }
  v = bv;
  e = be;
}

// Grouping of a one-token batch, written by the top-k wave itself (no grouping launch): the same
// outputs as k_group, whose stable scatter reduces for T = 1 to the rank of each chosen expert
// among the chosen ones.
struct Group1Out {
  int *counts, *offsets, *pairs, *inv, *act, *n_active;
  int act_stride, has_shared;
};

// The selection itself, on the token's logits v (NV = expert slots per lane, E <= 64 NV): logits
// stored, k rounds of a wave arg-max on (value, -index) with round j's id stored at once and its
// exp(value - first value) kept by lane j and divided by the sum at the end (no read-back), then
// (g1 given, T = 1) the grouping. Every store is skipped when `store` is false. Returns in lane
// j < topk the id chosen in round j and (g1 given) its rank among the chosen ids. The code is
// kept short (rolled loops): one wave runs it cold, so instruction fetch, not arithmetic, sets
// its time.
template <int NV>
__device__ __forceinline__ void topk_pick(float (&v)[NV], int lane, int t, int E, int topk,
                                          int renormalize, float *__restrict__ logits,
                                          int *__restrict__ ids, float *__restrict__ wts,
                                          const Group1Out &g1, bool store, int &id_out,
                                          int &rank_out) {
  rank_out = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (lane + 64 * i >= E) v[i] = -INFINITY;
    else if (store) logits[(int64_t)t * E + lane + 64 * i] = v[i];
  }
  // k rounds of a wave arg-max on (value, -index); round j's id is written at once, its
  // exp(value - first value) kept by lane j and divided by the sum at the end (no read-back)
  unsigned taken = 0;  // bit i: expert lane + 64 i already selected
  float sel0 = 0.f, denom = 0.f, my_w = 0.f;
  int my_id = 0x7FFFFFFF;  // lane j < topk: the id chosen in round j
  for (int j = 0; j < topk; ++j) {
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + 64 * i;
      // a NaN logit ranks below every number (ties to the lower index as usual), so the chosen
      // id is always an unchosen expert in [0, E); its weight then comes out NaN
      const float vi = v[i] == v[i] ? v[i] : -INFINITY;
      if (e < E && !(taken >> i & 1u) && better(vi, e, bv, be)) {
        bv = vi;
        be = e;
      }
    }
    wave_argmax(bv, be);
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (j == 0) sel0 = bv;
    const float ej = expf(bv - sel0);
    if (lane == j) {
      my_id = be;
      my_w = ej;
    }
    if (renormalize) denom += ej;
    if (store && lane == 0) ids[(int64_t)t * topk + j] = be;
  }
  if (!renormalize) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (lane + 64 * i < E) s += expf(v[i] - sel0);
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    denom = s;
  }
  if (store && lane < topk) wts[(int64_t)t * topk + lane] = my_w / denom;
  id_out = my_id;
  if (g1.counts != nullptr) {  // T = 1 (the launch has a single wave at work)
    // rank of lane j's expert among the chosen ones: its position in expert order
    int rank = 0;
    for (int q = 0; q < topk; ++q) rank += __builtin_amdgcn_readlane(my_id, q) < my_id ? 1 : 0;
    rank_out = rank;
    if (!store) return;
    if (lane < topk) {
      g1.pairs[rank] = lane;
      g1.inv[lane] = rank;
      g1.act[rank] = my_id;
      g1.act[g1.act_stride + rank] = rank;
      g1.act[2 * g1.act_stride + rank] = 1;
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + 64 * i;
      if (e < E) {
        int below = 0;
        for (int q = 0; q < topk; ++q) below += __builtin_amdgcn_readlane(my_id, q) < e ? 1 : 0;
        g1.counts[e] = (int)(taken >> i & 1u);
        g1.offsets[e] = below;
      }
    }
    if (lane == 0) {
      g1.offsets[E] = topk;
      int na = topk;
      if (g1.has_shared) {  // the shared expert's one position, after the routed pairs
        g1.act[na] = E;
        g1.act[g1.act_stride + na] = topk;
        g1.act[2 * g1.act_stride + na] = 1;
        ++na;
      }
      *g1.n_active = na;
    }
  }
}

// The one-token selection made inside the expert launch: router partial sums in, the routing
// outputs of the top-k kernel's one-token path out (stored by one workgroup only).
struct Route1Args {
  const float *part;  // the router's partial sums, [hsplit][8][E] (token row 0)
  int E, hsplit, renormalize;
  float *logits, *wts;
  int *ids;
  Group1Out g1;
};

// Every workgroup of the launch adds the router's partial sums of the token (expert 64 w + lane in
// wave w, the same additions in the same order as the top-k kernel), wave 0 makes the selection,
// and the workgroup learns the expert of active slot `slot` (the chosen experts in ascending id
// order, then the shared expert E). Only a workgroup with `store` set writes the routing outputs.
// E <= 256.
__device__ __forceinline__ int route_one_token(const Route1Args &r, int topk, int slot, bool store) {
  constexpr int NV = 4;
  __shared__ float lg[NV * 64];
  __shared__ int chosen;
  const int lane = threadIdx.x & 63, w0 = (int)(threadIdx.x >> 6), nw = (int)(blockDim.x >> 6);
  for (int w = w0; w < NV; w += nw) {
    const int e = min(lane + 64 * w, r.E - 1);
    float b[kMaxHSplit];
#pragma unroll
    for (int q = 0; q < kMaxHSplit; ++q) b[q] = r.part[(int64_t)min(q, r.hsplit - 1) * 8 * r.E + e];
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < kMaxHSplit; ++q) sum += q < r.hsplit ? b[q] : 0.f;
    lg[64 * w + lane] = sum;
  }
  __syncthreads();
  if (w0 == 0) {
    float v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = lg[64 * i + lane];
    int my_id, rank;
    topk_pick<NV>(v, lane, 0, r.E, topk, r.renormalize, r.logits, r.ids, r.wts, r.g1, store, my_id,
                  rank);
    if (lane < topk && rank == slot) chosen = my_id;
    if (lane == 0 && slot >= topk) chosen = r.E;
  }
  __syncthreads();
  return chosen;
}

}  // namespace tq
