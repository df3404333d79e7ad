// tq_moe.hip -- top-k routed MoE expert FFN: router logits, top-k, expert grouping, grouped
// expert GEMV over the selected experts, SwiGLU, and the weighted combine.
//
// Decode path, all on one stream and without host synchronisation:
//   k_router        logits partial sums (fp32), lane per expert row, tokens through scalar loads
//   k_router_kl     the same for T <= 8, lanes along the hidden dimension (coalesced rows)
//   k_router_mf     the same for T > 8 and E >= 64 on the fp32 matrix cores
//   k_topk          one wave per token: logits = sum of the partials, k largest (ties to the lower
//                   expert index), softmax weights renormalised over the selected experts
//   k_group         one workgroup: per-expert counts, exclusive offsets and a stable scatter of the
//                   (token, slot) pairs sorted by (expert, token); the list of active experts
//   k_moe_gemv      grouped GEMV over (active expert, matrix, row group, k slice) work items;
//                   empty items (experts beyond the active count) return at once
//   k_moe_swiglu    h = silu(gate) * up from the gate/up slices
//   k_moe_combine   y[t] = sum_j w[t][j] * o[pair (t, j)] + o_shared[t], slots in order
//   k_moe_combine4  the same sums, a workgroup per token and 16-byte column runs
// No atomic operation decides any order, so every output is deterministic.
#include <stdlib.h>

#include "tq_gemv_core.h"
#include "tq_gemv_mf.h"
#include "tq_launch.h"
#include "tq_moe.h"
#include "tq_prefill.h"
#include "tq_qmm.h"
#include "tq_route.h"

namespace tq {

// ---- router logits ------------------------------------------------------------------------------
// Grid: x = (expert row group, h slice), y = token tile of 8. partial layout [tile][hs][8][E].
__global__ __launch_bounds__(256) void k_router(const float *__restrict__ wr, int E, int H,
                                                const float *__restrict__ x, int T, int hsplit,
                                                int hpk, float *__restrict__ part) {
  __shared__ float red[4][8][64];
  const int rgs = blockIdx.x / hsplit, hs = blockIdx.x - rgs * hsplit;
  const int tile = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = wave_index(), nw = blockDim.x >> 6;
  const int e = min(rgs * 64 + lane, E - 1);
  const int h0 = hs * hpk, h1 = min(h0 + hpk, H);
  const int per_wave = ((h1 - h0 + nw - 1) / nw + 3) & ~3;
  const int a0 = h0 + wave * per_wave, a1 = min(a0 + per_wave, h1);
  const float *xr[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) xr[t] = x + (int64_t)min(tile * 8 + t, T - 1) * H;
  float acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = 0.f;
  const float *wrow = wr + (int64_t)e * H;
  for (int h = a0; h < a1; h += 4) {
    const float4 wv = *reinterpret_cast<const float4 *>(wrow + h);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      acc[t] = __builtin_fmaf(wv.x, xr[t][h], acc[t]);
      acc[t] = __builtin_fmaf(wv.y, xr[t][h + 1], acc[t]);
      acc[t] = __builtin_fmaf(wv.z, xr[t][h + 2], acc[t]);
      acc[t] = __builtin_fmaf(wv.w, xr[t][h + 3], acc[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  for (int i = threadIdx.x; i < 8 * 64; i += blockDim.x) {
    const int t = i >> 6, l = i & 63;
    float s = 0.f;
    for (int v = 0; v < nw; ++v) s += red[v][t][l];
    const int ee = rgs * 64 + l;
    if (ee < E) part[(((int64_t)tile * hsplit + hs) * 8 + t) * E + ee] = s;
  }
}


// Router for decode-sized batches (T <= 8): lanes along the hidden dimension, so a wave's loads
// of its expert rows are coalesced 1 KB runs, all of a slice's loads in flight at once. Workgroup
// = 4 waves x 4 expert rows, one hidden slice of hpk values (a multiple of 256); each lane adds
// its 4 values per 256-value step, then a halving butterfly over the wave leaves row r's slice sum
// in lane 16 r. Output layout as k_router's (tile 0): part[(hs * 8 + t) * E + e].
// NT = token rows the kernel carries (8, or 1 for one token: the same sums with an eighth of the
// activation loads and accumulators).
template <int NT>
__global__ __launch_bounds__(256) void k_router_kl(const float *__restrict__ wr, int E, int H,
                                                   const float *__restrict__ x, int T, int hsplit,
                                                   int hpk, float *__restrict__ part) {
  constexpr int RW = 4;
  const int rg = blockIdx.x / hsplit, hs = blockIdx.x - rg * hsplit;
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int e0 = rg * 16 + wave * RW;
  const int h0 = hs * hpk, h1 = min(h0 + hpk, H);
  const float *wrow[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) wrow[r] = wr + (int64_t)min(e0 + r, E - 1) * H;
  float acc[RW][NT];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[r][t] = 0.f;
  for (int h = h0 + 4 * lane; h < h1; h += 256) {
    float4 wv[RW], xv[NT];
#pragma unroll
    for (int r = 0; r < RW; ++r) wv[r] = *reinterpret_cast<const float4 *>(wrow[r] + h);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      xv[t] = *reinterpret_cast<const float4 *>(x + (int64_t)min(t, T - 1) * H + h);
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float a = acc[r][t];
        a = __builtin_fmaf(wv[r].x, xv[t].x, a);
        a = __builtin_fmaf(wv[r].y, xv[t].y, a);
        a = __builtin_fmaf(wv[r].z, xv[t].z, a);
        a = __builtin_fmaf(wv[r].w, xv[t].w, a);
        acc[r][t] = a;
      }
  }
  // per token: 4 rows -> 2 (lanes 32 apart), -> 1 (16 apart), then plain sums over 8, 4, 2, 1
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const bool up32 = (lane & 32) != 0, up16 = (lane & 16) != 0;
    float a0 = (up32 ? acc[2][t] : acc[0][t]) + __shfl_xor(up32 ? acc[0][t] : acc[2][t], 32);
    float a1 = (up32 ? acc[3][t] : acc[1][t]) + __shfl_xor(up32 ? acc[1][t] : acc[3][t], 32);
    float b = (up16 ? a1 : a0) + __shfl_xor(up16 ? a0 : a1, 16);
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1) b += __shfl_xor(b, d);
    const int e = e0 + (up32 ? 2 : 0) + (up16 ? 1 : 0);
    if ((lane & 15) == 0 && t < T && e < E) part[((int64_t)hs * 8 + t) * E + e] = b;
  }
}

// Router for many tokens and experts (T > 8, E >= 64) on the fp32 matrix cores: the logits are
// the dense product x[T][H] . wr[E][H]^T, fp32 products and sums as in the vector routers, in
// another order. One wave per (64-token tile, 64-expert tile, hidden slice of hpk values, a
// multiple of 16); v_mfma_f32_16x16x4_f32 with A = 16 token rows x 4 k, B = 4 k x 16 expert
// rows, 4 x 4 such blocks per wave. Lane l = 16 g + t loads, per 16-value step of the slice, the
// 4 values at h + 4 g of token rows 16 i + t and expert rows 16 j + t (one 16-byte load each), so
// the 4 components of a load feed 4 consecutive MFMAs: every value of the step meets its partner
// once. The lane receives D[token 4 g + c][expert t]. The next step's 8 loads are issued before
// the current step's 64 MFMAs (two register sets in turn). Rows beyond T or E are clamped on load
// and not stored. The 4 expert tiles of one (token tile, slice) are dealt to one XCD in a row, so
// they share its L2 for the token rows. Output layout as k_router's:
// part[((tok / 8 * hsplit + hs) * 8 + tok % 8) * E + e].
typedef float f32x4r __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64) void k_router_mf(const float *__restrict__ wr, int E, int H,
                                                  const float *__restrict__ x, int T, int hsplit,
                                                  int hpk, float *__restrict__ part) {
  const int nte = (E + 63) >> 6, ntt = (T + 63) >> 6;
  const int b = blockIdx.x, grp = (b >> 3) / nte * 8 + (b & 7), te = (b >> 3) % nte;
  if (grp >= ntt * hsplit) return;
  const int tt = grp / hsplit, hs = grp - tt * hsplit;
  const int lane = threadIdx.x, g = lane >> 4, t = lane & 15;
  const int h0 = hs * hpk, h1 = min(h0 + hpk, H);
  const float *xp[4], *wp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xp[i] = x + (int64_t)min(tt * 64 + 16 * i + t, T - 1) * H + 4 * g;
    wp[i] = wr + (int64_t)min(te * 64 + 16 * i + t, E - 1) * H + 4 * g;
  }
  f32x4r acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4r{0.f, 0.f, 0.f, 0.f};
  // two register sets in turn; the scheduling barriers keep each set's loads ahead of the
  // other set's MFMAs (left to itself the compiler sinks them to the end of the step)
  f32x4r xa[4], wa[4], xb[4], wb[4];
  const int n = (h1 - h0) >> 4;
  auto load = [&](f32x4r *xv, f32x4r *wv, int step) {
    const int h = h0 + 16 * min(step, n - 1);  // past the end: reload the last step
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xv[i] = *reinterpret_cast<const f32x4r *>(xp[i] + h);
      wv[i] = *reinterpret_cast<const f32x4r *>(wp[i] + h);
    }
  };
  auto mma = [&](const f32x4r *xv, const f32x4r *wv) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[i][c], wv[j][c], acc[i][j], 0, 0, 0);
  };
  load(xa, wa, 0);
  for (int st = 0; st + 1 < n; st += 2) {
    load(xb, wb, st + 1);
    mma(xa, wa);
    __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);   // the 8 loads first
    __builtin_amdgcn_sched_group_barrier(0x008, 64, 0);  // then the 64 MFMAs
    load(xa, wa, st + 2);
    mma(xb, wb);
    __builtin_amdgcn_sched_group_barrier(0x020, 8, 1);
    __builtin_amdgcn_sched_group_barrier(0x008, 64, 1);
  }
  if (n & 1) mma(xa, wa);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = te * 64 + 16 * j + t;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int tok = tt * 64 + 16 * i + 4 * g + c;
        if (tok < T && e < E)
          part[(((int64_t)(tok >> 3) * hsplit + hs) * 8 + (tok & 7)) * E + e] = acc[i][j][c];
      }
    }
}


// ---- top-k and softmax weights -----------------------------------------------------------------
// One wave per token (the selection itself: tq_route.h).
template <int NV>
__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ part, int T, int E,
                                              int hsplit, int topk, int renormalize,
                                              float *__restrict__ logits, int *__restrict__ ids,
                                              float *__restrict__ wts, Group1Out g1) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x >> 6) + (int)(threadIdx.x >> 6);
  // logits: the hidden slices' partial sums, added in slice order. They were just written by the
  // router's workgroups on every XCD, so each dependent batch of loads costs a memory round trip:
  // up to 4 slots per lane every slice's load goes out at once (HB = all 32), beyond 8 at a time.
  constexpr int HB = NV <= 4 ? kMaxHSplit : 8;
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = 0.f;
  if (NV > 1 && NV <= 4 && T == 1) {
    // One token: the workgroup's 4 waves share the sums (wave w: experts 64 w .. 64 w + 63, the
    // same additions in the same order as below, the padded slices' +0 included), so each lane
    // issues hsplit loads instead of NV hsplit; then wave 0 goes on alone.
    __shared__ float lg[4 * 64];
    const int w = (int)(threadIdx.x >> 6), e = min(lane + 64 * w, E - 1);
    float sum = 0.f;
    float b[HB];
#pragma unroll
    for (int q = 0; q < HB; ++q) b[q] = part[(int64_t)min(q, hsplit - 1) * 8 * E + e];
#pragma unroll
    for (int q = 0; q < HB; ++q) sum += q < hsplit ? b[q] : 0.f;
    lg[64 * w + lane] = sum;
    __syncthreads();
    if (t != 0) return;  // waves 1..3
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = lg[64 * i + lane];
  } else {
    if (t >= T) return;  // whole wave
    const int tile = t >> 3, tt = t & 7;
    const float *pbase = part + ((int64_t)tile * hsplit * 8 + tt) * E;
    for (int h0 = 0; h0 < hsplit; h0 += HB) {
      float b[NV][HB];
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int e = min(lane + 64 * i, E - 1);
#pragma unroll
        for (int q = 0; q < HB; ++q) b[i][q] = pbase[(int64_t)min(h0 + q, hsplit - 1) * 8 * E + e];
      }
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int q = 0; q < HB; ++q) v[i] += h0 + q < hsplit ? b[i][q] : 0.f;
    }
  }
  int my_id, rank;
  topk_pick<NV>(v, lane, t, E, topk, renormalize, logits, ids, wts, g1, true, my_id, rank);
}

// ---- grouping --------------------------------------------------------------------------------------
// An expert id read back from the top-k output, kept inside [0, E) so that no table is ever
// indexed past its end (the top-k kernel only writes ids in range).
__device__ __forceinline__ int id_at(const int *ids, int i, int E) {
  const unsigned e = (unsigned)ids[i];
  return (int)(e < (unsigned)E ? e : (unsigned)(E - 1));
}

// One workgroup of 8 waves. Tokens are taken in chunks of 64, one per lane of a wave; a token
// picks k distinct experts, so for one expert every lane of a chunk appears at most once.
//   mask[e]    (per wave) the lanes of the current chunk routed to e, built with LDS atomic ORs,
//              which commute, so the mask does not depend on the order of the updates.
//   tab[c][e]  first the number of pairs of chunk c routed to e (popcount of the mask), then
//              in place the number routed to e by the chunks before c.
//   pairs[offsets[e] + tab[c][e] + r] = t*k + j, r = lanes of chunk c routed to e below t's lane.
// act (stride S = act_stride): [0, S) expert id, [S, 2S) first position, [2S, 3S) count, for the
// active experts in ascending expert order, then the shared expert (id E, positions T*k ..
// T*k+T-1) as entries of at most shared_piece consecutive positions each, so that no single
// entry carries all T tokens.
__global__ __launch_bounds__(512) void k_group(const int *__restrict__ ids, int T, int topk, int E,
                                               int has_shared, int act_stride, int shared_piece,
                                               int *__restrict__ counts,
                                               int *__restrict__ offsets, int *__restrict__ pairs,
                                               int *__restrict__ inv, int *__restrict__ act,
                                               int *__restrict__ n_active) {
  extern __shared__ unsigned long long smem64[];
  const int nchunks = (T + 63) >> 6;
  unsigned long long *masks = smem64;                                   // [8][E]
  int *off = reinterpret_cast<int *>(masks + 8 * E);                    // [E]
  unsigned short *tab = reinterpret_cast<unsigned short *>(off + E);    // [nchunks][E]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  unsigned long long *mymask = masks + wave * E;
  for (int i = threadIdx.x; i < 8 * E; i += blockDim.x) masks[i] = 0ull;
  for (int i = threadIdx.x; i < nchunks * E; i += blockDim.x) tab[i] = 0;
  __syncthreads();
  // per-chunk counts
  for (int c = wave; c < nchunks; c += nw) {
    const int t = c * 64 + lane;
    const bool live = t < T;
    if (live)
      for (int j = 0; j < topk; ++j) atomicOr(&mymask[id_at(ids, t * topk + j, E)], 1ull << lane);
    __builtin_amdgcn_wave_barrier();
    if (live)
      for (int j = 0; j < topk; ++j) {
        const int e = id_at(ids, t * topk + j, E);
        tab[c * E + e] = (unsigned short)__popcll(mymask[e]);
      }
    __builtin_amdgcn_wave_barrier();
    if (live)
      for (int j = 0; j < topk; ++j) mymask[id_at(ids, t * topk + j, E)] = 0ull;
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    unsigned run = 0;
    for (int c = 0; c < nchunks; ++c) {
      const unsigned v = tab[c * E + e];
      tab[c * E + e] = (unsigned short)run;
      run += v;
    }
    off[e] = (int)run;  // the count, for now
  }
  __syncthreads();
  // counts -> exclusive offsets, and the active-list index of every expert with a non-zero count:
  // two exclusive scans over the experts, each thread owning two consecutive experts
  int *scan = off + E + ((nchunks * E + 1) >> 1);  // [2][blockDim]: position and active counts
  {
    const int e0 = 2 * (int)threadIdx.x, e1 = e0 + 1;
    const int c0 = e0 < E ? off[e0] : 0, c1 = e1 < E ? off[e1] : 0;
    const int nt = blockDim.x;
    int sp = c0 + c1, sa = (c0 > 0) + (c1 > 0);
    scan[threadIdx.x] = sp;
    scan[nt + threadIdx.x] = sa;
    __syncthreads();
    for (int d = 1; d < nt; d <<= 1) {  // inclusive scans of the per-thread totals
      const int vp = threadIdx.x >= (unsigned)d ? scan[threadIdx.x - d] : 0;
      const int va = threadIdx.x >= (unsigned)d ? scan[nt + threadIdx.x - d] : 0;
      __syncthreads();
      scan[threadIdx.x] += vp;
      scan[nt + threadIdx.x] += va;
      __syncthreads();
    }
    const int pos0 = scan[threadIdx.x] - sp, act0 = scan[nt + threadIdx.x] - sa;
    const int total = scan[nt - 1], nact = scan[2 * nt - 1];
    __syncthreads();  // every thread has read the scans (off is rewritten below)
    if (e0 < E) {
      counts[e0] = c0;
      offsets[e0] = pos0;
      off[e0] = pos0;
      if (c0 > 0) {
        act[act0] = e0;
        act[act_stride + act0] = pos0;
        act[2 * act_stride + act0] = c0;
      }
    }
    if (e1 < E) {
      const int a1 = act0 + (c0 > 0);
      counts[e1] = c1;
      offsets[e1] = pos0 + c0;
      off[e1] = pos0 + c0;
      if (c1 > 0) {
        act[a1] = e1;
        act[act_stride + a1] = pos0 + c0;
        act[2 * act_stride + a1] = c1;
      }
    }
    if (threadIdx.x == 0) {
      int na = nact;
      offsets[E] = total;
      if (has_shared)
        for (int t0 = 0; t0 < T; t0 += shared_piece) {
          act[na] = E;
          act[act_stride + na] = total + t0;
          act[2 * act_stride + na] = min(shared_piece, T - t0);
          ++na;
        }
      *n_active = na;
    }
  }
  __syncthreads();
  // stable scatter
  for (int c = wave; c < nchunks; c += nw) {
    const int t = c * 64 + lane;
    const bool live = t < T;
    if (live)
      for (int j = 0; j < topk; ++j) atomicOr(&mymask[id_at(ids, t * topk + j, E)], 1ull << lane);
    __builtin_amdgcn_wave_barrier();
    if (live) {
      const unsigned long long below = (1ull << lane) - 1ull;
      for (int j = 0; j < topk; ++j) {
        const int e = id_at(ids, t * topk + j, E);
        const int pos = off[e] + (int)tab[c * E + e] + __popcll(mymask[e] & below);
        pairs[pos] = t * topk + j;
        inv[t * topk + j] = pos;
      }
    }
    __builtin_amdgcn_wave_barrier();
    if (live)
      for (int j = 0; j < topk; ++j) mymask[id_at(ids, t * topk + j, E)] = 0ull;
    __builtin_amdgcn_wave_barrier();
  }
}

size_t group_lds_bytes(int64_t T, int64_t E) {
  const int64_t nchunks = (T + 63) / 64;
  // masks [8][E] u64, off [E] int, tab [nchunks][E] u16 (padded to ints), scan [2][512] int
  return (size_t)(8 * E * 8 + E * 4 + ((nchunks * E + 1) / 2) * 4 + 2 * 512 * 4);
}

// ---- grouped expert GEMV -----------------------------------------------------------------------
// Work item = ((active slot a, matrix m), row group, k slice); the grid covers the largest
// possible number of active experts and items past the actual count return at once. The token
// rows of an expert are processed in tiles of up to 8.

struct MoeGemvArgs {
  const MoeExpertPtrs *experts;  // device table [E]
  MoeExpertPtrs shared;          // by value (id E)
  const uint8_t *staging;        // non-null: routed expert a's blobs at staging + a * stage_stride
  int64_t stage_stride;
  int64_t stage_off[3];          // offsets of gate / up / down inside one staged expert
  const int *act;
  const int *n_active;
  const int *pairs;
  int slot0;                     // first active slot of this launch
  int act_stride;
  int E, topk, Tk;
  int mat0, nmat;                // matrices m = mat0 .. mat0 + nmat - 1 (0 gate, 1 up, 2 down)
  int n_rows, units;             // rows of each matrix, units of 256 weights along k
  int64_t row_bytes;
  int rowgroups, ksplit, upk, upw;
  const float *xsrc;             // activation rows: by token (gate/up) or by position (down)
  int64_t ldx;
  int x_by_token;
  float *out;                    // [nmat][ksplit][P][n_rows]
  int64_t P;
};

// One tile of up to NT token rows (nt valid ones; the rest repeat the last valid row and their
// results are dropped).
template <int FMT, int NT>
__device__ __forceinline__ void moe_tile(const MoeGemvArgs &a, const uint8_t *w, int m, int rg,
                                         int ks, int p0, int nt, float *lds) {
  const int row0 = rg * 64;
  const int ku0 = ks * a.upk, ku1 = min(ku0 + a.upk, a.units);
  const float *xr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int p = p0 + min(t, nt - 1);
    int64_t r = p;
    if (a.x_by_token) r = p >= a.Tk ? p - a.Tk : a.pairs[p] / a.topk;
    xr[t] = a.xsrc + r * a.ldx;
  }
  gemv_tile<FMT, NT>(w, a.row_bytes, a.n_rows, row0, ku0, ku1, a.upw, xr, lds);
  float *o = a.out + ((int64_t)(m - a.mat0) * a.ksplit + ks) * a.P * a.n_rows;
  for (int i = threadIdx.x; i < nt * 64; i += blockDim.x) {
    const int t = i >> 6, l = i & 63;
    if (row0 + l < a.n_rows) o[(int64_t)(p0 + t) * a.n_rows + row0 + l] = lds[i];
  }
  __syncthreads();  // lds is reused by the next tile
}

// Tiles of NT tokens (a compile-time size per launch: one body, no per-tile dispatch, so the
// kernel keeps the registers of a single tile shape).
template <int FMT, int NT>
__global__ __launch_bounds__(512) void k_moe_gemv(MoeGemvArgs a) {
  extern __shared__ float lds[];
  const int per_slot = a.nmat * a.rowgroups * a.ksplit;
  const int slot = a.slot0 + (int)blockIdx.x / per_slot;
  if (slot >= *a.n_active) return;
  int r = (int)blockIdx.x - (slot - a.slot0) * per_slot;
  const int mi = r / (a.rowgroups * a.ksplit);
  r -= mi * a.rowgroups * a.ksplit;
  const int rg = r / a.ksplit, ks = r - rg * a.ksplit;
  const int m = a.mat0 + mi;
  const int e = a.act[slot], p0 = a.act[a.act_stride + slot], cnt = a.act[2 * a.act_stride + slot];
  const uint8_t *w;
  if (e == a.E) {
    w = (const uint8_t *)a.shared.m[m];
  } else if (a.staging != nullptr) {
    w = a.staging + (int64_t)slot * a.stage_stride + a.stage_off[m];
  } else {
    w = (const uint8_t *)a.experts[e].m[m];
  }
  for (int t0 = 0; t0 < cnt; t0 += NT) moe_tile<FMT, NT>(a, w, m, rg, ks, p0 + t0, min(NT, cnt - t0), lds);
}

// ---- SwiGLU over the gate/up slices and the combine ---------------------------------------------

__global__ __launch_bounds__(256) void k_moe_swiglu(const float *__restrict__ gu, int ksplit,
                                                    int64_t P, int F, int64_t pos0, int64_t npos,
                                                    float *__restrict__ h) {
  const int64_t end = (pos0 + npos) * F, stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t slice = P * F;
  for (int64_t i = pos0 * F + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < end; i += stride) {
    float g = 0.f, u = 0.f;
    for (int q = 0; q < ksplit; ++q) {
      g += gu[(int64_t)q * slice + i];
      u += gu[((int64_t)ksplit + q) * slice + i];
    }
    h[i] = g * u / (1.f + expf(-g));
  }
}

__global__ __launch_bounds__(256) void k_moe_combine(const float *__restrict__ o, int ksplit,
                                                     int64_t P, int H, const int *__restrict__ inv,
                                                     const float *__restrict__ wts, int T,
                                                     int topk, int has_shared,
                                                     float *__restrict__ y) {
  const int64_t total = (int64_t)T * H, stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t slice = P * H;
  const int Tk = T * topk;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int t = (int)(i / H), c = (int)(i - (int64_t)t * H);
    float acc = 0.f;
    for (int j = 0; j < topk; ++j) {
      const int64_t pos = inv[t * topk + j];
      float s = 0.f;
      for (int q = 0; q < ksplit; ++q) s += o[q * slice + pos * H + c];
      acc = __builtin_fmaf(wts[t * topk + j], s, acc);
    }
    if (has_shared) {
      float s = 0.f;
      for (int q = 0; q < ksplit; ++q) s += o[q * slice + (int64_t)(Tk + t) * H + c];
      acc += s;
    }
    y[i] = acc;
  }
}

// The same sums with one workgroup per (token, run of 4 x 256 columns): the token's pair
// positions and weights are uniform (scalar loads) and each thread adds 4 adjacent columns with
// 16-byte loads, up to 8 slots' loads in flight at once; slots, and k slices within a slot, are
// added in the same order as k_moe_combine, so the results are bitwise the same. y 16-byte
// aligned.
__global__ __launch_bounds__(256) void k_moe_combine4(const float *__restrict__ o, int ksplit,
                                                      int64_t P, int H,
                                                      const int *__restrict__ inv,
                                                      const float *__restrict__ wts, int T,
                                                      int topk, int has_shared,
                                                      float *__restrict__ y) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (c >= H) return;
  const int64_t slice = P * H;
  const int *ip = inv + (int64_t)t * topk;
  const float *wp = wts + (int64_t)t * topk;
  auto ld = [&](int64_t pos, int q) {
    return *reinterpret_cast<const f32x4r *>(o + q * slice + pos * H + c);
  };
  f32x4r acc = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < topk; j0 += 8) {
    f32x4r s[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] = ld(ip[min(j0 + j, topk - 1)], 0);
    for (int q = 1; q < ksplit; ++q)
#pragma unroll
      for (int j = 0; j < 8; ++j) s[j] += ld(ip[min(j0 + j, topk - 1)], q);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j0 + j < topk) {
        const float w = wp[j0 + j];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(w, 0.f + s[j][e], acc[e]);
      }
  }
  if (has_shared) {
    const int64_t pos = (int64_t)T * topk + t;
    f32x4r s = ld(pos, 0);
    for (int q = 1; q < ksplit; ++q) s += ld(pos, q);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += 0.f + s[e];
  }
  *reinterpret_cast<f32x4r *>(y + (int64_t)t * H + c) = acc;
}

// ---- host side ---------------------------------------------------------------------------------


MoePlan plan_moe(const MoeShape &s) {
  MoePlan p;
  p.s = s;
  const int64_t T = s.tokens, E = s.n_experts, k = s.top_k;
  p.P = T * k + (s.has_shared ? T : 0);
  // the shared expert's T positions as entries of at most shared_piece: 16 on the fp32 grouped
  // path (two tiles of 8), all T elsewhere (one token, or the matrix-core chunk table)
  // Q4_K steps of two or more tokens: the fp32-accurate fp16 matrix-core kernels, which read each
  // active expert's weights once per chunk of 16 or 32 positions instead of running VALU dot
  // products per token (with host-resident experts: one launch once every copy has landed)
  p.qmm = !s.mfma && s.type == FMT_Q4_K && T > 1 && qmm_shape_ok(s.hidden, s.ffn);
  p.qmm = p.qmm && knob(TQ_KNOB_MOE_QMM, 1) != 0;  // 0: grouped GEMV
  p.qmm_nt = (T * k + E - 1) / E > 12 ? 2 : 1;
  if (const int v = knob(TQ_KNOB_QMM_NT, 0)) p.qmm_nt = v == 2 ? 2 : 1;
  p.shared_piece = (int)(!s.mfma && !p.qmm && T > 16 ? 16 : T);
  const int nsh = s.has_shared ? (int)((T + p.shared_piece - 1) / p.shared_piece) : 0;
  p.max_active = (int)((E < T * k ? E : T * k) + nsh);
  p.act_stride = (int)E + (nsh > 1 ? nsh : 1);
  // token rows per tile of the grouped GEMV: one at T = 1, else about the mean per expert
  const int64_t mean = (T * k + E - 1) / E;
  p.nt = T == 1 ? 1 : mean >= 12 ? 8 : mean >= 2 ? 4 : 2;  // measured: Mixtral T=16, 64; DeepSeek T=256
  if (const int n = knob(TQ_KNOB_MOE_NT, 0))  // tuning override: 1, 2, 4 or 8
    if (n == 1 || n == 2 || n == 4 || n == 8) p.nt = n;
  p.klane = !s.mfma && moe_klane_ok(s.type, s.hidden, s.ffn, s.tokens);
  // router: 64 expert rows per workgroup, token tiles of 8, h split to fill the chip
  p.rtiles = (int)((T + 7) / 8);
  const int rrg = (int)((E + 63) / 64);
  int hs = (512 + rrg * p.rtiles - 1) / (rrg * p.rtiles);
  hs = clampi(hs, 1, (int)(s.hidden / 256 < kMaxHSplit ? s.hidden / 256 : kMaxHSplit));
  p.hpk = (int)(((s.hidden + hs - 1) / hs + 3) & ~3);
  p.hsplit = (int)((s.hidden + p.hpk - 1) / p.hpk);
  // decode-sized batches: the lanes-along-hidden router, slices of whole 256-value steps, as many
  // as the partial-sum table allows
  p.router_kl = T <= 8 && s.hidden % 256 == 0 && knob(TQ_KNOB_ROUTER_KL, 1) != 0;
  if (p.router_kl) {
    const int steps = (int)(s.hidden / 256);
    const int per = clampi(knob(TQ_KNOB_ROUTER_STEPS, 1), 1, steps);  // 256-value steps per slice
    const int hsk = clampi((steps + per - 1) / per, 1, kMaxHSplit);
    p.hpk = (int)(((steps + hsk - 1) / hsk) * 256);
    p.hsplit = (int)((s.hidden + p.hpk - 1) / p.hpk);
  }
  // many tokens and 64 or more experts: the matrix-core router, hidden slices (multiples of 16)
  // so that about 2048 waves run
  p.router_mf = !p.router_kl && T > 8 && E >= 64 && knob(TQ_KNOB_ROUTER_MF, 1) != 0;
  if (p.router_mf) {
    const int64_t tiles = ((T + 63) / 64) * ((E + 63) / 64);
    int hsm = (int)((2048 + tiles - 1) / tiles);
    hsm = clampi(hsm, 1, (int)(s.hidden / 256 < kMaxHSplit ? s.hidden / 256 : kMaxHSplit));
    p.hpk = (int)(((s.hidden + hsm - 1) / hsm + 15) & ~15);
    p.hsplit = (int)((s.hidden + p.hpk - 1) / p.hpk);
  }
  // gate/up: F rows over k = hidden; down: hidden rows over k = F
  auto split = [&](int64_t rows, int64_t kdim, int nmat, int &rowgroups, int &ks, int &upk,
                   int &waves, int &upw) {
    const int units = (int)(kdim / 256);
    rowgroups = (int)((rows + 63) / 64);
    const int64_t items = (int64_t)p.max_active * nmat * rowgroups;
    int want = (int)((1024 + items - 1) / items);
    want = clampi(want, 1, units);
    upk = (units + want - 1) / want;
    ks = (units + upk - 1) / upk;
    int w = clampi(upk, 1, 4);
    upw = (upk + w - 1) / w;
    waves = (upk + upw - 1) / upw;
  };
  split(s.ffn, s.hidden, 2, p.gu_rg, p.gu_ks, p.gu_upk, p.gu_waves, p.gu_upw);
  split(s.hidden, s.ffn, 1, p.d_rg, p.d_ks, p.d_upk, p.d_waves, p.d_upw);
  if (p.klane) p.d_ks = 1;  // the lanes-along-k kernel writes whole sums
  // workspace carve-up
  int64_t o = 0;
  auto take = [&](int64_t bytes) {
    const int64_t at = o;
    o = align256(o + bytes);
    return at;
  };
  p.off_rpart = take((int64_t)p.rtiles * p.hsplit * 8 * E * 4);
  p.off_logits = take(T * E * 4);
  p.off_ids = take(T * k * 4);
  p.off_wts = take(T * k * 4);
  p.off_counts = take(E * 4);
  p.off_offsets = take((E + 1) * 4);
  p.off_pairs = take(T * k * 4);
  p.off_inv = take(T * k * 4);
  p.off_act = take((int64_t)3 * p.act_stride * 4);
  p.off_nact = take(4);
  if (s.mfma) {
    p.d_ks = 1;
    p.max_chunks = prefill_max_chunks(p.P, p.max_active);
    p.off_xb = take(T * s.hidden * 2);
    p.off_hb = take(p.P * s.ffn * 2);
    p.off_chunks = take((int64_t)3 * p.max_chunks * 4);
    p.off_nchunks = take(4);
  } else if (p.qmm) {
    p.d_ks = 1;
    p.max_chunks = max_chunks_for(p.P, p.max_active, qmm_chunk_rows(p.qmm_nt));
    p.off_xsplit = take((int64_t)split_rows_bytes(T, s.hidden));
    p.off_hsplit = take((int64_t)split_rows_bytes(p.P, s.ffn));
    p.off_h = take(p.P * s.ffn * 4);
    p.off_chunks = take((int64_t)3 * p.max_chunks * 4);
    p.off_nchunks = take(4);
  } else {
    p.off_gu = take((int64_t)2 * p.gu_ks * p.P * s.ffn * 4);
    p.off_h = take(p.P * s.ffn * 4);
  }
  p.off_o = take((int64_t)p.d_ks * p.P * s.hidden * 4);
  // one token: arrival counters for the combine fused into the down launch, one per row range
  // (a range holds at least 4 rows, so hidden / 4 + 1 always suffice)
  p.nctr = T == 1 && p.klane ? (int)(s.hidden / 4 + 1) : 0;
  p.route1 = T == 1 && p.klane && E <= 256 && s.top_k <= E && knob(TQ_KNOB_MOE_ROUTE1, 1) != 0 &&
             knob(TQ_KNOB_GROUP1, 1) != 0 && moe_mf_ok(s.type, s.hidden, s.ffn);
  p.off_ctr = take((int64_t)p.nctr * 4);
  p.stage_stride = align256(s.expert_bytes);
  p.off_stage = take(s.experts_on_host ? (int64_t)(p.max_active) * p.stage_stride : 0);
  // host-resident experts with a residency cache: the call's device table of expert pointers
  p.off_table = take(s.experts_on_host ? E * (int64_t)sizeof(MoeExpertPtrs) : 0);
  p.bytes = o;
  return p;
}

template <int FMT, int NT>
static int moe_gemv_launch(MoeGemvArgs a, int nslots, int waves, hipStream_t st) {
  const int grid = nslots * a.nmat * a.rowgroups * a.ksplit;
  const size_t lds = (size_t)4 * gemv_tile_lds_floats<FMT>(NT, a.upk, waves);
  if (lds > 65536) return -2;
  hipLaunchKernelGGL((k_moe_gemv<FMT, NT>), dim3((unsigned)grid), dim3(64 * waves), lds, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int FMT>
static int moe_gemv_nt(const MoeGemvArgs &a, int nt, int nslots, int waves, hipStream_t st) {
  if constexpr (FMT == FMT_Q5_K) {
    return moe_gemv_launch<FMT, 1>(a, nslots, waves, st);  // one token per pass
  } else {
    switch (nt) {
      case 1: return moe_gemv_launch<FMT, 1>(a, nslots, waves, st);
      case 2: return moe_gemv_launch<FMT, 2>(a, nslots, waves, st);
      case 4: return moe_gemv_launch<FMT, 4>(a, nslots, waves, st);
      default: return moe_gemv_launch<FMT, 8>(a, nslots, waves, st);
    }
  }
}

static int moe_gemv_dispatch(int fmt, const MoeGemvArgs &a, int nt, int nslots, int waves,
                             hipStream_t st) {
  switch (fmt) {
    case FMT_Q4_K: return moe_gemv_nt<FMT_Q4_K>(a, nt, nslots, waves, st);
    case FMT_Q6_K: return moe_gemv_nt<FMT_Q6_K>(a, nt, nslots, waves, st);
    case FMT_Q5_K: return moe_gemv_nt<FMT_Q5_K>(a, nt, nslots, waves, st);
    case FMT_Q4_0: return moe_gemv_nt<FMT_Q4_0>(a, nt, nslots, waves, st);
    default: return moe_gemv_nt<FMT_Q8_0>(a, nt, nslots, waves, st);
  }
}

// The one-token grouping outputs in the workspace (written by the top-k wave).
static Group1Out group1_out(const MoePlan &p, char *ws) {
  Group1Out g1{};
  g1.counts = (int *)(ws + p.off_counts);
  g1.offsets = (int *)(ws + p.off_offsets);
  g1.pairs = (int *)(ws + p.off_pairs);
  g1.inv = (int *)(ws + p.off_inv);
  g1.act = (int *)(ws + p.off_act);
  g1.n_active = (int *)(ws + p.off_nact);
  g1.act_stride = p.act_stride;
  g1.has_shared = p.s.has_shared ? 1 : 0;
  return g1;
}

int launch_moe_routing(const MoePlan &p, const float *router_w, const float *x, char *ws,
                       hipStream_t st, bool route1) {
  const MoeShape &s = p.s;
  const int E = (int)s.n_experts, H = (int)s.hidden, T = (int)s.tokens, k = (int)s.top_k;
  float *rpart = (float *)(ws + p.off_rpart);
  if (p.router_kl && ((uintptr_t)x & 15) == 0 && ((uintptr_t)router_w & 15) == 0) {
    const dim3 grid((unsigned)(((E + 15) / 16) * p.hsplit));
    if (T == 1)
      hipLaunchKernelGGL(k_router_kl<1>, grid, dim3(256), 0, st, router_w, E, H, x, T, p.hsplit,
                         p.hpk, rpart);
    else
      hipLaunchKernelGGL(k_router_kl<8>, grid, dim3(256), 0, st, router_w, E, H, x, T, p.hsplit,
                         p.hpk, rpart);
  } else if (p.router_mf && ((uintptr_t)x & 15) == 0 && ((uintptr_t)router_w & 15) == 0) {
    const int64_t groups = ((T + 63) / 64) * (int64_t)p.hsplit;
    const int64_t blocks = (groups + 7) / 8 * 8 * ((E + 63) / 64);
    hipLaunchKernelGGL(k_router_mf, dim3((unsigned)blocks), dim3(64), 0, st, router_w, E, H, x, T,
                       p.hsplit, p.hpk, rpart);
  } else {
    const dim3 rgrid((unsigned)(((E + 63) / 64) * p.hsplit), (unsigned)p.rtiles);
    hipLaunchKernelGGL(k_router, rgrid, dim3(256), 0, st, router_w, E, H, x, T, p.hsplit, p.hpk,
                       rpart);
  }
  if (route1) return hipGetLastError() == hipSuccess ? 0 : -1;  // the selection: in the gate/up launch
  {
    const dim3 g((unsigned)((T + 3) / 4));
    float *lg = (float *)(ws + p.off_logits), *wt = (float *)(ws + p.off_wts);
    int *id = (int *)(ws + p.off_ids);
    Group1Out g1{};
    if (T == 1 && knob(TQ_KNOB_GROUP1, 1) != 0) g1 = group1_out(p, ws);
    if (E <= 64)
      hipLaunchKernelGGL(k_topk<1>, g, dim3(256), 0, st, rpart, T, E, p.hsplit, k, s.renormalize, lg, id, wt, g1);
    else if (E <= 256)
      hipLaunchKernelGGL(k_topk<4>, g, dim3(256), 0, st, rpart, T, E, p.hsplit, k, s.renormalize, lg, id, wt, g1);
    else
      hipLaunchKernelGGL(k_topk<16>, g, dim3(256), 0, st, rpart, T, E, p.hsplit, k, s.renormalize, lg, id, wt, g1);
    if (g1.counts != nullptr) return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  const size_t glds = group_lds_bytes(s.tokens, s.n_experts);
  if (glds > 65536 &&
      hipFuncSetAttribute((const void *)k_group, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)glds) != hipSuccess)
    return -2;
  hipLaunchKernelGGL(k_group, dim3(1), dim3(512), glds, st, (const int *)(ws + p.off_ids), T, k, E,
                     s.has_shared, p.act_stride, p.shared_piece, (int *)(ws + p.off_counts), (int *)(ws + p.off_offsets),
                     (int *)(ws + p.off_pairs), (int *)(ws + p.off_inv), (int *)(ws + p.off_act),
                     (int *)(ws + p.off_nact));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_moe_combine(const MoePlan &p, char *ws, float *y, hipStream_t st) {
  const MoeShape &s = p.s;
  const int T = (int)s.tokens, k = (int)s.top_k;
  if (((uintptr_t)y & 15) == 0 && knob(TQ_KNOB_COMBINE4, 1) != 0) {
    const int quads = (int)(s.hidden / 4), threads = T >= 64 ? 256 : 64;
    hipLaunchKernelGGL(k_moe_combine4, dim3((unsigned)((quads + threads - 1) / threads), T),
                       dim3(threads), 0, st, (const float *)(ws + p.off_o), p.d_ks, p.P,
                       (int)s.hidden, (const int *)(ws + p.off_inv),
                       (const float *)(ws + p.off_wts), T, k, s.has_shared, y);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  const int64_t total = (int64_t)T * s.hidden;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)blocks), dim3(256), 0, st,
                     (const float *)(ws + p.off_o), p.d_ks, p.P, (int)s.hidden,
                     (const int *)(ws + p.off_inv), (const float *)(ws + p.off_wts), T, k,
                     s.has_shared, y);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

bool moe_fuse_combine_ok(const MoePlan &p) {
  return p.nctr > 0 && p.klane && p.s.tokens == 1 && p.d_ks == 1 &&
         knob(TQ_KNOB_FUSE_COMBINE, 1) != 0;
}

int launch_moe_experts(const MoePlan &p, const MoeExpertPtrs *experts_dev,
                       const MoeExpertPtrs &shared, const uint8_t *staging, const float *x,
                       char *ws, hipStream_t st, const SlotRange *range, float *fuse_y,
                       bool route1) {
  const MoeShape &s = p.s;
  const int E = (int)s.n_experts, T = (int)s.tokens, k = (int)s.top_k;
  MoeGemvArgs a{};
  a.experts = experts_dev;
  a.shared = shared;
  a.staging = staging;
  a.stage_stride = p.stage_stride;
  a.stage_off[0] = 0;
  a.stage_off[1] = s.gate_bytes;
  a.stage_off[2] = 2 * s.gate_bytes;
  a.act = (const int *)(ws + p.off_act);
  a.n_active = (const int *)(ws + p.off_nact);
  a.pairs = (const int *)(ws + p.off_pairs);
  a.slot0 = range ? range->slot0 : 0;
  a.act_stride = p.act_stride;
  const int nslots = range ? range->nslots : p.max_active;
  const int64_t pos0 = range ? range->pos0 : 0, npos = range ? range->npos : p.P;
  a.E = E;
  a.topk = k;
  a.Tk = T * k;
  a.P = p.P;
  if (s.mfma) {
    PrefillArgs b{};
    b.experts = experts_dev;
    b.shared = shared;
    b.act = a.act;
    b.n_active = a.n_active;
    b.act_stride = p.act_stride;
    b.chunks = (const int *)(ws + p.off_chunks);
    b.n_chunks = (const int *)(ws + p.off_nchunks);
    b.pairs = a.pairs;
    b.E = E;
    b.topk = k;
    b.Tk = T * k;
    b.staging = staging;
    b.stage_stride = p.stage_stride;
    for (int m = 0; m < 3; ++m) b.stage_off[m] = a.stage_off[m];
    return launch_prefill(p.max_chunks, b, x, T, s.hidden, s.ffn, (uint16_t *)(ws + p.off_xb),
                          (uint16_t *)(ws + p.off_hb), (float *)(ws + p.off_o), st);
  }
  if (p.qmm) {
    if (range != nullptr) return -2;  // whole steps only (routed experts in device memory)
    QmmArgs q{};
    q.experts = experts_dev;
    q.shared = shared;
    q.staging = staging;
    q.stage_stride = p.stage_stride;
    for (int m = 0; m < 3; ++m) q.stage_off[m] = a.stage_off[m];
    q.act = a.act;
    q.n_active = a.n_active;
    q.act_stride = p.act_stride;
    q.chunks = (const int *)(ws + p.off_chunks);
    q.n_chunks = (const int *)(ws + p.off_nchunks);
    q.pairs = a.pairs;
    q.E = E;
    q.topk = k;
    q.Tk = T * k;
    return launch_qmm_moe(q, p.qmm_nt, p.max_chunks, x, T, p.P, s.hidden, s.ffn,
                          ws + p.off_xsplit, ws + p.off_hsplit, (float *)(ws + p.off_h),
                          (float *)(ws + p.off_o), st);
  }
  if (p.klane) {
    MoeKlArgs g{};
    g.experts = experts_dev;
    g.shared = shared;
    g.staging = staging;
    g.stage_stride = p.stage_stride;
    for (int m = 0; m < 3; ++m) g.stage_off[m] = a.stage_off[m];
    g.act = a.act;
    g.n_active = a.n_active;
    g.pairs = a.pairs;
    g.slot0 = a.slot0;
    g.act_stride = p.act_stride;
    g.E = E;
    g.topk = k;
    g.Tk = T * k;
    MoeKlArgs d = g;
    g.gate_up = 1;
    g.rows = (int)(2 * s.ffn);
    g.row_bytes = s.hidden / 256 * 144;
    g.x = x;
    g.ldx = s.hidden;
    g.out = (float *)(ws + p.off_h);
    g.ldo = s.ffn;
    if (fuse_y != nullptr) {
      if (!moe_fuse_combine_ok(p) || range != nullptr) return -2;
      g.ctr = d.ctr = (unsigned *)(ws + p.off_ctr);
      g.nctr = p.nctr;  // d.nctr stays 0: only the gate/up launch clears them
      g.ctr_cap = d.ctr_cap = p.nctr;
      d.fuse_y = fuse_y;
      d.wts = (const float *)(ws + p.off_wts);
      d.inv = (const int *)(ws + p.off_inv);
      d.has_shared = s.has_shared ? 1 : 0;
    }
    if (route1) {  // the selection made by the gate/up launch (matrix-core kernel only)
      if (!p.route1 || range != nullptr || staging != nullptr || a.slot0 != 0) return -2;
      g.route1 = 1;
      g.route.part = (const float *)(ws + p.off_rpart);
      g.route.E = E;
      g.route.hsplit = p.hsplit;
      g.route.renormalize = s.renormalize;
      g.route.logits = (float *)(ws + p.off_logits);
      g.route.wts = (float *)(ws + p.off_wts);
      g.route.ids = (int *)(ws + p.off_ids);
      g.route.g1 = group1_out(p, ws);
      const int rc = launch_moe_mf(g, s.hidden, nslots, st);
      if (rc) return rc;
    } else {
      // the matrix-core kernel where it takes the shape, else lanes along k (the two launches may
      // differ: either kind of down launch counts on counters the gate/up launch cleared)
      int rc = launch_moe_mf(g, s.hidden, nslots, st);
      if (rc == -2) rc = launch_moe_kl(g, s.hidden, nslots, st);
      if (rc) return rc;
    }
    d.gate_up = 0;
    d.rows = (int)s.hidden;
    d.row_bytes = s.ffn / 256 * 144;
    d.x = (const float *)(ws + p.off_h);
    d.ldx = s.ffn;
    d.out = (float *)(ws + p.off_o);
    d.ldo = s.hidden;
    const int rc = launch_moe_mf(d, s.ffn, nslots, st);
    return rc == -2 ? launch_moe_kl(d, s.ffn, nslots, st) : rc;
  }
  // gate and up
  a.mat0 = 0;
  a.nmat = 2;
  a.n_rows = (int)s.ffn;
  a.units = (int)(s.hidden / 256);
  a.row_bytes = s.hidden / fmt_block_weights(s.type) * fmt_block_bytes(s.type);
  a.rowgroups = p.gu_rg;
  a.ksplit = p.gu_ks;
  a.upk = p.gu_upk;
  a.upw = p.gu_upw;
  a.xsrc = x;
  a.ldx = s.hidden;
  a.x_by_token = 1;
  a.out = (float *)(ws + p.off_gu);
  int rc = moe_gemv_dispatch(s.type, a, p.nt, nslots, p.gu_waves, st);
  if (rc) return rc;
  float *h = (float *)(ws + p.off_h);
  {
    const int64_t total = npos * s.ffn;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(k_moe_swiglu, dim3((unsigned)blocks), dim3(256), 0, st, (const float *)a.out,
                       p.gu_ks, p.P, (int)s.ffn, pos0, npos, h);
  }
  // down
  a.mat0 = 2;
  a.nmat = 1;
  a.n_rows = (int)s.hidden;
  a.units = (int)(s.ffn / 256);
  a.row_bytes = s.ffn / fmt_block_weights(s.type) * fmt_block_bytes(s.type);
  a.rowgroups = p.d_rg;
  a.ksplit = p.d_ks;
  a.upk = p.d_upk;
  a.upw = p.d_upw;
  a.xsrc = h;
  a.ldx = s.ffn;
  a.x_by_token = 0;
  a.out = (float *)(ws + p.off_o);
  return moe_gemv_dispatch(s.type, a, p.nt, nslots, p.d_waves, st);
}

}  // namespace tq
