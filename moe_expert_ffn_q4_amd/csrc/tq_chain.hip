// tq_chain.hip -- a chain of batch-1 Q4_K products run by one persistent launch.
//
// A decode step is a chain: every product's input is derived from an earlier product's output
// (q|k|v -> attention -> o -> residual and norm -> gate|up -> SwiGLU -> down -> residual and norm
// -> the next layer). KTransformers replays each decode step as one CUDA graph (its page,
// "KTransformers 的技术原理", "CUDA Graph 优化"); here the whole chain is one kernel launch. The
// weights never depend on activations, so the waves that multiply keep requesting weights of
// later work while the chain waits at the boundary between two products, where separate
// launches would drain and refill the machine.
//
// Work: each product ("op") is cut into items of 16 rows. Items of all ops are numbered in chain
// order and dealt round robin to the workgroups (item t -> workgroup t mod grid), which must all
// be resident at once: the grid is at most what the device holds. In a workgroup, wave 0 is the
// control wave and the seven others multiply:
//   * multiplying wave c owns slice c of k (blocks c nblk / 7 .. (c + 1) nblk / 7) of every item,
//     streams it block by block with the next blocks' weights in flight in registers, waits only
//     for its own loads and for LDS flags, and leaves its slice's row sums in an LDS ring. The
//     products run on the int8 matrix cores with exact operands (the GEMV core of tq_gemv_i8.h:
//     the nibbles as int8, each 256-value block of x as four 7-bit digits after a power-of-two
//     scale, one fp32 fold per block), so the waves' vector ALUs are not what bounds them;
//   * the control wave stages each op's x in LDS, adds the seven slice sums of each row in slice
//     order, stores the op's outputs (device-scope stores), and when the workgroup's last item of
//     an op is stored and its stores have completed, adds the workgroup's items to one of eight
//     per-op counters. Before staging an op's x it waits until the counters of the op before it
//     reach that op's item count; an x that no earlier op writes is requested before that wait.
//     It has no weight loads of its own, so its waits for completed stores cost only the stores.
// Every wait is bounded: after about a second without progress it sets the plan's error word and
// gives up, so the launch always ends; the host reads the error word with tq_chain_status.
#include "tq_chain.h"
#include "tq_gemv_core.h"
#include "tq_gemv_i8.h"

#include <vector>

namespace tq {

namespace {

constexpr int kWaves = 8;          // waves per workgroup
constexpr int kDepth = 4;          // blocks of weights per multiplying wave in registers
constexpr int kSub = 8;            // counters per op (a workgroup uses counter blockIdx % 8)
constexpr int kLine = 128;         // bytes between counters
constexpr unsigned kPollLimit = 1u << 22;  // polls (each a memory round trip and a short sleep)

// The plan as the kernel sees it: the header and op table (read only, so scalar loads), and the
// counters and error word (written) through a second pointer into the same buffer.
struct Plan {
  const char *__restrict__ ro;
  char *__restrict__ rw;
};

// An op's table entry, read with scalar loads into scalar registers. The compiler would read it
// with vector loads (it cannot prove that the output stores, through pointers loaded from this
// same table, leave the table alone), and every wait for those would also wait for all the weight
// loads in flight. The asm waits for its own results.
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
static_assert(sizeof(ChainOp) == 136 && offsetof(ChainOp, y) == 32 && offsetof(ChainOp, x) == 64 &&
                  offsetof(ChainOp, cum) == 80 && offsetof(ChainOp, nparts) == 100 &&
                  offsetof(ChainOp, item0) == 124 && offsetof(ChainOp, dep) == 128 &&
                  offsetof(ChainOp, x_dep) == 132,
              "ChainOp is read as 16 + 16 + 2 dwords");
__device__ __forceinline__ ChainOp op_at(const Plan &p, int o) {
  const char *e = p.ro + kChainOpsOffset + (int64_t)o * sizeof(ChainOp);
  u32x16 a, b;
  u32x2 c;
  asm volatile("s_load_dwordx16 %0, %3, 0x0\n\ts_load_dwordx16 %1, %3, 0x40\n\t"
               "s_load_dwordx2 %2, %3, 0x80\n\ts_waitcnt lgkmcnt(0)"
               : "=s"(a), "=s"(b), "=s"(c)
               : "s"(e)
               : "memory");
  // fields by dword position (static_asserts below check the layout)
  auto u64 = [](uint32_t lo, uint32_t hi) { return ((uint64_t)hi << 32) | lo; };
  ChainOp op;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    op.w[q] = (const uint8_t *)u64(a[2 * q], a[2 * q + 1]);
    op.y[q] = (float *)u64(a[8 + 2 * q], a[9 + 2 * q]);
  }
  op.x = (const float *)u64(b[0], b[1]);
  op.row_bytes = (int64_t)u64(b[2], b[3]);
#pragma unroll
  for (int q = 0; q < 5; ++q) op.cum[q] = (int)b[4 + q];
  op.nparts = (int)b[9];
  op.swiglu = (int)b[10];
  op.total = (int)b[11];
  op.nblk = (int)b[12];
  op.rows_per_item = (int)b[13];
  op.items = (int)b[14];
  op.item0 = (int)b[15];
  op.dep = (int)c[0];
  op.x_dep = (int)c[1];
  return op;
}
// Only the first item of op o (one scalar load).
__device__ __forceinline__ int op_item0(const Plan &p, int o) {
  const char *e = p.ro + kChainOpsOffset + (int64_t)o * sizeof(ChainOp) + offsetof(ChainOp, item0);
  uint32_t v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(e) : "memory");
  return (int)v;
}
__device__ __forceinline__ unsigned *counter(const Plan &p, int o, int sub) {
  uint32_t off;
  asm volatile("s_load_dword %0, %1, 0x8\n\ts_waitcnt lgkmcnt(0)" : "=s"(off) : "s"(p.ro) : "memory");
  return reinterpret_cast<unsigned *>(p.rw + off + ((int64_t)o * kSub + sub) * kLine);
}
__device__ __forceinline__ unsigned *error_word(const Plan &p) {
  return reinterpret_cast<unsigned *>(p.rw + kChainErrorOffset);
}
// A wait that gave up: the first one is recorded as (kind << 24) | op (see tq_chain.h).
__device__ __forceinline__ void give_up(const Plan &p, int kind, int o) {
  unsigned expected = 0;
  __hip_atomic_compare_exchange_strong(error_word(p), &expected, ((unsigned)kind << 24) | ((unsigned)o & 0xFFFFFFu),
                                       __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Rows of one op: up to four matrices back to back, or gate and up rows alternating (swiglu).
struct ChainMap {
  const uint8_t *w0, *w1, *w2, *w3;
  float *y0, *y1, *y2, *y3;
  int c1, c2, c3;
  int swiglu, total;
  int64_t row_bytes;

  __device__ __forceinline__ void init(const ChainOp &op) {
    w0 = op.w[0];
    w1 = op.w[1];
    w2 = op.w[2];
    w3 = op.w[3];
    y0 = op.y[0];
    y1 = op.y[1];
    y2 = op.y[2];
    y3 = op.y[3];
    c1 = op.nparts > 1 ? op.cum[1] : 1 << 30;
    c2 = op.nparts > 2 ? op.cum[2] : 1 << 30;
    c3 = op.nparts > 3 ? op.cum[3] : 1 << 30;
    swiglu = op.swiglu;
    total = op.total;
    row_bytes = op.row_bytes;
  }
  __device__ __forceinline__ const uint8_t *row(int v) const {
    const uint8_t *p0 = w0, *p1 = w1, *p2 = w2, *p3 = w3;
    if (swiglu) return ((v & 1) ? p1 : p0) + (int64_t)(v >> 1) * row_bytes;
    const uint8_t *b = v >= c3 ? p3 : v >= c2 ? p2 : v >= c1 ? p1 : p0;
    const int first = v >= c3 ? c3 : v >= c2 ? c2 : v >= c1 ? c1 : 0;
    return b + (int64_t)(v - first) * row_bytes;
  }
  __device__ __forceinline__ float *out(int v) const {
    float *p0 = y0, *p1 = y1, *p2 = y2, *p3 = y3;
    float *b = v >= c3 ? p3 : v >= c2 ? p2 : v >= c1 ? p1 : p0;
    const int first = v >= c3 ? c3 : v >= c2 ? c2 : v >= c1 ? c1 : 0;
    return b + (v - first);
  }
};

// Outputs are read by later ops of the same launch on other XCDs: stored and loaded at device
// scope (the L2 of each XCD is not coherent with the others').
__device__ __forceinline__ void put(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) float lds_float;

// Copies x [k] of op `op` into LDS as stored, with system-scope loads (cache policy sc0 sc1: no
// cache of this XCD answers them) straight into LDS, one wave, 1 KB pieces.
__device__ __forceinline__ void x_to_lds(const ChainOp &op, float *xs, int lane) {
  for (int q = 0; q < op.nblk; ++q)
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(op.x + 256 * q + 4 * lane),
                                     (lds_float *)(xs + 256 * q), 16, 0, 17);
}

// Wave 0: wait until every item of op `dep` has been stored (bounded; see the file comment).
__device__ __forceinline__ void wait_op(const Plan &plan, int dep, unsigned need, int lane) {
  unsigned *err = error_word(plan);
  for (unsigned polls = 0;; ++polls) {
    unsigned v = 0;
    // read-modify-write atomics: performed where the counters live, never answered from a copy
    // of the line that a cache of this XCD may still hold
    if (lane < kSub) v = __hip_atomic_fetch_add(counter(plan, dep, lane), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (lane == kSub) v = __hip_atomic_fetch_add(err, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned sum = 0;
#pragma unroll
    for (int s = 0; s < kSub; ++s) sum += __builtin_amdgcn_readlane(v, s);
    const unsigned failed = __builtin_amdgcn_readlane(v, kSub);
    if (sum >= need || failed) return;
    if (polls >= kPollLimit) {
      if (lane == 0) give_up(plan, kWaitDep, dep);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// The op holding item t, searching forward from op o.
__device__ __forceinline__ int op_of(const Plan &plan, int o, int nops, int t) {
  while (o + 1 < nops && t >= op_item0(plan, o + 1)) ++o;
  return o;
}

constexpr int kNC = kWaves - 1;  // multiplying waves of a workgroup
constexpr int kTile = 16;        // rows per item
constexpr int kRing = 16;        // items of slice sums between the multiplying waves and the control

// Blocks [b0, b1) of k that multiplying wave c owns in an op of nblk blocks.
__device__ __forceinline__ int slice_begin(int nblk, int c) { return (c * nblk) / kNC; }

// LDS shared by the waves of a workgroup. It is a file-scope variable, so every access in the
// functions below is an LDS instruction: through a generic pointer it would be a flat access,
// which the compiler also counts as a vector-memory access, so that every wait for it would wait
// for all the weight loads in flight as well.
struct Shared {
  float xs[kChainMaxK];                        // x of the current op, as stored
  uint8_t dig[kChainMaxK / 256][kLdsBlock];    // int8 digits of every block of x (each wave its own)
  float part[kRing][kNC][kTile];               // slice sums of the last kRing items
  unsigned filled[kRing];                      // multiplying waves done with each ring slot
  unsigned xready;                             // op whose x is in xs, plus one (0: none)
  unsigned consumed;                           // items the control wave has stored
};
__shared__ __attribute__((aligned(16))) Shared g_sh;

__device__ __forceinline__ unsigned lds_get(const unsigned &w) {
  return __hip_atomic_load(&w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_set(unsigned &w, unsigned v) {
  __hip_atomic_store(&w, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Bounded spin on an LDS word until `done(value)`; gives up (and flags the plan) after the
// limit, or at once when a wait elsewhere has already failed.
template <class F>
__device__ __forceinline__ void lds_wait(const Plan &plan, const unsigned &word, int lane, int kind,
                                         int o, F done) {
  // the flag is the same for every lane: made uniform, so the loop exit is too
  for (unsigned polls = 1; !done(__builtin_amdgcn_readfirstlane(lds_get(word))); ++polls) {
    if ((polls & 1023) == 0) {
      if (__builtin_amdgcn_readfirstlane(__hip_atomic_fetch_add(error_word(plan), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) break;
      if (polls >= kPollLimit) {
        if (lane == 0) give_up(plan, kind, o);
        break;
      }
    }
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");  // later LDS reads stay after the wait
}

// One block of weights of a 16-row tile, as loaded by one lane: the row's block header and its
// half (l / 32) of each of the four 32-byte quant groups; zero for lanes l % 32 >= 16.
struct Blk {
  u32x4 head, q[4];
};

// A position in a multiplying wave's walk: item t (sequence number s in the workgroup), its op,
// and block i of the wave's slice of that op.
struct Cursor {
  int t, s, o, i, b0, nb, item0, end;  // end: first item past op o
};

// A multiplying wave: wave c + 1 of the workgroup, slice c of every item; D blocks of weights in
// registers (D - 1 in flight while one is computed).
template <int D>
struct Mul {
  Plan plan;
  int nops, total, G, c, lane;
  Cursor cc;      // compute side
  Cursor lc;      // load side (ahead of cc by D - 1 blocks)
  ChainMap lm;    // rows of the load side's op
  int entered;    // op whose digits this wave has made (-1: none)
  float acc;

  // fill o, b0, nb, item0, end for k.t; the op table is read only when k.t has left op k.o
  __device__ __forceinline__ void locate(Cursor &k) {
    if (k.t < k.end && k.t >= k.item0) return;
    k.o = op_of(plan, k.o, nops, k.t);
    const ChainOp op = op_at(plan, k.o);
    k.b0 = slice_begin(op.nblk, c);
    k.nb = slice_begin(op.nblk, c + 1) - k.b0;
    k.item0 = op.item0;
    k.end = op.item0 + op.items;
  }
  // the load cursor's next block: across items (skipping items where the slice is empty)
  __device__ __forceinline__ void advance_load() {
    if (lc.i + 1 < lc.nb) {
      ++lc.i;
      return;
    }
    Cursor k = lc;
    k.i = 0;
    for (;;) {
      k.t += G;
      if (k.t >= total) return;  // no further block: the last one is read again (never computed)
      locate(k);
      if (k.nb > 0) break;
    }
    if (k.o != lc.o) lm.init(op_at(plan, k.o));
    lc = k;
  }
  // Straight-line loads (no branch around them, so the compiler keeps exact counts of the loads in
  // flight): lanes l % 32 >= 16 read the row of lane l - 16 again (cache hits) and their operands
  // are zeroed when the block is computed; past the last item the last block is read again.
  __device__ __forceinline__ void load(Blk &b) {
    const int n = lane & 15, h = lane >> 5;
    const int row = min((lc.t - lc.item0) * kTile + n, lm.total - 1);
    const uint8_t *p = lm.row(row) + (int64_t)(lc.b0 + lc.i) * 144;
    b.head = gload(p);
#pragma unroll
    for (int g = 0; g < 4; ++g) b.q[g] = gload(p + 16 + 32 * g + 16 * h);
  }
  __device__ __forceinline__ void issue(Blk &b) {
    advance_load();
    load(b);
  }
  // item s's slot in the ring is free once the control wave has stored item s - kRing
  __device__ __forceinline__ void ring_room(int s) {
    const unsigned need = (unsigned)(s - kRing + 1);
    if (s >= kRing) lds_wait(plan, g_sh.consumed, lane, kWaitRing, cc.o, [need](unsigned x) { return (int)(x - need) >= 0; });
  }
  // this wave's sums of item s (rows in lanes 0..15) into the ring
  __device__ __forceinline__ void put_sums(int s, float v) {
    ring_room(s);
    if (lane < kTile) g_sh.part[s % kRing][c][lane] = v;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the sums are in LDS before the count
    if (lane == 0) __hip_atomic_fetch_add(&g_sh.filled[s % kRing], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  // move the compute cursor to the next item, giving zero sums for items with an empty slice
  __device__ __forceinline__ bool next_item() {
    cc.i = 0;
    for (;;) {
      cc.t += G;
      ++cc.s;
      if (cc.t >= total) return false;
      locate(cc);
      if (cc.nb > 0) return true;
      put_sums(cc.s, 0.f);
    }
  }
  // entering an op: wait for its x in LDS, then make the digits of this wave's blocks
  __device__ __forceinline__ void enter(int o) {
    entered = o;
    const unsigned want = (unsigned)o + 1;
    lds_wait(plan, g_sh.xready, lane, kWaitX, o, [want](unsigned x) { return x == want; });
    for (int p = 0; p < cc.nb; p += 4) {
      const int b = cc.b0 + p + (lane >> 4);
      if (b < cc.b0 + cc.nb) make_digits(g_sh.xs + 256 * b, lane & 15, g_sh.dig[b]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  template <int J>
  __device__ __forceinline__ bool step(Blk (&v)[D]) {
    issue(v[(J + D - 1) % D]);  // the weights D - 1 blocks ahead, before any wait
    if (cc.i == 0) {
      if (cc.o != entered) enter(cc.o);
      acc = 0.f;
    }
    const int b = cc.b0 + cc.i, n = lane & 31, h = lane >> 5;
    const uint8_t *l = g_sh.dig[b];
    const u32x4 xa = *reinterpret_cast<const u32x4 *>(l + n * 32 + 16 * h);
    const u32x4 S = *reinterpret_cast<const u32x4 *>(l + kDigitBytes + 16 * h);
    const float us = *reinterpret_cast<const float *>(l + kDigitBytes + 32);
    const bool live = n < kTile;
    const u32x4 z = {0u, 0u, 0u, 0u};
    const u32x4 q4[4] = {live ? v[J].q[0] : z, live ? v[J].q[1] : z, live ? v[J].q[2] : z,
                         live ? v[J].q[3] : z};
    acc += i8_block(live ? v[J].head : z, q4, xa, S, us, n >> 2, h);
    if (++cc.i < cc.nb) return true;
    // the item's slice is done: the two sub-block parities of each row, then the ring
    const float row = acc + __shfl_xor(acc, 32);
    put_sums(cc.s, row);
    return next_item();
  }
  template <int J>
  __device__ __forceinline__ bool steps(Blk (&v)[D]) {
    if (!step<J>(v)) return false;
    if constexpr (J + 1 < D) return steps<J + 1>(v);
    return true;
  }
  __device__ __forceinline__ void run(int t0) {
    entered = -1;
    cc = Cursor{t0, 0, 0, 0, 0, 0, 0, 0};
    locate(cc);
    if (cc.nb == 0) {  // leading items with an empty slice
      put_sums(cc.s, 0.f);
      if (!next_item()) return;
    }
    lc = cc;
    lm.init(op_at(plan, lc.o));
    Blk v[D];
    load(v[0]);
#pragma unroll
    for (int i = 1; i < D - 1; ++i) issue(v[i]);
    while (steps<0>(v)) {
    }
  }
};

// The control wave: dependencies, x, the slice sums' totals, output stores and counts.
__device__ __forceinline__ void control(const Plan &plan, int nops, int total, int G, int lane) {
  int co = -1, end = 0;
  ChainMap m;
  ChainOp op;
  for (int t = (int)blockIdx.x, s = 0; t < total; t += G, ++s) {
    const int o = t < end ? co : op_of(plan, co < 0 ? 0 : co, nops, t);
    if (o != co) {
      co = o;
      op = op_at(plan, o);
      end = op.item0 + op.items;
      m.init(op);
      // every multiplying wave is done with the previous op's x and digits: all earlier items
      // are stored
      if (!op.x_dep) x_to_lds(op, g_sh.xs, lane);  // x from outside the chain: read it at once
      if (op.dep >= 0) wait_op(plan, op.dep, (unsigned)op_at(plan, op.dep).items, lane);
      if (op.x_dep) x_to_lds(op, g_sh.xs, lane);   // x written by an earlier op
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // x has landed in LDS
      if (lane == 0) lds_set(g_sh.xready, (unsigned)co + 1);
    }
    const int slot = s % kRing;
    lds_wait(plan, g_sh.filled[slot], lane, kWaitSums, co, [](unsigned x) { return x == (unsigned)kNC; });
    // row r (lane r < 16): the slices' sums added in slice order
    float v = 0.f;
    if (lane < kTile)
#pragma unroll
      for (int cw = 0; cw < kNC; ++cw) v += g_sh.part[slot][cw][lane];
    const int r0 = (t - op.item0) * kTile, r = r0 + lane;
    if (m.swiglu) {  // gate / up rows alternate: the pair (r, r + 1) for even r
      const float u = __shfl_down(v, 1);
      if (lane < kTile && (lane & 1) == 0 && r < m.total) put(m.y0 + (r >> 1), silu_mul(v, u));
    } else if (lane < kTile && r < m.total) {
      put(m.out(r), v);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the sums are read before the slot is freed
    if (lane == 0) {
      lds_set(g_sh.filled[slot], 0u);
      lds_set(g_sh.consumed, (unsigned)s + 1);
    }
    const bool last_of_op = t + G >= total || t + G >= op.item0 + op.items;
    if (last_of_op) {
      // the outputs were stored at device scope and have completed before the counter moves; a
      // release fence would also write back the whole L2 of the XCD, which costs more than the
      // products themselves
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      const int first = ((int)blockIdx.x - op.item0 % G + G) % G;  // this workgroup's first item
      const int mine = (op.items - 1 - first) / G + 1;
      if (lane == 0)
        __hip_atomic_fetch_add(counter(plan, co, blockIdx.x % kSub), (unsigned)mine,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

// kWaves waves per workgroup (wave 0 controls, the others multiply), D blocks of weights in
// registers per multiplying wave.
template <int D>
__global__ __launch_bounds__(64 * kWaves) void k_chain(const char *__restrict__ ro, char *__restrict__ rw) {
  const Plan plan{ro, rw};
  u32x2 hd;
  asm volatile("s_load_dwordx2 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(hd) : "s"(ro) : "memory");
  const int nops = (int)hd[0], total = (int)hd[1], G = (int)gridDim.x;
  const int wave = wave_index(), lane = (int)threadIdx.x & 63;
  if ((int)blockIdx.x >= total) return;
  if (threadIdx.x < kRing) g_sh.filled[threadIdx.x] = 0u;
  if (threadIdx.x == 0) {
    g_sh.xready = 0u;
    g_sh.consumed = 0u;
  }
  __syncthreads();
  if (wave == 0) {
    control(plan, nops, total, G, lane);
    return;
  }
  Mul<D> mw;
  mw.plan = plan;
  mw.nops = nops;
  mw.total = total;
  mw.G = G;
  mw.c = wave - 1;
  mw.lane = lane;
  mw.run((int)blockIdx.x);
}

// Clears the counters of a plan before a run (a fill kernel rather than a memset, so that the
// pair can be captured into a graph and replayed).
__global__ __launch_bounds__(256) void k_chain_reset(char *__restrict__ plan) {
  const ChainHeader &h = *reinterpret_cast<const ChainHeader *>(plan);
  for (int i = (int)(blockIdx.x * blockDim.x + threadIdx.x); i < h.nops * kSub;
       i += (int)(gridDim.x * blockDim.x))
    *reinterpret_cast<unsigned *>(plan + h.ctr_off + (int64_t)i * kLine) = 0u;
}

int chain_counters_offset(int nops) {
  return (int)((kChainOpsOffset + (int64_t)nops * sizeof(ChainOp) + 255) & ~(int64_t)255);
}

size_t chain_plan_bytes(int nops) {
  return (size_t)chain_counters_offset(nops) + (size_t)nops * kSub * kLine;
}

int chain_build(const ChainOpDesc *ops, int nops, std::vector<char> &buf) {
  buf.assign(chain_plan_bytes(nops), 0);
  ChainHeader &h = *reinterpret_cast<ChainHeader *>(buf.data());
  ChainOp *tab = reinterpret_cast<ChainOp *>(buf.data() + kChainOpsOffset);
  int64_t item0 = 0;
  for (int i = 0; i < nops; ++i) {
    const ChainOpDesc &d = ops[i];
    ChainOp &o = tab[i];
    const int nparts = d.swiglu ? 2 : d.nparts;
    int64_t rows = 0;
    for (int p = 0; p < 4; ++p) {
      o.w[p] = p < nparts ? (const uint8_t *)d.w[p] : (const uint8_t *)d.w[0];
      o.y[p] = p < nparts ? d.y[p] : d.y[0];
      o.cum[p] = (int)rows;
      if (p < nparts) rows += d.n[p];
    }
    o.cum[4] = (int)rows;
    o.nparts = nparts;
    o.swiglu = d.swiglu ? 1 : 0;
    o.total = d.swiglu ? (int)(2 * d.n[0]) : (int)rows;
    o.x = d.x;
    o.nblk = (int)(d.k / 256);
    o.row_bytes = (int64_t)o.nblk * 144;
    o.rows_per_item = kTile;
    o.items = (o.total + o.rows_per_item - 1) / o.rows_per_item;
    o.item0 = (int)item0;
    o.dep = i - 1;
    // x written by an earlier op of the chain (then it is read only after the op before this one)
    o.x_dep = 0;
    const char *xb = (const char *)d.x, *xe = xb + 4 * d.k;
    for (int j = 0; j < i && !o.x_dep; ++j)
      for (int p = 0; p < (ops[j].swiglu ? 1 : ops[j].nparts); ++p) {
        const char *yb = (const char *)ops[j].y[p], *ye = yb + 4 * ops[j].n[p];
        if (yb < xe && xb < ye) o.x_dep = 1;
      }
    item0 += o.items;
  }
  if (item0 > (int64_t)1 << 30) return -1;
  h.nops = nops;
  h.total_items = (int)item0;
  h.ctr_off = chain_counters_offset(nops);
  h.magic = kChainMagic;
  return 0;
}

#define kChainKernel (k_chain<kDepth>)

int chain_grid(int *grid) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(kChainKernel),
                                                   64 * kWaves, 0) != hipSuccess)
    return -1;
  if (per_cu < 1 || cus < 1) return -1;
  const int want = 8 / kWaves;  // two waves per SIMD
  *grid = cus * (per_cu < want ? per_cu : want);
  return 0;
}

int launch_chain(void *plan, hipStream_t s) {
  int grid = 0;
  if (chain_grid(&grid)) return -1;
  hipLaunchKernelGGL(k_chain_reset, dim3(8), dim3(256), 0, s, (char *)plan);
  if (hipGetLastError() != hipSuccess) return -1;
  hipLaunchKernelGGL(kChainKernel, dim3((unsigned)grid), dim3(64 * kWaves), 0, s, (const char *)plan,
                     (char *)plan);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace tq
