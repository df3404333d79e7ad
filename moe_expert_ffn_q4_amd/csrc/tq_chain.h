// tq_chain.h -- the plan of a chain of batch-1 Q4_K products (internal to libtq). The host writes
// it once (tq_chain_prepare); the persistent kernel reads it on every run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

namespace tq {

// Plan layout (device memory, 256-byte aligned):
//   [0, 64)                  ChainHeader
//   [kChainErrorOffset, +4)  error word: 0, or (kind << 24) | op of the first wait that gave up
//                            (kind: kWait*), sticky until read
//   [kChainOpsOffset, ...)   ChainOp[nops]
//   [ctr_off, ...)           nops x 8 completion counters, 128 bytes apart
struct ChainHeader {
  int nops, total_items, ctr_off, magic;
};
constexpr int kChainMagic = 0x54514348;  // "TQCH"
constexpr int kChainErrorOffset = 128;
constexpr int kChainOpsOffset = 256;
constexpr int kChainMaxOps = 4096;
// Kinds of waits that can give up (recorded in the error word).
enum { kWaitDep = 1, kWaitX = 2, kWaitRing = 3, kWaitSums = 4 };
constexpr int kChainMaxK = 16384;  // the activation vector of an op is staged whole in LDS

struct ChainOp {
  const uint8_t *w[4];  // blobs of the matrices (swiglu: gate, up)
  float *y[4];          // outputs (swiglu: y[0] = h)
  const float *x;       // input [k]
  int64_t row_bytes;    // bytes of one row (k / 256 * 144)
  int cum[5];           // first row of each matrix among the op's rows
  int nparts, swiglu;
  int total;            // rows (swiglu: 2 n, gate and up rows alternating)
  int nblk;             // k / 256
  int rows_per_item;    // 16
  int items, item0;     // items of the op, index of its first item in the chain
  int dep;              // op that must have stored all its outputs first (-1: none)
  int x_dep;            // 1: x overlaps the outputs of an earlier op
};

// One product of a chain as the caller describes it (the fields of tq_chain_op).
struct ChainOpDesc {
  int nparts, swiglu;
  const void *w[4];
  int64_t n[4];
  float *y[4];
  int64_t k;
  const float *x;
};

size_t chain_plan_bytes(int nops);
// The plan bytes for ops (every field already checked): 0, or -1 if the chain is too long.
int chain_build(const ChainOpDesc *ops, int nops, std::vector<char> &buf);
int chain_counters_offset(int nops);
int launch_chain(void *plan, hipStream_t s);

}  // namespace tq
