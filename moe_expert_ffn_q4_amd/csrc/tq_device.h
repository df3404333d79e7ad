// tq_device.h -- small device helpers shared by the libtq kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

// Four dwords, 16-byte aligned.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// Four dwords loaded with only 4-byte alignment guaranteed (rows of Q6_K / Q8_0 blobs).
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));

// Loads and stores through the global address space. Pointers read from a device table, or
// passed through an asm statement (the scalar-register selects of the row maps), are generic to
// the compiler, and generic (flat) accesses count against lgkmcnt as well as vmcnt: every wait
// for a scalar load or an LDS access would then also wait for the weight prefetch in flight.
typedef const u32x4 __attribute__((address_space(1))) *gu32x4;
typedef const u32x4a4 __attribute__((address_space(1))) *gu32x4a4;

__device__ __forceinline__ u32x4 gload(const void *p) { return *(gu32x4)p; }
__device__ __forceinline__ void gstore(float *p, float v) {
  *(__attribute__((address_space(1))) float *)p = v;
}

// IEEE binary16 bits (low 16 bits of `bits`) -> fp32. Exact; subnormals are kept because HIP
// kernels run with fp16 denormals enabled.
__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}

// Byte e (0..3) of w as an fp32 integer value (compiles to v_cvt_f32_ubyteN).
__device__ __forceinline__ float byte_to_float(uint32_t w, int e) {
  return (float)((w >> (8 * e)) & 0xFFu);
}

// Bytes 2h and 2h+1 of w, each holding a value 0..15, converted to fp32 by the fp8 (e4m3)
// conversion unit: a byte b < 16 is either the subnormal b * 2^-9 (exponent field 0) or the normal
// (1 + (b-8)/8) * 2^-6 = b * 2^-9 (exponent field 1), so the result is exactly b times a power of
// two, two values per instruction. nibble_fp8_unit() is that power of two (read back from the
// hardware so that either fp8 exponent bias works).
template <bool HIGH_HALF>
__device__ __forceinline__ void nibbles_to_float(uint32_t w, float &a, float &b) {
  const auto v = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HIGH_HALF);
  a = v[0];
  b = v[1];
}
__device__ __forceinline__ float nibble_fp8_unit() {
  return __builtin_amdgcn_cvt_pk_f32_fp8(1, false)[0];
}

// w with what the compiler knows about its bits forgotten. After masking a dword down to four
// nibbles, this keeps the four byte conversions as one v_cvt_f32_ubyteN each; otherwise the
// compiler re-derives each nibble with its own shift/mask before converting.
__device__ __forceinline__ uint32_t opaque(uint32_t w) {
  asm("" : "+v"(w));
  return w;
}

// The dword that starts two bytes into the 8-byte pair (hi:lo).
__device__ __forceinline__ uint32_t shift2(uint32_t lo, uint32_t hi) {
  return __builtin_amdgcn_alignbyte(hi, lo, 2);
}

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t float_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

// SwiGLU of one gate/up pair: silu(g) * u = g * u / (1 + e^-g).
__device__ __forceinline__ float silu_mul(float g, float u) { return g * u / (1.f + expf(-g)); }

__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Completion counters of the k-sliced products: the workgroup that finishes a row group's last k
// slice adds the slices' partial sums. Every arrival adds D = (token << 16) + 1 to its row group's
// 8-byte word, the token being the launch's (never zero, different for every launch the host
// makes: call_tag()). A word that only this launch's arrivals have touched since it was zero
// therefore holds exactly count * D (mod 2^64), and one fetch-add both counts an arrival and
// shows that; whatever bytes a fresh workspace holds pass that test only by a 2^-48 chance. The
// last workgroup sets its word back to zero (done_arrivals): a launch recorded in a HIP graph
// keeps its token on every replay, and zero is 0 * D for any token. Nothing has to be cleared by
// the caller.
struct Arrivals {
  unsigned long long *ctr;  // one 8-byte word per row group
  unsigned long long tag;   // token << 16
};
constexpr unsigned long long kArrivalCountMask = 0xFFFFull;

// Counts the calling workgroup on row group g and returns true for the one that brings the count
// to `parts` (< 65536). One thread calls it, after the workgroup's partial sums have completed at
// agent scope. An add that lands on a word that is not count * D (bytes another call or another
// use of the memory left) turns it into 1 * D by compare-and-swap, or, when another workgroup of
// this launch has done that in the meantime, counts itself on that word (its add on the old word
// is dropped with the old word).
__device__ inline bool arrive_last(const Arrivals &a, int g, unsigned parts) {
  unsigned long long *p = a.ctr + g;
  const unsigned long long D = a.tag | 1ull;
  auto ours = [D](unsigned long long v) { return v == (v & kArrivalCountMask) * D; };
  unsigned long long w = __hip_atomic_fetch_add(p, D, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!ours(w)) {
    w += D;  // what the word holds if nobody else touched it
    for (;;) {
      if (__hip_atomic_compare_exchange_strong(p, &w, D, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT))
        return parts == 1u;
      if (ours(w)) {  // claimed by another workgroup of this launch
        w = __hip_atomic_fetch_add(p, D, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  return (unsigned)(w & kArrivalCountMask) + 1u == parts;
}

// The last workgroup of row group g, once done: the word back to zero for the next launch.
__device__ inline void done_arrivals(const Arrivals &a, int g) {
  __hip_atomic_store(a.ctr + g, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace tq
