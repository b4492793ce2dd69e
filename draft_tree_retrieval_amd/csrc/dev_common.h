// Device helpers shared by the libtr kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tr_internal.h"

namespace tr {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- numbers
// Order-preserving map of an IEEE float bit pattern to uint32 (larger value
// -> larger code).  The folded form maps -0.0 onto +0.0 so that equal
// values compare equal.
__device__ __forceinline__ uint32_t ord_nofold(uint32_t bits) {
  return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}
__device__ __forceinline__ uint32_t ord_fold(uint32_t bits) {
  return ord_nofold(bits == 0x80000000u ? 0u : bits);
}
// Selection key: value first, then the lower token id wins ties.
__device__ __forceinline__ uint64_t make_key(uint32_t bits, uint32_t id) {
  return (uint64_t(ord_fold(bits)) << 32) | uint32_t(~id);
}
__device__ __forceinline__ uint32_t key_id(uint64_t key) { return ~uint32_t(key); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {  // round to nearest even
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// ---------------------------------------------------------------- waves
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor(uint32_t(v), m, 64);
  uint32_t hi = __shfl_xor(uint32_t(v >> 32), m, 64);
  return (uint64_t(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = max(v, (uint32_t)__shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Sorted (descending) list of the KM best keys seen by one lane.
template <int KM>
struct TopList {
  uint64_t v[KM];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int i = 0; i < KM; ++i) v[i] = 0;
  }
  // One bubble pass: keeps the KM largest of list + {x}, sorted.
  __device__ __forceinline__ void insert(uint64_t x) {
#pragma unroll
    for (int i = 0; i < KM; ++i) {
      uint64_t hi = v[i] > x ? v[i] : x;
      uint64_t lo = v[i] > x ? x : v[i];
      v[i] = hi;
      x = lo;
    }
  }
  __device__ __forceinline__ void pop() {
#pragma unroll
    for (int i = 0; i < KM - 1; ++i) v[i] = v[i + 1];
    v[KM - 1] = 0;
  }
};

// The KM best keys over the lists of all 64 lanes, best first; every lane
// returns the same array.  Real keys are unique (distinct token ids).
template <int KM>
__device__ __forceinline__ void wave_merge(TopList<KM>& L, uint64_t* out) {
#pragma unroll
  for (int r = 0; r < KM; ++r) {
    uint64_t m = wave_max_u64(L.v[0]);
    out[r] = m;
    if (m != 0 && L.v[0] == m) L.pop();
  }
}

// ---------------------------------------------------------------- handshake
// Called by every thread of a block after it wrote its results.  Returns
// true in every thread of the block that arrives last among `total`
// blocks sharing `counter`; that block sees the others' writes, and the
// counter is back to zero for the next call.
__device__ __forceinline__ bool last_block_arrives(uint32_t* counter, uint32_t total) {
  __shared__ uint32_t s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t prev = atomicAdd(counter, 1u);
    bool last = (prev == total - 1);
    if (last) atomicExch(counter, 0u);
    s_last = last ? 1u : 0u;
  }
  __syncthreads();
  bool last = s_last != 0;
  if (last) __threadfence();
  return last;
}

__device__ __forceinline__ void set_flag(uint8_t* ws, uint32_t bit) {
  if (ws) atomicOr(reinterpret_cast<uint32_t*>(ws), bit);
}

}  // namespace tr
