// Device helpers shared by the libtr kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tr_internal.h"

namespace tr {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- numbers
// Order code of an IEEE float bit pattern: a larger value gets a larger
// code, -0.0 and +0.0 get the same code (0x80000000), and every non-NaN
// value gets a code above 0 (so 0 can mark "empty").  Negative values map
// to the two's complement negation of their bits, the others to the bits
// plus 2^31.
__device__ __forceinline__ uint32_t ord32(uint32_t bits) {
  return (bits & 0x80000000u) ? (0u - bits) : (bits + 0x80000000u);
}
// The same code for each bfloat16 half of a word (16-bit arithmetic per
// half): ord16(h) << 16 == ord32(h << 16).
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef int16_t i16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t ord16x2(uint32_t w) {
  const u16x2 x = __builtin_bit_cast(u16x2, w);
  const uint32_t neg_mask = __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, w) >> (int16_t)15);
  const uint32_t neg = __builtin_bit_cast(uint32_t, (u16x2)(0) - x);
  const uint32_t pos = __builtin_bit_cast(uint32_t, x + (u16x2)(0x8000));
  return (neg & neg_mask) | (pos & ~neg_mask);
}
__device__ __forceinline__ uint32_t max16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}
// Selection key: value first, then the lower token id wins ties.
__device__ __forceinline__ uint64_t key_of(uint32_t code, uint32_t id) {
  return (uint64_t(code) << 32) | uint32_t(~id);
}
__device__ __forceinline__ uint64_t make_key(uint32_t bits, uint32_t id) { return key_of(ord32(bits), id); }
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
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  uint32_t lo = __shfl(uint32_t(v), src, 64);
  uint32_t hi = __shfl(uint32_t(v >> 32), src, 64);
  return (uint64_t(hi) << 32) | lo;
}
// Lane src's value (src the same in every lane).
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int src) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v)), src));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v >> 32)), src));
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
// Maximum over the wave, in every lane, without the LDS crossbar: DPP
// within each 16-lane row (swap neighbours, swap pairs, mirror the halves,
// mirror the row: after each step a lane holds the maximum over 2, 4, 8,
// 16 lanes), then gfx950's permlane swaps across rows and halves.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0xB1, 0xF, 0xF, false)));   // quad_perm 1,0,3,2
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x4E, 0xF, 0xF, false)));   // quad_perm 2,3,0,1
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x141, 0xF, 0xF, false)));  // row_half_mirror
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x140, 0xF, 0xF, false)));  // row_mirror
  const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(uint32_t(r16[0]), uint32_t(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(uint32_t(r32[0]), uint32_t(r32[1]));
}
// Reductions over lanes l, l^16 (x16) or l, l^32 (x32) with gfx950's
// permlane swaps (VALU, no trip through the LDS crossbar).  With both
// operands equal to v, permlane16_swap returns (even 16-lane rows of v in
// both rows of each pair, odd rows likewise) and permlane32_swap returns
// (lower half in both halves, upper half likewise).
__device__ __forceinline__ float xmax16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xmax32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xsum16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xsum32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
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

// In-wave bitonic sort of one 64-bit key per lane, largest at lane 0.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t o = shfl_xor_u64(v, j);
      const bool keep_max = ((lane & j) == 0) == ((lane & k) == 0);
      v = keep_max ? (o > v ? o : v) : (o < v ? o : v);
    }
  }
  return v;
}

// ---------------------------------------------------------------- handshake
// Blocks of one launch hand results to the block that arrives last.  The
// L2 caches of the XCDs are not coherent with each other, and a device-scope
// fence would write back and invalidate a whole L2, so nothing here uses
// one.  Instead every value handed over is written with a device-scope
// atomic exchange (performed at the device's coherence point) by thread 0
// of the writing block, which waits for those atomics to complete before it
// counts the block in; the last block reads the values with device-scope
// atomic loads, which do not hit stale L2 lines.
__device__ __forceinline__ void put_dev(uint64_t* p, uint64_t v) {
  __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_dev(int32_t* p, int32_t v) {
  __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get_dev(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t get_dev(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Called by every thread of a block after thread 0 wrote its hand-over
// values with put_dev.  Returns true in every thread of the block that
// arrives last among `total` blocks sharing `counter`; the counter is back
// to zero afterwards.
__device__ __forceinline__ bool last_block_arrives(uint32_t* counter, uint32_t total) {
  __shared__ uint32_t s_last;
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_s_waitcnt(0);     // this thread's put_dev atomics have completed
    const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = (prev == total - 1);
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last ? 1u : 0u;
  }
  __syncthreads();
  return s_last != 0;
}

__device__ __forceinline__ void set_flag(uint8_t* ws, uint32_t bit) {
  if (ws) atomicOr(reinterpret_cast<uint32_t*>(ws), bit);
}

}  // namespace tr
