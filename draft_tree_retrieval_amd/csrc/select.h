// Block-level selection helpers shared by the top-k kernels: ranking a
// few candidate keys held in LDS, and merging per-lane sorted lists.
#pragma once

#include "dev_common.h"

namespace tr {

constexpr int kCandW = 64;   // candidate slots per wave

// The KM largest of n <= blockDim.x distinct keys held contiguously in LDS,
// best first, into out[KM] (LDS; zero where n < KM): key t is ranked by
// thread t.
template <int KM>
__device__ __forceinline__ void rank_select(const uint64_t* keys, int n, uint64_t* out) {
  const int tid = threadIdx.x;
  if (tid < KM) out[tid] = 0;
  __syncthreads();
  if (tid < n) {
    const uint64_t mine = keys[tid];
    int rank = 0;
    for (int j = 0; j < n; ++j) rank += keys[j] > mine ? 1 : 0;
    if (rank < KM) out[rank] = mine;
  }
  __syncthreads();
}

// The same over NW per-wave lists: list w holds cnt[w] keys from
// keys + w * kCandW; n = cnt[0] + ... + cnt[NW-1] <= blockDim.x.
template <int KM, int NW>
__device__ __forceinline__ void rank_select_lists(const uint64_t* keys, const uint32_t* cnt, int n,
                                                  uint64_t* out) {
  const int tid = threadIdx.x;
  if (tid < KM) out[tid] = 0;
  __syncthreads();
  if (tid < n) {
    int w = 0, idx = tid;
    while (idx >= int(cnt[w])) { idx -= int(cnt[w]); ++w; }
    const uint64_t mine = keys[w * kCandW + idx];
    int rank = 0;
    for (int v = 0; v < NW; ++v) {
      const uint64_t* kv = keys + v * kCandW;
      const int c = int(cnt[v]);
      for (int j = 0; j < c; ++j) rank += kv[j] > mine ? 1 : 0;
    }
    if (rank < KM) out[rank] = mine;
  }
  __syncthreads();
}

// Block merge of per-lane lists: each wave's KM best, then the block's,
// into out[KM] (LDS).
template <int KM, int NW>
__device__ __forceinline__ void block_merge(TopList<KM>& L, uint64_t (*s_keys)[KM], uint64_t* out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t best[KM];
  wave_merge<KM>(L, best);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < KM; ++r) s_keys[wave][r] = best[r];
  }
  __syncthreads();
  if (wave == 0) {
    L.clear();
    if (lane < NW) {
#pragma unroll
      for (int r = 0; r < KM; ++r) L.v[r] = s_keys[lane][r];
    }
    wave_merge<KM>(L, best);
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < KM; ++r) out[r] = best[r];
    }
  }
  __syncthreads();
}

}  // namespace tr
