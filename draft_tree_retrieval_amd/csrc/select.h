// Block-level selection shared by the top-k kernels: the k best of one
// segment of a logit row (select_block), ranking a few candidate keys held
// in LDS, and merging per-lane sorted lists.
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


// Largest 64-bit key over the wave, in every lane: the codes' maximum,
// then the largest low word among the lanes holding that code (two DPP and
// permlane reductions instead of six 64-bit shuffles).
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v) {
  const uint32_t hi = uint32_t(v >> 32);
  const uint32_t mh = wave_max_u32(hi);
  const uint32_t ml = wave_max_u32(hi == mh ? uint32_t(v) : 0u);
  return (uint64_t(mh) << 32) | ml;
}

// Flip codes of two bfloat16 halves (16-bit arithmetic per half) or of one
// float: unsigned order = value order, -0.0 one below +0.0.
__device__ __forceinline__ uint32_t flip16x2(uint32_t w) {
  const uint32_t s = __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, w) >> (int16_t)15);
  return w ^ (s | 0x80008000u);
}
__device__ __forceinline__ uint32_t flip32(uint32_t w) {
  return w ^ (uint32_t(int32_t(w) >> 31) | 0x80000000u);
}
// The order code (ord32, which merges -0.0 and +0.0) of a flip code: equal
// for non-negative values, one more for negative ones.
__device__ __forceinline__ uint32_t ord_of_flip16(uint32_t u) { return (u < 0x8000u ? u + 1u : u) << 16; }
__device__ __forceinline__ uint32_t ord_of_flip32(uint32_t u) { return u < 0x80000000u ? u + 1u : u; }

// x[i] for a per-lane i, by a binary tree of selects on the bits of i
// (indexing the register array itself would move it to scratch memory).
template <int N>
__device__ __forceinline__ u32x4 pick(const u32x4 (&x)[N], int i) {
  u32x4 a[N];
#pragma unroll
  for (int q = 0; q < N; ++q) a[q] = x[q];
#pragma unroll
  for (int s = 0, w = N; w > 1; ++s, w >>= 1) {
    const bool up = ((i >> s) & 1) != 0;
#pragma unroll
    for (int q = 0; q < w / 2; ++q) a[q] = up ? a[2 * q + 1] : a[2 * q];
  }
  return a[0];
}

// The k best elements of the segment [s0, s1) of a logit row (rowp: the
// row's first element), value descending, ties to the lower id, -0.0 equal
// to +0.0 (the argtopk of the Chinese summary of "Token Recycling", section
// Method; softmax is increasing, so the ids are selected on the raw
// logits).  One block of NT threads, every element read once into registers
// (NV 16-byte vectors per lane, so s1 - s0 <= NT * NV * 16 / element size):
//   1. every element becomes a flip code and every vector keeps its largest;
//   2. with FIRST, the block's largest code gives the best element (the
//      lowest id among those with that code), reported at once through
//      out.first(id) by thread 0 before the rest of the selection; then
//      each wave bisects its lane maxima for the k-th largest and keeps its
//      k largest;
//   3. T = the k-th largest of the waves' kept maxima is reached by k
//      elements, so every one of the k best reaches it (lowered by one when
//      it is +0.0's flip code, so -0.0 passes too): only vectors whose
//      maximum reaches T are opened, one per lane and pass, and their
//      elements >= T go to per-wave candidate lists in LDS by ballot;
//   4. wave 0 ranks the candidates in registers; tie-heavy rows overflowing
//      a list fall back to exact per-lane insertion.
// Results go out through out.put(r, key) for ranks r < KM (key_of codes;
// key 0 for places past the segment's elements; with FIRST, ranks from 1).
// The code is loops rather than unrolled copies: each block runs it once,
// latency-bound, from a cold instruction cache.
template <bool BF16, int KM, int NT, int NV, bool FIRST, typename Out>
__device__ __forceinline__ void select_block(const uint8_t* __restrict__ rowp, int64_t s0,
                                             int64_t s1, int32_t k, Out& out) {
  constexpr int NW = NT / 64;
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int VE = 16 / ESZ;
  constexpr uint32_t kZeroPos = BF16 ? 0x8000u : 0x80000000u;   // flip code of +0.0
  static_assert(NV <= 32, "the hit mask holds 32 vectors");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  __shared__ uint64_t s_cand[NW * kCandW];
  __shared__ uint64_t s_keys[NW][KM];
  __shared__ uint64_t s_best[KM];
  __shared__ uint32_t s_top[NW * KM];
  __shared__ uint32_t s_mx[NW];
  __shared__ uint32_t s_am[NW];
  __shared__ uint32_t s_wcnt[NW];

  // aligned vectors [a0, a1) inside [s0, s1); fewer than VE loose elements
  // on either side, loaded first from clamped (always valid) indices
  const uintptr_t addr0 = reinterpret_cast<uintptr_t>(rowp + s0 * ESZ);
  int64_t a0 = s0 + int64_t(((16 - (addr0 & 15)) & 15) / ESZ);
  if (a0 > s1) a0 = s1;
  const int nv = int((s1 - a0) / VE);
  const int64_t a1 = a0 + int64_t(nv) * VE;
  const int64_t hid = s0 + tid, tl = a1 + tid;
  const bool hvalid = hid < a0, tvalid = tl < s1;
  uint32_t hraw, traw;
  if (BF16) {
    hraw = reinterpret_cast<const uint16_t*>(rowp)[min(hid, s1 - 1)];
    traw = reinterpret_cast<const uint16_t*>(rowp)[min(tl, s1 - 1)];
  } else {
    hraw = reinterpret_cast<const uint32_t*>(rowp)[min(hid, s1 - 1)];
    traw = reinterpret_cast<const uint32_t*>(rowp)[min(tl, s1 - 1)];
  }
  const u32x4* vp = reinterpret_cast<const u32x4*>(rowp + a0 * ESZ);
  u32x4 x[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = i * NT + tid;
    x[i] = idx < nv ? __builtin_nontemporal_load(vp + idx) : u32x4{0, 0, 0, 0};
  }

  // ---- 1. flip codes in place (0: no element), vector and lane maxima
  uint32_t vm[NV];
  uint32_t lm = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const uint32_t keep = (i * NT + tid < nv) ? ~0u : 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) x[i][j] = (BF16 ? flip16x2(x[i][j]) : flip32(x[i][j])) & keep;
    if (BF16) {
      vm[i] = max16x2(max16x2(x[i][0], x[i][1]), max16x2(x[i][2], x[i][3]));
      lm = max16x2(lm, vm[i]);
    } else {
      vm[i] = max(max(x[i][0], x[i][1]), max(x[i][2], x[i][3]));
      lm = max(lm, vm[i]);
    }
  }
  const uint32_t hu = hvalid ? (BF16 ? (flip16x2(hraw) & 0xFFFFu) : flip32(hraw)) : 0u;
  const uint32_t tu = tvalid ? (BF16 ? (flip16x2(traw) & 0xFFFFu) : flip32(traw)) : 0u;
  if (BF16) lm = max(lm & 0xFFFFu, lm >> 16);
  lm = max(lm, max(hu, tu));

  // ---- 2. with FIRST, the best element before the rest of the selection
  if (FIRST) {
    const uint32_t wmx = wave_max_u32(lm);
    if (lane == 0) s_mx[wave] = wmx;
    __syncthreads();
    // the best element: Ma admits the block's largest code (and -0.0 with
    // +0.0); each lane holding such an element finds its lowest id (head,
    // then its vectors in order, then tail), the block the lowest of those
    uint32_t Mx = s_mx[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) Mx = max(Mx, s_mx[w]);
    const uint32_t Ma = Mx == kZeroPos ? kZeroPos - 1 : Mx;
    uint32_t inv = 0;                                  // ~id of the lane's first element >= Ma
    if (lm >= Ma) {
      if (hu >= Ma) {
        inv = ~uint32_t(hid);
      } else {
        const uint32_t bm = BF16 ? (Ma - 1) * 0x10001u : Ma - 1;
        uint32_t am = 0;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const bool hit = BF16 ? (max16x2(vm[i], bm) ^ bm) != 0u : vm[i] > bm;
          am |= hit ? (1u << i) : 0u;
        }
        if (am) {
          const int i0 = __builtin_ctz(am);
          const u32x4 v = pick<NV>(x, i0);
          int e = 0;
#pragma unroll
          for (int j = 3; j >= 0; --j) {
            if (BF16) {
              if ((v[j] >> 16) >= Ma) e = 2 * j + 1;
              if ((v[j] & 0xFFFFu) >= Ma) e = 2 * j;
            } else if (v[j] >= Ma) {
              e = j;
            }
          }
          inv = ~uint32_t(a0 + int64_t(i0 * NT + tid) * VE + e);
        } else {
          inv = ~uint32_t(tl);
        }
      }
    }
    inv = wave_max_u32(inv);
    if (lane == 0) s_am[wave] = inv;
    __syncthreads();
    if (tid == 0) {
      uint32_t best = s_am[0];
#pragma unroll
      for (int w = 1; w < NW; ++w) best = max(best, s_am[w]);
      out.first(~best);
    }
  }

  // ---- 2b. the wave's k-th largest lane maximum and its k largest
  constexpr int kBits = BF16 ? 16 : 32;
  uint32_t lo = 0;
#pragma unroll
  for (int bit = kBits - 1; bit >= 0; --bit) {
    const uint32_t c = lo | (1u << bit);
    if (__popcll(__ballot(lm >= c)) >= k) lo = c;
  }
  {
    const uint64_t gt = __ballot(lm > lo);               // fewer than k lanes
    const int ngt = __popcll(gt);
    const uint32_t below =
        __builtin_amdgcn_mbcnt_hi(uint32_t(gt >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(gt), 0u));
    if (lm > lo) s_top[wave * KM + below] = lm;
    if (lane >= ngt && lane < k) s_top[wave * KM + lane] = lo;
  }
  __syncthreads();

  // ---- 3. T = the block's k-th largest lane maximum (the k-th largest of
  // the waves' k largest).  Candidates: elements at or above T.
  constexpr int NTOP = NW * KM;
  constexpr int NTV = (NTOP + 63) / 64;
  uint32_t tv[NTV];
#pragma unroll
  for (int h = 0; h < NTV; ++h) {
    const int i = lane + 64 * h;
    tv[h] = (i < NTOP && (i % KM) < k) ? s_top[min(i, NTOP - 1)] : 0u;
  }
  uint32_t T = 0;
#pragma unroll
  for (int bit = kBits - 1; bit >= 0; --bit) {
    const uint32_t c = T | (1u << bit);
    int reach = 0;
#pragma unroll
    for (int h = 0; h < NTV; ++h) reach += __popcll(__ballot(tv[h] >= c));
    if (reach >= k) T = c;
  }
  if (T == kZeroPos) T = kZeroPos - 1;                 // -0.0 ties with +0.0
  if (T == 0) T = 1;                                   // 0 marks "no element"
  uint64_t* wc = s_cand + wave * kCandW;
  uint32_t wpos = 0;                                   // wave-uniform
  auto put = [&](bool pred, uint32_t code, int64_t id) {
    const uint64_t m = __ballot(pred);
    if (m) {
      const uint32_t off =
          wpos + __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
      if (pred && off < uint32_t(kCandW)) wc[off] = key_of(code, uint32_t(id));
      wpos += uint32_t(__popcll(m));
    }
  };
  // per lane, the vectors whose maximum reaches T; then one such vector
  // per lane and pass, taken out of the registers by a select tree
  const uint32_t below2 = BF16 ? (T - 1) * 0x10001u : T - 1;
  uint32_t hm = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const bool hit = BF16 ? (max16x2(vm[i], below2) ^ below2) != 0u : vm[i] > below2;
    hm |= hit ? (1u << i) : 0u;
  }
  while (__ballot(hm != 0u) != 0) {
    const bool act = hm != 0u;
    const int i = act ? __builtin_ctz(hm) : 0;
    hm &= hm - 1u;
    const u32x4 v = pick<NV>(x, i);
    const int64_t id = a0 + int64_t(i * NT + tid) * VE;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (BF16) {
        const uint32_t u0 = v[j] & 0xFFFFu, u1 = v[j] >> 16;
        put(act && u0 >= T, ord_of_flip16(u0), id + 2 * j);
        put(act && u1 >= T, ord_of_flip16(u1), id + 2 * j + 1);
      } else {
        put(act && v[j] >= T, ord_of_flip32(v[j]), id + j);
      }
    }
  }
  put(hu >= T, BF16 ? ord_of_flip16(hu) : ord_of_flip32(hu), hid);
  put(tu >= T, BF16 ? ord_of_flip16(tu) : ord_of_flip32(tu), tl);
  if (lane == 0) s_wcnt[wave] = wpos;
  __syncthreads();
  uint32_t n = 0, most = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    n += s_wcnt[w];
    most = max(most, s_wcnt[w]);
  }
  const bool overflow = most > uint32_t(kCandW);
  constexpr int r0 = FIRST ? 1 : 0;

  // ---- 4. rank
  if (!overflow && n <= 64u) {
    if (wave == 0) {
      uint32_t c[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) c[w] = s_wcnt[w];
      int src = -1, before = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        if (src < 0 && lane < before + int(c[w])) src = w * kCandW + (lane - before);
        before += int(c[w]);
      }
      const uint64_t key = src >= 0 ? s_cand[src] : 0ull;
      int rank = 0;
      for (int j = 0; j < int(n); ++j) rank += readlane_u64(key, j) > key ? 1 : 0;
      if (lane >= int(n)) rank = lane;                 // places past the elements hold key 0
      if (rank >= r0 && rank < KM) out.put(rank, key);
    }
    return;
  }
  if (!overflow && n <= uint32_t(NT)) {
    rank_select_lists<KM, NW>(s_cand, s_wcnt, int(n), s_best);
  } else {
    TopList<KM> L;
    L.clear();
    if (!overflow) {
      for (int c = tid; c < NW * kCandW; c += NT)
        if (uint32_t(c % kCandW) < s_wcnt[c / kCandW]) L.insert(s_cand[c]);
    } else {
      // too many ties at the threshold: exact insertion from the registers
#pragma unroll 1
      for (int i = 0; i < NV; ++i) {
        const u32x4 v = pick<NV>(x, i);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t id = a0 + int64_t(i * NT + tid) * VE + (BF16 ? 2 * j : j);
          if (BF16) {
            const uint32_t u0 = v[j] & 0xFFFFu, u1 = v[j] >> 16;
            if (u0 >= T) L.insert(key_of(ord_of_flip16(u0), uint32_t(id)));
            if (u1 >= T) L.insert(key_of(ord_of_flip16(u1), uint32_t(id + 1)));
          } else if (v[j] >= T) {
            L.insert(key_of(ord_of_flip32(v[j]), uint32_t(id)));
          }
        }
      }
      if (hu >= T) L.insert(key_of(BF16 ? ord_of_flip16(hu) : ord_of_flip32(hu), uint32_t(hid)));
      if (tu >= T) L.insert(key_of(BF16 ? ord_of_flip16(tu) : ord_of_flip32(tu), uint32_t(tl)));
    }
    block_merge<KM, NW>(L, s_keys, s_best);
  }
  if (tid >= r0 && tid < KM) out.put(tid, s_best[tid]);
}

}  // namespace tr
