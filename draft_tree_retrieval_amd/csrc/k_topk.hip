// argtopk over vocabulary-wide logit rows, fused with the per-sequence tail
// of a TR step (verification, update of M, commit, next retrieval).
//
// The update M[x~_i] = argtopk(p~_{i+1}) needs the k best token ids of
// every tree node's next-token distribution (Chinese summary of "Token
// Recycling", section Method).  Softmax is increasing, so the ids are
// selected on the raw logits.  The scan is bound by HBM bandwidth: every
// logit is read once, with 16-byte loads, and a lane keeps its own sorted
// list of the best keys in registers.  A cheap filter on the value code
// (maximum of a loaded vector against the lane's current k-th best) skips
// almost every element; since a lane visits ids in increasing order, an
// element equal to the k-th best value always loses the tie, so a strict
// test is exact.
//
// Launch: grid (segments, rows), 256 threads.  Rows are split into
// segments so that short vocabularies still fill the 256 CUs; the last
// segment block of a row merges the segment lists, and the last row block
// of a sequence runs that sequence's tail.
#include "tail.h"

namespace tr {

TopkPlan plan_topk(int64_t rows, int64_t V, int32_t k) {
  TopkPlan p{};
  p.rows = rows;
  p.kmax = k <= 8 ? 8 : 16;
  // about two blocks per CU, segments of at least 2048 logits, at most 64
  int64_t want = (512 + rows - 1) / rows;
  int64_t by_len = V / 2048;
  int64_t segs = want < by_len ? want : by_len;
  if (segs < 1) segs = 1;
  if (segs > 64) segs = 64;
  int64_t len = (V + segs - 1) / segs;
  len = (len + 7) & ~int64_t(7);
  segs = (V + len - 1) / len;
  p.segs = int32_t(segs);
  p.seg_len = len;
  size_t off = kDataOff;
  p.part_off = off;
  off = align256(off + size_t(rows) * segs * p.kmax * 8);
  p.ids_off = off;
  off = align256(off + size_t(rows) * k * 4);
  p.end = off;
  return p;
}

template <bool BF16, int KM>
__device__ __forceinline__ void scan_vec(const u32x4& x, uint32_t id0, TopList<KM>& L, uint32_t& thr) {
  uint32_t w[4] = {x[0], x[1], x[2], x[3]};
  constexpr int NE = BF16 ? 8 : 4;
  uint32_t bits[NE];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (BF16) {
      bits[2 * j] = w[j] << 16;
      bits[2 * j + 1] = w[j] & 0xFFFF0000u;
    } else {
      bits[j] = w[j];
    }
  }
  uint32_t m = 0;
#pragma unroll
  for (int e = 0; e < NE; ++e) m = max(m, ord_nofold(bits[e]));
  if (m > thr) {
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      uint64_t key = make_key(bits[e], id0 + e);
      if (key > L.v[KM - 1]) L.insert(key);
    }
    thr = uint32_t(L.v[KM - 1] >> 32);
  }
}

template <bool BF16, int KM>
__device__ __forceinline__ void scan_one(uint32_t raw, uint32_t id, TopList<KM>& L) {
  uint32_t bits = BF16 ? (raw << 16) : raw;
  uint64_t key = make_key(bits, id);
  if (key > L.v[KM - 1]) L.insert(key);
}

template <bool BF16, int KM>
__global__ __launch_bounds__(256) void topk_kernel(const void* __restrict__ logits, int64_t V,
                                                   int32_t k, int32_t segs, int64_t seg_len,
                                                   int32_t* __restrict__ ids_out,
                                                   uint64_t* __restrict__ part, uint8_t* ws,
                                                   TreeDev tree, TailArgs tail) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int VE = 16 / ESZ;             // elements per 16-byte vector
  constexpr int U = 4;                     // vectors in flight per lane
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.y;
  const int seg = blockIdx.x;
  const int64_t s0 = int64_t(seg) * seg_len;
  const int64_t s1 = min(V, s0 + seg_len);
  const uint8_t* rowp = reinterpret_cast<const uint8_t*>(logits) + row * V * ESZ;

  TopList<KM> L;
  L.clear();
  uint32_t thr = 0;

  // aligned vector range [a0, a1) inside [s0, s1)
  const uintptr_t addr0 = reinterpret_cast<uintptr_t>(rowp + s0 * ESZ);
  int64_t a0 = s0 + int64_t(((16 - (addr0 & 15)) & 15) / ESZ);
  if (a0 > s1) a0 = s1;
  const int64_t nv = (s1 - a0) / VE;
  const int64_t a1 = a0 + nv * VE;
  auto raw_at = [&](int64_t i) -> uint32_t {
    return BF16 ? uint32_t(reinterpret_cast<const uint16_t*>(rowp)[i])
                : reinterpret_cast<const uint32_t*>(rowp)[i];
  };
  // head (lowest ids) first, then vectors, then the tail: ids rise per lane
  if (s0 + tid < a0) scan_one<BF16, KM>(raw_at(s0 + tid), uint32_t(s0 + tid), L);
  thr = uint32_t(L.v[KM - 1] >> 32);
  const u32x4* vp = reinterpret_cast<const u32x4*>(rowp + a0 * ESZ);
  for (int64_t base = 0; base < nv; base += int64_t(256) * U) {
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * 256 + tid;
      x[u] = i < nv ? __builtin_nontemporal_load(vp + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * 256 + tid;
      if (i < nv) scan_vec<BF16, KM>(x[u], uint32_t(a0 + i * VE), L, thr);
    }
  }
  if (a1 + tid < s1) scan_one<BF16, KM>(raw_at(a1 + tid), uint32_t(a1 + tid), L);

  // block merge: each wave's KM best, then the block's KM best
  __shared__ uint64_t s_keys[4][KM];
  uint64_t best[KM];
  wave_merge<KM>(L, best);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < KM; ++r) s_keys[wave][r] = best[r];
  }
  __syncthreads();
  if (wave == 0) {
    L.clear();
    if (lane < 4) {
#pragma unroll
      for (int r = 0; r < KM; ++r) L.v[r] = s_keys[lane][r];
    }
    wave_merge<KM>(L, best);
  }

  if (segs > 1) {
    if (wave == 0 && lane == 0) {
#pragma unroll
      for (int r = 0; r < KM; ++r) part[(row * segs + seg) * KM + r] = best[r];
    }
    uint32_t* row_cnt = reinterpret_cast<uint32_t*>(ws + kRowCntOff);
    if (!last_block_arrives(row_cnt + row, uint32_t(segs))) return;
    if (wave == 0) {
      L.clear();
      if (lane < segs) {
#pragma unroll
        for (int r = 0; r < KM; ++r) L.v[r] = part[(row * segs + lane) * KM + r];
      }
      wave_merge<KM>(L, best);
    }
  }
  if (wave == 0 && lane == 0) {
#pragma unroll
    for (int r = 0; r < KM; ++r)
      if (r < k) ids_out[row * k + r] = int32_t(key_id(best[r]));
  }
  if (tail.mode == TAIL_NONE) return;

  // ---- per-sequence tail, run by the last row block of the sequence
  const int b = int(row / tree.T);
  uint32_t* seq_cnt = reinterpret_cast<uint32_t*>(ws + kSeqCntOff);
  if (!last_block_arrives(seq_cnt + b, uint32_t(tree.T))) return;

  __shared__ TailShared S;
  const int32_t* topk_b = ids_out + int64_t(b) * tree.T * k;
  int32_t* tok_b = tail.tree_tok + int64_t(b) * tree.T;
  const size_t msz = tail.m_is64 ? 8 : 4;
  void* M_b = reinterpret_cast<uint8_t*>(tail.M) + size_t(b) * size_t(V) * size_t(k) * msz;
  tail_load(S, tree, tok_b, topk_b, k);
  if (tail.mode == TAIL_STEP) {
    tail_verify(S, tree);
    tail_write_verdict(S, tree, b, tail.accept_len, tail.accept_path, nullptr, tail.emitted);
  }
  tail_update(S, tree, topk_b, k, M_b, tail.m_is64, V, ws);
  if (tail.mode != TAIL_STEP) return;
  tail_commit(S, tree, b, tail, ws);
  __threadfence();
  __syncthreads();
  tail_retrieve(S, tree, S.bonus, M_b, tail.m_is64, V, k, tok_b, ws);
  if (threadIdx.x == 0) tail.root_tok[b] = S.bonus;
}

hipError_t launch_topk(const TreeDev& tree, int32_t B, const void* logits, int l_is_bf16, int64_t V,
                       int32_t k, int32_t* topk_ids, const TailArgs& tail, uint8_t* ws,
                       const TopkPlan& plan, hipStream_t s) {
  dim3 grid(plan.segs, unsigned(plan.rows));
  uint64_t* part = reinterpret_cast<uint64_t*>(ws + plan.part_off);
#define TR_TOPK(BF, KMV)                                                                       \
  hipLaunchKernelGGL((topk_kernel<BF, KMV>), grid, dim3(256), 0, s, logits, V, k, plan.segs, \
                     plan.seg_len, topk_ids, part, ws, tree, tail)
  if (l_is_bf16) {
    if (plan.kmax == 8) TR_TOPK(true, 8); else TR_TOPK(true, 16);
  } else {
    if (plan.kmax == 8) TR_TOPK(false, 8); else TR_TOPK(false, 16);
  }
#undef TR_TOPK
  return hipGetLastError();
}

}  // namespace tr
