// argtopk over vocabulary-wide logit rows, fused with the per-sequence tail
// of a TR step (verification, update of M, commit, next retrieval).
//
// The update M[x~_i] = argtopk(p~_{i+1}) needs the k best token ids of
// every tree node's next-token distribution (Chinese summary of "Token
// Recycling", section Method).  Softmax is increasing, so the ids are
// selected on the raw logits.  Ties go to the lower id, -0.0 equals +0.0.
//
// The scan is bound by HBM bandwidth, so every logit is read once and kept
// in registers.  A block owns one segment of a row (at most 16 x 16 bytes
// per lane) and selects in three steps:
//   1. every lane turns its values into order codes in place and takes
//      their maximum;
//   2. the lanes of a wave form KM groups; each group's maximum is reached
//      by one of its elements, so the smallest of the KM group maxima is
//      reached by KM distinct elements and nothing below it can be among
//      the KM best.  The block threshold is the largest of the four waves'
//      values;
//   3. only elements at or above the threshold -- usually a few dozen --
//      go to a candidate list in LDS, where each is ranked against the
//      others.
// Rows full of ties can overflow the candidate list; the block then falls
// back to exact per-lane insertion of every element above the threshold.
//
// Launch: grid (segments, rows), 256 threads.  Segments spread short
// vocabularies over the CUs; the last segment block of a row merges the
// segment lists, and the last row block of a sequence runs that sequence's
// tail (hand-over through device-scope atomics, see dev_common.h).
#include "tail.h"

namespace tr {

constexpr int kNV = 16;       // 16-byte vectors per lane per segment
constexpr int kCand = 512;    // candidate slots per block

TopkPlan plan_topk(int64_t rows, int64_t V, int32_t k, int32_t esz) {
  TopkPlan p{};
  p.rows = rows;
  p.kmax = k <= 8 ? 8 : 16;
  const int64_t cap = int64_t(256) * kNV * (16 / esz);   // largest segment a block holds
  const int64_t max_segs = 256 / p.kmax;                 // the final merge ranks <= 256 keys
  int64_t need = (V + cap - 1) / cap;
  int64_t want = (256 + rows - 1) / rows;         // about one block per CU
  int64_t by_len = V / 4096;                      // but segments of >= 4096 logits
  int64_t segs = want < by_len ? want : by_len;
  if (segs < need) segs = need;
  if (segs < 1) segs = 1;
  if (segs > max_segs) segs = max_segs;
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

// The KM largest of n <= blockDim.x distinct keys held in LDS, best first,
// into out[KM] (LDS; zero where n < KM): key t is ranked by thread t.
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

// Block merge of per-lane lists: each wave's KM best, then the block's,
// into out[KM] (LDS).
template <int KM>
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
    if (lane < 4) {
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

template <bool BF16, int KM>
__global__ __launch_bounds__(256) void topk_kernel(const void* __restrict__ logits, int64_t V,
                                                   int32_t k, int32_t segs, int64_t seg_len,
                                                   int32_t* __restrict__ ids_out,
                                                   uint64_t* __restrict__ part, uint8_t* ws,
                                                   TreeDev tree, TailArgs tail) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int VE = 16 / ESZ;             // elements per 16-byte vector
  constexpr int GL = 64 / KM;              // lanes per threshold group
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.y;
  const int seg = blockIdx.x;
  const int64_t s0 = int64_t(seg) * seg_len;
  const int64_t s1 = min(V, s0 + seg_len);
  const uint8_t* rowp = reinterpret_cast<const uint8_t*>(logits) + row * V * ESZ;

  __shared__ uint64_t s_cand[kCand];
  __shared__ uint64_t s_keys[4][KM];
  __shared__ uint64_t s_best[KM];
  __shared__ uint32_t s_cnt;
  __shared__ uint32_t s_lo[4];
  if (tid == 0) s_cnt = 0;

  // aligned vector range [a0, a1) inside [s0, s1); at most VE-1 loose
  // elements on each side
  const uintptr_t addr0 = reinterpret_cast<uintptr_t>(rowp + s0 * ESZ);
  int64_t a0 = s0 + int64_t(((16 - (addr0 & 15)) & 15) / ESZ);
  if (a0 > s1) a0 = s1;
  const int nv = int((s1 - a0) / VE);
  const int64_t a1 = a0 + int64_t(nv) * VE;
  auto code_at = [&](int64_t i) -> uint32_t {
    return BF16 ? ord32(uint32_t(reinterpret_cast<const uint16_t*>(rowp)[i]) << 16)
                : ord32(reinterpret_cast<const uint32_t*>(rowp)[i]);
  };

  // ---- 1. load, order codes in place (0 marks "no element"), lane maximum
  const u32x4* vp = reinterpret_cast<const u32x4*>(rowp + a0 * ESZ);
  u32x4 x[kNV];
#pragma unroll
  for (int i = 0; i < kNV; ++i) {
    const int idx = i * 256 + tid;
    x[i] = idx < nv ? __builtin_nontemporal_load(vp + idx) : u32x4{0, 0, 0, 0};
  }
  uint32_t loose_code[2] = {0, 0};       // head and tail elements
  const int64_t loose_id[2] = {s0 + tid, a1 + tid};
  if (loose_id[0] < a0) loose_code[0] = code_at(loose_id[0]);
  if (loose_id[1] < s1) loose_code[1] = code_at(loose_id[1]);
  uint32_t mt = max(loose_code[0], loose_code[1]);
  uint32_t m2 = 0;
#pragma unroll
  for (int i = 0; i < kNV; ++i) {
    const uint32_t keep = (i * 256 + tid < nv) ? ~0u : 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (BF16) {
        x[i][j] = ord16x2(x[i][j]) & keep;
        m2 = max16x2(m2, x[i][j]);
      } else {
        x[i][j] = ord32(x[i][j]) & keep;
        mt = max(mt, x[i][j]);
      }
    }
  }
  if (BF16) mt = max(mt, max(m2 & 0xFFFFu, m2 >> 16) << 16);

  // ---- 2. threshold
  uint32_t gm = mt;
#pragma unroll
  for (int sh = 1; sh < GL; sh <<= 1) gm = max(gm, (uint32_t)__shfl_xor(gm, sh, 64));
#pragma unroll
  for (int sh = GL; sh < 64; sh <<= 1) gm = min(gm, (uint32_t)__shfl_xor(gm, sh, 64));
  if (lane == 0) s_lo[wave] = gm;
  __syncthreads();
  const uint32_t lo = max(max(s_lo[0], s_lo[1]), max(s_lo[2], s_lo[3]));

  // ---- 3. candidates
  auto push = [&](uint32_t code, int64_t id) {
    const uint32_t slot = atomicAdd(&s_cnt, 1u);
    if (slot < uint32_t(kCand)) s_cand[slot] = key_of(code, uint32_t(id));
  };
  if (BF16) {
    const uint32_t lo16 = lo >> 16;
    const uint32_t below2 = lo16 ? (lo16 - 1) * 0x10001u : 0u;   // lo16-1 in both halves
#pragma unroll
    for (int i = 0; i < kNV; ++i) {
      const uint32_t vmx = max16x2(max16x2(x[i][0], x[i][1]), max16x2(x[i][2], x[i][3]));
      const bool hit = lo16 ? max16x2(vmx, below2) != below2 : vmx != 0u;
      if (hit) {
        const int64_t id = a0 + int64_t(i * 256 + tid) * VE;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t c0 = x[i][j] & 0xFFFFu, c1 = x[i][j] >> 16;
          if (c0 && c0 >= lo16) push(c0 << 16, id + 2 * j);
          if (c1 && c1 >= lo16) push(c1 << 16, id + 2 * j + 1);
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kNV; ++i) {
      const uint32_t vmx = max(max(x[i][0], x[i][1]), max(x[i][2], x[i][3]));
      if (vmx && vmx >= lo) {
        const int64_t id = a0 + int64_t(i * 256 + tid) * VE;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (x[i][j] && x[i][j] >= lo) push(x[i][j], id + j);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h)
    if (loose_code[h] && loose_code[h] >= lo) push(loose_code[h], loose_id[h]);
  __syncthreads();
  const uint32_t n = s_cnt;

  // ---- the block's KM best into s_best
  if (n <= 256u) {
    rank_select<KM>(s_cand, int(n), s_best);
  } else {
    TopList<KM> L;
    L.clear();
    if (n <= uint32_t(kCand)) {
      for (uint32_t c = tid; c < n; c += 256) L.insert(s_cand[c]);
    } else {
      // too many ties at the threshold: exact insertion from the registers
#pragma unroll
      for (int i = 0; i < kNV; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t id = a0 + int64_t(i * 256 + tid) * VE + (BF16 ? 2 * j : j);
          if (BF16) {
            const uint32_t c0 = (x[i][j] & 0xFFFFu) << 16, c1 = x[i][j] & 0xFFFF0000u;
            if (c0 && c0 >= lo) L.insert(key_of(c0, uint32_t(id)));
            if (c1 && c1 >= lo) L.insert(key_of(c1, uint32_t(id + 1)));
          } else if (x[i][j] && x[i][j] >= lo) {
            L.insert(key_of(x[i][j], uint32_t(id)));
          }
        }
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (loose_code[h] && loose_code[h] >= lo) L.insert(key_of(loose_code[h], uint32_t(loose_id[h])));
    }
    block_merge<KM>(L, s_keys, s_best);
  }

  // ---- segments of a row meet in the last one
  if (segs > 1) {
    if (tid == 0) {
#pragma unroll
      for (int r = 0; r < KM; ++r) put_dev(&part[(row * segs + seg) * KM + r], s_best[r]);
    }
    uint32_t* row_cnt = reinterpret_cast<uint32_t*>(ws + kRowCntOff);
    if (!last_block_arrives(row_cnt + row, uint32_t(segs))) return;
    const int nk = segs * KM;                   // <= 256 by the plan
    for (int c = tid; c < nk; c += 256) s_cand[c] = get_dev(&part[row * segs * KM + c]);
    __syncthreads();
    rank_select<KM>(s_cand, nk, s_best);
  }
  if (tid == 0) {
#pragma unroll
    for (int r = 0; r < KM; ++r)
      if (r < k) put_dev(&ids_out[row * k + r], int32_t(key_id(s_best[r])));
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
  __syncthreads();          // the M rows written above are read below by this block
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
