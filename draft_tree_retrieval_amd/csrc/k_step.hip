// The greedy TR step for few logit rows (a single sequence or a handful:
// fewer than 256 rows of at most 32768 logits), where the step's time is
// latency, not bandwidth.
//
// One launch holds three kinds of blocks, each waiting only on blocks of
// lower index:
//   * row blocks (one per tree node of every sequence): the argtopk of the
//     node's logit row (the M[x~_i] = argtopk(p~_{i+1}) update of the
//     Chinese summary of "Token Recycling", section Method; softmax is
//     increasing, so ids are selected on the raw logits, ties to the lower
//     id, -0.0 equal to +0.0), published to a mailbox of self-validating
//     words (bit 31 set on a written id);
//   * one tail block per sequence: reads the template, the tree tokens and
//     the prefix length and builds the update map while the rows are
//     selected, then polls the mailbox, verifies, updates M and retrieves
//     the next draft tree; it publishes the verdict for
//   * commit blocks (when a key/value cache is given): they copy the
//     accepted path's key/value rows into the cache, in parallel with the
//     retrieval.
// Blocks are dispatched in index order on each XCD, and a block only ever
// waits for blocks of lower index, which never wait for it: every wait
// ends.  The waits are bounded all the same (TR_FLAG_HANDOVER).
//
// A row block (256 threads, one row of up to 32768 elements, every element
// read once into registers) selects in four steps:
//   1. every element becomes a flip code (an unsigned integer in the order
//      of the values: negative values bit-inverted, others with the sign bit
//      set; -0.0 sits one below +0.0) and every 16-byte vector keeps its
//      largest code;
//   2. each wave bisects over its 64 lane maxima for the k-th largest and
//      keeps its k largest lane maxima; the block's largest code gives the
//      greedy token (rank 0), published at once;
//   3. T = the k-th largest of all the waves' kept maxima (lowered by one
//      when it is +0.0's code, so that -0.0 passes with +0.0) is reached by
//      k elements, so every one of the k best reaches it: only vectors whose
//      maximum reaches T are looked into, and their elements at or above T
//      go to per-wave candidate lists in LDS;
//   4. wave 0 ranks the candidates (order codes with -0.0 == +0.0, then the
//      lower id) in registers.
// Rows full of ties overflow a list; the block then falls back to exact
// per-lane insertion of every element at or above T.
#include "select.h"
#include "tail.h"

namespace tr {

constexpr int kStepNT = 256;
constexpr int kStepVecs = 16;            // bfloat16: 16-byte vectors per lane (fp32: twice as many)
constexpr int kCommitPerBlock = kStepNT * 4;   // 16-byte units one commit block copies per pass
constexpr int kMaxCommitBlocks = 32;
constexpr int64_t kHelperBytes = 128 * 1024;   // of M one helper block reads
constexpr int kMaxHelpers = 16;

StepPlan plan_step(int32_t B, const TreeDev& tree, int64_t V, int32_t k, int32_t esz, bool sample,
                   const TailArgs& tail) {
  StepPlan p{};
  const int64_t rows = int64_t(B) * tree.T;
  (void)esz;                                           // both types hold rows of kStepMaxV
  p.use = !sample && rows < 256 && B <= kMaxStepSeq && k <= kMaxK && V <= kStepMaxV;
  p.rows = int32_t(rows);
  p.B = B;
  p.commit = 0;
  if (tail.mode == TAIL_STEP && tail.k_cache) {
    const int64_t units = int64_t(2) * (tree.D + 1) * tail.Hkv * (tail.row_bytes / 16) * tail.n_layers;
    int64_t c = (units + kCommitPerBlock - 1) / kCommitPerBlock;
    p.commit = int32_t(c < 1 ? 1 : c > kMaxCommitBlocks ? kMaxCommitBlocks : c);
  }
  // helpers: H per sequence, in groups of 8 blocks (one per XCD) placed so
  // that sequence b's helpers share its tail block's XCD
  const int64_t mbytes = V * k * (tail.m_is64 ? 8 : 4);
  int64_t h = (mbytes + kHelperBytes - 1) / kHelperBytes;
  p.helpers = tail.mode == TAIL_STEP ? int32_t(h < 1 ? 1 : h > kMaxHelpers ? kMaxHelpers : h) : 0;
  p.help_base = (p.rows + B + B * p.commit + 7) / 8 * 8;
  p.grid = p.help_base + 8 * p.helpers * ((B + 7) / 8);
  return p;
}

namespace {

// Flip codes of two bfloat16 halves (16-bit arithmetic per half) or of one
// float: unsigned order = value order, -0.0 one below +0.0.
__device__ __forceinline__ uint32_t flip16x2(uint32_t w) {
  const uint32_t s = __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, w) >> (int16_t)15);
  return w ^ (s | 0x80008000u);
}
__device__ __forceinline__ uint32_t flip32(uint32_t w) {
  return w ^ (uint32_t(int32_t(w) >> 31) | 0x80000000u);
}
// The order code (ord32 of dev_common.h, which merges -0.0 and +0.0) of a
// flip code: equal for non-negative values, one more for negative ones.
__device__ __forceinline__ uint32_t ord_of_flip16(uint32_t u) { return (u < 0x8000u ? u + 1u : u) << 16; }
__device__ __forceinline__ uint32_t ord_of_flip32(uint32_t u) { return u < 0x80000000u ? u + 1u : u; }

__device__ __forceinline__ void mail_put(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t mail_get(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void verdict_put(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t verdict_get(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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

// ---------------------------------------------------------------- rows
template <bool BF16, int KM>
__device__ __forceinline__ void step_row(const void* __restrict__ logits, int64_t V, int32_t k,
                                         int row, int32_t* __restrict__ ids_out, uint32_t* mail) {
  constexpr int NT = kStepNT, NW = NT / 64;
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int VE = 16 / ESZ;
  constexpr int NV = BF16 ? kStepVecs : 2 * kStepVecs;   // both: kStepMaxV elements
  static_assert(int64_t(NV) * NT * VE == kStepMaxV, "row length");
  constexpr uint32_t kZeroPos = BF16 ? 0x8000u : 0x80000000u;   // flip code of +0.0
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint8_t* rowp = reinterpret_cast<const uint8_t*>(logits) + int64_t(row) * V * ESZ;

  __shared__ uint64_t s_cand[NW * kCandW];
  __shared__ uint64_t s_keys[NW][KM];
  __shared__ uint64_t s_best[KM];
  __shared__ uint32_t s_top[NW * KM];
  __shared__ uint32_t s_mx[NW];
  __shared__ uint32_t s_am[NW];
  __shared__ uint32_t s_wcnt[NW];

  // aligned vectors [a0, a1); fewer than VE loose elements on either side
  const uintptr_t addr0 = reinterpret_cast<uintptr_t>(rowp);
  int64_t a0 = int64_t(((16 - (addr0 & 15)) & 15) / ESZ);
  if (a0 > V) a0 = V;
  const int nv = int((V - a0) / VE);
  const int64_t a1 = a0 + int64_t(nv) * VE;
  // loose elements first, from clamped (always valid) indices: their use
  // comes after the vectors', so no wait lands between the loads
  const int64_t hid = tid, tl = a1 + tid;
  const bool hvalid = hid < a0, tvalid = tl < V;
  uint32_t hraw, traw;
  if (BF16) {
    hraw = reinterpret_cast<const uint16_t*>(rowp)[min(hid, V - 1)];
    traw = reinterpret_cast<const uint16_t*>(rowp)[min(tl, V - 1)];
  } else {
    hraw = reinterpret_cast<const uint32_t*>(rowp)[min(hid, V - 1)];
    traw = reinterpret_cast<const uint32_t*>(rowp)[min(tl, V - 1)];
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

  // ---- 2. the wave's k-th largest lane maximum
  constexpr int kBits = BF16 ? 16 : 32;
  uint32_t lo = 0;
#pragma unroll
  for (int bit = kBits - 1; bit >= 0; --bit) {
    const uint32_t c = lo | (1u << bit);
    if (__popcll(__ballot(lm >= c)) >= k) lo = c;
  }
  // the wave's k largest lane maxima (those above lo, then copies of lo)
  {
    const uint64_t gt = __ballot(lm > lo);               // fewer than k lanes
    const int ngt = __popcll(gt);
    const uint32_t below =
        __builtin_amdgcn_mbcnt_hi(uint32_t(gt >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(gt), 0u));
    if (lm > lo) s_top[wave * KM + below] = lm;
    if (lane >= ngt && lane < k) s_top[wave * KM + lane] = lo;
  }
  const uint32_t wmx = wave_max_u32(lm);
  if (lane == 0) s_mx[wave] = wmx;
  __syncthreads();
  uint32_t* mrow = mail + int64_t(row) * k;
  int32_t* orow = ids_out + int64_t(row) * k;

  // ---- the greedy token (rank 0) goes out first: the tail verifies on it
  // while the other ranks are selected.  Ma admits the block's largest code
  // (and -0.0 with +0.0); each lane that holds such an element finds its
  // lowest id (head, then its vectors in order, then tail), the block the
  // lowest of those.
  uint32_t Mx = s_mx[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) Mx = max(Mx, s_mx[w]);
  const uint32_t Ma = Mx == kZeroPos ? kZeroPos - 1 : Mx;
  uint32_t inv = 0;                                    // ~id of the lane's first element >= Ma
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
    orow[0] = int32_t(~best);
    mail_put(mrow, ~best | 0x80000000u);
  }

  // ---- 3. T = the block's k-th largest lane maximum (the k-th largest of
  // the waves' k largest): k elements reach it, so every one of the k best
  // does.  Candidates: elements at or above T, by ballot into the lists.
  constexpr int NTOP = NW * KM;                        // 32 or 64: one per lane
  const uint32_t tv = (lane < NTOP && (lane % KM) < k) ? s_top[min(lane, NTOP - 1)] : 0u;
  uint32_t T = 0;
#pragma unroll
  for (int bit = kBits - 1; bit >= 0; --bit) {
    const uint32_t c = T | (1u << bit);
    if (__popcll(__ballot(tv >= c)) >= k) T = c;
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
  // per lane and pass, taken out of the registers by a select tree.  The
  // pass is a loop, not unrolled code: a block runs it once, from a cold
  // instruction cache, so its length is what it costs.
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
      if (lane < int(n) && rank < k && rank > 0) {         // rank 0 is out already
        const uint32_t id = key_id(key);
        orow[rank] = int32_t(id);
        mail_put(mrow + rank, id | 0x80000000u);
      }
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
  if (tid > 0 && tid < k) {
    const uint32_t id = key_id(s_best[tid]);
    orow[tid] = int32_t(id);
    mail_put(mrow + tid, id | 0x80000000u);
  }
}

// ---------------------------------------------------------------- tail
// Per-launch LDS of the tail block beyond the shared tail state: the
// update map as a direct table (token -> node whose top-k row M now holds
// for it; 0xFF none), the nodes in layer order as packed descriptors
// (node | parent << 8 | rank << 16) with each layer's first index, and a
// flag per node once its whole top-k row is in S.topk.
struct StepShared {
  alignas(16) uint8_t wtab[kStepMaxV];
  uint32_t desc[kMaxNodes];
  int32_t lst[kMaxNodes + 2];
  uint8_t pos[kMaxNodes];        // a node's index within its layer's list
  uint32_t rowok[kMaxNodes];
  int32_t narrow;                // every layer fits in one wave (and D + 2 <= 64)
};

// The direct map table from the hash map the claims built (one wave; nodes
// lane, lane+64): the winner of each token writes itself.
__device__ __forceinline__ void step_map_table(const TailShared& S, StepShared& X,
                                               const TreeDev& tree, int64_t V) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int n = lane + 64 * h;
    const int32_t t = n < tree.T ? S.tok[n] : -1;
    if (t >= 0 && int64_t(t) < V && map_get(S, t) == n) X.wtab[t] = uint8_t(n);
  }
}

// The layer lists from the template in LDS (wave 0; nodes lane, lane+64).
__device__ __forceinline__ void step_layers(const TailShared& S, StepShared& X, const TreeDev& tree) {
  const int lane = threadIdx.x & 63;
  int dep[2];
  uint32_t dsc[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int n = lane + 64 * h;
    const bool in = n < tree.T;
    dep[h] = in ? S.dep[n] : -1;
    dsc[h] = in ? uint32_t(n) | (uint32_t(S.par[n] == 0xFF ? 0 : S.par[n]) << 8) |
                      (uint32_t(S.rnk[n]) << 16) : 0u;
  }
  int at = 0, widest = 0;
  int idx[2] = {-1, -1};                               // each node's place in the lists
  for (int d = 1; d <= tree.D; ++d) {
    if (lane == 0) X.lst[d] = at;
    const int start = at;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint64_t m = __ballot(dep[h] == d);
      const int below = int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
      if (dep[h] == d) {
        idx[h] = at + below;
        X.pos[lane + 64 * h] = uint8_t(at + below - start);
      }
      at += __popcll(m);
    }
    widest = max(widest, at - start);
  }
  if (lane == 0) {
    X.lst[tree.D + 1] = at;
    X.pos[0] = 0;
    X.narrow = (widest <= 64 && tree.D + 2 <= 64) ? 1 : 0;
  }
  wave_lds_sync();
  // descriptors, with the parent's place in its layer in bits 24..31
#pragma unroll
  for (int h = 0; h < 2; ++h)
    if (idx[h] >= 0) X.desc[idx[h]] = dsc[h] | (uint32_t(X.pos[(dsc[h] >> 8) & 0xFFu]) << 24);
}

// The value of node n at layer d > 1 from its parent token p (valid or
// not), its rank, and the M entry mv loaded for it: a map hit's row (from
// LDS once its flag is set, else from the mailbox), the root's prefetched
// row at layer 1, else M.  Shared by both retrieval loops.
template <typename MT>
__device__ __forceinline__ int32_t step_value(TailShared& S, const StepShared& X, int d, int32_t p,
                                              bool pv, int rnk, MT mv, int pre_row, int32_t k,
                                              int64_t V, const uint32_t* mail, uint8_t* ws,
                                              bool& bad) {
  const uint32_t wt = X.wtab[pv ? p : 0];
  const int w = pv && wt != 0xFFu ? int(wt) : -1;
  const bool late = w >= 0 && rnk > 0 &&
                    __hip_atomic_load(&X.rowok[w], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0u;
  int32_t alt = (w >= 0 ? S.topk + w * k : S.pre + pre_row)[rnk];
  if (__ballot(late) != 0 && late) {
    // the row may have reached LDS since the first look: read it there
    // then (the value read before its flag was set is not the row's)
    if (__hip_atomic_load(&X.rowok[w], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != 0u) {
      alt = S.topk[w * k + rnk];
    } else {
      const uint32_t* word = mail + w * k + rnk;
      uint32_t v = 0;
      for (int spin = 0; spin <= kSpinLimit; ++spin) {
        v = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (v >> 31) break;
      }
      if ((v >> 31) == 0u) set_flag(ws, TR_FLAG_HANDOVER);
      alt = (v >> 31) ? int32_t(v & 0x7FFFFFFFu) : -1;
    }
  }
  const int64_t v = !pv ? -1 : (w >= 0 || d == 1) ? int64_t(alt) : int64_t(mv);
  const bool ok = v >= 0 && v < V;
  bad = bad || (p >= 0 && !pv) || (pv && !ok);
  return ok ? int32_t(v) : -1;
}

// The next draft tree when every layer fits in one wave: lane i holds the
// value of the i-th node of the current layer in a register, and a node
// takes its parent's token from the parent's lane (a cross-lane permute),
// so a layer's chain is: permute, then the M entry and the map table
// together, then the hit's value.  The tokens also go to S.nxt for the
// output, off the chain.
template <typename MT>
__device__ __forceinline__ void step_retrieve_narrow(TailShared& S, const StepShared& X,
                                                     const TreeDev& tree, int32_t root,
                                                     const void* M_b, int64_t V, int32_t k,
                                                     int32_t* out_b, uint8_t* ws,
                                                     const uint32_t* mail) {
  const int lane = threadIdx.x & 63;
  const int pre_row = S.best * k;
  const int D = tree.D;
  const int lstv = lane <= D + 1 ? X.lst[lane] : 0;     // lane d: layer d's first index
  bool bad = lane == 0 && (root < 0 || int64_t(root) >= V);
  if (lane == 0) S.nxt[0] = root;
  int32_t val = root;                                  // the previous layer's tokens, by place
  int beg = __builtin_amdgcn_readlane(lstv, 1), end = __builtin_amdgcn_readlane(lstv, 2);
  uint32_t desc = D >= 1 && lane < end - beg ? X.desc[beg + lane] : 0u;
  for (int d = 1; d <= D; ++d) {
    const bool act = lane < end - beg;
    const uint32_t dsc = desc;
    // the next layer's descriptors, off the chain
    if (d < D) {
      const int nb = __builtin_amdgcn_readlane(lstv, d + 1), ne = __builtin_amdgcn_readlane(lstv, d + 2);
      desc = lane < ne - nb ? X.desc[nb + lane] : 0u;
      beg = nb;
      end = ne;
    }
    const int n = int(dsc & 0xFFu), rnk = int((dsc >> 16) & 0xFFu), ppos = int(dsc >> 24);
    const int32_t pp = __shfl(val, ppos, 64);
    const int32_t p = act ? (d == 1 ? root : pp) : -1;
    const bool pv = p >= 0 && int64_t(p) < V;
    MT mv = MT(0);
    if (d > 1) mv = reinterpret_cast<const MT*>(M_b)[pv ? int64_t(p) * k + rnk : 0];
    const int32_t v = step_value<MT>(S, X, d, p, pv, rnk, mv, pre_row, k, V, mail, ws, bad);
    if (act) S.nxt[n] = v;
    val = v;
  }
  if (bad) set_flag(ws, TR_FLAG_BAD_TOKEN);
  wave_lds_sync();
#pragma unroll
  for (int h = 0; h < 2; ++h)
    if (lane + 64 * h < tree.T) out_b[lane + 64 * h] = S.nxt[lane + 64 * h];
}

// The next draft tree: nxt[0] = root, then layer by layer nxt[n] =
// M'[nxt[parent n]][rank n], M' = M after this step's update (Chinese
// summary, Method, draft retrieval).  Wave 0, one node of the layer per
// lane (more passes for a layer wider than 64).
//
// The layers are a chain of dependent reads, so a layer's common path is
// short: the node's descriptor (read ahead, off the chain); the parent's
// token; then, together, its M row entry (from the L2 the helper blocks
// filled) and its entry in the direct map table; then the value a map hit
// or the root's prefetched row supplies.  A map hit's row is in LDS once
// waves 1..3 have it (rowok set after the row); a hit whose row is not in
// yet reads its word from the mailbox (the slow path: one wave-uniform
// branch).  Bad tokens set the flag once, after the loop.
template <typename MT>
__device__ __forceinline__ void step_retrieve(TailShared& S, const StepShared& X,
                                              const TreeDev& tree, int32_t root, const void* M_b,
                                              int64_t V, int32_t k, int32_t* out_b, uint8_t* ws,
                                              const uint32_t* mail) {
  const int lane = threadIdx.x & 63;
  const int pre_row = S.best * k;
  if (lane == 0) S.nxt[0] = root;
  bool bad = lane == 0 && (root < 0 || int64_t(root) >= V);
  uint32_t desc = 0u;
  if (tree.D >= 1) desc = X.lst[1] + lane < X.lst[2] ? X.desc[X.lst[1] + lane] : 0u;
  wave_lds_sync();
  for (int d = 1; d <= tree.D; ++d) {
    const int beg = X.lst[d], end = X.lst[d + 1];
    for (int base = beg; base < end; base += 64) {
      const bool act = base + lane < end;
      const uint32_t dsc = base == beg ? desc : (act ? X.desc[base + lane] : 0u);
      const int n = int(dsc & 0xFFu), par = int((dsc >> 8) & 0xFFu), rnk = int((dsc >> 16) & 0xFFu);
      const int32_t p = act ? S.nxt[par] : -1;
      const bool pv = p >= 0 && int64_t(p) < V;
      MT mv = MT(0);
      if (d > 1) mv = reinterpret_cast<const MT*>(M_b)[pv ? int64_t(p) * k + rnk : 0];
      const uint32_t wt = X.wtab[pv ? p : 0];
      const int w = pv && wt != 0xFFu ? int(wt) : -1;
      const bool late = w >= 0 && rnk > 0 &&
                        __hip_atomic_load(&X.rowok[w], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0u;
      int32_t alt = (w >= 0 ? S.topk + w * k : S.pre + pre_row)[rnk];
      if (__ballot(late) != 0 && late) {
        // the row may have reached LDS since the first look: read it there
        // then (the value read before its flag was set is not the row's)
        if (__hip_atomic_load(&X.rowok[w], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != 0u) {
          alt = S.topk[w * k + rnk];
        } else {
          const uint32_t* word = mail + w * k + rnk;
          uint32_t v = 0;
          for (int spin = 0; spin <= kSpinLimit; ++spin) {
            v = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (v >> 31) break;
          }
          if ((v >> 31) == 0u) set_flag(ws, TR_FLAG_HANDOVER);
          alt = (v >> 31) ? int32_t(v & 0x7FFFFFFFu) : -1;
        }
      }
      if (act) {
        const int64_t v = !pv ? -1 : (w >= 0 || d == 1) ? int64_t(alt) : int64_t(mv);
        const bool ok = v >= 0 && v < V;
        bad = bad || (p >= 0 && !pv) || (pv && !ok);
        S.nxt[n] = ok ? int32_t(v) : -1;
      }
    }
    if (d < tree.D) {                                   // the next layer's first descriptors, off the chain
      const int nb = X.lst[d + 1], ne = X.lst[d + 2];
      desc = nb + lane < ne ? X.desc[nb + lane] : 0u;
    }
    wave_lds_sync();
  }
  if (bad) set_flag(ws, TR_FLAG_BAD_TOKEN);
#pragma unroll
  for (int h = 0; h < 2; ++h)
    if (lane + 64 * h < tree.T) out_b[lane + 64 * h] = S.nxt[lane + 64 * h];
}

// Verdict word handed to the commit blocks: bit 63 set once written, bit 62
// whether the accepted rows fit in the cache, bits 32..38 the accepted
// (deepest) node, bits 0..31 the prefix length before the commit.
__device__ __forceinline__ uint64_t verdict_word(bool fits, int best, int32_t P) {
  return (uint64_t(1) << 63) | (uint64_t(fits ? 1 : 0) << 62) | (uint64_t(best) << 32) | uint32_t(P);
}

template <typename MT, int KM>
__device__ __forceinline__ void step_tail(const TreeDev& tree, int b, int32_t k, int64_t V,
                                          uint32_t* mail, const TailArgs& tail, uint8_t* ws,
                                          uint64_t* verdict, bool commit) {
  __shared__ TailShared S;
  __shared__ StepShared X;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int T = tree.T;
  const bool step = tail.mode == TAIL_STEP;
  const bool path_only = step && tail.update_mode == UPDATE_ACCEPTED;
  void* M_b = reinterpret_cast<MT*>(tail.M) + int64_t(b) * V * k;
  int32_t* tok_b = tail.tree_tok + int64_t(b) * T;

  // ---- set-up while the rows are being selected: template, tokens,
  // prefix length, and (unless only the accepted path is recycled) the
  // update map, which depends on the tokens alone
  const int32_t tok = tok_b[min(tid, T - 1)];
  const int32_t P = (step && tail.k_cache) ? tail.prefix_len[b] : 0;
  if (wave == 0) tail_tree_wave(S, tree);
  map_clear(S);
  if (tid < T) S.tok[tid] = tok;
  if (tid < kMaxNodes) X.rowok[tid] = 0u;
  if (step) {
    for (int i = tid; i < kStepMaxV / 16; i += kStepNT)
      reinterpret_cast<u32x4*>(X.wtab)[i] = u32x4{~0u, ~0u, ~0u, ~0u};
  }
  if (tid == 0) S.P = P;
  __syncthreads();
  if (wave == 1 && !path_only) {
    tail_update_claim(S, tree, V, ws, false);
    if (step) {
      wave_lds_sync();
      step_map_table(S, X, tree, V);
    }
  }
  if (wave == 0 && step) {
    wave_lds_sync();                                   // the template tail_tree_wave wrote
    step_layers(S, X, tree);
  }

  // ---- the rows.  Whole step: thread n waits for row n's greedy token
  // g(n) (rank 0, published first), then fetches the row of M the next
  // tree's first layer takes if n is accepted, M[g(n)].  Update only:
  // thread n waits for all k ranks of row n.
  uint32_t* mseq = mail + int64_t(b) * T * k;
  bool timed_out = false;
  MT pre[KM];
  bool pre_ok = false;
  const int nw = step ? 1 : k;                         // words waited for here
  if (tid < T) {
    const uint32_t* m = mseq + tid * k;
    uint32_t v[KM];
    for (int spin = 0;; ++spin) {
      bool ok = true;
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (j < nw) {
          v[j] = mail_get(m + j);
          ok = ok && (v[j] >> 31) != 0u;
        }
      }
      if (ok) break;
      if (spin == kSpinLimit) {
        timed_out = true;
        break;
      }
    }
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j < nw) S.topk[tid * k + j] = int32_t(v[j] & 0x7FFFFFFFu);
    if (step) {
      const int32_t g = int32_t(v[0] & 0x7FFFFFFFu);
      pre_ok = int64_t(g) < V;
      const int64_t base = pre_ok ? int64_t(g) * k : 0;    // row 0 stands in: no branch
#pragma unroll
      for (int j = 0; j < KM; ++j) pre[j] = reinterpret_cast<const MT*>(M_b)[base + min(j, k - 1)];
    }
  }
  if (__syncthreads_or(timed_out)) {                   // rows (or greedy tokens) in LDS unless a wait gave up
    if (tid == 0) {
      set_flag(ws, TR_FLAG_HANDOVER);
      if (commit) verdict_put(verdict + b, verdict_word(false, 0, 0));
    }
    return;
  }
  if (!step) {                                         // update of M only
    if (wave == 0) tail_update_store<MT>(S, tree, k, M_b, V);
    for (int i = tid - 64; i >= 0 && i < T * k; i += kStepNT - 64) mail_put(mseq + i, 0u);
    return;
  }

  // ---- verification (wave 0) while the prefetched rows land
  Verdict vd{};
  if (wave == 0) {
    vd = tail_verify_wave(S, tree, k);
    if (path_only) {
      wave_lds_sync();
      tail_update_claim(S, tree, V, ws, true);
      wave_lds_sync();
      step_map_table(S, X, tree, V);
    }
  }
  if (tid < T) {
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const int64_t x = int64_t(pre[j]);
      if (j < k) S.pre[tid * k + j] = !pre_ok ? -1 : (x >= 0 && x < V) ? int32_t(x) : -2;
    }
  }
  __syncthreads();                                     // verdict, update map, prefetched rows

  if (wave == 0) {
    // the next tree (loads only); a map hit's ranks come from the mailbox
    const bool fits = tail_commit_fits(S, tail, vd.L);
    if (X.narrow)
      step_retrieve_narrow<MT>(S, X, tree, vd.bonus, M_b, V, k, tok_b, ws, mseq);
    else
      step_retrieve<MT>(S, X, tree, vd.bonus, M_b, V, k, tok_b, ws, mseq);
    if (tid == 0) {
      tail.root_tok[b] = vd.bonus;
      if (fits) tail.prefix_len[b] = int32_t(S.P + vd.L + 1);
    }
  } else {
    if (tid == 64 && tail.k_cache) {
      const bool fits = tail_commit_fits(S, tail, S.L);
      if (commit) verdict_put(verdict + b, verdict_word(fits, S.best, S.P));
      if (!fits) set_flag(ws, TR_FLAG_CACHE_FULL);
    }
    tail_write_verdict(S, tree, b, tail.accept_len, tail.accept_path, nullptr, tail.emitted, 64);
    // thread 64 + n: the rest of row n, then M[tok n] = row n if n wins its token
    const int n = tid - 64;
    if (n < T) {
      const uint32_t* m = mseq + n * k;
      uint32_t v[KM];
      bool ok = true;
      for (int spin = 0;; ++spin) {
        ok = true;
#pragma unroll
        for (int j = 1; j < KM; ++j) {
          if (j < k) {
            v[j] = mail_get(m + j);
            ok = ok && (v[j] >> 31) != 0u;
          }
        }
        if (ok || spin == kSpinLimit) break;
      }
      if (!ok) set_flag(ws, TR_FLAG_HANDOVER);
      if (ok) {                                        // the row for the retrieval, then its flag
#pragma unroll
        for (int j = 1; j < KM; ++j)
          if (j < k) S.topk[n * k + j] = int32_t(v[j] & 0x7FFFFFFFu);
        __hip_atomic_store(&X.rowok[n], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      const int32_t t = S.tok[n];
      if (ok && t >= 0 && int64_t(t) < V && map_get(S, t) == n) {
        m_store<MT>(M_b, int64_t(t) * k, S.topk[n * k]);
#pragma unroll
        for (int j = 1; j < KM; ++j)
          if (j < k) m_store<MT>(M_b, int64_t(t) * k + j, int32_t(v[j] & 0x7FFFFFFFu));
      }
    }
  }
  __syncthreads();                                     // the retrieval's last mailbox read is done
  for (int i = tid; i < T * k; i += kStepNT) mail_put(mseq + i, 0u);   // ready for the next call
}

// ---------------------------------------------------------------- commit
// Commit block c of C for sequence b: waits for the tail's verdict, copies
// its share of the accepted rows; the last of the C blocks clears the
// verdict for the next call.
__device__ __forceinline__ void step_commit(const TreeDev& tree, int b, int c, int C,
                                            const TailArgs& a, uint8_t* ws, uint64_t* verdict,
                                            uint32_t* done) {
  __shared__ int32_t s_path[kMaxNodes];
  __shared__ uint64_t s_hdr;
  const int tid = threadIdx.x;
  if (tid == 0) {
    uint64_t h = 0;
    for (int spin = 0;; ++spin) {
      h = verdict_get(verdict + b);
      if (h >> 63) break;
      if (spin == kSpinLimit) {
        set_flag(ws, TR_FLAG_HANDOVER);
        h = 0;
        break;
      }
    }
    s_hdr = h;
  }
  __syncthreads();
  const uint64_t h = s_hdr;
  if ((h >> 62) & 1u) {                                // the rows fit
    const int best = int((h >> 32) & 0x7Fu);
    const int64_t P = int64_t(uint32_t(h));
    const uint64_t a0 = tree.anc[best][0], a1 = tree.anc[best][1];
    for (int t = tid; t < tree.T; t += kStepNT)
      if (((t < 64 ? a0 >> t : a1 >> (t - 64)) & 1u) != 0u) s_path[tree.depth[t]] = t;
    __syncthreads();
    commit_rows(s_path, int(tree.depth[best]), P, tree, b, a, ws, c * kStepNT + tid, C * kStepNT);
  }
  if (h >> 63) {
    if (last_block_arrives(done + b, uint32_t(C)) && tid == 0) verdict_put(verdict + b, 0);
  }
}

// ---------------------------------------------------------------- helpers
// Helper h of H for sequence b reads its share of M_b with ordinary loads,
// which leaves it in the L2 of the XCD the helper runs on -- the tail
// block's -- before the retrieval's chain of dependent row reads starts.
// Only the 16-byte aligned interior of M_b is read; the data is dropped.
template <typename MT>
__device__ __forceinline__ void step_helper(int b, int h, int H, int64_t V, int32_t k,
                                            const TailArgs& tail) {
  constexpr int U = 16;                                // loads in flight per thread
  const uintptr_t beg = reinterpret_cast<uintptr_t>(reinterpret_cast<const MT*>(tail.M) +
                                                    int64_t(b) * V * k);
  const uintptr_t lo = (beg + 15) & ~uintptr_t(15);
  const uintptr_t hi = (beg + uintptr_t(V * k) * sizeof(MT)) & ~uintptr_t(15);
  if (hi <= lo) return;
  const int64_t n16 = int64_t(hi - lo) / 16;
  const int64_t per = (n16 + H - 1) / H;
  const int64_t i0 = int64_t(h) * per, i1 = min(n16, i0 + per);
  const u32x4* p = reinterpret_cast<const u32x4*>(lo);
  uint32_t acc = 0;
  for (int64_t i = i0 + threadIdx.x; i < i1; i += int64_t(kStepNT) * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t idx = i + int64_t(u) * kStepNT;
      v[u] = idx < i1 ? p[idx] : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  asm volatile("" ::"v"(acc));                         // the loads must complete
}

}  // namespace

template <bool BF16, int KM, typename MT>
__global__ __launch_bounds__(kStepNT) void step_kernel(const void* __restrict__ logits, int64_t V,
                                                       int32_t k, int32_t* ids_out, uint8_t* ws,
                                                       TreeDev tree, TailArgs tail, int32_t rows,
                                                       int32_t B, int32_t C, int32_t help_base,
                                                       int32_t H) {
  uint32_t* mail = reinterpret_cast<uint32_t*>(ws + kMailOff);
  uint64_t* verdict = reinterpret_cast<uint64_t*>(ws + kVerdictOff);
  int bid = int(blockIdx.x);
  if (bid < rows) {
    step_row<BF16, KM>(logits, V, k, bid, ids_out, mail);
    return;
  }
  bid -= rows;
  if (bid < B) {
    step_tail<MT, KM>(tree, bid, k, V, mail, tail, ws, verdict, C > 0);
    return;
  }
  bid -= B;
  if (bid < B * C) {
    step_commit(tree, bid / C, bid % C, C, tail, ws, verdict,
                reinterpret_cast<uint32_t*>(ws + kCommitCntOff));
    return;
  }
  // helper region: block help_base + 8 * g + x runs on XCD x; group g is
  // helper g % H of the sequences of round g / H, and slot x serves the
  // sequence whose tail block (index rows + b) is on XCD x
  const int j = int(blockIdx.x) - help_base;
  if (j < 0 || H == 0) return;                          // padding up to the region
  const int g = j / 8, x = j % 8;
  const int b = (g / H) * 8 + ((x - rows % 8) + 8) % 8;
  if (b < B) step_helper<MT>(b, g % H, H, V, k, tail);
}

hipError_t launch_step(const TreeDev& tree, const void* logits, int l_is_bf16, int64_t V,
                       int32_t k, int32_t* topk_ids, const TailArgs& tail, uint8_t* ws,
                       const StepPlan& plan, hipStream_t s) {
#define TR_STEP(BF, KMV, MTV)                                                                    \
  hipLaunchKernelGGL((step_kernel<BF, KMV, MTV>), dim3(unsigned(plan.grid)), dim3(kStepNT), 0, s, \
                     logits, V, k, topk_ids, ws, tree, tail, plan.rows, plan.B, plan.commit,     \
                     plan.help_base, plan.helpers)
#define TR_STEP_M(BF, KMV)                            \
  do {                                                \
    if (tail.m_is64) TR_STEP(BF, KMV, int64_t);       \
    else TR_STEP(BF, KMV, int32_t);                   \
  } while (0)
  prof_begin(s, TR_KERNEL_TOPK);
  if (l_is_bf16) {
    if (k <= 8) TR_STEP_M(true, 8); else TR_STEP_M(true, 16);
  } else {
    if (k <= 8) TR_STEP_M(false, 8); else TR_STEP_M(false, 16);
  }
  prof_end(s);
#undef TR_STEP_M
#undef TR_STEP
  return hipGetLastError();
}

}  // namespace tr
