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
// read once into registers) selects with select_block (select.h), which
// reports the greedy token (rank 0) as soon as the block's largest element
// is known, before the other ranks.
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

// ---------------------------------------------------------------- rows
// A row block: the row's top-k (select_block), its greedy token published
// first, the other ranks after; each written to the output and to the
// mailbox word the tail block polls.
struct StepRowOut {
  int32_t* orow;
  uint32_t* mrow;
  int32_t k;
  __device__ __forceinline__ void first(uint32_t id) const {
    orow[0] = int32_t(id);
    mail_put(mrow, id | 0x80000000u);
  }
  __device__ __forceinline__ void put(int r, uint64_t key) const {
    if (r < 1 || r >= k) return;
    const uint32_t id = key_id(key);
    orow[r] = int32_t(id);
    mail_put(mrow + r, id | 0x80000000u);
  }
};

template <bool BF16, int KM>
__device__ __forceinline__ void step_row(const void* __restrict__ logits, int64_t V, int32_t k,
                                         int row, int32_t* __restrict__ ids_out, uint32_t* mail) {
  constexpr int NV = BF16 ? kStepVecs : 2 * kStepVecs;   // both: kStepMaxV elements
  static_assert(int64_t(NV) * kStepNT * (BF16 ? 8 : 4) == kStepMaxV, "row length");
  const uint8_t* rowp = reinterpret_cast<const uint8_t*>(logits) + int64_t(row) * V * (BF16 ? 2 : 4);
  StepRowOut out{ids_out + int64_t(row) * k, mail + int64_t(row) * k, k};
  select_block<BF16, KM, kStepNT, NV, true>(rowp, 0, V, k, out);
}

// A row block of the LM head's step: the row's candidates are the 8 best
// keys of every 128-id vocabulary slice, descending per slice
// (lmhead_topk_kernel), and thread t holds slice t's list (V <= 32768: at
// most 256 slices).  Each wave takes its lists' 8 best in 8 rounds (the
// largest head, popped from its list); wave 0 merges the four waves' lists
// the same way and publishes rank 0 (the greedy token) at its first round.
template <int KM>
__device__ __forceinline__ void step_row_cand(const uint64_t* __restrict__ part, int64_t V,
                                              int32_t k, int row, int32_t* __restrict__ ids_out,
                                              uint32_t* mail) {
  constexpr int NW = kStepNT / 64, NL = 8;             // lists of 8 keys per slice
  static_assert(KM <= NL, "ranks within one slice list");
  __shared__ uint64_t s_lists[NW][NL];
  const int nvs = int((V + 127) / 128);
  StepRowOut out{ids_out + int64_t(row) * k, mail + int64_t(row) * k, k};
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t v[NL];
  if (tid < nvs) {
    const u64x2* p = reinterpret_cast<const u64x2*>(part + (int64_t(row) * nvs + tid) * NL);
#pragma unroll
    for (int q = 0; q < NL / 2; ++q) {
      const u64x2 x = p[q];
      v[2 * q] = x[0];
      v[2 * q + 1] = x[1];
    }
  } else {
#pragma unroll
    for (int i = 0; i < NL; ++i) v[i] = 0;
  }
  auto pop = [&](uint64_t (&l)[NL]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NL - 1; ++i) l[i] = l[i + 1];
    l[NL - 1] = 0;
  };
  uint64_t best[NL];
#pragma unroll
  for (int r = 0; r < NL; ++r) {
    const uint64_t m = wave_max_key(v[0]);
    best[r] = m;
    if (m != 0 && v[0] == m) pop(v);                   // keys are distinct: one lane pops
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < NL; ++r) s_lists[wave][r] = best[r];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int r = 0; r < NL; ++r) v[r] = lane < NW ? s_lists[lane][r] : 0;
#pragma unroll
    for (int r = 0; r < KM; ++r) {
      const uint64_t m = wave_max_key(v[0]);
      if (lane == 0) {
        if (r == 0) out.first(key_id(m));
        else out.put(r, m);
      }
      if (m != 0 && v[0] == m) pop(v);
    }
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
    if (tid == 0 && tail.k_cache) {                    // the verdict, before the prefetched rows land
      const bool fits = tail_commit_fits(S, tail, vd.L);
      if (commit) verdict_put(verdict + b, verdict_word(fits, vd.best, S.P));
      if (!fits) set_flag(ws, TR_FLAG_CACHE_FULL);
    }
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
// its share of the accepted rows; the last of the C blocks to read the
// verdict clears it for the next call (before the copies, so nothing waits
// for the copies' stores before the kernel ends).
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
    // counted in once the verdict is read: the last of the C blocks clears
    // it for the next call while the rows are still being copied
    if (h >> 63) {
      const uint32_t prev = __hip_atomic_fetch_add(done + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (prev == uint32_t(C - 1)) {
        __hip_atomic_store(done + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        verdict_put(verdict + b, 0);
      }
    }
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

// CAND: the rows are the LM head's slice lists (step_row_cand), not logits.
template <bool BF16, int KM, typename MT, bool CAND>
__global__ __launch_bounds__(kStepNT) void step_kernel(const void* __restrict__ logits, int64_t V,
                                                       int32_t k, int32_t* ids_out, uint8_t* ws,
                                                       TreeDev tree, TailArgs tail, int32_t rows,
                                                       int32_t B, int32_t C, int32_t help_base,
                                                       int32_t H) {
  uint32_t* mail = reinterpret_cast<uint32_t*>(ws + kMailOff);
  uint64_t* verdict = reinterpret_cast<uint64_t*>(ws + kVerdictOff);
  int bid = int(blockIdx.x);
  if (bid < rows) {
    if constexpr (CAND)
      step_row_cand<KM>(static_cast<const uint64_t*>(logits), V, k, bid, ids_out, mail);
    else
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
  hipLaunchKernelGGL((step_kernel<BF, KMV, MTV, false>), dim3(unsigned(plan.grid)), dim3(kStepNT), \
                     0, s, logits, V, k, topk_ids, ws, tree, tail, plan.rows, plan.B, plan.commit, \
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

hipError_t launch_step_lmhead(const TreeDev& tree, const uint64_t* part, int64_t V, int32_t k,
                              int32_t* topk_ids, const TailArgs& tail, uint8_t* ws,
                              const StepPlan& plan, hipStream_t s) {
  prof_begin(s, TR_KERNEL_LMHEAD_MERGE);
  if (tail.m_is64)
    hipLaunchKernelGGL((step_kernel<true, 8, int64_t, true>), dim3(unsigned(plan.grid)),
                       dim3(kStepNT), 0, s, part, V, k, topk_ids, ws, tree, tail, plan.rows,
                       plan.B, plan.commit, plan.help_base, plan.helpers);
  else
    hipLaunchKernelGGL((step_kernel<true, 8, int32_t, true>), dim3(unsigned(plan.grid)),
                       dim3(kStepNT), 0, s, part, V, k, topk_ids, ws, tree, tail, plan.rows,
                       plan.B, plan.commit, plan.help_base, plan.helpers);
  prof_end(s);
  return hipGetLastError();
}

}  // namespace tr
