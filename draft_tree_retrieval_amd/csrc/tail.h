// Per-sequence integer work of a TR step, run by one workgroup of at least
// 256 threads: verification, the recycling update of M, the commit of the
// accepted path's key/value rows and the retrieval of the next draft tree.
//
// The work is a chain of dependent steps, each waiting on memory, so the
// code keeps independent memory traffic off that chain: the M rows the next
// tree's first layer may need are fetched while verification runs, and
// after verification wave 0 alone does the tree work (update, retrieval;
// two nodes per lane, at most 128 nodes, synchronised through LDS inside
// the wave) while the other waves write every output and copy the accepted
// rows into the cache.  A wave's memory counter covers its stores as well
// as its loads, and a store completes far later than a load returns, so
// wave 0 stores nothing until the retrieval is done.
#pragma once

#include "dev_common.h"

namespace tr {

// LDS writes of a wave are visible to its later LDS reads (the LDS unit
// runs one wave's operations in order); this keeps the compiler from moving
// LDS accesses across the point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int kMapSlots = 512;          // LDS map: 128 groups of 4 slots
constexpr int kSpinLimit = 1 << 22;     // polls before a hand-over wait gives up (seconds)

struct TailShared {
  uint64_t anc[kMaxNodes][2];           // bit m of anc[n]: m lies on the path root..n (n included)
  uint8_t par[kMaxNodes];               // the template (LDS copy: indexed reads of the
  uint8_t dep[kMaxNodes];               // kernel argument would each be a memory
  uint8_t rnk[kMaxNodes];               // round trip)
  int32_t tok[kMaxNodes];               // this step's tree tokens
  int32_t topk[kMaxNodes * kMaxK];      // this step's top-k rows, [T][k]
  int32_t pre[kMaxNodes * kMaxK];       // M row of each node's greedy token, as before the update
  int32_t nxt[kMaxNodes];               // next tree tokens
  int32_t path[kMaxNodes];              // accepted path, root first
  alignas(16) int32_t hkey[kMapSlots];  // token -> node whose row M now holds
  alignas(16) int32_t hval[kMapSlots];
  uint32_t red[16];
  int32_t best, L, bonus, P;
};

// M holds int32 or int64 ids (MT); the element type is a template
// parameter so that no load sits behind a branch on it (the compiler waits
// for a load before such a branch joins).
template <typename MT>
__device__ __forceinline__ int64_t m_load(const void* M, int64_t idx) {
  return int64_t(reinterpret_cast<const MT*>(M)[idx]);
}
template <typename MT>
__device__ __forceinline__ void m_store(void* M, int64_t idx, int32_t v) {
  reinterpret_cast<MT*>(M)[idx] = MT(v);
}

// Small open-addressing map in LDS from a token to the highest tree node
// carrying it (the node whose top-k row M holds for that token after this
// step's update): at most 128 keys in 512 slots, linear probing that starts
// at the first slot of the token's aligned group of four, so a lookup reads
// a whole group (keys, then values) in one 16-byte LDS access each and
// rarely needs the next group.
__device__ __forceinline__ uint32_t tok_group(int32_t t) {
  return (uint32_t(t) * 2654435761u) >> 25;           // 128 groups
}
__device__ __forceinline__ void map_clear(TailShared& S) {
  for (int i = threadIdx.x; i < kMapSlots; i += blockDim.x) {
    S.hkey[i] = -1;
    S.hval[i] = -1;
  }
}
// Slot of token t, claimed if t is not in the map yet.
__device__ __forceinline__ uint32_t map_claim(TailShared& S, int32_t t) {
  uint32_t slot = tok_group(t) * 4;
  while (true) {
    const int32_t prev = atomicCAS(&S.hkey[slot], -1, t);
    if (prev == -1 || prev == t) return slot;
    slot = (slot + 1) & uint32_t(kMapSlots - 1);
  }
}
// Lookup within one group: the value of t, -1 when an empty slot ends the
// probe first, -2 when all four slots hold other keys (go on to the next).
__device__ __forceinline__ int32_t group_find(const i32x4& keys, const i32x4& vals, int32_t t) {
  int32_t w = -2;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int32_t hit = keys[j] == t ? vals[j] : keys[j] == -1 ? -1 : -2;
    w = w == -2 ? hit : w;
  }
  return w;
}
__device__ __forceinline__ int32_t map_get_from(const TailShared& S, int32_t t, uint32_t g) {
  while (true) {
    const i32x4 keys = reinterpret_cast<const i32x4*>(S.hkey)[g];
    const i32x4 vals = reinterpret_cast<const i32x4*>(S.hval)[g];
    const int32_t w = group_find(keys, vals, t);
    if (w != -2) return w;
    g = (g + 1) & uint32_t(kMapSlots / 4 - 1);
  }
}
__device__ __forceinline__ int32_t map_get(const TailShared& S, int32_t t) {
  return map_get_from(S, t, tok_group(t));
}

// The template into LDS; the caller synchronises before use.
__device__ __forceinline__ void tail_tree(TailShared& S, const TreeDev& tree) {
  for (int n = threadIdx.x; n < tree.T; n += blockDim.x) {
    S.par[n] = tree.parent[n];
    S.dep[n] = tree.depth[n];
    S.rnk[n] = tree.rank[n];
  }
}

// The template and every node's ancestor set into LDS, by one wave (nodes
// lane and lane + 64).  Indexed reads of the kernel argument are memory
// round trips: they leave together with the caller's other loads.
__device__ __forceinline__ void tail_tree_wave(TailShared& S, const TreeDev& tree) {
  const int lane = threadIdx.x & 63;
  uint8_t par[2], dep[2], rnk[2];
  uint64_t a0[2], a1[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {               // every index < kMaxNodes: no branch
    const int n = lane + 64 * h;
    par[h] = tree.parent[n];
    dep[h] = tree.depth[n];
    rnk[h] = tree.rank[n];
    a0[h] = tree.anc[n][0];
    a1[h] = tree.anc[n][1];
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int n = lane + 64 * h;
    if (n >= tree.T) continue;
    S.par[n] = par[h];
    S.dep[n] = dep[h];
    S.rnk[n] = rnk[h];
    S.anc[n][0] = a0[h];
    S.anc[n][1] = a1[h];
  }
}

// tok <- tree_tok_b, the template with its ancestor sets, the sequence's
// top-k rows and (when given) its prefix length into LDS.  The rows were
// handed over by other blocks of the same launch: read them with get_dev,
// all in flight at once, while wave 0 builds the template.
// NT = blockDim.x >= 256 (T * k <= 2048 ids, at most 8 per thread).
template <int NT>
__device__ __forceinline__ void tail_load(TailShared& S, const TreeDev& tree, const int32_t* tok_b,
                                          const int32_t* topk_b, int32_t k,
                                          const int32_t* prefix_len_b = nullptr) {
  static_assert(NT >= 256 && kMaxNodes * kMaxK % NT == 0, "tail_load: 256, 512 or 1024 threads");
  constexpr int kPer = kMaxNodes * kMaxK / NT;
  const int nk = tree.T * k;
  const int n = threadIdx.x;
  int32_t v[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r)                 // clamped: every load in bounds, none branched
    v[r] = get_dev(topk_b + min(n + r * NT, nk - 1));
  const int32_t t = tok_b[min(n, tree.T - 1)];
  const int32_t P = prefix_len_b ? *prefix_len_b : 0;
  if ((threadIdx.x >> 6) == 0) tail_tree_wave(S, tree);
  map_clear(S);
#pragma unroll
  for (int r = 0; r < kPer; ++r)
    if (n + r * NT < nk) S.topk[n + r * NT] = v[r];
  if (n < tree.T) S.tok[n] = t;
  if (n == 0) S.P = P;
  __syncthreads();
}

// S.pre[n] = M[g(n)] as before the update (g = the node's greedy token),
// for node n by the calling thread: the next tree's root is g(best) for
// the accepted node best, so its first layer is one of these rows.  Run by
// waves that are idle during verification, so the loads overlap it and
// the rows are in LDS at the barrier that publishes the verdict.
// Out-of-range ids become -2 (flagged where used), rows of invalid tokens -1.
// KM >= k bounds the row length (8 or 16).
template <typename MT, int KM>
__device__ __forceinline__ void tail_prefetch(TailShared& S, const TreeDev& tree, int32_t k,
                                              const void* M_b, int64_t V, int n) {
  if (n >= tree.T) return;
  const int32_t g = S.topk[n * k];
  const bool ok = g >= 0 && int64_t(g) < V;
  const int64_t base = ok ? int64_t(g) * k : 0;          // row 0 stands in: no branch
  MT v[KM];
  if (KM == 8 && sizeof(MT) == 4 && k == 8) {            // two aligned 16-byte loads
    const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const MT*>(M_b) + base);
    const u32x4 x = p[0], y = p[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = MT(x[j]);
      v[4 + j] = MT(y[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < KM; ++j) v[j] = reinterpret_cast<const MT*>(M_b)[base + min(j, k - 1)];
  }
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const int64_t x = int64_t(v[j]);
    if (j < k) S.pre[n * k + j] = !ok ? -1 : (x >= 0 && x < V) ? int32_t(x) : -2;
  }
}

// Greedy verification: node n is accepted when every node m on its path
// below the root carries the greedy token of its parent, tok(m) == g(par m);
// best = deepest accepted node, ties to the lowest index; path root..best.
// Run by one wave (nodes lane and lane + 64) without a block barrier: the
// per-node matches form a 128-bit ballot mask, a node is accepted when its
// ancestor set lies inside that mask, and the path is best's ancestor set,
// each member writing itself at its depth.  S.best, S.L, S.bonus and S.path
// become visible to the other waves at the caller's next barrier; the
// values are returned for the calling wave.
struct Verdict {
  int best, L, bonus;
};
__device__ __forceinline__ Verdict tail_verify_wave(TailShared& S, const TreeDev& tree, int32_t k) {
  const int lane = threadIdx.x & 63;
  int dep[2];
  bool match[2];
  uint64_t a[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int n = lane + 64 * h;
    const bool in = n < tree.T;
    const int p = in ? S.par[n] : 0;
    dep[h] = in ? S.dep[n] : 0;
    a[h][0] = in ? S.anc[n][0] : 0;
    a[h][1] = in ? S.anc[n][1] : 0;
    const int32_t t = in ? S.tok[n] : 0;
    const int32_t g = (in && n != 0) ? S.topk[p * k] : 0;
    match[h] = in && (n == 0 || t == g);
  }
  const uint64_t m0 = __ballot(match[0]), m1 = __ballot(match[1]);
  uint32_t key = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int n = lane + 64 * h;
    const bool ok = n < tree.T && ((a[h][0] & ~m0) | (a[h][1] & ~m1)) == 0;
    if (ok) key = max(key, (uint32_t(dep[h]) << 8) | uint32_t(255 - n));
  }
  key = wave_max_u32(key);
  Verdict v;
  v.best = 255 - int(key & 255u);
  v.L = int(key >> 8);
  const uint64_t on0 = S.anc[v.best][0], on1 = S.anc[v.best][1];
  v.bonus = S.topk[v.best * k];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int n = lane + 64 * h;
    if (n < tree.T && (((h ? on1 : on0) >> lane) & 1u)) S.path[dep[h]] = n;
  }
  if (lane == 0) {
    S.best = v.best;
    S.L = v.L;
    S.bonus = v.bonus;
  }
  return v;
}
// The same for a whole block: wave 0 decides, then every thread sees it.
__device__ __forceinline__ void tail_verify(TailShared& S, const TreeDev& tree, int32_t k) {
  if ((threadIdx.x >> 6) == 0) tail_verify_wave(S, tree, k);
  __syncthreads();
}

// Verification outputs of sequence b, written by the threads [first,
// blockDim.x).
__device__ __forceinline__ void tail_write_verdict(const TailShared& S, const TreeDev& tree, int b,
                                                   int32_t* accept_len, int32_t* accept_path,
                                                   int32_t* bonus, int32_t* emitted, int first = 0) {
  const int W = tree.D + 1;
  const int me = int(threadIdx.x) - first, count = int(blockDim.x) - first;
  if (me < 0) return;
  for (int i = me; i < W; i += count) {
    if (accept_path) accept_path[int64_t(b) * W + i] = (i <= S.L) ? S.path[i] : -1;
    if (emitted)
      emitted[int64_t(b) * W + i] = (i < S.L) ? S.tok[S.path[i + 1]] : (i == S.L ? S.bonus : -1);
  }
  if (me == 0) {
    if (accept_len) accept_len[b] = S.L;
    if (bonus) bonus[b] = S.bonus;
  }
}

// M[tok n] = topk[n], where among nodes carrying the same token the one
// with the highest index wins: every node enters its token into the LDS
// map with an atomic maximum of its index (tail_update_claim), and after
// the map is complete the winners write their rows (tail_update_store).
// Invalid tokens raise the flag and write nothing.  Each part is run by one
// wave (nodes lane and lane + 64).  With path_only (the ablation that
// recycles the accepted tokens only) just the nodes of the accepted path
// enter the map; a node is on it when the path holds it at its depth.  A
// child's index exceeds its parent's, so the highest index is the deepest.
__device__ __forceinline__ void tail_update_claim(TailShared& S, const TreeDev& tree, int64_t V,
                                                  uint8_t* ws, bool path_only = false) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int n = lane + 64 * h;
    const int32_t t = n < tree.T ? S.tok[n] : -1;
    if (n >= tree.T) continue;
    if (t < 0 || int64_t(t) >= V) {
      set_flag(ws, TR_FLAG_BAD_TOKEN);
      continue;
    }
    if (path_only) {
      const int dn = S.dep[n];
      if (dn > S.L || S.path[dn] != n) continue;
    }
    atomicMax(&S.hval[map_claim(S, t)], n);
  }
}
template <typename MT>
__device__ __forceinline__ void tail_update_store(const TailShared& S, const TreeDev& tree,
                                                  int32_t k, void* M_b, int64_t V) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int n = lane + 64 * h;
    const int32_t t = n < tree.T ? S.tok[n] : -1;
    if (t < 0 || int64_t(t) >= V || map_get(S, t) != n) continue;
    for (int j = 0; j < k; ++j) m_store<MT>(M_b, int64_t(t) * k + j, S.topk[n * k + j]);
  }
}

// Whether the accepted rows fit in the cache: the prefix length advances
// (and the rows are copied) only then.
__device__ __forceinline__ bool tail_commit_fits(const TailShared& S, const TailArgs& a, int L) {
  return a.k_cache && S.P >= 0 && int64_t(S.P) + L + 1 <= a.cap;
}

// Copy of the key/value rows of path[0..L] (LDS) to cache positions
// P..P+L: 16-byte units me, me + count, ... of the copy, R units per thread
// in flight.  The caller has checked that the rows fit.  A paged cache
// copies every layer's rows, each position into row p % page_size of page
// table[b][p / page_size] of that layer's pool.
__device__ __forceinline__ void commit_rows(const int32_t* path, int L, int64_t P,
                                            const TreeDev& tree, int b, const TailArgs& a,
                                            uint8_t* ws, int me, int count) {
  const int nrows = L + 1;
  const bool paged = a.paged.table != nullptr;
  const int upr = a.row_bytes >> 4;               // 16-byte units per row
  const int per_node = a.Hkv * upr;
  const int per_layer = 2 * nrows * per_node;      // keys then values
  const int total = per_layer * a.n_layers;
  constexpr int R = 4;
  for (int u0 = me; u0 < total; u0 += R * count) {
    u32x4 buf[R];
    int64_t dst_off[R];
    bool dst_v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int u = min(u0 + r * count, total - 1);   // clamped: loads stay in bounds
      const int layer = u / per_layer;
      const int ul = u - layer * per_layer;
      const bool isv = ul >= per_layer / 2;
      const int uu = isv ? ul - per_layer / 2 : ul;
      const int i = uu / per_node, rem = uu - i * per_node;
      const int h = rem / upr, c = rem - h * upr;
      const int node = path[i];
      const uint8_t* src = (isv ? a.v_tree : a.k_tree) + layer * a.tree_layer_bytes +
                           ((int64_t(b) * tree.T + node) * a.Hkv + h) * a.row_bytes + c * 16;
      if (paged) {
        const int64_t pos = P + i;
        int64_t pg = a.paged.table[int64_t(b) * a.paged.max_pages + (pos >> a.paged.ps_log2)];
        if (pg < 0 || pg >= a.paged.num_pages) {       // stays inside the pool
          set_flag(ws, TR_FLAG_BAD_PAGE);
          pg = 0;
        }
        dst_off[r] = layer * a.cache_layer_bytes +
                     ((pg * a.Hkv + h) * a.paged.page_size + (pos & (a.paged.page_size - 1))) *
                         a.row_bytes + c * 16;
      } else {
        dst_off[r] = ((int64_t(b) * a.Hkv + h) * a.cap + P + i) * a.row_bytes + c * 16;
      }
      dst_v[r] = isv;
      buf[r] = *reinterpret_cast<const u32x4*>(src);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (u0 + r * count >= total) break;
      uint8_t* dst = (dst_v[r] ? a.v_cache : a.k_cache) + dst_off[r];
      *reinterpret_cast<u32x4*>(dst) = buf[r];
    }
  }
}

// The commit of sequence b by the threads [first, blockDim.x); thread first
// raises the flag when the rows do not fit (tail_commit_fits).  S.L
// (verification) and S.P (tail_load) must be visible.
__device__ __forceinline__ void tail_commit(const TailShared& S, const TreeDev& tree, int b,
                                            const TailArgs& a, uint8_t* ws, int first) {
  const int me = int(threadIdx.x) - first, count = int(blockDim.x) - first;
  if (!a.k_cache || me < 0) return;
  const int64_t P = S.P;
  if (P < 0 || P + S.L + 1 > a.cap) {
    if (me == 0) set_flag(ws, TR_FLAG_CACHE_FULL);
    return;
  }
  commit_rows(S.path, S.L, P, tree, b, a, ws, me, count);
}

// Draft tree retrieval: nxt[0] = root; layer by layer
// nxt[n] = M[nxt[parent n]][rank n].  Run by one wave (nodes lane and
// lane + 64).  With use_map, rows written by this block's update come from
// LDS (every other row of M is unchanged by it); with use_pre, the first
// layer's row M[root] comes from S.pre[S.best] (root = g(best)).  Invalid
// tokens propagate as -1.  S holds the template (tail_tree).
//
// The layers form a chain of dependent reads, so each layer keeps its
// chain short: the nodes' template data sit in registers, both nodes of a
// lane are resolved side by side, and each layer's M load leaves before
// the map probe that may make it unnecessary.
//
// With mail (the few-row step kernel), S.topk holds only each node's
// greedy token (rank 0) when the retrieval starts: a map hit's other ranks
// are read from the mailbox word its row block publishes (bit 31 set once
// written), waiting for it if need be (bounded: TR_FLAG_HANDOVER).
template <typename MT>
__device__ __forceinline__ void tail_retrieve(TailShared& S, const TreeDev& tree, int32_t root,
                                              const void* M_b, int64_t V, int32_t k,
                                              int32_t* out_b, uint8_t* ws, bool use_map,
                                              bool use_pre = false,
                                              const uint32_t* mail = nullptr) {
  const int lane = threadIdx.x & 63;
  int n[2], dep[2], par[2], rnk[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    n[h] = lane + 64 * h;
    const bool in = n[h] < tree.T;
    dep[h] = in ? S.dep[n[h]] : 0;               // 0: the root or no node
    par[h] = in ? S.par[n[h]] : 0;
    rnk[h] = in ? S.rnk[n[h]] : 0;
  }
  const int pre_row = use_pre ? S.best * k : 0;
  if (lane == 0) S.nxt[0] = root;
  wave_lds_sync();
  for (int d = 1; d <= tree.D; ++d) {
    // Three LDS round trips per layer: the parent tokens; the map group of
    // each (keys and values together) while M is read; the value a map hit
    // or the prefetched first layer supplies.  The M load leaves before the
    // probe and is waited for last (a map hit discards it); row 0 stands in
    // for lanes without a valid parent token.
    int32_t p[2], w[2], alt[2];
    bool pv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      p[h] = dep[h] == d ? S.nxt[par[h]] : -1;
      pv[h] = p[h] >= 0 && int64_t(p[h]) < V;
    }
    const bool first_pre = use_pre && d == 1;
    MT mv[2] = {MT(0), MT(0)};
    if (!first_pre) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        mv[h] = reinterpret_cast<const MT*>(M_b)[pv[h] ? int64_t(p[h]) * k + rnk[h] : 0];
    }
    // the home group only; a full group without the token (rare) is
    // probed further below, after the M load has been waited for: a loop
    // here would make the compiler wait for that load before entering it
    uint32_t g[2] = {0u, 0u};
    if (use_map) {
      i32x4 keys[2], vals[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        g[h] = tok_group(pv[h] ? p[h] : 0);
        keys[h] = reinterpret_cast<const i32x4*>(S.hkey)[g[h]];
        vals[h] = reinterpret_cast<const i32x4*>(S.hval)[g[h]];
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) w[h] = pv[h] ? group_find(keys[h], vals[h], p[h]) : -1;
    } else {
      w[0] = w[1] = -1;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int32_t* src = w[h] >= 0 ? S.topk + w[h] * k : S.pre + pre_row;
      alt[h] = src[rnk[h]];
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (w[h] == -2) {
        w[h] = map_get_from(S, p[h], (g[h] + 1) & uint32_t(kMapSlots / 4 - 1));
        alt[h] = (w[h] >= 0 ? S.topk + w[h] * k : S.pre + pre_row)[rnk[h]];
      }
    }
    if (mail) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (dep[h] != d || w[h] < 0 || rnk[h] == 0) continue;
        const uint32_t* word = mail + w[h] * k + rnk[h];
        uint32_t v = 0;
        for (int spin = 0; spin <= kSpinLimit; ++spin) {
          v = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (v >> 31) break;
        }
        if ((v >> 31) == 0u) set_flag(ws, TR_FLAG_HANDOVER);
        alt[h] = (v >> 31) ? int32_t(v & 0x7FFFFFFFu) : -1;
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (dep[h] != d) continue;
      if (p[h] >= 0 && !pv[h]) set_flag(ws, TR_FLAG_BAD_TOKEN);
      const int64_t v = !pv[h] ? -1 : (w[h] >= 0 || first_pre) ? int64_t(alt[h]) : int64_t(mv[h]);
      const bool ok = v >= 0 && v < V;
      if (pv[h] && !ok) set_flag(ws, TR_FLAG_BAD_TOKEN);
      S.nxt[n[h]] = ok ? int32_t(v) : -1;
    }
    wave_lds_sync();
  }
  if (lane == 0 && (root < 0 || int64_t(root) >= V)) set_flag(ws, TR_FLAG_BAD_TOKEN);
#pragma unroll
  for (int h = 0; h < 2; ++h)
    if (n[h] < tree.T) out_b[n[h]] = S.nxt[n[h]];
}

}  // namespace tr
