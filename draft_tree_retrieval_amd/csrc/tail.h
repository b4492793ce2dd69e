// Per-sequence integer work of a TR step, run by one workgroup
// (blockDim.x >= number of tree nodes): verification, the recycling update
// of M, the commit of the accepted path's key/value rows and the retrieval
// of the next draft tree.
#pragma once

#include "dev_common.h"

namespace tr {

struct TailShared {
  int32_t tok[kMaxNodes];    // this step's tree tokens
  int32_t g[kMaxNodes];      // target's top-1 after each node
  int32_t acc[kMaxNodes];    // accepted?
  int32_t nxt[kMaxNodes];    // next tree tokens
  int32_t path[kMaxNodes];   // accepted path, root first
  uint32_t red[16];
  int32_t best, L, bonus, P;
};

__device__ __forceinline__ int64_t m_load(const void* M, int m_is64, int64_t idx) {
  return m_is64 ? reinterpret_cast<const int64_t*>(M)[idx]
                : int64_t(reinterpret_cast<const int32_t*>(M)[idx]);
}
__device__ __forceinline__ void m_store(void* M, int m_is64, int64_t idx, int32_t v) {
  if (m_is64) reinterpret_cast<int64_t*>(M)[idx] = int64_t(v);
  else reinterpret_cast<int32_t*>(M)[idx] = v;
}

// tok <- tree_tok_b, g <- column 0 of topk_b.  The top-k rows may have been
// handed over by other blocks of the same launch: read them with get_dev.
__device__ __forceinline__ void tail_load(TailShared& S, const TreeDev& tree, const int32_t* tok_b,
                                          const int32_t* topk_b, int32_t k) {
  for (int n = threadIdx.x; n < tree.T; n += blockDim.x) {
    S.tok[n] = tok_b[n];
    S.g[n] = get_dev(topk_b + int64_t(n) * k);
  }
  __syncthreads();
}

// Greedy verification: acc(0); acc(n) = acc(parent) && tok(n) == g(parent);
// best = deepest accepted node, ties to the lowest index; path root..best.
__device__ __forceinline__ void tail_verify(TailShared& S, const TreeDev& tree) {
  const int tid = threadIdx.x;
  if (tid == 0) S.acc[0] = 1;
  __syncthreads();
  for (int d = 1; d <= tree.D; ++d) {
    for (int n = tid; n < tree.T; n += blockDim.x) {
      if (tree.depth[n] == d) {
        int p = tree.parent[n];
        S.acc[n] = S.acc[p] && (S.tok[n] == S.g[p]);
      }
    }
    __syncthreads();
  }
  uint32_t key = 0;
  for (int n = tid; n < tree.T; n += blockDim.x)
    if (S.acc[n]) key = max(key, (uint32_t(tree.depth[n]) << 8) | uint32_t(255 - n));
  key = wave_max_u32(key);
  const int nw = blockDim.x >> 6;
  if ((tid & 63) == 0) S.red[tid >> 6] = key;
  __syncthreads();
  if (tid == 0) {
    uint32_t m = S.red[0];
    for (int w = 1; w < nw; ++w) m = max(m, S.red[w]);
    int best = 255 - int(m & 255u);
    int L = tree.depth[best];
    int n = best;
    for (int i = L; i >= 0; --i) {
      S.path[i] = n;
      n = (n == 0) ? 0 : tree.parent[n];
    }
    S.best = best;
    S.L = L;
    S.bonus = S.g[best];
  }
  __syncthreads();
}

// Verification outputs of sequence b.
__device__ __forceinline__ void tail_write_verdict(const TailShared& S, const TreeDev& tree, int b,
                                                   int32_t* accept_len, int32_t* accept_path,
                                                   int32_t* bonus, int32_t* emitted) {
  const int W = tree.D + 1;
  for (int i = threadIdx.x; i < W; i += blockDim.x) {
    if (accept_path) accept_path[int64_t(b) * W + i] = (i <= S.L) ? S.path[i] : -1;
    if (emitted)
      emitted[int64_t(b) * W + i] = (i < S.L) ? S.tok[S.path[i + 1]] : (i == S.L ? S.bonus : -1);
  }
  if (threadIdx.x == 0) {
    if (accept_len) accept_len[b] = S.L;
    if (bonus) bonus[b] = S.bonus;
  }
}

// M[tok n] = topk[n] for every node n whose token no later node repeats
// (the node with the highest index wins on duplicated tokens).
__device__ __forceinline__ void tail_update(const TailShared& S, const TreeDev& tree,
                                            const int32_t* topk_b, int32_t k, void* M_b,
                                            int m_is64, int64_t V, uint8_t* ws) {
  for (int n = threadIdx.x; n < tree.T; n += blockDim.x) {
    const int32_t t = S.tok[n];
    bool winner = true;
    for (int m = n + 1; m < tree.T; ++m) winner = winner && (S.tok[m] != t);
    if (!winner) continue;
    if (t < 0 || int64_t(t) >= V) {
      set_flag(ws, TR_FLAG_BAD_TOKEN);
      continue;
    }
    for (int j = 0; j < k; ++j) m_store(M_b, m_is64, int64_t(t) * k + j, get_dev(topk_b + int64_t(n) * k + j));
  }
}

// Copy the key/value rows of path[0..L] to cache positions P..P+L.
__device__ __forceinline__ void tail_commit(TailShared& S, const TreeDev& tree, int b,
                                            const TailArgs& a, uint8_t* ws) {
  if (!a.k_cache) return;
  if (threadIdx.x == 0) S.P = a.prefix_len[b];
  __syncthreads();
  const int64_t P = S.P;
  const int nrows = S.L + 1;
  if (P < 0 || P + nrows > a.cap) {
    if (threadIdx.x == 0) set_flag(ws, TR_FLAG_CACHE_FULL);
    return;
  }
  const int upr = a.row_bytes >> 4;               // 16-byte units per row
  const int per_node = a.Hkv * upr;
  const int total = 2 * nrows * per_node;          // keys then values
  constexpr int R = 4;                             // units in flight per thread
  for (int u0 = threadIdx.x; u0 < total; u0 += R * blockDim.x) {
    u32x4 buf[R];
    int64_t dst_off[R];
    bool dst_v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int u = min(u0 + r * int(blockDim.x), total - 1);   // clamped: loads stay in bounds
      const bool isv = u >= total / 2;
      const int uu = isv ? u - total / 2 : u;
      const int i = uu / per_node, rem = uu - i * per_node;
      const int h = rem / upr, c = rem - h * upr;
      const int node = S.path[i];
      const uint8_t* src = (isv ? a.v_tree : a.k_tree) +
                           ((int64_t(b) * tree.T + node) * a.Hkv + h) * a.row_bytes + c * 16;
      dst_off[r] = ((int64_t(b) * a.Hkv + h) * a.cap + P + i) * a.row_bytes + c * 16;
      dst_v[r] = isv;
      buf[r] = *reinterpret_cast<const u32x4*>(src);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (u0 + r * int(blockDim.x) >= total) break;
      uint8_t* dst = (dst_v[r] ? a.v_cache : a.k_cache) + dst_off[r];
      *reinterpret_cast<u32x4*>(dst) = buf[r];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) a.prefix_len[b] = int32_t(P + nrows);
}

// Draft tree retrieval: nxt[0] = root; layer by layer
// nxt[n] = M[nxt[parent n]][rank n].  Invalid tokens propagate as -1.
__device__ __forceinline__ void tail_retrieve(TailShared& S, const TreeDev& tree, int32_t root,
                                              const void* M_b, int m_is64, int64_t V, int32_t k,
                                              int32_t* out_b, uint8_t* ws) {
  if (threadIdx.x == 0) S.nxt[0] = root;
  __syncthreads();
  for (int d = 1; d <= tree.D; ++d) {
    for (int n = threadIdx.x; n < tree.T; n += blockDim.x) {
      if (tree.depth[n] == d) {
        const int32_t p = S.nxt[tree.parent[n]];
        int32_t t = -1;
        if (p >= 0 && int64_t(p) < V) {
          int64_t v = m_load(M_b, m_is64, int64_t(p) * k + tree.rank[n]);
          if (v >= 0 && v < V) t = int32_t(v);
          else set_flag(ws, TR_FLAG_BAD_TOKEN);
        } else if (p >= 0) {
          set_flag(ws, TR_FLAG_BAD_TOKEN);
        }
        S.nxt[n] = t;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0 && (root < 0 || int64_t(root) >= V)) set_flag(ws, TR_FLAG_BAD_TOKEN);
  for (int n = threadIdx.x; n < tree.T; n += blockDim.x) out_b[n] = S.nxt[n];
}

}  // namespace tr
