// Stochastic verification of a TR step (the speculative-sampling rule of
// the speculative-decoding lesson -- accept a draft x with min(1, p(x)/q(x)),
// otherwise draw from the normalised positive part of p - q and stop --
// applied to a draft tree whose drafts come from M, so q is a point mass on
// each drafted token).
//
// p_n = softmax(z_n / temperature) after node n.  From the root, the
// children of the current node are tried in rank order: child c with token
// x is accepted when u_c * (Z - R) < e_x, where e_x = exp(z_x - max) /
// temperature scaled, Z the sum of e over the row and R the mass of the
// distinct siblings rejected before it (r(x) = e_x / (Z - R) is x's
// probability in the residual).  A duplicate of a rejected sibling has
// residual probability 0.  The first accepted child becomes the current
// node; when none is accepted (or there are none) the bonus token is drawn
// from the residual of that node with its second uniform, by inverse CDF
// over the ids in increasing order.
//
// Work split: every top-k block hands over (max, sum of e) of its row
// segment with the top-k ids; the tail merges them per node, gathers each
// child's logit in its parent's row, walks the tree with wave 0 (one ballot
// per level) and draws with the whole block: every wave sums 512-id buckets
// of the stop node's row, then wave 0 finds the bucket, the lane and the
// id, each level continuing the running sum of the level above, so a
// crossing is found whenever the draw lies below the total.  Where rounding
// leaves a level without a crossing, the last unit there with positive mass
// is taken.
#pragma once

#include "tail.h"

namespace tr {

struct SampleShared {
  float sm[kMaxNodes];          // row maximum of each node's logits
  float sz[kMaxNodes];          // sum over the row of exp2((z - max) * scale)
  float pe[kMaxNodes];          // node c's token's e in its parent's row
  float u0[kMaxNodes];          // uniforms: acceptance as a child
  float u1[kMaxNodes];          //           the draw when the walk stops here
  int32_t excl[kMaxK];          // tokens taken out of the stop node's residual
  int32_t nex;
  float bucket[kMaxBuckets];    // e summed over each 512-id bucket of the stop row
};

// Inverse of ord32: the float whose order code is `code` (-0.0 comes back
// as +0.0).
__device__ __forceinline__ float ord_to_f32(uint32_t code) {
  return __uint_as_float(code >= 0x80000000u ? code - 0x80000000u : 0u - code);
}

// e = exp2(z * scale + off), off = -max * scale: every place that weighs a
// logit uses this one expression, so equal logits get equal bits.  The
// hardware exp2 flushes results below 2^-126 to zero; the row maximum
// weighs 1, so such terms are below float rounding of any sum they join.
__device__ __forceinline__ float soft_weight(float z, float scale, float off) {
  return __builtin_amdgcn_exp2f(fmaf(z, scale, off));
}

// Running sums in lane order: lane i gets v_0 + ... + v_{i-1} added onto
// `base` one lane at a time (every lane performs the same additions, so
// the sum after lane i is bit for bit the one lane i+1 starts from), and
// `end` the sum after all 64.
__device__ __forceinline__ float lane_running_sum(float v, float base, float& end) {
  const int lane = threadIdx.x & 63;
  float run = base, mine = base;
#pragma unroll 8
  for (int i = 0; i < 64; ++i) {
    const float vi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), i));
    mine = i == lane ? run : mine;
    run += vi;
  }
  end = run;
  return mine;
}

template <bool BF16>
__device__ __forceinline__ float logit_at(const void* logits, int64_t idx) {
  if constexpr (BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(logits)[idx]);
  else return reinterpret_cast<const float*>(logits)[idx];
}

// Per-node statistics, children's probabilities and uniforms into LDS (all
// threads; needs blockDim.x >= tree.T).  stat holds [rows][segs] (max, sum)
// pairs handed over by the top-k blocks.
template <bool BF16>
__device__ __forceinline__ void sample_prepare(const TailShared& S, SampleShared& SS,
                                               const TreeDev& tree, int b, int64_t V,
                                               const void* logits, const uint64_t* stat,
                                               int32_t segs, const TailArgs& a) {
  const int n = threadIdx.x;
  const float s2 = a.temp_scale;
  float zc = 0.f;
  if (n < tree.T) {
    const int64_t row = int64_t(b) * tree.T + n;
    const int32_t x = S.tok[n];
    const bool ok = n > 0 && x >= 0 && int64_t(x) < V;
    if (ok) zc = logit_at<BF16>(logits, (int64_t(b) * tree.T + S.par[n]) * V + x);
    SS.u0[n] = a.uniforms[row * 2];
    SS.u1[n] = a.uniforms[row * 2 + 1];
    float m = -__builtin_inff(), z = 0.f;
    for (int g = 0; g < segs; ++g) {             // segments in order
      const uint64_t st = get_dev(stat + row * segs + g);
      const float mg = __uint_as_float(uint32_t(st)), sg = __uint_as_float(uint32_t(st >> 32));
      if (mg > m) {
        z = z * exp2f((m - mg) * s2) + sg;
        m = mg;
      } else {
        z += sg * exp2f((mg - m) * s2);
      }
    }
    SS.sm[n] = m;
    SS.sz[n] = z;
  }
  __syncthreads();
  if (n > 0 && n < tree.T) {
    const int32_t x = S.tok[n];
    const bool ok = x >= 0 && int64_t(x) < V;
    const float mp = SS.sm[S.par[n]];
    SS.pe[n] = ok ? soft_weight(zc, s2, -mp * s2) : 0.f;
  }
  __syncthreads();
}

// The walk, by wave 0: S.path, S.L, S.best (the stop node) and the stop
// node's excluded tokens.
__device__ __forceinline__ void sample_walk(TailShared& S, SampleShared& SS, const TreeDev& tree,
                                            int64_t V) {
  const int lane = threadIdx.x & 63;
  const int pa = (lane > 0 && lane < tree.T) ? S.par[lane] : -1;
  const int pb = (lane + 64 < tree.T) ? S.par[lane + 64] : -1;
  int n = 0, L = 0;
  while (true) {
    const uint64_t ma = __ballot(pa == n), mb = __ballot(pb == n);
    const int nc = __popcll(ma) + __popcll(mb);   // <= k: children hold distinct ranks below k
    const int c0 = ma ? int(__builtin_ctzll(ma)) : 64 + int(__builtin_ctzll(mb | (1ull << 63)));
    const bool has = lane < nc;
    int32_t x = -1;
    float e = 0.f, u = 1.f;
    if (has) {                                  // children are consecutive nodes, in rank order
      x = S.tok[c0 + lane];
      e = SS.pe[c0 + lane];
      u = SS.u0[c0 + lane];
    }
    const bool valid = has && x >= 0 && int64_t(x) < V;
    bool dup = false;
    for (int i = 0; i < nc; ++i) dup = dup || (i < lane && __builtin_amdgcn_readlane(x, i) == x);
    const float ev = (valid && !dup) ? e : 0.f;
    float pre = 0.f;                            // rejected mass before this sibling, in rank order
    for (int i = 0; i < nc; ++i) {
      const float ei = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ev), i));
      pre += i < lane ? ei : 0.f;
    }
    const float Z = SS.sz[n];
    const uint64_t am = __ballot(valid && !dup && u * (Z - pre) < e);
    if (am) {
      n = c0 + int(__builtin_ctzll(am));
      ++L;
      if (lane == 0) S.path[L] = n;
      continue;
    }
    if (has) SS.excl[lane] = valid ? x : -1;
    if (lane == 0) {
      SS.nex = nc;
      S.path[0] = 0;
      S.best = n;
      S.L = L;
    }
    return;
  }
}

// Raw bits of ids i0 .. i0+7 of a row (16-byte loads where the row is
// aligned and the ids are inside it, single loads otherwise; ids past the
// row read nothing).
template <bool BF16>
__device__ __forceinline__ void draw_load(const uint8_t* rowp, int64_t i0, int64_t V, bool vec_ok,
                                          u32x4 (&v)[2]) {
  v[0] = u32x4{0, 0, 0, 0};
  v[1] = u32x4{0, 0, 0, 0};
  if (vec_ok && i0 + 8 <= V) {
    const u32x4* p = reinterpret_cast<const u32x4*>(rowp + i0 * (BF16 ? 2 : 4));
    v[0] = p[0];
    if (!BF16) v[1] = p[1];
    return;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (i0 + j >= V) break;
    if (BF16) {
      const uint32_t h = reinterpret_cast<const uint16_t*>(rowp)[i0 + j];
      v[0][j >> 1] |= (j & 1) ? (h << 16) : h;
    } else {
      v[j >> 2][j & 3] = reinterpret_cast<const uint32_t*>(rowp)[i0 + j];
    }
  }
}

// e of ids i0 .. i0+7 (0 past the row and for excluded ids).
template <bool BF16>
__device__ __forceinline__ void draw_weights(const u32x4 (&v)[2], int64_t i0, int64_t V, float s2,
                                             float off, const SampleShared& SS, int nex,
                                             float (&w)[8]) {
  uint32_t skip = 0;
  for (int q = 0; q < nex; ++q) {
    const int64_t d = int64_t(SS.excl[q]) - i0;
    if (SS.excl[q] >= 0 && d >= 0 && d < 8) skip |= 1u << uint32_t(d);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float z = BF16 ? __uint_as_float((j & 1) ? (v[0][j >> 1] & 0xFFFF0000u) : (v[0][j >> 1] << 16))
                         : __uint_as_float(v[j >> 2][j & 3]);
    const bool in = i0 + j < V && !((skip >> j) & 1u);
    w[j] = in ? soft_weight(z, s2, off) : 0.f;
  }
}

// The draw at the stop node S.best into S.bonus (all threads call it; the
// caller synchronises afterwards).
template <bool BF16>
__device__ __forceinline__ void sample_draw(TailShared& S, SampleShared& SS, const TreeDev& tree,
                                            int b, int32_t k, int64_t V, const void* logits,
                                            float s2) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = int(blockDim.x >> 6);
  const int s = S.best;
  const uint8_t* rowp = reinterpret_cast<const uint8_t*>(logits) +
                        (int64_t(b) * tree.T + s) * V * (BF16 ? 2 : 4);
  const bool vec_ok = (reinterpret_cast<uintptr_t>(rowp) & 15) == 0;
  const float off = -SS.sm[s] * s2;
  const int nex = SS.nex;
  const int nb = int((V + kDrawBucket - 1) / kDrawBucket);

  // pass 1: bucket sums, eight buckets of a wave in flight at once
  constexpr int kChunk = 8;
  for (int c0 = wave; c0 < nb; c0 += kChunk * nw) {
    u32x4 raw[kChunk][2];
#pragma unroll
    for (int q = 0; q < kChunk; ++q) {
      const int bk = c0 + q * nw;
      if (bk < nb) draw_load<BF16>(rowp, int64_t(bk) * kDrawBucket + lane * 8, V, vec_ok, raw[q]);
    }
#pragma unroll
    for (int q = 0; q < kChunk; ++q) {
      const int bk = c0 + q * nw;
      if (bk >= nb) break;
      float w[8];
      draw_weights<BF16>(raw[q], int64_t(bk) * kDrawBucket + lane * 8, V, s2, off, SS, nex, w);
      float ls = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) ls += w[j];
      const float tot = wave_sum_f32(ls);
      if (lane == 0) SS.bucket[bk] = tot;
    }
  }
  __syncthreads();
  if (wave != 0) return;

  // pass 2 (wave 0): running sums over the buckets in order (64 at a time,
  // bucket lane + 64 q in lane `lane`), the total, then the first bucket
  // whose running sum passes tau = r * total
  const float r = SS.u1[s];
  constexpr int kQ = kMaxBuckets / 64;
  float bv[kQ], bstart[kQ];
  float tot = 0.f;
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    if (q * 64 >= nb) break;                   // wave-uniform
    const int i = q * 64 + lane;
    bv[q] = i < nb ? SS.bucket[i] : 0.f;
    bstart[q] = lane_running_sum(bv[q], tot, tot);
  }
  const float tau = r * tot;
  int bsel = -1, blast = -1;
  float before = 0.f;
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    if (q * 64 >= nb) break;
    const uint64_t cross = __ballot(bv[q] > 0.f && bstart[q] + bv[q] > tau);
    const uint64_t pos = __ballot(bv[q] > 0.f);
    if (pos) blast = q * 64 + 63 - int(__builtin_clzll(pos));
    if (bsel < 0 && cross) {
      const int j = int(__builtin_ctzll(cross));
      bsel = q * 64 + j;
      before = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bstart[q]), j));
    }
  }
  if (bsel < 0 && blast >= 0) {                // tau within rounding of the total
    bsel = blast;
    const int q = blast >> 6, j = blast & 63;
#pragma unroll
    for (int qq = 0; qq < kQ; ++qq)
      if (qq == q) before = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bstart[qq]), j));
  }
  if (bsel < 0) {                              // no mass outside the excluded ids
    if (lane == 0) {
      int32_t pick = S.topk[s * k];
      for (int i = k - 1; i >= 0; --i) {
        const int32_t c = S.topk[s * k + i];
        bool ex = false;
        for (int q = 0; q < nex; ++q) ex = ex || SS.excl[q] == c;
        if (!ex) pick = c;
      }
      S.bonus = pick;
    }
    return;
  }

  // the lane of the bucket: running sums in lane order, continued from before
  const int64_t i0 = int64_t(bsel) * kDrawBucket + lane * 8;
  u32x4 raw[2];
  draw_load<BF16>(rowp, i0, V, vec_ok, raw);
  float w[8];
  draw_weights<BF16>(raw, i0, V, s2, off, SS, nex, w);
  float ls = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) ls += w[j];
  float bend;
  const float mine = lane_running_sum(ls, before, bend);   // running sum after lanes 0..lane-1
  const uint64_t cross = __ballot(mine + ls > tau && ls > 0.f);
  const uint64_t pos = __ballot(ls > 0.f);
  int lsel;
  if (cross) {
    // the first lane whose running sum passes tau (lanes before it do not)
    lsel = int(__builtin_ctzll(cross));
  } else {
    lsel = pos ? 63 - int(__builtin_clzll(pos)) : 0;
  }
  if (lane == lsel) {
    float acc = mine;
    int pick = -1, lastpos = -1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (w[j] > 0.f) lastpos = j;
      acc += w[j];
      if (pick < 0 && w[j] > 0.f && acc > tau) pick = j;
    }
    if (pick < 0) pick = lastpos >= 0 ? lastpos : 0;
    S.bonus = int32_t(i0 + pick);
  }
}

}  // namespace tr
