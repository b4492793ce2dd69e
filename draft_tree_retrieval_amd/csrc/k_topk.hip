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
//   2. every wave finds, by bisection on the code bits with ballot counts
//      over all the block's lane maxima (shared through LDS), the largest
//      code t that at least k lane maxima reach: k distinct elements are
//      >= t, so nothing below t is among the k best;
//   3. only elements at or above t -- usually k or a few more -- are
//      written, by ballot, to per-wave candidate lists in LDS; one wave
//      ranks them in registers (all threads rank them when there are many).
// Rows full of ties can overflow a candidate list; the block then falls
// back to exact per-lane insertion of every element above the threshold.
//
// Launch: grid (segments, rows).  Many rows: 256 threads holding 16
// vectors per lane, segments spreading short vocabularies over the CUs.
// Few rows (latency-bound): 512 threads holding 8 vectors per lane, so two
// waves per SIMD share the selection work.  The last segment block of
// a row merges the
// segment lists, and the last row block of a sequence runs that sequence's
// tail (hand-over through device-scope atomics, see dev_common.h).
#include "sample.h"
#include "select.h"

namespace tr {

TopkPlan plan_topk(int64_t rows, int64_t V, int32_t k, int32_t esz) {
  TopkPlan p{};
  p.rows = rows;
  p.kmax = k <= 8 ? 8 : 16;
  p.threads = rows < 256 ? 1024 : 256;
  const int64_t nv = p.threads == 1024 ? 4 : 16;          // vectors per lane
  const int64_t cap = int64_t(p.threads) * nv * (16 / esz);  // largest segment a block holds
  const int64_t max_segs = 256 / p.kmax;                 // the final merge ranks <= 256 keys
  p.seg_cap = cap;
  p.max_v = max_segs * cap;                              // longer rows are refused on the host
  int64_t need = (V + cap - 1) / cap;
  // Few rows: one block per row when a row fits, so no segment hand-over
  // (a round trip through device memory) stands between the scan and the
  // step's tail.  Many rows: about one block per CU, segments of >= 4096.
  int64_t want = (256 + rows - 1) / rows;
  int64_t by_len = V / 4096;
  int64_t segs = rows < 256 ? 1 : (want < by_len ? want : by_len);
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
  p.stat_off = off;
  off = align256(off + size_t(rows) * segs * 8);
  p.end = off;
  return p;
}

// The per-sequence tail: update only (TAIL_UPDATE) or the whole step
// (TAIL_STEP: verification, update, commit, next retrieval).  Needs at
// least 256 threads.  After verification, wave 0 retrieves the next tree
// while waves 1.. write the verdict, wave 1 the updated rows of M and
// waves 1.. copy the accepted key/value rows, so retrieval's loads never
// wait behind their stores.
template <typename MT, int KM, int NT, bool BF16, bool SAMPLE>
__device__ __forceinline__ void seq_tail(TailShared& S, const TreeDev& tree, int b, int32_t k,
                                         int64_t V, const int32_t* topk_b, int32_t* tok_b,
                                         const TailArgs& tail, uint8_t* ws, const void* logits,
                                         const uint64_t* stat, int32_t segs) {
  static_assert(NT >= 256, "the tail's roles take four waves");
  void* M_b = reinterpret_cast<MT*>(tail.M) + int64_t(b) * V * k;
  const int wave = threadIdx.x >> 6;
  if constexpr (SAMPLE) {
    // verification by sampling: no greedy token to prefetch M rows for
    __shared__ SampleShared SS;
    tail_load<NT>(S, tree, tok_b, topk_b, k, tail.k_cache ? tail.prefix_len + b : nullptr);
    sample_prepare<BF16>(S, SS, tree, b, V, logits, stat, segs, tail);
    if (wave == 0) sample_walk(S, SS, tree, V);
    __syncthreads();
    sample_draw<BF16>(S, SS, tree, b, k, V, logits, tail.temp_scale);
    __syncthreads();
    tail_write_verdict(S, tree, b, tail.accept_len, tail.accept_path, nullptr, tail.emitted, 64);
    if (wave == 0) tail_update_claim(S, tree, V, ws, tail.update_mode == UPDATE_ACCEPTED);
    __syncthreads();
    if (wave != 0) {
      tail_commit(S, tree, b, tail, ws, 64);
      if (wave == 1) tail_update_store<MT>(S, tree, k, M_b, V);
      return;
    }
    const bool fits = tail_commit_fits(S, tail, S.L);
    tail_retrieve<MT>(S, tree, S.bonus, M_b, V, k, tok_b, ws, true, false);
    if (threadIdx.x == 0) {
      tail.root_tok[b] = S.bonus;
      if (fits) tail.prefix_len[b] = int32_t(S.P + S.L + 1);
    }
    return;
  }
  if (tail.mode != TAIL_STEP) {
    tail_load<NT>(S, tree, tok_b, topk_b, k);
    if (wave == 0) {
      tail_update_claim(S, tree, V, ws);
      wave_lds_sync();
      tail_update_store<MT>(S, tree, k, M_b, V);
    }
    return;
  }
  tail_load<NT>(S, tree, tok_b, topk_b, k, tail.k_cache ? tail.prefix_len + b : nullptr);
  // wave 0 verifies while waves 2 and 3 fetch the rows the next tree's
  // first layer may take; wave 1 fills the update map meanwhile unless only
  // the accepted path is recycled (that map needs the verdict)
  const bool path_only = tail.update_mode == UPDATE_ACCEPTED;
  Verdict vd{};
  if (wave == 0) {
    vd = tail_verify_wave(S, tree, k);
    if (path_only) {
      wave_lds_sync();
      tail_update_claim(S, tree, V, ws, true);
    }
  } else if (wave == 1) {
    if (!path_only) tail_update_claim(S, tree, V, ws, false);
  } else if (wave < 4) {
    tail_prefetch<MT, KM>(S, tree, k, M_b, V, int(threadIdx.x) - 128);
  }
  __syncthreads();                                   // verdict, update map, prefetched rows
  if (wave != 0) {                                   // outputs and stores
    tail_write_verdict(S, tree, b, tail.accept_len, tail.accept_path, nullptr, tail.emitted, 64);
    tail_commit(S, tree, b, tail, ws, 64);
    if (wave == 1) tail_update_store<MT>(S, tree, k, M_b, V);
    return;
  }
  const bool fits = tail_commit_fits(S, tail, vd.L);
  tail_retrieve<MT>(S, tree, vd.bonus, M_b, V, k, tok_b, ws, true, true);
  if (threadIdx.x == 0) {
    tail.root_tok[b] = vd.bonus;
    if (fits) tail.prefix_len[b] = int32_t(S.P + vd.L + 1);
  }
}

// The sampling instantiations are held to three waves per SIMD (at most
// 168 VGPRs), as many as the greedy ones reach by themselves: with many
// rows the blocks of a launch run in rounds, so occupancy is throughput.
// Where a top-k block's results go: with several segments per row, its KM
// best keys (key 0 past the segment's elements) to the row's partial lists,
// else the k ids to the output; written with device-scope atomics by wave 0
// for the last-arriving block (dev_common.h).
template <int KM>
struct TopkOut {
  uint64_t* part;
  int32_t* ids;
  int64_t row;
  int seg, segs;
  int32_t k;
  __device__ __forceinline__ void first(uint32_t) const {}
  __device__ __forceinline__ void put(int r, uint64_t key) const {
    if (segs > 1) put_dev(&part[(row * segs + seg) * KM + r], key);
    else if (r < k) put_dev(&ids[row * k + r], int32_t(key_id(key)));
  }
};

template <bool BF16, int KM, int NT, int NV, bool SAMPLE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(SAMPLE ? 3 : 1))) void topk_kernel(const void* __restrict__ logits, int64_t V,
                                                   int32_t k, int32_t segs, int64_t seg_len,
                                                   int32_t* __restrict__ ids_out,
                                                   uint64_t* __restrict__ part, uint64_t* stat,
                                                   uint8_t* ws, TreeDev tree, TailArgs tail,
                                                   int32_t defer) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int VE = 16 / ESZ;             // elements per 16-byte vector
  constexpr int NW = NT / 64;              // waves
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.y;
  const int seg = blockIdx.x;
  const int64_t s0 = int64_t(seg) * seg_len;
  const int64_t s1 = min(V, s0 + seg_len);
  const uint8_t* rowp = reinterpret_cast<const uint8_t*>(logits) + row * V * ESZ;

  constexpr int kCand = NW * kCandW;
  __shared__ uint64_t s_cand[kCand];
  __shared__ uint64_t s_keys[NW][KM];
  __shared__ uint64_t s_best[KM];
  __shared__ uint32_t s_wcnt[NW];
  __shared__ uint32_t s_top[NW * KM];
  __shared__ float s_wsum[NW];

  if constexpr (!SAMPLE) {
    // greedy steps and top-k alone: the compact selection of select.h
    TopkOut<KM> out{part, ids_out, row, seg, segs, k};
    select_block<BF16, KM, NT, NV, false>(rowp, s0, s1, k, out);
  } else {
    // sampling: the same selection, with each segment's softmax statistics
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
    u32x4 x[NV];
  #pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = i * NT + tid;
      x[i] = idx < nv ? __builtin_nontemporal_load(vp + idx) : u32x4{0, 0, 0, 0};
    }
    uint32_t loose_code[2] = {0, 0};       // head and tail elements
    const int64_t loose_id[2] = {s0 + tid, a1 + tid};
    if (loose_id[0] < a0) loose_code[0] = code_at(loose_id[0]);
    if (loose_id[1] < s1) loose_code[1] = code_at(loose_id[1]);
    uint32_t mt = max(loose_code[0], loose_code[1]);
    uint32_t m2 = 0;
  #pragma unroll
    for (int i = 0; i < NV; ++i) {
      const uint32_t keep = (i * NT + tid < nv) ? ~0u : 0u;
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

    // ---- 2. threshold: the largest code reached by at least k lane maxima
    // of the block, i.e. the k-th largest lane maximum.  Each wave bisects
    // over its own 64 lanes for its k-th largest and puts its k largest lane
    // maxima into LDS (those above it, then copies of it); the block's k-th
    // largest is the k-th largest of these NW * k values (the block's k
    // largest are among them), found by every wave with a second bisection.
    constexpr int kLowBit = BF16 ? 16 : 0;
    uint32_t lo = 0;
  #pragma unroll
    for (int bit = 31; bit >= kLowBit; --bit) {
      const uint32_t c = lo | (1u << bit);
      if (__popcll(__ballot(mt >= c)) >= k) lo = c;
    }
    {
      const uint64_t gt = __ballot(mt > lo);            // fewer than k lanes
      const int ngt = __popcll(gt);
      const uint32_t below = __builtin_amdgcn_mbcnt_hi(uint32_t(gt >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(gt), 0u));
      if (mt > lo) s_top[wave * KM + below] = mt;
      if (lane >= ngt && lane < k) s_top[wave * KM + lane] = lo;
    }
    __syncthreads();
    constexpr int NTOP = NW * KM;                       // 32 .. 256
    constexpr int NTV = (NTOP + 63) / 64;
    uint32_t tv[NTV];
  #pragma unroll
    for (int h = 0; h < NTV; ++h) {
      const int i = lane + 64 * h;
      tv[h] = (i < NTOP && (i % KM) < k) ? s_top[min(i, NTOP - 1)] : 0u;
    }

    // sampling: softmax statistics of the segment, (max, sum of
    // exp2((z - max) * scale)), handed over with the ids
    float seg_max = 0.f;
    if constexpr (SAMPLE) {
      uint32_t bm = tv[0];
  #pragma unroll
      for (int h = 1; h < NTV; ++h) bm = max(bm, tv[h]);
      bm = wave_max_u32(bm);
      seg_max = ord_to_f32(bm);
      const float s2 = tail.temp_scale, off = -seg_max * s2;
      float acc = 0.f;
  #pragma unroll
      for (int i = 0; i < NV; ++i)
  #pragma unroll
        for (int j = 0; j < 4; ++j) {
          // an opaque copy: were the halves extracted here shared with the
          // candidate scan below, all of them would stay live across the
          // threshold search (twice the registers of x)
          uint32_t word = x[i][j];
          asm volatile("" : "+v"(word));
          if (BF16) {
            const uint32_t c0 = (word & 0xFFFFu) << 16, c1 = word & 0xFFFF0000u;
            acc += c0 ? soft_weight(ord_to_f32(c0), s2, off) : 0.f;
            acc += c1 ? soft_weight(ord_to_f32(c1), s2, off) : 0.f;
          } else {
            acc += word ? soft_weight(ord_to_f32(word), s2, off) : 0.f;
          }
        }
  #pragma unroll
      for (int h = 0; h < 2; ++h)
        acc += loose_code[h] ? soft_weight(ord_to_f32(loose_code[h]), s2, off) : 0.f;
      acc = wave_sum_f32(acc);
      if (lane == 0) s_wsum[wave] = acc;
    }
    lo = 0;
  #pragma unroll
    for (int bit = 31; bit >= kLowBit; --bit) {
      const uint32_t c = lo | (1u << bit);
      int reach = 0;
  #pragma unroll
      for (int h = 0; h < NTV; ++h) reach += __popcll(__ballot(tv[h] >= c));
      if (reach >= k) lo = c;
    }

    // ---- 3. candidates: each element at or above lo gets the next slot of
    // its wave's list, in lane order (ballot + lane-masked bit count)
    uint64_t* wc = s_cand + wave * kCandW;
    uint32_t wpos = 0;                        // wave-uniform
    auto put = [&](bool pred, uint32_t code, int64_t id) {
      const uint64_t m = __ballot(pred);
      if (m) {
        const uint32_t off =
            wpos + __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
        if (pred && off < uint32_t(kCandW)) wc[off] = key_of(code, uint32_t(id));
        wpos += uint32_t(__popcll(m));
      }
    };
    const uint32_t lo16 = lo >> 16;
    const uint32_t below2 = lo16 ? (lo16 - 1) * 0x10001u : 0u;     // bf16: lo16-1 in both halves
  #pragma unroll
    for (int i = 0; i < NV; ++i) {
      uint32_t hv[4];                          // nonzero where an element reaches lo
      bool hit = false;
  #pragma unroll
      for (int j = 0; j < 4; ++j) {
        hv[j] = BF16 ? (max16x2(x[i][j], below2) ^ below2) : ((x[i][j] && x[i][j] >= lo) ? 1u : 0u);
        hit = hit || hv[j] != 0u;
      }
      if (__ballot(hit) == 0) continue;
      const int64_t id = a0 + int64_t(i * NT + tid) * VE;
  #pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (BF16) {
          put((hv[j] & 0xFFFFu) != 0u, (x[i][j] & 0xFFFFu) << 16, id + 2 * j);
          put(hv[j] > 0xFFFFu, x[i][j] & 0xFFFF0000u, id + 2 * j + 1);
        } else {
          put(hv[j] != 0u, x[i][j], id + j);
        }
      }
    }
  #pragma unroll
    for (int h = 0; h < 2; ++h) put(loose_code[h] && loose_code[h] >= lo, loose_code[h], loose_id[h]);
    if (lane == 0) s_wcnt[wave] = wpos;
    __syncthreads();
    uint32_t n = 0, most = 0;
  #pragma unroll
    for (int w = 0; w < NW; ++w) {
      n += s_wcnt[w];
      most = max(most, s_wcnt[w]);
    }
    const bool overflow = most > uint32_t(kCandW);
    if constexpr (SAMPLE) {
      if (tid == 0) {
        float tot = 0.f;
  #pragma unroll
        for (int w = 0; w < NW; ++w) tot += s_wsum[w];
        put_dev(&stat[row * segs + seg], (uint64_t(__float_as_uint(tot)) << 32) | __float_as_uint(seg_max));
      }
    }

    // ---- the block's KM best
    if (!overflow && n <= 64u) {
      // one wave: lane i ranks candidate i against the others in registers
      if (wave == 0) {
        // lane i takes candidate i: its list and place from the list sizes,
        // read at once (not one dependent LDS read per list)
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
        if (lane >= int(n)) rank = lane;           // empty places n.. hold key 0
        if (rank < KM) {
          if (segs > 1) put_dev(&part[(row * segs + seg) * KM + rank], key);
          else if (rank < k) put_dev(&ids_out[row * k + rank], int32_t(key_id(key)));
        }
      }
    } else {
      if (!overflow && n <= uint32_t(NT)) {
        rank_select_lists<KM, NW>(s_cand, s_wcnt, int(n), s_best);
      } else {
        TopList<KM> L;
        L.clear();
        if (!overflow) {
          for (int c = tid; c < kCand; c += NT)
            if (uint32_t(c % kCandW) < s_wcnt[c / kCandW]) L.insert(s_cand[c]);
        } else {
          // too many ties at the threshold: exact insertion from the registers
  #pragma unroll
          for (int i = 0; i < NV; ++i)
  #pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int64_t id = a0 + int64_t(i * NT + tid) * VE + (BF16 ? 2 * j : j);
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
        block_merge<KM, NW>(L, s_keys, s_best);
      }
      if (tid == 0) {
  #pragma unroll
        for (int r = 0; r < KM; ++r) {
          if (segs > 1) put_dev(&part[(row * segs + seg) * KM + r], s_best[r]);
          else if (r < k) put_dev(&ids_out[row * k + r], int32_t(key_id(s_best[r])));
        }
      }
    }
  }

  // ---- segments of a row meet in the last one (defer: in topk_seq_kernel,
  // launched next, so no block holds its slot through a hand-over)
  if (segs > 1) {
    if (defer) return;
    uint32_t* row_cnt = reinterpret_cast<uint32_t*>(ws + kRowCntOff);
    if (!last_block_arrives(row_cnt + row, uint32_t(segs))) return;
    const int nk = segs * KM;                   // <= 256 by the plan
    for (int c = tid; c < nk; c += NT) s_cand[c] = get_dev(&part[row * segs * KM + c]);
    __syncthreads();
    rank_select<KM>(s_cand, nk, s_best);
    if (tid == 0) {
#pragma unroll
      for (int r = 0; r < KM; ++r)
        if (r < k) put_dev(&ids_out[row * k + r], int32_t(key_id(s_best[r])));
    }
  }
  if (tail.mode == TAIL_NONE) return;

  // ---- per-sequence tail, run by the last row block of the sequence
  const int b = int(row / tree.T);
  uint32_t* seq_cnt = reinterpret_cast<uint32_t*>(ws + kSeqCntOff);
  if (!last_block_arrives(seq_cnt + b, uint32_t(tree.T))) return;

  __shared__ TailShared S;
  const int32_t* topk_b = ids_out + int64_t(b) * tree.T * k;
  int32_t* tok_b = tail.tree_tok + int64_t(b) * tree.T;
  if (tail.m_is64)
    seq_tail<int64_t, KM, NT, BF16, SAMPLE>(S, tree, b, k, V, topk_b, tok_b, tail, ws, logits, stat, segs);
  else
    seq_tail<int32_t, KM, NT, BF16, SAMPLE>(S, tree, b, k, V, topk_b, tok_b, tail, ws, logits, stat, segs);
}

// Second half of the fused LM head: one block per row merges the 8 best
// keys of every vocabulary slice (written by lmhead_topk_kernel) into the
// row's top-k ids; the last row block of a sequence then runs the step's
// tail as topk_kernel does.  Keys are read eight per thread at a time, all
// loads of a batch in flight together.
__global__ __launch_bounds__(512) void lmhead_merge_kernel(const uint64_t* __restrict__ part,
                                                            int32_t nvs, int64_t V, int32_t k,
                                                            int32_t* __restrict__ ids_out,
                                                            uint8_t* ws, TreeDev tree,
                                                            TailArgs tail) {
  constexpr int KM = 8, NT = 512, NW = NT / 64, kBatch = 8;
  __shared__ uint64_t s_keys[NW][KM];
  __shared__ uint64_t s_best[KM];
  const int64_t row = blockIdx.x;
  const int n = nvs * KM;
  const uint64_t* pr = part + row * int64_t(n);
  TopList<KM> L;
  L.clear();
  for (int i0 = threadIdx.x; i0 < n; i0 += kBatch * NT) {
    uint64_t v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) v[j] = pr[min(i0 + j * NT, n - 1)];
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (i0 + j * NT < n) L.insert(v[j]);
  }
  block_merge<KM, NW>(L, s_keys, s_best);
  if (threadIdx.x == 0)
    for (int r = 0; r < k; ++r) put_dev(&ids_out[row * k + r], int32_t(key_id(s_best[r])));
  if (tail.mode == TAIL_NONE) return;
  const int b = int(row / tree.T);
  uint32_t* seq_cnt = reinterpret_cast<uint32_t*>(ws + kSeqCntOff);
  if (!last_block_arrives(seq_cnt + b, uint32_t(tree.T))) return;
  __shared__ TailShared S;
  const int32_t* topk_b = ids_out + int64_t(b) * tree.T * k;
  int32_t* tok_b = tail.tree_tok + int64_t(b) * tree.T;
  if (tail.m_is64)
    seq_tail<int64_t, 8, 512, true, false>(S, tree, b, k, V, topk_b, tok_b, tail, ws, nullptr, nullptr, 1);
  else
    seq_tail<int32_t, 8, 512, true, false>(S, tree, b, k, V, topk_b, tok_b, tail, ws, nullptr, nullptr, 1);
}

hipError_t launch_lmhead_merge(const TreeDev& tree, int64_t rows, const uint64_t* part, int32_t nvs,
                               int64_t V, int32_t k, int32_t* ids, const TailArgs& tail,
                               uint8_t* ws, hipStream_t s) {
  prof_begin(s, TR_KERNEL_LMHEAD_MERGE);
  hipLaunchKernelGGL(lmhead_merge_kernel, dim3(unsigned(rows)), dim3(512), 0, s, part, nvs, V, k,
                     ids, ws, tree, tail);
  prof_end(s);
  return hipGetLastError();
}

// The segment lists of every row of sequence b meet here, one block per
// sequence, which then runs the step's tail (greedy steps and updates after
// topk_kernel with defer set).  The sequence's T x segs x KM keys (at most
// kSeqKeys, segs <= kSeqSegs) come into LDS in one pass; then one thread
// per row merges the row's segs descending lists: the largest of the lists'
// heads is the next rank, and that list's next key (one LDS read) replaces
// its head.
constexpr int kSeqKeys = 4096;
constexpr int kSeqSegs = 8;
template <int KM, typename MT>
__global__ __launch_bounds__(512) void topk_seq_kernel(const uint64_t* __restrict__ part,
                                                       int32_t segs, int64_t V, int32_t k,
                                                       int32_t* __restrict__ ids_out, uint8_t* ws,
                                                       TreeDev tree, TailArgs tail) {
  constexpr int NT = 512, NL = kSeqKeys / (2 * NT);  // pair loads per thread
  __shared__ __attribute__((aligned(16))) uint64_t s_keys[kSeqKeys];
  const int b = int(blockIdx.x);
  const int tid = threadIdx.x;
  const int nk = segs * KM;                          // keys per row
  const int total = tree.T * nk;                     // <= kSeqKeys (the launch checks)
  const uint64_t* ps = part + int64_t(b) * total;
  u64x2 x[NL];
#pragma unroll
  for (int q = 0; q < NL; ++q) {                     // nk is even: pairs stay in range
    const int i = 2 * (tid + q * NT);
    if (i < total) x[q] = *reinterpret_cast<const u64x2*>(ps + i);
  }
#pragma unroll
  for (int q = 0; q < NL; ++q) {
    const int i = 2 * (tid + q * NT);
    if (i < total) *reinterpret_cast<u64x2*>(s_keys + i) = x[q];
  }
  __syncthreads();
  for (int n = tid; n < tree.T; n += NT) {
    const uint64_t* pr = s_keys + n * nk;
    uint64_t hd[kSeqSegs];
#pragma unroll
    for (int l = 0; l < kSeqSegs; ++l) hd[l] = l < segs ? pr[l * KM] : 0ull;
    uint32_t pos = 0;                                // 4 bits per list: its head's index
    const int64_t row = int64_t(b) * tree.T + n;
#pragma unroll
    for (int r = 0; r < KM; ++r) {
      uint64_t m = hd[0];
      int ml = 0;
#pragma unroll
      for (int l = 1; l < kSeqSegs; ++l)
        if (hd[l] > m) {
          m = hd[l];
          ml = l;
        }
      if (r < k) put_dev(&ids_out[row * k + r], int32_t(key_id(m)));
      const uint32_t nx = ((pos >> (4 * ml)) & 15u) + 1u;
      pos += 1u << (4 * ml);
      const uint64_t nh = nx < uint32_t(KM) ? pr[ml * KM + int(nx)] : 0ull;
#pragma unroll
      for (int l = 0; l < kSeqSegs; ++l) hd[l] = l == ml ? nh : hd[l];
    }
  }
  __builtin_amdgcn_s_waitcnt(0);                     // the ids' device-scope stores completed
  __syncthreads();
  __shared__ TailShared S;
  const int32_t* topk_b = ids_out + int64_t(b) * tree.T * k;
  int32_t* tok_b = tail.tree_tok + int64_t(b) * tree.T;
  seq_tail<MT, KM, NT, true, false>(S, tree, b, k, V, topk_b, tok_b, tail, ws, nullptr, nullptr, segs);
}

hipError_t launch_topk(const TreeDev& tree, int32_t B, const void* logits, int l_is_bf16, int64_t V,
                       int32_t k, int32_t* topk_ids, const TailArgs& tail, uint8_t* ws,
                       const TopkPlan& plan, hipStream_t s) {
  dim3 grid(plan.segs, unsigned(plan.rows));
  uint64_t* part = reinterpret_cast<uint64_t*>(ws + plan.part_off);
  uint64_t* stat = reinterpret_cast<uint64_t*>(ws + plan.stat_off);
  // greedy steps and updates with several segments per row: the rows'
  // segments meet in a second launch, one block per sequence
  const int defer = !tail.sample && plan.segs > 1 && tail.mode != TAIL_NONE &&
                    int64_t(B) * tree.T == plan.rows &&
                    int64_t(tree.T) * plan.segs * plan.kmax <= kSeqKeys && plan.segs <= kSeqSegs ? 1 : 0;
#define TR_TOPK(BF, KMV, NTV, NVV, SMP)                                                         \
  hipLaunchKernelGGL((topk_kernel<BF, KMV, NTV, NVV, SMP>), grid, dim3(NTV), 0, s, logits, V,   \
                     k, plan.segs, plan.seg_len, topk_ids, part, stat, ws, tree, tail, defer)
#define TR_TOPK_NT(BF, KMV)                                                 \
  do {                                                                      \
    if (tail.sample) {                                                      \
      if (plan.threads == 1024) TR_TOPK(BF, KMV, 1024, 4, true);            \
      else TR_TOPK(BF, KMV, 256, 16, true);                                 \
    } else {                                                                \
      if (plan.threads == 1024) TR_TOPK(BF, KMV, 1024, 4, false);           \
      else TR_TOPK(BF, KMV, 256, 16, false);                                \
    }                                                                       \
  } while (0)
  prof_begin(s, TR_KERNEL_TOPK);
  if (l_is_bf16) {
    if (plan.kmax == 8) TR_TOPK_NT(true, 8); else TR_TOPK_NT(true, 16);
  } else {
    if (plan.kmax == 8) TR_TOPK_NT(false, 8); else TR_TOPK_NT(false, 16);
  }
  if (defer) {
#define TR_SEQ(KMV, MTV)                                                                        \
  hipLaunchKernelGGL((topk_seq_kernel<KMV, MTV>), dim3(unsigned(B)), dim3(512), 0, s, part,     \
                     plan.segs, V, k, topk_ids, ws, tree, tail)
    if (plan.kmax == 8) {
      if (tail.m_is64) TR_SEQ(8, int64_t); else TR_SEQ(8, int32_t);
    } else {
      if (tail.m_is64) TR_SEQ(16, int64_t); else TR_SEQ(16, int32_t);
    }
#undef TR_SEQ
  }
  prof_end(s);
#undef TR_TOPK_NT
#undef TR_TOPK
  return hipGetLastError();
}

}  // namespace tr
