// Tree attention for the merged draft sequence.
//
// Every tree node attends to the whole prefix and to its own ancestors
// (itself included), never to a sibling branch ("Token Recycling" summary,
// Method, third module; walk-through, workflow step 3).  Per (sequence, kv
// head) the query rows are the (node, query head) pairs of that kv head; the
// keys are the prefix followed by the tree nodes, and a tree key is visible to
// a row exactly when it lies in the row's ancestor set.
//
// bf16 path: one pass over the keys with matrix cores, then a merge.
//  * The keys of every (sequence, kv head) unit are cut into 64-key
//    sub-blocks, the prefix's first and then ceil(T / 64) sub-blocks of tree
//    nodes, each row masked to its ancestor set there.  The flat list of all
//    units' sub-blocks is cut into equal contiguous ranges, one per block, and
//    the blocks stay resident (one per CU), so every CU does the same amount
//    of work whatever the prefix lengths.  The cut is computed on the device
//    from the prefix lengths at every call.
//  * A unit's query rows are split into equal row tiles of at most sixteen
//    16-row strips; every tile has its own set of blocks ("lane"), and the
//    blocks of the lanes that read the same keys at the same time share an XCD
//    (and its L2).
//  * A unit that lies wholly inside one block's range is finished there and
//    written out.  A unit cut by range boundaries leaves one (m, l, O) partial
//    per block; the merge kernel combines them in block order.
//  * Inside a block the keys and values stream HBM -> LDS by LDS DMA through a
//    four-slot ring, with one barrier per two slots; each wave holds one or two 16-row query strips and
//    computes S^T = K Q^T and O^T = V^T P^T with v_mfma_f32_16x16x32_bf16, so
//    a lane's output column is its query row and the softmax statistics stay
//    in the lane.  K sits in LDS as [key][d] (16-byte chunks XOR-swizzled by
//    row); V also as [key][d], read with the transposed LDS read
//    ds_read_b64_tr_b16, which delivers the V^T operand directly.
//
// fp32 path (the small fp32 workload): split-K prefix chunks on
// v_mfma_f32_16x16x4_f32, the tree keys merged in the combine pass together
// with the chunk partials.
#include "dev_common.h"

namespace tr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kSub = 64;          // fp32 chunk boundaries are multiples of this many keys
constexpr int kWaves = 8;         // waves per bf16 prefix block
constexpr int kSpw = 2;           // 16-row strips per wave (fp32 kernel)
constexpr int kRowsPerTile = 4 * kSpw * 16;   // fp32 kernel: 4 waves
constexpr int kTileStrips = 16;   // bf16: strips per row tile (8 waves x 2)
constexpr int kBlocks = 256;      // bf16: resident blocks (one per CU)
constexpr size_t kLdsBytes = 160 * 1024;           // LDS of a CU (gfx950)
// static LDS of the bf16 prefix kernel (ring 8 x 16 KB, ancestor sets
// 256 x 16 B, wave sums) and a margin
constexpr size_t kAttnStaticLds = 8 * 16384 + 256 * 16 + 32 + 1024;
constexpr float kLog2e = 1.4426950408889634f;

// Cost of one 64-key sub-block for a bf16 row tile of ns strips, in units
// of ~0.1 strip-times: wave w holds strips w and w + 8 (w + 4 when ns <= 8,
// waves 4..7 then only stream keys) and runs on SIMD w % 4, so SIMD s
// carries strips s, s+4, s+8, s+12 (matrix and vector work of a strip: 10);
// every computing wave reads the whole K and V sub-block from LDS (3 on the
// CU's LDS port).  The larger of the two bounds the step.
static int tile_cost(int ns) {
  const int simd = (ns + 3) / 4;
  const int waves = ns > 8 ? 8 : (ns < 4 ? ns : 4);
  return 10 * simd > 3 * waves ? 10 * simd : 3 * waves;
}

AttnPlan plan_attn(int32_t T, int32_t B, int32_t Hq, int32_t Hkv, int64_t cap, int is_bf16) {
  AttnPlan p{};
  p.G = Hq / Hkv;
  p.R = T * p.G;
  if (is_bf16) {
    // row tiles: the fewest that minimise tiles x per-tile step cost, the
    // time of the pass with every tile's lane running side by side
    const int S = (p.R + 15) / 16;
    int best = 0, cost = 0;
    for (int nt = (S + kTileStrips - 1) / kTileStrips; nt <= S; ++nt) {
      const int c = nt * tile_cost((S + nt - 1) / nt);
      if (best == 0 || c < cost) { best = nt; cost = c; }
      if (nt >= kBlocks) break;
    }
    p.nt = best;
    p.S = S;
    p.tstrips = (S + best - 1) / best;
    // blocks per lane: with the lanes' blocks of one index on one XCD, at
    // most 32 per XCD (its CUs), else a block would wait for a whole one
    if (best <= 32) {
      p.xpair = 1;
      p.gl = 8 * (32 / best);
    } else {
      p.xpair = 0;
      p.gl = kBlocks / best > 0 ? kBlocks / best : 1;
    }
    p.grid = best * p.gl;
    // dynamic LDS: the per-sequence scan (2 B + 1 ints, 16-byte padded) and,
    // for 5- or 6-strip tiles when it fits, the key halves' hand-over
    const size_t scan = size_t(2 * B + 1 + 3) / 4 * 16;
    const size_t hand = size_t(2) * 64 * 36 * 4;
    p.split = kAttnStaticLds + scan + hand <= kLdsBytes ? 1 : 0;
    p.lds_dyn = scan + (p.split ? hand : 0);
    p.tree_keys = 1;
    const size_t slots = size_t(best) * 2 * p.gl * p.tstrips * 16;   // 2 partials per block
    size_t off = kDataOff;
    p.o_off = off;                                   // bf16 [nt][2 gl][tstrips*16][128]
    off = align256(off + slots * kHeadDim * 2);
    p.ml_off = off;                                  // float2 [nt][2 gl][tstrips*16]
    off = align256(off + slots * 8);
    p.rec_off = off;                                 // int4 [nt][gl] merge records
    off = align256(off + size_t(best) * p.gl * 16);
    p.end = off;
    return p;
  }
  p.spw = kSpw;
  p.tile_rows = kRowsPerTile;
  p.row_tiles = (p.R + p.tile_rows - 1) / p.tile_rows;
  int64_t base = int64_t(B) * Hkv * p.row_tiles;
  // at most one block per CU; the combine merges the chunks and the tree keys
  int64_t chunks = kBlocks / base;
  int64_t by_cap = (cap + kSub - 1) / kSub;
  if (chunks > by_cap) chunks = by_cap;
  if (chunks > 64) chunks = 64;
  if (chunks < 1) chunks = 1;
  p.chunks = int32_t(chunks);
  p.tree_keys = 0;
  const size_t rpad = size_t(p.row_tiles) * p.tile_rows;
  const size_t units = size_t(B) * Hkv * p.chunks * rpad;
  size_t off = kDataOff;
  p.o_off = off;                                    // fp32 partials
  off = align256(off + units * kHeadDim * 4);
  p.ml_off = off;
  off = align256(off + units * 8);
  p.end = off;
  return p;
}

__device__ __forceinline__ int chunk_len(int P, int chunks, int sub) {
  int cs = (P + chunks - 1) / chunks;
  return (cs + sub - 1) / sub * sub;
}

// prefix_len outside [0, cap] is a caller error: clamp it (so no read
// leaves the cache) and raise the sticky flag once per sequence.
__device__ __forceinline__ int clamp_prefix(int P, int64_t cap, uint8_t* ws, bool report) {
  if (P < 0 || int64_t(P) > cap) {
    if (report) set_flag(ws, TR_FLAG_BAD_PREFIX);
    P = P < 0 ? 0 : int(cap);
  }
  return P;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A chunk with no keys for its sequence still marks its rows' partials as
// empty (weight 0), so the merge can read every chunk without knowing the
// prefix length.
__device__ __forceinline__ void mark_empty(float2* part_ml, int64_t unit0, int rows) {
  for (int r = threadIdx.x; r < rows; r += blockDim.x) part_ml[unit0 + r] = make_float2(-INFINITY, 0.f);
}

// ---------------------------------------------------------------- bf16 prefix
// 8 waves.  The keys and values of a block's range stream HBM -> LDS through
// the LDS DMA (global_load_lds_dwordx4) in 64-key sub-blocks (16 KB of K and
// 16 KB of V) into a ring of four LDS slots, three sub-blocks in flight ahead
// of the one in use; nothing passes through registers and nothing is
// restaged.
//  * K is stored [key][d] with the 16-byte column chunk c of row r at
//    position c ^ (r & 15): the S^T = K Q^T operand reads (16 rows, one
//    chunk) are conflict-free.
//  * V is stored [key][d] with chunk c of row r at c ^ 2 (r & 7), and the
//    O^T = V^T P^T operand is read with ds_read_b64_tr_b16: within each
//    16-lane group, lane i receives element e from the address of lane
//    4 e + i / 4 plus i % 4 elements, so lanes pointing at rows k0 ..
//    k0+3 (four lanes a row, 4 d apart) deliver to lane i the four keys
//    k0 .. k0+3 of column d0 + i: the V^T layout the product needs.
// The key order inside the second product's K dimension is permuted
// consistently on both operands (k-index 8 g + m is key 4 g + m of the
// first 16-key tile of the 32-key block for m < 4, of the second for
// m >= 4) so that the probabilities need no cross-lane moves.
// Waits are explicit: a workgroup fence would wait for every DMA in flight,
// so the loop synchronises with a bare barrier after its own vmcnt wait, and
// each ring slot is its own LDS array named statically (one array would make
// the compiler wait for DMAs into the other slots before every read).  One
// barrier serves two 64-key steps: at an even step both of the pair's
// sub-blocks have landed, and the two slots the previous pair read are
// refilled with the next pair, which has two to three steps to land.
constexpr int kSB = 64;                   // keys per sub-block
constexpr float kLazy = 8.f;              // lazy rescaling threshold (log2 units)
constexpr int kRingSlots = 4;
constexpr int kSubBytes = kSB * kHeadDim * 2;   // 16 KB
// Transposed LDS read (ds_read_b64_tr_b16) of the 8 bytes at LDS address
// p: four 16-bit values, delivered across each 16-lane group as described
// above.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p));
}
// LDS DMA of 16 bytes per lane: lane l's src lands at lds_base + 16 l
// (lds_base wave-uniform).  These gfx950 builtins sit in plain device
// functions: inside a kernel template the host compilation pass cannot
// instantiate them and drops the kernel's launch stub without a word.
__device__ __forceinline__ void lds_dma16(const void* src, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
}
// Sum of two bf16 values added to c (v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float add_bf16x2(bf16x2 p, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(p, bf16x2{(__bf16)1.f, (__bf16)1.f}, c, false);
}
// Page id of the sub-block of sequence b that starts at key kb, read
// through the scalar cache (a wave-uniform address); an id outside the pool
// reads page 0 and raises the sticky flag.
__device__ __forceinline__ int32_t page_id(const PagedArgs& pg, int b, int kb, uint8_t* ws) {
  typedef const __attribute__((address_space(4))) int32_t* cptr;
  const cptr tb = (cptr)pg.table;
  int32_t id = tb[int64_t(b) * pg.max_pages + (kb >> pg.ps_log2)];
  if (id < 0 || int64_t(id) >= pg.num_pages) {
    set_flag(ws, TR_FLAG_BAD_PAGE);
    id = 0;
  }
  return id;
}

template <int N>
struct IntC {
  static constexpr int value = N;
};

// Rows of row tile t: strips [st0, st0 + ns) of the unit's S strips
// (tiles as equal as whole strips allow, the larger ones first).
__device__ __forceinline__ void tile_rows_of(int t, int nt, int S, int R, int& row0, int& rows) {
  const int Sb = S / nt, Sr = S - Sb * nt;
  const int ns = Sb + (t < Sr ? 1 : 0);
  row0 = (t * Sb + min(t, Sr)) * 16;
  rows = min(ns * 16, R - row0);
}
// The block of a lane whose range [beg(i), beg(i+1)), beg(i) =
// floor(i W / nb), holds flat position x.
__device__ __forceinline__ int block_of(int64_t x, int64_t W, int nb) {
  return int(((x + 1) * nb - 1) / W);
}

// Position of the walk over a lane's flat (sequence, kv head, sub-block)
// order: sub-block s of unit (b, kvh), whose sequence has n sub-blocks and
// prefix length P.  All fields are wave-uniform.
struct Walk {
  int b, kvh, s, n, P;
};

// Merge record of a block: the unit whose partials it gathers (the block
// after the one a cut unit starts in): {b * Hkv + kvh, first block, blocks,
// 1 if the unit starts inside the first block (its partial is that
// block's second)}; x = -1: none.
// (q is not __restrict__: loads through a const __restrict__ pointer may be
// moved across the explicit waits below, which must cover them.)
template <bool PAGED>
__global__ __launch_bounds__(512) void attn_prefix_bf16(
    const uint16_t* q, const uint16_t* kc, const uint16_t* vc, const uint16_t* kt,
    const uint16_t* vt, TreeDev tree, int64_t cap, const int32_t* __restrict__ prefix_len, int B,
    int Hq, int Hkv, int G, int R, int nt, int S, int tstrips, int gl, int xpair, int split,
    float sl2, uint16_t* __restrict__ part_o, float2* __restrict__ part_ml,
    int4* __restrict__ rec, uint16_t* __restrict__ out, uint8_t* ws, PagedArgs pg) {
  const int T = tree.T;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, g = lane >> 4;
  // Blocks are dealt to the 8 XCDs round-robin by block index.  With xpair,
  // block (lane t, index i) gets grid slot 8 (nt (i / 8) + t) + i % 8, so the
  // lanes' blocks of the same index, which read the same keys at the same
  // time, run on the same XCD and share its L2 (gl = 8 floor(32 / nt): no
  // XCD gets more than its 32 CUs); else slot i nt + t.
  int t, bil;
  if (xpair) {
    const int xcd = blockIdx.x & 7, qd = blockIdx.x >> 3;
    t = qd % nt;
    bil = (qd / nt) * 8 + xcd;
  } else {
    t = blockIdx.x % nt;
    bil = blockIdx.x / nt;
  }
  if (bil >= gl) return;
  int trow0, trows;
  tile_rows_of(t, nt, S, R, trow0, trows);
  const int ns = (trows + 15) / 16;                 // strips of this tile
  const int ntt = (T + kSB - 1) / kSB;              // tree sub-blocks of a unit

  // ---- sub-blocks per sequence and their running sum (every block does
  // the same scan, so the cut needs no other launch)
  // dynamic LDS: s_cb [B + 1] sub-blocks of sequences < b, s_p [B] clamped
  // prefix lengths, then (split) the key halves' hand-over buffer
  extern __shared__ __attribute__((aligned(16))) int32_t s_dyn[];
  int32_t* s_cb = s_dyn;
  int32_t* s_p = s_dyn + B + 1;
  float* s_mo = reinterpret_cast<float*>(s_dyn + ((2 * B + 1 + 3) & ~3));   // [2][64][36]
  __shared__ int32_t s_wsum[kWaves];
  __shared__ uint64_t s_anc[kTileStrips * 16][2];   // ancestor sets of the tile's rows
  if (tid < ns * 16) {
    const int n = min(trow0 + tid, R - 1) / G;
    s_anc[tid][0] = tree.anc[n][0];
    s_anc[tid][1] = tree.anc[n][1];
  }
  int carry = 0;
  bool same = true;                                 // every sequence has as many sub-blocks
  int n_first;                                      // sub-blocks of sequence 0
  if (B <= 64) {
    // one wave scans; one barrier
    if (w == 0) {
      int nsub = 0;
      if (lane < B) {
        // prefix_len outside [0, cap] is a caller error: clamped (no read
        // leaves the cache), flagged once
        const int P = clamp_prefix(prefix_len[lane], cap, ws, blockIdx.x == 0);
        s_p[lane] = P;
        nsub = (P + kSB - 1) / kSB + ntt;
      }
      const int x = int(wave_incl_scan(uint32_t(nsub)));
      if (lane < B) s_cb[lane] = x - nsub;
      if (lane == B - 1) s_cb[B] = x;
      const int n0 = __builtin_amdgcn_readfirstlane(nsub);
      s_wsum[0] = __all(lane >= B || nsub == n0) ? 1 : 0;
    }
    __syncthreads();
    carry = s_cb[B];
    n_first = s_cb[1];
    same = s_wsum[0] != 0;
  } else {
    n_first = (clamp_prefix(prefix_len[0], cap, ws, false) + kSB - 1) / kSB + ntt;
    for (int base = 0; base < B; base += 64 * kWaves) {
      const int bb = base + tid;
      int nsub = 0;
      if (bb < B) {
        const int P = clamp_prefix(prefix_len[bb], cap, ws, blockIdx.x == 0);
        s_p[bb] = P;
        nsub = (P + kSB - 1) / kSB + ntt;
      }
      const int x = int(wave_incl_scan(uint32_t(nsub)));
      if (lane == 63) s_wsum[w] = x;
      __syncthreads();
      int off = carry, tot = 0;
#pragma unroll
      for (int i = 0; i < kWaves; ++i) {
        const int v = s_wsum[i];
        off += i < w ? v : 0;
        tot += v;
      }
      if (bb < B) s_cb[bb] = off + x - nsub;
      carry += tot;
      same = same && (bb >= B || nsub == n_first);
      __syncthreads();
    }
    if (tid == 0) s_cb[B] = carry;
    same = __syncthreads_and(same);
  }

  // ---- this block's range of the lane's W sub-blocks (no block empty).
  // Units of equal length, no more of them than blocks: as many blocks as
  // fit whole per unit, so no block crosses from one unit into the next.
  // Merge records are kept per unit when units are no more than blocks
  // (each cut unit's record at its index, a whole unit's cleared by the
  // block that finishes it), else per block.
  const int64_t W = int64_t(carry) * Hkv;
  const int U = B * Hkv;
  const bool byunit = U <= gl;
  const int nb = same && byunit ? U * min(gl / U, n_first) : int(min<int64_t>(gl, W));
  if (bil >= nb) {
    if (tid == 0 && !byunit) rec[t * gl + bil] = make_int4(-1, 0, 0, 0);
    return;
  }
  const int64_t g0 = int64_t(bil) * W / nb, g1 = int64_t(bil + 1) * W / nb;
  const int nj = int(g1 - g0);
  // the unit holding g0: the last sequence whose first sub-block is <= g0
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (int64_t(s_cb[mid]) * Hkv <= g0) lo = mid; else hi = mid - 1;
  }
  Walk w0;
  w0.b = __builtin_amdgcn_readfirstlane(lo);
  w0.n = __builtin_amdgcn_readfirstlane(s_cb[w0.b + 1] - s_cb[w0.b]);
  w0.P = __builtin_amdgcn_readfirstlane(s_p[w0.b]);
  {
    const int64_t rel = g0 - int64_t(s_cb[w0.b]) * Hkv;
    w0.kvh = __builtin_amdgcn_readfirstlane(int(rel / w0.n));
    w0.s = __builtin_amdgcn_readfirstlane(int(rel - int64_t(w0.kvh) * w0.n));
  }
  if (tid == 0) {
    // this block merges its first unit when that unit started in the block
    // before it
    int4 r = make_int4(-1, 0, 0, 0);
    const int64_t ustart = g0 - w0.s;
    if (w0.s > 0 && block_of(ustart, W, nb) == bil - 1) {
      const int first = bil - 1;
      const int last = block_of(ustart + w0.n - 1, W, nb);
      r = make_int4(w0.b * Hkv + w0.kvh, first, last - first + 1,
                    ustart > int64_t(first) * W / nb ? 1 : 0);
    }
    if (!byunit) rec[t * gl + bil] = r;
    else if (r.x >= 0) rec[t * gl + r.x] = r;
  }
  auto advance = [&](Walk& it) {
    if (++it.s == it.n) {
      it.s = 0;
      if (++it.kvh == Hkv) {
        it.kvh = 0;
        ++it.b;
        const int bb = min(it.b, B - 1);
        it.n = __builtin_amdgcn_readfirstlane(s_cb[bb + 1] - s_cb[bb]);
        it.P = __builtin_amdgcn_readfirstlane(s_p[bb]);
      }
    }
  };

  // ---- the wave's query strips.  Tiles of more than 8 strips: wave w holds
  // strips w and w + 8.  5 or 6 strips with the key split: waves 0..3 hold
  // strip w; waves 4..7 hold strip 4 + (w & 1) over key half (w >> 1) & 1
  // (keys 32 h .. 32 h + 31 of every sub-block), so each SIMD (wave w runs on
  // SIMD w % 4) carries 1.5 strips rather than two of them carrying 2; the
  // halves merge through LDS when a unit ends.  Else wave w < 4 holds
  // strips w and w + 4 and waves 4..7 only stream keys.
  split = split && (ns == 5 || ns == 6);            // LDS for the hand-over fits
  const bool hw = split && w >= 4;                  // a half-key wave
  const int kh = hw ? (w >> 1) & 1 : 0;             // its key half
  int stride, strip0, nstr;
  if (ns > 8) {
    stride = 8;
    strip0 = w;
    nstr = w + 8 < ns ? 2 : 1;
  } else if (split) {
    stride = 0;
    strip0 = w < 4 ? w : 4 + (w & 1);
    nstr = strip0 < ns ? 1 : 0;
  } else {
    stride = 4;
    strip0 = w;
    nstr = w < 4 ? (w + 4 < ns ? 2 : (w < ns ? 1 : 0)) : 0;
  }

  __shared__ __attribute__((aligned(16))) uint8_t Ks0[kSubBytes];
  __shared__ __attribute__((aligned(16))) uint8_t Ks1[kSubBytes];
  __shared__ __attribute__((aligned(16))) uint8_t Ks2[kSubBytes];
  __shared__ __attribute__((aligned(16))) uint8_t Ks3[kSubBytes];
  __shared__ __attribute__((aligned(16))) uint8_t Vs0[kSubBytes];
  __shared__ __attribute__((aligned(16))) uint8_t Vs1[kSubBytes];
  __shared__ __attribute__((aligned(16))) uint8_t Vs2[kSubBytes];
  __shared__ __attribute__((aligned(16))) uint8_t Vs3[kSubBytes];
  auto kslot = [&](int i) -> uint8_t* { return i == 0 ? Ks0 : i == 1 ? Ks1 : i == 2 ? Ks2 : Ks3; };
  auto vslot = [&](int i) -> uint8_t* { return i == 0 ? Vs0 : i == 1 ? Vs1 : i == 2 ? Vs2 : Vs3; };

  // Sub-block `it` into ring slot sl: 1024 16-byte slots of K and of V, two
  // of each per thread (wave w, pass q: slots (8 q + w) * 64 + lane).
  // Prefix rows past P repeat row P-1 (finite data the key mask gives
  // probability 0); a tree sub-block reads node rows of kt / vt
  // ([B][T][Hkv][d]; nodes past T repeat the last, masked like keys past P).
  // PAGED: kc / vc are page pools [num_pages][Hkv][page_size][d]; pid is the
  // page of the sub-block's rows (a 64-key sub-block never straddles pages).
  // A full prefix sub-block (the common case) is a wave-uniform base plus
  // each lane's fixed byte offset (row r = p / 16 of the sub-block, its
  // swizzled 16-byte chunk), computed once here; the second pass is 32 rows
  // on with the same swizzle, 8 KB further.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  uint32_t offk, offv;
  {
    const int r = (w * 64 + lane) >> 4, pos = lane & 15;
    offk = uint32_t(r * 256 + ((pos ^ (r & 15)) << 4));
    offv = uint32_t(r * 256 + ((pos ^ ((r & 7) << 1)) << 4));
  }
  auto dma = [&](const Walk& it, int pid, int sl) {
    const int ntp = (it.P + kSB - 1) / kSB;
    const int kb = it.s * kSB;
    if (it.s < ntp) {
      const uint16_t* kp;
      const uint16_t* vp;
      int row_base = 0;
      if constexpr (PAGED) {
        const int64_t pool_off = (int64_t(pid) * Hkv + it.kvh) * pg.page_size * kHeadDim;
        kp = kc + pool_off;
        vp = vc + pool_off;
        row_base = (kb >> pg.ps_log2) << pg.ps_log2;   // first position of the page
      } else {
        const int64_t head_off = (int64_t(it.b) * Hkv + it.kvh) * cap * kHeadDim;
        kp = kc + head_off;
        vp = vc + head_off;
      }
      if (kb + kSB <= it.P) {
        const uint8_t* kbase = reinterpret_cast<const uint8_t*>(kp + int64_t(kb - row_base) * kHeadDim);
        const uint8_t* vbase = reinterpret_cast<const uint8_t*>(vp + int64_t(kb - row_base) * kHeadDim);
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          const int base = (q2 * kWaves + wu) * 64;    // wave-uniform first slot
          lds_dma16(kbase + q2 * 8192 + offk, kslot(sl) + base * 16);
          lds_dma16(vbase + q2 * 8192 + offv, vslot(sl) + base * 16);
        }
      } else {
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          const int base = (q2 * kWaves + wu) * 64;
          const int p = base + lane;
          const int r = p >> 4, pos = p & 15;
          const int64_t row = min(kb + r, it.P - 1) - row_base;
          const int ck = pos ^ (r & 15), cv = pos ^ ((r & 7) << 1);
          lds_dma16(kp + row * kHeadDim + ck * 8, kslot(sl) + base * 16);
          lds_dma16(vp + row * kHeadDim + cv * 8, vslot(sl) + base * 16);
        }
      }
    } else {
      const int nb0 = (it.s - ntp) * kSB;
      const int64_t node_stride = int64_t(Hkv) * kHeadDim;
      const uint16_t* kt_b = kt + (int64_t(it.b) * T * Hkv + it.kvh) * kHeadDim;
      const uint16_t* vt_b = vt + (int64_t(it.b) * T * Hkv + it.kvh) * kHeadDim;
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const int base = (q2 * kWaves + wu) * 64;
        const int p = base + lane;
        const int r = p >> 4, pos = p & 15;
        const int64_t node = min(nb0 + r, T - 1);
        const int ck = pos ^ (r & 15), cv = pos ^ ((r & 7) << 1);
        lds_dma16(kt_b + node * node_stride + ck * 8, kslot(sl) + base * 16);
        lds_dma16(vt_b + node * node_stride + cv * 8, vslot(sl) + base * 16);
      }
    }
    asm volatile("" ::: "memory");
  };
  // page of a prefix sub-block (0 for tree sub-blocks and unpaged caches)
  auto page = [&](const Walk& it) -> int {
    if constexpr (PAGED) {
      if (it.b < B && it.s * kSB < it.P) return __builtin_amdgcn_readfirstlane(page_id(pg, it.b, it.s * kSB, ws));
    }
    return 0;
  };

  // The compute for waves holding NS strips (1 or 2); waves without a strip
  // run it with `active` false and only stream keys.
  auto body = [&](auto ns_c) {
    constexpr int NS = decltype(ns_c)::value;
    const bool active = nstr > 0;
    int srow[NS];                                   // the strips' first rows in the tile
#pragma unroll
    for (int s = 0; s < NS; ++s) srow[s] = (strip0 + s * stride) * 16;

    bf16x8 qb[NS][4];
    floatx4 acc[NS][8];
    float mrow[NS], lrow[NS], moff[NS], thr[NS];
    // queries of the unit (b, kvh): rows past the tile read any row, never stored
    auto qload = [&](int b, int kvh) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int r = trow0 + min(srow[s] + li, trows - 1);
        const int n = r / G, gq = r - n * G;
        const uint16_t* qp = q + ((int64_t(b) * T + n) * Hq + kvh * G + gq) * kHeadDim;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          qb[s][ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32 + g * 8);
      }
    };
    auto reset = [&]() {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        mrow[s] = -INFINITY;
        moff[s] = 0.f;
        thr[s] = -INFINITY;
        lrow[s] = 0.f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acc[s][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    };
    // S^T = K Q^T for NTL 16-key tiles from tile tb on (sacc[s][t] holds
    // tile tb + t); operands read two tiles ahead of the products
    auto qk = [&](const uint8_t* Ks, floatx4 (&sacc)[NS][4], auto ntl, int tb) {
      constexpr int NTL = decltype(ntl)::value;
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int t4 = 0; t4 < NTL; ++t4) sacc[s][t4] = floatx4{0.f, 0.f, 0.f, 0.f};
      constexpr int KT = 2;
#pragma unroll
      for (int t0 = 0; t0 < NTL; t0 += KT) {
        bf16x8 ka[KT][4];
#pragma unroll
        for (int tt = 0; tt < KT; ++tt)
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            ka[tt][ks] = *reinterpret_cast<const bf16x8*>(
                Ks + ((tb + t0 + tt) * 16 + li) * 256 + (((4 * ks + g) ^ li) << 4));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int tt = 0; tt < KT; ++tt)
#pragma unroll
            for (int s = 0; s < NS; ++s)
              sacc[s][t0 + tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[tt][ks], qb[s][ks], sacc[s][t0 + tt], 0, 0, 0);
      }
    };
    // V^T operands (transposed LDS reads), read while the softmax runs:
    // rows kr .. kr+3 with kr = 32 pp + 4 g (+16 for the second half),
    // lane li at row kr + li / 4, columns 16 dt + 4 (li % 4) .. +3.  NPP
    // 32-key blocks from block pb0 on (va[i][p] holds block pb0 + p).
    constexpr int VG = 2;
    bf16x8 va[VG][2];
    auto read_v = [&](const uint8_t* Vs, int dt0, auto npp, int pb0) {
      constexpr int NPP = decltype(npp)::value;
#pragma unroll
      for (int i = 0; i < VG; ++i) {
        const int dt = dt0 + i;
        const int cch = 2 * dt + ((li >> 1) & 1), half = (li & 1) * 8;
#pragma unroll
        for (int pp = 0; pp < NPP; ++pp) {
          uint32_t u[4];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int row = 32 * (pb0 + pp) + 16 * hh + 4 * g + (li >> 2);
            const uint8_t* addr = Vs + row * 256 + ((cch ^ ((row & 7) << 1)) << 4) + half;
            const u32x2 r2 = lds_read_tr16(addr);
            u[2 * hh] = r2[0];
            u[2 * hh + 1] = r2[1];
          }
          va[i][pp] = __builtin_bit_cast(bf16x8, u32x4{u[0], u[1], u[2], u[3]});
        }
      }
    };
    // Sub-block s of a unit with prefix length P: prefix keys past P (a
    // ragged last sub-block) get score -inf; in a tree sub-block a row sees
    // only its ancestor set.
    auto mask = [&](floatx4 (&sacc)[NS][4], int s, int P, auto ntl, int tb) {
      constexpr int NTL = decltype(ntl)::value;
      const int ntp = (P + kSB - 1) / kSB;
      if (s < ntp) {
        const int nk = P - s * kSB;
        if (nk < kSB) {
          const int nrel = nk - 4 * g - 16 * tb;      // keys t*16 + i of the lane's tiles
#pragma unroll
          for (int ss = 0; ss < NS; ++ss)
#pragma unroll
            for (int t4 = 0; t4 < NTL; ++t4)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (t4 * 16 + i >= nrel) sacc[ss][t4][i] = -INFINITY;
        }
      } else {
        const int hi = s - ntp > 0 ? 1 : 0;           // nodes 64 .. 127
#pragma unroll
        for (int ss = 0; ss < NS; ++ss) {
          const uint64_t bits = s_anc[srow[ss] + li][hi] >> (4 * g + 16 * tb);
#pragma unroll
          for (int t4 = 0; t4 < NTL; ++t4) {
            const uint32_t nib = uint32_t(bits >> (t4 * 16));   // keys (tb+t4)*16+4g .. +3
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (!((nib >> i) & 1u)) sacc[ss][t4][i] = -INFINITY;
          }
        }
      }
    };
    // Online softmax per query row (the lane's column) on raw scores:
    // scale > 0, so max(scale s) = scale max(s) and p = 2^(s sl2 - m).
    // Lazy rescaling: a row's reference maximum m moves only when a score
    // passes it by more than kLazy (log2 units), so the probabilities stay
    // below 2^kLazy and the accumulators are rarely rescaled; the partial
    // (m, l, O) is consistent for any reference m.  A lane compares its own
    // maximum with the raw-score threshold (m + kLazy) / sl2; only when some
    // lane passes it does the wave reduce the maxima over the column's four
    // lane groups and move m.  l is summed per lane (over its own keys) and
    // over the lane groups when the unit ends; it adds the probabilities as
    // rounded to bf16, the weights the second product uses.
    bf16x8 pb[NS][2];
    auto softmax = [&](const floatx4 (&sacc)[NS][4], auto ntl, bool fresh) {
      constexpr int NTL = decltype(ntl)::value;
      float lm[NS];
      bool pass = false;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float mt[NTL];
#pragma unroll
        for (int t4 = 0; t4 < NTL; ++t4)
          mt[t4] = fmaxf(fmaxf(sacc[s][t4][0], sacc[s][t4][1]), fmaxf(sacc[s][t4][2], sacc[s][t4][3]));
        float m = mt[0];
#pragma unroll
        for (int t4 = 1; t4 < NTL; ++t4) m = fmaxf(m, mt[t4]);
        lm[s] = m;
        pass |= m > thr[s];
      }
      if (__any(pass)) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const float mcand = xmax32(xmax16(lm[s])) * sl2;
          const bool bump = mcand > mrow[s] + kLazy;
          const float mnew = bump ? mcand : mrow[s];
          const float alpha = bump ? fast_exp2(mrow[s] - mnew) : 1.f;
          mrow[s] = mnew;
          // a row that has seen no visible key yet keeps m = -inf: offset 0
          // gives p = 2^-inf = 0 for its masked scores, not NaN
          moff[s] = mnew == -INFINITY ? 0.f : mnew;
          thr[s] = (mnew + kLazy) / sl2;
          lrow[s] *= alpha;
          if (!fresh && __any(bump)) {
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) acc[s][dt] *= alpha;
          }
        }
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        __bf16 ph[4][4];
#pragma unroll
        for (int t4 = 0; t4 < NTL; ++t4)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            ph[t4][i] = (__bf16)fast_exp2(__builtin_fmaf(sacc[s][t4][i], sl2, -moff[s]));
        float ls = lrow[s];
#pragma unroll
        for (int t4 = 0; t4 < NTL; ++t4) {
          ls = add_bf16x2(bf16x2{ph[t4][0], ph[t4][1]}, ls);
          ls = add_bf16x2(bf16x2{ph[t4][2], ph[t4][3]}, ls);
        }
        lrow[s] = ls;
#pragma unroll
        for (int pp = 0; pp < NTL / 2; ++pp)
          pb[s][pp] = bf16x8{ph[2 * pp][0], ph[2 * pp][1], ph[2 * pp][2], ph[2 * pp][3],
                             ph[2 * pp + 1][0], ph[2 * pp + 1][1], ph[2 * pp + 1][2], ph[2 * pp + 1][3]};
      }
    };
    // O^T += V^T P^T over NPP 32-key blocks from pb0 on (va holds dt 0, 1
    // on entry)
    auto pv = [&](const uint8_t* Vs, auto npp, int pb0) {
      constexpr int NPP = decltype(npp)::value;
#pragma unroll
      for (int dt0 = 0; dt0 < 8; dt0 += VG) {
        if (dt0 > 0) {
          read_v(Vs, dt0, npp, pb0);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int pp = 0; pp < NPP; ++pp)
#pragma unroll
          for (int i = 0; i < VG; ++i)
#pragma unroll
            for (int s = 0; s < NS; ++s)
              acc[s][dt0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[i][pp], pb[s][pp], acc[s][dt0 + i], 0, 0, 0);
      }
    };
    // one sub-block: all 64 keys, or (half-key waves) keys 32 kh .. 32 kh + 31:
    // scores and probabilities first, then (after the step's DMA has been
    // issued, while the scores are no longer live) the second product
    auto probs = [&](const uint8_t* Ks, const uint8_t* Vs, int s, int P, bool fresh) {
      floatx4 sc[NS][4];
      if (NS == 2 || !hw) {
        qk(Ks, sc, IntC<4>{}, 0);
        mask(sc, s, P, IntC<4>{}, 0);
        read_v(Vs, 0, IntC<2>{}, 0);
        __builtin_amdgcn_sched_barrier(0);
        softmax(sc, IntC<4>{}, fresh);
      } else {
        qk(Ks, sc, IntC<2>{}, 2 * kh);
        mask(sc, s, P, IntC<2>{}, 2 * kh);
        read_v(Vs, 0, IntC<1>{}, kh);
        __builtin_amdgcn_sched_barrier(0);
        softmax(sc, IntC<2>{}, fresh);
      }
    };
    auto weigh = [&](const uint8_t* Vs) {
      if (NS == 2 || !hw) pv(Vs, IntC<2>{}, 0);
      else pv(Vs, IntC<1>{}, kh);
    };
    // The unit (b, kvh) ends in this block: a unit wholly inside the range
    // is normalised and written out; a cut one leaves its partial in the
    // block's slot (0 for the block's first unit, 1 for its last).  With the
    // key split the second key half first hands (m, l, O) of its strip to
    // the first through LDS (every wave meets the barrier).
    auto finish = [&](int b, int kvh, bool whole, int slot) {
      if (NS == 1 && split) {
        float* mo = s_mo + ((w & 1) * 64 + lane) * 36;
        if (hw && kh == 1 && active) {
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<floatx4*>(mo + 4 * dt) = acc[0][dt];
          mo[32] = mrow[0];
          mo[33] = lrow[0];
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);        // lgkmcnt(0)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (hw && kh == 0 && active) {
          const float m1 = mo[32], l1 = mo[33];
          if (m1 != -INFINITY) {                    // the second half saw a visible key
            if (mrow[0] == -INFINITY) {
              mrow[0] = m1;
              lrow[0] = l1;
#pragma unroll
              for (int dt = 0; dt < 8; ++dt) acc[0][dt] = *reinterpret_cast<const floatx4*>(mo + 4 * dt);
            } else {
              const float mn = fmaxf(mrow[0], m1);
              const float a0 = fast_exp2(mrow[0] - mn), a1 = fast_exp2(m1 - mn);
              lrow[0] = lrow[0] * a0 + l1 * a1;
              mrow[0] = mn;
#pragma unroll
              for (int dt = 0; dt < 8; ++dt)
                acc[0][dt] = acc[0][dt] * a0 + *reinterpret_cast<const floatx4*>(mo + 4 * dt) * a1;
            }
          }
        }
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const float l = xsum32(xsum16(lrow[s]));
        int rt = srow[s] + li;                        // row in the tile
        // (opaque, so the output-address arithmetic of this rare path is not
        // hoisted out of the loop into long-lived registers)
        asm volatile("" : "+v"(rt));
        if (!active || (hw && kh == 1) || rt >= trows) continue;
        if (whole) {
          const float inv = __builtin_amdgcn_rcpf(l);  // 1 ulp: far below the bf16 rounding
          const int r = trow0 + rt;
          const int n = r / G, gq = r - n * G;
          uint16_t* po = out + ((int64_t(b) * T + n) * Hq + kvh * G + gq) * kHeadDim;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
            const u32x2 v = {uint32_t(__builtin_bit_cast(uint16_t, (__bf16)(acc[s][dt][0] * inv))) |
                                 (uint32_t(__builtin_bit_cast(uint16_t, (__bf16)(acc[s][dt][1] * inv))) << 16),
                             uint32_t(__builtin_bit_cast(uint16_t, (__bf16)(acc[s][dt][2] * inv))) |
                                 (uint32_t(__builtin_bit_cast(uint16_t, (__bf16)(acc[s][dt][3] * inv))) << 16)};
            *reinterpret_cast<u32x2*>(po + dt * 16 + 4 * g) = v;
          }
        } else {
          const int64_t unit = (int64_t(t) * 2 * gl + 2 * bil + slot) * (tstrips * 16) + rt;
          uint16_t* po = part_o + unit * kHeadDim;   // bf16: the partial sums round once
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
            const u32x2 v = {uint32_t(__builtin_bit_cast(uint16_t, (__bf16)acc[s][dt][0])) |
                                 (uint32_t(__builtin_bit_cast(uint16_t, (__bf16)acc[s][dt][1])) << 16),
                             uint32_t(__builtin_bit_cast(uint16_t, (__bf16)acc[s][dt][2])) |
                                 (uint32_t(__builtin_bit_cast(uint16_t, (__bf16)acc[s][dt][3])) << 16)};
            *reinterpret_cast<u32x2*>(po + dt * 16 + 4 * g) = v;
          }
          if (g == 0) part_ml[unit] = make_float2(mrow[s], l);
        }
      }
    };

    int pnext = 0;                                  // page of the next sub-block to stream
    Walk wc = w0;                                   // the sub-block being computed
    Walk wd = w0;                                   // the next sub-block to stream
    bool whole = wc.s == 0;                         // the unit starts in this block
    int slot = 0;                                   // the block's first unit: slot 0
    bool fresh = true;
    reset();
    // two sub-blocks in flight before the loop (the pages of the first three looked up at once)
    {
      Walk w1 = wd, w2;
      advance(w1);
      w2 = w1;
      advance(w2);
      const int p0 = page(wd), p1 = nj > 1 ? page(w1) : 0, p2 = nj > 2 ? page(w2) : 0;
      dma(wd, p0, 0);
      if (nj > 1) dma(w1, p1, 1);
      wd = w2;
      pnext = p2;
    }
    // the first unit's queries, then everything landed before the loop (an
    // explicit wait: otherwise the compiler waits for all loads in flight,
    // the ring's DMA included, before every step's products)
    if (active) qload(wc.b, wc.kvh);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070);            // vmcnt(0) lgkmcnt(0)
    asm volatile("" ::: "memory");
    const int nround = (nj + kRingSlots - 1) / kRingSlots * kRingSlots;
    for (int j0 = 0; j0 < nround; j0 += kRingSlots) {
#pragma unroll
      for (int jj = 0; jj < kRingSlots; ++jj) {
        const int j = j0 + jj;
        // even steps: sub-blocks j and j + 1 landed (nothing younger is in
        // flight yet), then one barrier for both steps
        if ((jj & 1) == 0) {
          __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0)
          asm volatile("" ::: "memory");
          __builtin_amdgcn_s_barrier();
          asm volatile("" ::: "memory");
        }
        // this step's DMA is issued after the scores and probabilities, so
        // its issue overlaps the matrix cores instead of holding every wave
        // back right after the barrier
        if (j < nj && active) probs(kslot(jj), vslot(jj), wc.s, wc.P, fresh);
        if ((jj & 1) == 0) {                       // the slots of steps j - 2 and j - 1
          if (j + 2 < nj) {
            dma(wd, pnext, (jj + 2) % kRingSlots);
            advance(wd);
            if (j + 3 < nj) pnext = page(wd);
          }
          if (j + 3 < nj) {
            dma(wd, pnext, (jj + 3) % kRingSlots);
            advance(wd);
            if (j + 4 < nj) pnext = page(wd);
          }
        }
        if (j < nj) {
          if (active) weigh(vslot(jj));
          fresh = false;
          if (wc.s == wc.n - 1 || j == nj - 1) {
            const bool unit_whole = whole && wc.s == wc.n - 1;
            finish(wc.b, wc.kvh, unit_whole, slot);
            if (byunit && unit_whole && tid == 0) rec[t * gl + wc.b * Hkv + wc.kvh] = make_int4(-1, 0, 0, 0);
            slot = 1;
            if (j < nj - 1) {                       // the next unit starts here
              advance(wc);
              if (active) qload(wc.b, wc.kvh);
              reset();
              whole = true;
              fresh = true;
            }
            // the stores (and the next unit's queries) complete here, on
            // this rare path: left pending, the compiler would make every
            // later step wait for all loads in flight, the ring's DMA
            // included, before reusing the stores' source registers or
            // reading the queries
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(0x0F70);    // vmcnt(0)
            asm volatile("" ::: "memory");
          } else {
            advance(wc);
          }
        }
        // this step's LDS reads (and page lookups) are done before the next barrier
        __builtin_amdgcn_s_waitcnt(0xC07F);        // lgkmcnt(0), vm/exp not waited
        asm volatile("" ::: "memory");
      }
    }
  };
  if (nstr == 2) body(IntC<2>{});
  else body(IntC<1>{});
}

// ---------------------------------------------------------------- bf16 merge
// One block of 256 threads per (lane, merge record, 16 rows of the tile):
// the record (one per unit when units are no more than blocks, else one
// per block boundary) names a unit cut by block ranges and the blocks
// holding its partials; 16 lanes per output row (8 head-dimension
// values each) merge them in block order with an online softmax (run-to-run
// bit identical) and write the normalised row.
__global__ __launch_bounds__(256) void attn_merge_bf16(
    const int4* __restrict__ rec, int nt, int gl, int B_Hkv, int S, int tstrips, int R, int T, int G,
    int Hq, int Hkv, const uint16_t* __restrict__ part_o, const float2* __restrict__ part_ml,
    uint16_t* __restrict__ out) {
  constexpr int kBatch = 8;
  const int rg = blockIdx.x % tstrips;             // 16-row group of the tile
  const int li_rec = blockIdx.x / tstrips;         // t * records per lane + record
  const int nrec = B_Hkv <= gl ? B_Hkv : gl;
  const int t = li_rec / nrec;
  const int4 rc = rec[t * gl + li_rec % nrec];
  if (rc.x < 0) return;
  int trow0, trows;
  tile_rows_of(t, nt, S, R, trow0, trows);
  const int rt = rg * 16 + (threadIdx.x >> 4);     // row in the tile
  if (rt >= trows) return;                          // whole 16-lane groups leave together
  const int li = threadIdx.x & 15;                 // d = 8 li .. 8 li + 7
  const int b = rc.x / Hkv, kvh = rc.x - b * Hkv;
  const int first = rc.y, nc = rc.z, s0 = rc.w;
  const int64_t rows_t = int64_t(tstrips) * 16;
  float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  float2 ml[kBatch];
  u32x4 po[kBatch];
  for (int c0 = 0; c0 < nc; c0 += kBatch) {
    // (nc is the record's: a branch the whole block takes alike, so a
    // record of few partials issues only their loads)
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (c0 + i >= nc) break;
      const int c = c0 + i;
      const int slot = 2 * (first + c) + (c == 0 ? s0 : 0);
      const int64_t unit = (int64_t(t) * 2 * gl + slot) * rows_t + rt;
      ml[i] = part_ml[unit];
      po[i] = *reinterpret_cast<const u32x4*>(part_o + unit * kHeadDim + 8 * li);
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (c0 + i >= nc || !(ml[i].y > 0.f)) continue;   // past the list, or no visible key
      const float mn = fmaxf(m, ml[i].x);
      const float a = fast_exp2(m - mn), e = fast_exp2(ml[i].x - mn);
      l = l * a + ml[i].y * e;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[2 * j] = o[2 * j] * a + __uint_as_float(po[i][j] << 16) * e;
        o[2 * j + 1] = o[2 * j + 1] * a + __uint_as_float(po[i][j] & 0xFFFF0000u) * e;
      }
      m = mn;
    }
  }
  const float inv = 1.f / l;
  const int r = trow0 + rt;
  const int n = r / G, gq = r - n * G;
  const int64_t oe = ((int64_t(b) * T + n) * Hq + kvh * G + gq) * kHeadDim + 8 * li;
  u32x4 u;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    u[e] = uint32_t(f32_to_bf16(o[2 * e] * inv)) | (uint32_t(f32_to_bf16(o[2 * e + 1] * inv)) << 16);
  *reinterpret_cast<u32x4*>(out + oe) = u;
}

// ---------------------------------------------------------------- fp32 prefix
// Same decomposition with v_mfma_f32_16x16x4_f32: one value per lane per
// operand, so K and V are staged in their natural [key][d] layout; the
// product's K dimension for S^T is d = 32 g + step (a lane reads 32
// consecutive floats of its key row).
constexpr int kSub32 = 32;
constexpr int kStride32 = 132;

__global__ __launch_bounds__(256) void attn_prefix_f32(
    const float* __restrict__ q, const float* __restrict__ kc, const float* __restrict__ vc,
    int64_t cap, const int32_t* __restrict__ prefix_len, int T, int Hq, int Hkv, int G, int R,
    int chunks, float sl2, float* __restrict__ part_o, float2* __restrict__ part_ml, uint8_t* ws) {
  const int c = blockIdx.x, rt = blockIdx.y, z = blockIdx.z;
  const int b = z / Hkv, kvh = z - b * Hkv;
  const int P = clamp_prefix(prefix_len[b], cap, ws, c == 0 && rt == 0 && kvh == 0 && threadIdx.x == 0);
  const int cs = chunk_len(P, chunks, kSub);
  const int k0 = c * cs;
  const int k1 = min(P, k0 + cs);
  const int Rpad = gridDim.y * kRowsPerTile;
  if (k0 >= k1) {
    mark_empty(part_ml, (int64_t(z) * chunks + c) * Rpad + rt * kRowsPerTile,
               min(kRowsPerTile, R - rt * kRowsPerTile));
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, g = lane >> 4;

  __shared__ __attribute__((aligned(16))) float Ks[kSub32 * kStride32];
  __shared__ __attribute__((aligned(16))) float Vs[kSub32 * kStride32];

  float qf[kSpw][32];
#pragma unroll
  for (int s = 0; s < kSpw; ++s) {
    const int r = rt * kRowsPerTile + (w * kSpw + s) * 16 + li;
    const float* qp = nullptr;
    if (r < R) {
      const int n = r / G, gq = r - n * G;
      qp = q + ((int64_t(b) * T + n) * Hq + kvh * G + gq) * kHeadDim + 32 * g;
    }
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      floatx4 x = qp ? *reinterpret_cast<const floatx4*>(qp + 4 * v) : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[s][4 * v + e] = x[e];
    }
  }
  floatx4 acc[kSpw][8];
  float mrow[kSpw], lrow[kSpw];
#pragma unroll
  for (int s = 0; s < kSpw; ++s) {
    mrow[s] = -INFINITY;
    lrow[s] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[s][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  const int64_t head_off = (int64_t(b) * Hkv + kvh) * cap * kHeadDim;
  const float* kbase = kc + head_off;
  const float* vbase = vc + head_off;

  for (int kb = k0; kb < k1; kb += kSub32) {
    const int nk = min(kSub32, k1 - kb);
    __syncthreads();
    // 32 rows x 32 float4 per tensor: 4 float4 per thread each
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int u = tid + 256 * j;
      const int rk = u >> 5, c4 = u & 31;
      floatx4 kx = floatx4{0.f, 0.f, 0.f, 0.f}, vx = kx;
      if (rk < nk) {
        kx = *reinterpret_cast<const floatx4*>(kbase + int64_t(kb + rk) * kHeadDim + 4 * c4);
        vx = *reinterpret_cast<const floatx4*>(vbase + int64_t(kb + rk) * kHeadDim + 4 * c4);
      }
      *reinterpret_cast<floatx4*>(&Ks[rk * kStride32 + 4 * c4]) = kx;
      *reinterpret_cast<floatx4*>(&Vs[rk * kStride32 + 4 * c4]) = vx;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      floatx4 sacc[kSpw];
#pragma unroll
      for (int s = 0; s < kSpw; ++s) sacc[s] = floatx4{0.f, 0.f, 0.f, 0.f};
      const float* krow = &Ks[(t * 16 + li) * kStride32 + 32 * g];
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const floatx4 a4 = *reinterpret_cast<const floatx4*>(krow + 4 * v);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int s = 0; s < kSpw; ++s)
            sacc[s] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[e], qf[s][4 * v + e], sacc[s], 0, 0, 0);
      }
#pragma unroll
      for (int s = 0; s < kSpw; ++s) {
        float x[4];
        float mloc = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = t * 16 + 4 * g + i;
          x[i] = key < nk ? sacc[s][i] * sl2 : -INFINITY;
          mloc = fmaxf(mloc, x[i]);
        }
        mloc = xmax32(xmax16(mloc));
        const float mnew = fmaxf(mrow[s], mloc);
        const float alpha = fast_exp2(mrow[s] - mnew);
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = fast_exp2(x[i] - mnew);
          psum += x[i];
        }
        psum = xsum32(xsum16(psum));
        lrow[s] = lrow[s] * alpha + psum;
        mrow[s] = mnew;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          acc[s][dt] *= alpha;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float a = Vs[(t * 16 + 4 * g + i) * kStride32 + dt * 16 + li];
            acc[s][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, x[i], acc[s][dt], 0, 0, 0);
          }
        }
      }
    }
  }
#pragma unroll
  for (int s = 0; s < kSpw; ++s) {
    const int r = rt * kRowsPerTile + (w * kSpw + s) * 16 + li;
    if (r < R) {
      const int64_t unit = (int64_t(z) * chunks + c) * Rpad + r;
      float* po = part_o + unit * kHeadDim;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<floatx4*>(po + dt * 16 + 4 * g) = acc[s][dt];
      if (g == 0) part_ml[unit] = make_float2(mrow[s], lrow[s]);
    }
  }
}

// ---------------------------------------------------------------- combine
// 16 lanes per output row (b, n, h), 8 head-dimension values per lane.
// Merges the prefix chunk partials (all chunks in order; a chunk holding
// no keys of the sequence carries weight 0, so the prefix length is not
// needed and every load can be issued at once) and then the tree keys
// of n's path (n, its parent, ..., the root) with an online softmax.  All
// loads of a batch are issued before any of them is used.
__device__ __forceinline__ float row16_sum(float v) {
  // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  return v;
}

template <bool BF16>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float* f) {
  if (BF16) {
    const u32x4 u = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + elem);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = __uint_as_float(u[j] << 16);
      f[2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
    }
  } else {
    const floatx4 a = *reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(base) + elem);
    const floatx4 c = *reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(base) + elem + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[j] = a[j];
      f[4 + j] = c[j];
    }
  }
}

// Eight values as loaded (16 bytes of bf16 or 32 of fp32), unpacked only
// where they are used, so the loads of a batch all leave before the first
// wait.
template <bool BF16>
struct Raw8 {
  u32x4 u[BF16 ? 1 : 2];
};
template <bool BF16>
__device__ __forceinline__ void load_raw8(const void* base, int64_t elem, Raw8<BF16>& r) {
  const uint8_t* p = reinterpret_cast<const uint8_t*>(base) + elem * (BF16 ? 2 : 4);
#pragma unroll
  for (int i = 0; i < (BF16 ? 1 : 2); ++i) r.u[i] = reinterpret_cast<const u32x4*>(p)[i];
}
template <bool BF16>
__device__ __forceinline__ void unpack8(const Raw8<BF16>& r, float* f) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (BF16) {
      f[2 * j] = __uint_as_float(r.u[0][j] << 16);
      f[2 * j + 1] = __uint_as_float(r.u[0][j] & 0xFFFF0000u);
    } else {
      f[j] = __uint_as_float(r.u[0][j]);
      f[4 + j] = __uint_as_float(r.u[1][j]);
    }
  }
}

// UNIFORM_N: Hq is a multiple of four, so the four rows of a wave share
// their tree node n.  TREE: the path keys are merged here (the fp32 path,
// whose prefix pass does not take them; the bf16 prefix pass always does).
template <bool BF16, bool UNIFORM_N, bool TREE>
__global__ __launch_bounds__(128) void attn_combine(
    TreeDev tree, const void* __restrict__ q, const void* __restrict__ kt,
    const void* __restrict__ vt, int B, int Hq, int Hkv, int G, int chunks, int Rpad, float sl2,
    const void* __restrict__ part_o, const float2* __restrict__ part_ml, void* __restrict__ out) {
  constexpr int kBatch = 8;
  const int T = tree.T;
  const int64_t row = int64_t(blockIdx.x) * 8 + (threadIdx.x >> 4);
  if (row >= int64_t(B) * T * Hq) return;          // whole 16-lane groups leave together
  const int li = threadIdx.x & 15;                 // d = 8 li .. 8 li + 7
  const int h = int(row % Hq);
  const int n = int((row / Hq) % T);
  const int b = int(row / (int64_t(Hq) * T));
  const int kvh = h / G, gq = h - kvh * G;
  const int r = n * G + gq;
  const int z = b * Hkv + kvh;
  const int nc = chunks;                           // empty chunks carry weight 0

  float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  auto merge = [&](float ms, float ls, const float* os) {
    if (!(ls > 0.f)) return;                       // an empty chunk
    const float mn = fmaxf(m, ms);
    const float a = fast_exp2(m - mn), e = fast_exp2(ms - mn);
    l = l * a + ls * e;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = o[j] * a + os[j] * e;
    m = mn;
  };
  float2 ml[kBatch];
  Raw8<BF16> po[kBatch];
  auto load_parts = [&](int c0) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int c = max(0, min(c0 + i, nc - 1));
      const int64_t unit = (int64_t(z) * chunks + c) * Rpad + r;
      ml[i] = part_ml[unit];
      load_raw8<BF16>(part_o, unit * kHeadDim + 8 * li, po[i]);   // bf16 partials in the bf16 path
    }
  };
  // the nodes on n's path, n first and the root last: the bits of its
  // ancestor set (one indexed read of the kernel argument, in flight with
  // the partials), taken from the highest down
  uint64_t path[2];
  bool more = true;
  int idx[kBatch];
  int cnt = 0;
  Raw8<BF16> kx[kBatch], vx[kBatch];
  auto load_tree = [&]() {
    cnt = 0;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const bool hi = path[1] != 0;
      const uint64_t w = hi ? path[1] : path[0];
      const int bit = w ? 63 - __builtin_clzll(w) : 0;
      idx[i] = w ? (hi ? 64 : 0) + bit : 0;
      if (w) {
        ++cnt;
        if (hi) path[1] &= ~(uint64_t(1) << bit);
        else path[0] &= ~(uint64_t(1) << bit);
      }
    }
    more = (path[0] | path[1]) != 0;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int64_t kv_elem = ((int64_t(b) * T + idx[i]) * Hkv + kvh) * kHeadDim + 8 * li;
      load_raw8<BF16>(kt, kv_elem, kx[i]);
      load_raw8<BF16>(vt, kv_elem, vx[i]);
    }
  };
  auto merge_tree = [&](const float* qv) {
    float sc[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      float kf[8];
      unpack8<BF16>(kx[i], kf);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d += qv[e] * kf[e];
      sc[i] = row16_sum(d) * sl2;
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      float vf[8];
      unpack8<BF16>(vx[i], vf);
      if (i < cnt) merge(sc[i], 1.f, vf);
    }
  };

  // first batch of everything in flight at once, the ancestor set first
  // (the tree loads wait for it alone).  When the wave's rows share n the
  // set is a scalar load of the kernel argument, which does not wait
  // behind the vector loads.
  // When the prefix pass took the tree keys as sub-blocks of its chunks
  // (bf16), its partials already hold them; else (TREE) the path keys are
  // merged here.
  constexpr bool kTree = TREE;
  const int nw = UNIFORM_N ? __builtin_amdgcn_readfirstlane(n) : n;
  path[0] = kTree ? tree.anc[nw][0] : 0;
  path[1] = kTree ? tree.anc[nw][1] : 0;
  load_parts(0);                                   // chunks >= 1 (the plan's)
  Raw8<BF16> qraw;
  if constexpr (kTree) {
    load_raw8<BF16>(q, ((int64_t(b) * T + n) * Hq + h) * kHeadDim + 8 * li, qraw);
    load_tree();
  }
  // prefix chunk partials, chunks in order
  for (int c0 = 0; c0 < nc; c0 += kBatch) {
    if (c0 > 0) load_parts(c0);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      float pf[8];
      unpack8<BF16>(po[i], pf);
      if (c0 + i < nc) merge(ml[i].x, ml[i].y, pf);
    }
  }
  // tree keys on n's path: n, its parent, ..., the root
  if constexpr (kTree) {
    float qv[8];
    unpack8<BF16>(qraw, qv);
    merge_tree(qv);
    while (more) {
      load_tree();
      merge_tree(qv);
    }
  }

  const float inv = 1.f / l;
  const int64_t oe = ((int64_t(b) * T + n) * Hq + h) * kHeadDim + 8 * li;
  if (BF16) {
    u32x4 u;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      u[e] = uint32_t(f32_to_bf16(o[2 * e] * inv)) | (uint32_t(f32_to_bf16(o[2 * e + 1] * inv)) << 16);
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + oe) = u;
  } else {
    float* op = reinterpret_cast<float*>(out) + oe;
    *reinterpret_cast<floatx4*>(op) = floatx4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
    *reinterpret_cast<floatx4*>(op + 4) = floatx4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
  }
}

hipError_t launch_attn(const TreeDev& tree, int32_t B, int32_t Hq, int32_t Hkv, int is_bf16,
                       const void* q, const void* k_tree, const void* v_tree, const void* k_cache,
                       const void* v_cache, int64_t cap, const int32_t* prefix_len, float scale,
                       void* out, uint8_t* ws, const AttnPlan& plan, hipStream_t s,
                       const PagedArgs* paged, uint8_t* flags) {
  uint8_t* fl = flags ? flags : ws;                 // sticky flags
  void* part_o = ws + plan.o_off;
  float2* part_ml = reinterpret_cast<float2*>(ws + plan.ml_off);
  const float sl2 = scale * kLog2e;
  if (is_bf16) {
    const auto* qq = reinterpret_cast<const uint16_t*>(q);
    const auto* kk = reinterpret_cast<const uint16_t*>(k_cache);
    const auto* vv = reinterpret_cast<const uint16_t*>(v_cache);
    const auto* kt = reinterpret_cast<const uint16_t*>(k_tree);
    const auto* vt = reinterpret_cast<const uint16_t*>(v_tree);
    auto* po = reinterpret_cast<uint16_t*>(part_o);
    auto* rec = reinterpret_cast<int4*>(ws + plan.rec_off);
    auto* o = reinterpret_cast<uint16_t*>(out);
    const PagedArgs pa = paged ? *paged : PagedArgs{};
    prof_begin(s, TR_KERNEL_ATTN_PREFIX);
#define TR_PREFIX(PG)                                                                             \
  hipLaunchKernelGGL((attn_prefix_bf16<PG>), dim3(plan.grid), dim3(64 * kWaves), plan.lds_dyn, s, qq, \
                     kk, vv, kt, vt, tree, cap, prefix_len, B, Hq, Hkv, plan.G, plan.R, plan.nt,     \
                     plan.S, plan.tstrips, plan.gl, plan.xpair, plan.split, sl2, po, part_ml, rec, o, \
                     fl, pa)
    if (paged) TR_PREFIX(true); else TR_PREFIX(false);
#undef TR_PREFIX
    prof_end(s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    prof_begin(s, TR_KERNEL_ATTN_COMBINE);
    const int64_t U = int64_t(B) * Hkv;
    const int64_t recs = U <= plan.gl ? U : plan.gl;    // records per lane (per unit or per block)
    hipLaunchKernelGGL(attn_merge_bf16, dim3(unsigned(plan.nt * recs * plan.tstrips)), dim3(256), 0,
                       s, rec, plan.nt, plan.gl, int(U), plan.S, plan.tstrips, plan.R, tree.T, plan.G,
                       Hq, Hkv, po, part_ml, o);
    prof_end(s);
    return hipGetLastError();
  }
  dim3 grid(plan.chunks, plan.row_tiles, B * Hkv);
  prof_begin(s, TR_KERNEL_ATTN_PREFIX);
  hipLaunchKernelGGL(attn_prefix_f32, grid, dim3(256), 0, s, reinterpret_cast<const float*>(q),
                     reinterpret_cast<const float*>(k_cache), reinterpret_cast<const float*>(v_cache),
                     cap, prefix_len, tree.T, Hq, Hkv, plan.G, plan.R, plan.chunks, sl2,
                     reinterpret_cast<float*>(part_o), part_ml, fl);
  prof_end(s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = int64_t(B) * tree.T * Hq;
  dim3 cgrid(unsigned((rows + 7) / 8));
  const int Rpad = plan.row_tiles * plan.tile_rows;
  prof_begin(s, TR_KERNEL_ATTN_COMBINE);
#define TR_COMBINE(UN)                                                                        \
  hipLaunchKernelGGL((attn_combine<false, UN, true>), cgrid, dim3(128), 0, s, tree, q, k_tree, v_tree, \
                     B, Hq, Hkv, plan.G, plan.chunks, Rpad, sl2, part_o, part_ml, out)
  if (Hq % 4 == 0) TR_COMBINE(true); else TR_COMBINE(false);
#undef TR_COMBINE
  prof_end(s);
  return hipGetLastError();
}

}  // namespace tr
