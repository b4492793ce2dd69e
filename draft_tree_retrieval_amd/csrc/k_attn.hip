// Tree attention for the merged draft sequence.
//
// Every tree node attends to the whole prefix and to its own ancestors
// (itself included), never to a sibling branch ("Token Recycling" summary,
// Method, third module; walk-through, workflow step 3).  The prefix part is
// the same dense product for every query row of a key/value head, so it is
// computed with matrix cores over prefix chunks (split-K over the prefix,
// one block per (sequence, kv head, 128-row tile, chunk)); the tree part
// touches at most depth+1 keys per row and is folded into the combine pass
// that merges the chunk partials with an online softmax in a fixed order.
//
// Prefix pass layout (bf16).  Per 64-key sub-block the block stages K as
// [key][d] and V transposed as [d][key] in LDS.  Each wave owns 16-row
// query strips and computes S^T = K Q^T and O^T = V^T P^T with
// v_mfma_f32_16x16x32_bf16: in both products the lane's output column is
// its query row, so softmax statistics, the probabilities fed to the second
// product and the accumulator rows all stay in the same lane.  The key
// order inside the second product's K dimension is permuted consistently
// on both operands so that the probabilities need no cross-lane moves.
#include "dev_common.h"

namespace tr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kSub = 64;          // chunk boundaries are multiples of this many keys
constexpr int kWaves = 8;         // waves per bf16 prefix block
constexpr int kSpw = 2;           // 16-row strips per wave (fp32 kernel)
constexpr int kRowsPerTile = 4 * kSpw * 16;   // fp32 kernel: 4 waves
constexpr float kLog2e = 1.4426950408889634f;

AttnPlan plan_attn(int32_t T, int32_t B, int32_t Hq, int32_t Hkv, int64_t cap, int is_bf16) {
  AttnPlan p{};
  p.G = Hq / Hkv;
  p.R = T * p.G;
  if (is_bf16) {
    // two strips per wave once a head has more than one 128-row tile: each
    // key/value operand read from LDS then feeds twice the products and
    // fewer tiles re-read the same keys; one strip per wave below that, so
    // that more waves compute (one per SIMD at most otherwise)
    p.spw = p.R > 128 ? 2 : 1;
    p.tile_rows = kWaves * p.spw * 16;
  } else {
    p.spw = kSpw;
    p.tile_rows = kRowsPerTile;
  }
  p.row_tiles = (p.R + p.tile_rows - 1) / p.tile_rows;
  int64_t base = int64_t(B) * Hkv * p.row_tiles;
  // at most one block per CU: a block holds 131+ KB of LDS, so blocks past
  // the 256th would wait for a whole block to finish
  int64_t chunks = 256 / base;
  int64_t by_cap = (cap + kSub - 1) / kSub + (is_bf16 ? (T + kSub - 1) / kSub : 0);
  if (chunks > by_cap) chunks = by_cap;
  if (chunks > 64) chunks = 64;
  if (chunks < 1) chunks = 1;
  // bf16: at least two chunks, so that the tree keys always go to the
  // prefix pass (folded into the chunks' sub-blocks); left to the combine,
  // its per-row loop over them costs more than the extra chunk (32
  // sequences x 8 kv heads: combine 35 -> 17 us, prefix 234 -> 245 us)
  if (is_bf16 && chunks < 2) chunks = 2;
  p.chunks = int32_t(chunks);
  p.tree_keys = is_bf16 ? 1 : 0;
  const size_t rpad = size_t(p.row_tiles) * p.tile_rows;
  const size_t units = size_t(B) * Hkv * p.chunks * rpad;
  size_t off = kDataOff;
  p.o_off = off;                                    // bf16 path: bf16 partials
  off = align256(off + units * kHeadDim * (is_bf16 ? 2 : 4));
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
// 8 waves, two 16-row query strips per wave.  The keys and values of the
// chunk stream HBM -> LDS through the LDS DMA (global_load_lds_dwordx4) in
// 64-key sub-blocks (16 KB of K and 16 KB of V) into a ring of four LDS
// slots, three sub-blocks in flight ahead of the one in use; nothing passes
// through registers and nothing is restaged.
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
// so the loop synchronises with a bare barrier after vmcnt(8) (the two
// younger sub-blocks, 4 DMA loads each per wave, may still fly), and each
// ring slot is its own LDS array named statically (one array would make
// the compiler wait for DMAs into the other slots before every read).
constexpr int kSB = 64;                   // keys per sub-block
constexpr float kLazy = 8.f;              // lazy rescaling threshold (log2 units)
constexpr int kRingSlots = 4;
constexpr int kSubBytes = kSB * kHeadDim * 2;   // 16 KB
// PAGED: kc and vc are page pools [num_pages][Hkv][page_size][d] reached
// through the block table; the chunk's page ids are read into LDS first and
// each 64-key sub-block (inside one page: page sizes are powers of two of
// at least 64 keys) looks its page up once.
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

template <int N>
struct IntC {
  static constexpr int value = N;
};

// The chunks take the tree keys too: ceil(T / 64) sub-blocks after the
// prefix's, each row masked to its ancestor set.
template <int SPW, bool PAGED>
__global__ __launch_bounds__(512) void attn_prefix_bf16(
    const uint16_t* __restrict__ q, const uint16_t* kc,
    const uint16_t* vc, const uint16_t* kt, const uint16_t* vt, TreeDev tree, int64_t cap,
    const int32_t* __restrict__ prefix_len,
    int Hq, int Hkv, int G, int R, int chunks, float sl2, uint16_t* __restrict__ part_o,
    float2* __restrict__ part_ml, uint8_t* ws, int B, int row_tiles, PagedArgs pg) {
  const int T = tree.T;
  constexpr int kRows = kWaves * SPW * 16;        // query rows per tile
  // Blocks are dealt to the 8 XCDs round-robin by block index.  The row
  // tiles of one (sequence, kv head, chunk) group read the same keys and
  // values, so they are given consecutive slots on the same XCD and share
  // its L2: block i runs on XCD i % 8, slot i / 8 of that XCD.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int rt = slot % row_tiles;
  const int grp = (slot / row_tiles) * 8 + xcd;    // (sequence, kv head, chunk) group
  if (grp >= B * Hkv * chunks) return;
  const int z = grp / chunks, c = grp - z * chunks;
  const int b = z / Hkv, kvh = z - b * Hkv;
  // P gates every key load, so its load leaves first; the ancestor set of
  // each of the tile's rows (tree sub-block masks) is read while P is in
  // flight
  const int32_t p_raw = prefix_len[b];
  __shared__ uint64_t s_anc[kRows][2];
  if (int(threadIdx.x) < kRows) {
    const int n = min(rt * kRows + int(threadIdx.x), R - 1) / G;
    const uint64_t a0 = tree.anc[n][0], a1 = tree.anc[n][1];
    s_anc[threadIdx.x][0] = a0;
    s_anc[threadIdx.x][1] = a1;
  }
  const int P = clamp_prefix(p_raw, cap, ws, c == 0 && rt == 0 && kvh == 0 && threadIdx.x == 0);
  // The keys of a (sequence, kv head) are the prefix's ntp 64-key
  // sub-blocks followed by ntt sub-blocks of tree nodes (each row sees the
  // nodes of its ancestor set, itself included), dealt to the chunks as
  // evenly as whole sub-blocks allow: chunk c takes global sub-blocks
  // [s0, s0 + nsub).  The tree keys cost no pass of their own and the
  // combine merges partials only.
  const int ntp = (P + kSB - 1) / kSB, ntt = (T + kSB - 1) / kSB, ntot = ntp + ntt;
  const int sbase = ntot / chunks, srem = ntot - sbase * chunks;
  const int s0 = c * sbase + min(c, srem);
  const int nsub = sbase + (c < srem ? 1 : 0);
  const int k0 = s0 * kSB;                          // the chunk's prefix keys: [k0, k1)
  const int k1 = min(P, (s0 + nsub) * kSB);
  const int Rpad = row_tiles * kRows;
  if (nsub == 0) {
    mark_empty(part_ml, (int64_t(z) * chunks + c) * Rpad + rt * kRows, min(kRows, R - rt * kRows));
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, g = lane >> 4;
  // Strips of 16 query rows: wave w takes strip w.  With one strip per
  // wave and 5 or 6 strips in the tile, waves 4..7 instead split strips 4
  // and 5 by key halves (waves 4 + 2h and 5 + 2h take keys 32h .. 32h+31 of
  // every sub-block), so each SIMD (wave w runs on SIMD w % 4) carries 1.5
  // strips rather than two of them carrying 2; the halves merge at the end.
  const int tile_strips = (min(kRows, R - rt * kRows) + 15) / 16;
  const bool split = SPW == 1 && (tile_strips == 5 || tile_strips == 6);
  const bool hw = split && w >= 4;                  // a half-key wave
  const int kh = hw ? (w >> 1) & 1 : 0;             // its key half
  const int strip = hw ? 4 + (w & 1) : w;
  const int srow0 = strip * SPW * 16;               // the wave's first row in the tile
  const int row0 = rt * kRows + srow0;              // first query row of this wave
  const bool active = row0 < R;                    // waves past the last row only load

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
  __shared__ int32_t s_pg[PAGED ? kMaxChunkPages : 1];
  const int p0 = PAGED ? (k0 >> pg.ps_log2) : 0;    // first page of the chunk
  if constexpr (PAGED) {
    // <= kMaxChunkPages by the plan; none when the chunk holds tree keys only
    const int np = k1 > k0 ? ((k1 - 1) >> pg.ps_log2) - p0 + 1 : 0;
    for (int i = threadIdx.x; i < np; i += blockDim.x) {
      int32_t id = pg.table[int64_t(b) * pg.max_pages + p0 + i];
      if (id < 0 || int64_t(id) >= pg.num_pages) {     // stays inside the pool
        set_flag(ws, TR_FLAG_BAD_PAGE);
        id = 0;
      }
      s_pg[i] = id;
    }
    __syncthreads();
  }

  // (the query fragments are loaded before the DMAs; the compiler waits for
  // all loads in flight before entering the loop that uses them, so the
  // first step starts with the prologue's sub-blocks landed)
  bf16x8 qb[SPW][4];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const int r = min(row0 + s * 16 + li, R - 1);     // rows past R: any row, never stored
    const int n = r / G, gq = r - n * G;
    const uint16_t* qp = q + ((int64_t(b) * T + n) * Hq + kvh * G + gq) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qb[s][ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32 + g * 8);
  }
  asm volatile("" ::: "memory");

  floatx4 acc[SPW][8];
  float mrow[SPW], lrow[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    mrow[s] = -INFINITY;
    lrow[s] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[s][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  const int64_t head_off = PAGED ? 0 : (int64_t(b) * Hkv + kvh) * cap * kHeadDim;
  // Sub-block j into ring slot sl: 1024 16-byte slots of K and of V, two
  // of each per thread (wave w, pass q: slots (8 q + w) * 64 + lane).  Rows
  // past the chunk end repeat its last row (finite data the key mask gives
  // probability 0); sub-blocks past the end repeat the last one.
  // A tree sub-block reads node rows of kt / vt ([B][T][Hkv][d]; nodes past
  // T repeat the last, masked like the keys past P).
  const int64_t node_stride = int64_t(Hkv) * kHeadDim;
  const uint16_t* kt_b = kt + (int64_t(b) * T * Hkv + kvh) * kHeadDim;
  const uint16_t* vt_b = vt + (int64_t(b) * T * Hkv + kvh) * kHeadDim;
  auto dma = [&](int j, int sl) {
    const int gj = s0 + min(j, nsub - 1);
    if (gj < ntp) {
      const int kb = gj * kSB;
      // rows kb .. kb+63 (and the clamp P-1 >= kb) lie in one page
      const uint16_t* kp = kc + head_off;
      const uint16_t* vp = vc + head_off;
      int row_base = 0;
      if constexpr (PAGED) {
        const int64_t pool_off =
            (int64_t(s_pg[(kb >> pg.ps_log2) - p0]) * Hkv + kvh) * pg.page_size * kHeadDim;
        kp = kc + pool_off;
        vp = vc + pool_off;
        row_base = (kb >> pg.ps_log2) << pg.ps_log2;   // first position of the page
      }
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const int base = (q2 * kWaves + w) * 64;       // wave-uniform first slot
        const int p = base + lane;
        const int r = p >> 4, pos = p & 15;
        const int64_t row = min(kb + r, P - 1) - row_base;
        const int ck = pos ^ (r & 15), cv = pos ^ ((r & 7) << 1);
        lds_dma16(kp + row * kHeadDim + ck * 8, kslot(sl) + base * 16);
        lds_dma16(vp + row * kHeadDim + cv * 8, vslot(sl) + base * 16);
      }
    } else {
      const int nb = (gj - ntp) * kSB;
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const int base = (q2 * kWaves + w) * 64;
        const int p = base + lane;
        const int r = p >> 4, pos = p & 15;
        const int64_t node = min(nb + r, T - 1);
        const int ck = pos ^ (r & 15), cv = pos ^ ((r & 7) << 1);
        lds_dma16(kt_b + node * node_stride + ck * 8, kslot(sl) + base * 16);
        lds_dma16(vt_b + node * node_stride + cv * 8, vslot(sl) + base * 16);
      }
    }
    asm volatile("" ::: "memory");
  };

  // S^T = K Q^T for NTL tiles of 16 keys from tile tb on (sacc[s][t] holds
  // tile tb + t); operands read ahead of the products
  auto qk = [&](const uint8_t* Ks, floatx4 (&sacc)[SPW][4], auto ntl, int tb) {
    constexpr int NTL = decltype(ntl)::value;
#pragma unroll
    for (int s = 0; s < SPW; ++s)
#pragma unroll
      for (int t = 0; t < NTL; ++t) sacc[s][t] = floatx4{0.f, 0.f, 0.f, 0.f};
    constexpr int KT = 2;                             // key tiles read ahead
#pragma unroll
    for (int t0 = 0; t0 < NTL; t0 += KT) {
      bf16x8 ka[KT][4];
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          ka[t][ks] = *reinterpret_cast<const bf16x8*>(
              Ks + ((tb + t0 + t) * 16 + li) * 256 + (((4 * ks + g) ^ li) << 4));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
          for (int s = 0; s < SPW; ++s)
            sacc[s][t0 + t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[t][ks], qb[s][ks], sacc[s][t0 + t], 0, 0, 0);
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
      for (int p = 0; p < NPP; ++p) {
        const int pp = pb0 + p;
        uint32_t u[4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int row = 32 * pp + 16 * hh + 4 * g + (li >> 2);
          const uint8_t* addr = Vs + row * 256 + ((cch ^ ((row & 7) << 1)) << 4) + half;
          const u32x2 r2 = lds_read_tr16(addr);
          u[2 * hh] = r2[0];
          u[2 * hh + 1] = r2[1];
        }
        va[i][p] = __builtin_bit_cast(bf16x8, u32x4{u[0], u[1], u[2], u[3]});
      }
    }
  };
  // Global sub-block gj: prefix keys past P (a ragged last sub-block) get
  // score -inf; in a tree sub-block a row sees only its ancestor set.  (The
  // comparisons are against per-call values: sixteen loop-invariant key
  // indices or bit masks hoisted out of the loop would stay live.)
  auto mask = [&](floatx4 (&sacc)[SPW][4], int gj, auto ntl, int tb) {
    constexpr int NTL = decltype(ntl)::value;
    if (gj < ntp) {
      const int nk = P - gj * kSB;
      if (nk < kSB) {
        const int nrel = nk - 4 * g - 16 * tb;      // keys t*16 + i of the lane's tiles
#pragma unroll
        for (int s = 0; s < SPW; ++s)
#pragma unroll
          for (int t = 0; t < NTL; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (t * 16 + i >= nrel) sacc[s][t][i] = -INFINITY;
      }
    } else {
      const int hi = gj - ntp > 0 ? 1 : 0;          // nodes 64 .. 127
#pragma unroll
      for (int s = 0; s < SPW; ++s) {
        const uint64_t bits = s_anc[srow0 + s * 16 + li][hi] >> (4 * g + 16 * tb);
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
          const uint32_t nib = uint32_t(bits >> (t * 16));   // keys (tb+t)*16+4g .. +3
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (!((nib >> i) & 1u)) sacc[s][t][i] = -INFINITY;
        }
      }
    }
  };
  // online softmax per query row (the lane's column), on raw scores:
  // scale > 0, so max(scale s) = scale max(s) and p = 2^(s sl2 - m).
  // Lazy rescaling: a row's reference maximum moves only when a score
  // passes it by more than kLazy (log2 units), so the probabilities stay
  // below 2^kLazy and the accumulators are rarely rescaled; the partial
  // (m, l, O) stays consistent for any reference m.  No branch: the
  // rescale of the accumulators is left to the caller (alpha, bump).
  bf16x8 pb[SPW][2];
  float alpha[SPW];
  bool bump[SPW];
  auto softmax = [&](const floatx4 (&sacc)[SPW][4], auto ntl) {
    constexpr int NTL = decltype(ntl)::value;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      float mraw = -INFINITY;
#pragma unroll
      for (int t = 0; t < NTL; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) mraw = fmaxf(mraw, sacc[s][t][i]);
      mraw = xmax32(xmax16(mraw));
      const float mcand = mraw * sl2;
      bump[s] = mcand > mrow[s] + kLazy;           // always on the first sub-block
      const float mnew = bump[s] ? mcand : mrow[s];
      alpha[s] = bump[s] ? fast_exp2(mrow[s] - mnew) : 1.f;
      // a row that has seen no visible key yet (a tree sub-block hides all
      // of them from it) keeps m = -inf: offset 0 gives p = 0, not NaN
      const float off = mnew == -INFINITY ? 0.f : mnew;
      float psum = 0.f;
      __bf16 ph[4][4];
#pragma unroll
      for (int t = 0; t < NTL; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pr = fast_exp2(__builtin_fmaf(sacc[s][t][i], sl2, -off));
          psum += pr;
          ph[t][i] = (__bf16)pr;
        }
      psum = xsum32(xsum16(psum));
      lrow[s] = lrow[s] * alpha[s] + psum;
      mrow[s] = mnew;
#pragma unroll
      for (int pp = 0; pp < NTL / 2; ++pp)
        pb[s][pp] = bf16x8{ph[2 * pp][0], ph[2 * pp][1], ph[2 * pp][2], ph[2 * pp][3],
                           ph[2 * pp + 1][0], ph[2 * pp + 1][1], ph[2 * pp + 1][2], ph[2 * pp + 1][3]};
    }
  };
  // nothing to rescale on the first sub-block (acc is zero) or when no
  // lane's reference moved
  auto rescale = [&](bool first) {
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      if (!first && __any(bump[s])) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acc[s][dt] *= alpha[s];
      }
    }
  };
  // O^T += V^T P^T over NPP 32-key blocks from pb0 on (va holds dt 0, 1 on
  // entry)
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
          for (int s = 0; s < SPW; ++s)
            acc[s][dt0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[i][pp], pb[s][pp], acc[s][dt0 + i], 0, 0, 0);
    }
  };

  // three sub-blocks in flight, then per sub-block: wait, barrier, refill
  // the slot freed by the previous sub-block, compute.  (A software
  // pipeline that forms the next sub-block's scores during this one's
  // softmax measured slower here: the two waves of a SIMD already overlap
  // each other's matrix and VALU work.)
#pragma unroll
  for (int j = 0; j < kRingSlots - 1; ++j) dma(j, j);
  // the ancestor sets in LDS before the first step's barrier
  __builtin_amdgcn_s_waitcnt(0xC07F);              // lgkmcnt(0)
  asm volatile("" ::: "memory");
  const int nround = (nsub + kRingSlots - 1) / kRingSlots * kRingSlots;
  for (int j0 = 0; j0 < nround; j0 += kRingSlots) {
#pragma unroll
    for (int jj = 0; jj < kRingSlots; ++jj) {
      const int j = j0 + jj;
      __builtin_amdgcn_s_waitcnt(0x0F78);          // vmcnt(8), lgkm/exp not waited
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      dma(j + kRingSlots - 1, (jj + kRingSlots - 1) % kRingSlots);
      if (active && j < nsub) {
        floatx4 sc[SPW][4];
        if (!hw) {                                   // all 64 keys
          qk(kslot(jj), sc, IntC<4>{}, 0);
          mask(sc, s0 + j, IntC<4>{}, 0);
          read_v(vslot(jj), 0, IntC<2>{}, 0);
          __builtin_amdgcn_sched_barrier(0);
          softmax(sc, IntC<4>{});
          rescale(j == 0);
          pv(vslot(jj), IntC<2>{}, 0);
        } else {                                     // keys 32 kh .. 32 kh + 31
          qk(kslot(jj), sc, IntC<2>{}, 2 * kh);
          mask(sc, s0 + j, IntC<2>{}, 2 * kh);
          read_v(vslot(jj), 0, IntC<1>{}, kh);
          __builtin_amdgcn_sched_barrier(0);
          softmax(sc, IntC<2>{});
          rescale(j == 0);
          pv(vslot(jj), IntC<1>{}, kh);
        }
      }
      // this step's LDS reads are done before the next barrier
      __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0), vm/exp not waited
      asm volatile("" ::: "memory");
    }
  }

  if (split) {
    // the second key half of strips 4 and 5 hands its (m, l, O) to the
    // first through LDS; the first merges and stores
    __shared__ float s_mo[SPW == 1 ? 2 : 1][64][36];
    __shared__ float2 s_ml[SPW == 1 ? 2 : 1][64];
    if (hw && kh == 1 && active) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<floatx4*>(&s_mo[w & 1][lane][4 * dt]) = acc[0][dt];
      s_ml[w & 1][lane] = make_float2(mrow[0], lrow[0]);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (hw && kh == 0 && active) {
      const float2 ml1 = s_ml[w & 1][lane];
      if (ml1.y > 0.f) {
        if (!(lrow[0] > 0.f)) {
          mrow[0] = ml1.x;
          lrow[0] = ml1.y;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) acc[0][dt] = *reinterpret_cast<const floatx4*>(&s_mo[w & 1][lane][4 * dt]);
        } else {
          const float mn = fmaxf(mrow[0], ml1.x);
          const float a0 = fast_exp2(mrow[0] - mn), a1 = fast_exp2(ml1.x - mn);
          lrow[0] = lrow[0] * a0 + ml1.y * a1;
          mrow[0] = mn;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
            acc[0][dt] = acc[0][dt] * a0 + *reinterpret_cast<const floatx4*>(&s_mo[w & 1][lane][4 * dt]) * a1;
        }
      }
    }
  }
  if (!active || (hw && kh == 1)) return;
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const int r = row0 + s * 16 + li;
    if (r < R) {
      const int64_t unit = (int64_t(z) * chunks + c) * Rpad + r;
      uint16_t* po = part_o + unit * kHeadDim;     // bf16: the partial sums round once
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const u32x2 v = {uint32_t(__builtin_bit_cast(uint16_t, (__bf16)acc[s][dt][0])) |
                             (uint32_t(__builtin_bit_cast(uint16_t, (__bf16)acc[s][dt][1])) << 16),
                         uint32_t(__builtin_bit_cast(uint16_t, (__bf16)acc[s][dt][2])) |
                             (uint32_t(__builtin_bit_cast(uint16_t, (__bf16)acc[s][dt][3])) << 16)};
        *reinterpret_cast<u32x2*>(po + dt * 16 + 4 * g) = v;
      }
      if (g == 0) part_ml[unit] = make_float2(mrow[s], lrow[s]);
    }
  }
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
                       const PagedArgs* paged) {
  void* part_o = ws + plan.o_off;
  float2* part_ml = reinterpret_cast<float2*>(ws + plan.ml_off);
  const float sl2 = scale * kLog2e;
  dim3 grid(plan.chunks, plan.row_tiles, B * Hkv);
  const int64_t groups = int64_t(B) * Hkv * plan.chunks;
  dim3 grid1(unsigned((groups + 7) / 8 * 8 * plan.row_tiles));
  prof_begin(s, TR_KERNEL_ATTN_PREFIX);
  if (is_bf16) {
    const auto* qq = reinterpret_cast<const uint16_t*>(q);
    const auto* kk = reinterpret_cast<const uint16_t*>(k_cache);
    const auto* vv = reinterpret_cast<const uint16_t*>(v_cache);
    const PagedArgs pa = paged ? *paged : PagedArgs{};
    const auto* kt = reinterpret_cast<const uint16_t*>(k_tree);
    const auto* vt = reinterpret_cast<const uint16_t*>(v_tree);
#define TR_PREFIX(SPWV, PG)                                                                       \
  hipLaunchKernelGGL((attn_prefix_bf16<SPWV, PG>), grid1, dim3(64 * kWaves), 0, s, qq, kk, vv,  \
                     kt, vt, tree, cap, prefix_len, Hq, Hkv, plan.G, plan.R, plan.chunks, sl2,      \
                     reinterpret_cast<uint16_t*>(part_o), part_ml, ws, B, plan.row_tiles, pa)
    if (plan.spw == 2) {
      if (paged) TR_PREFIX(2, true); else TR_PREFIX(2, false);
    } else {
      if (paged) TR_PREFIX(1, true); else TR_PREFIX(1, false);
    }
#undef TR_PREFIX
  } else {
    hipLaunchKernelGGL(attn_prefix_f32, grid, dim3(256), 0, s, reinterpret_cast<const float*>(q),
                       reinterpret_cast<const float*>(k_cache), reinterpret_cast<const float*>(v_cache),
                       cap, prefix_len, tree.T, Hq, Hkv, plan.G, plan.R, plan.chunks, sl2,
                       reinterpret_cast<float*>(part_o), part_ml, ws);
  }
  prof_end(s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = int64_t(B) * tree.T * Hq;
  dim3 cgrid(unsigned((rows + 7) / 8));
  const int Rpad = plan.row_tiles * plan.tile_rows;
  prof_begin(s, TR_KERNEL_ATTN_COMBINE);
#define TR_COMBINE(BF, UN, TRV)                                                               \
  hipLaunchKernelGGL((attn_combine<BF, UN, TRV>), cgrid, dim3(128), 0, s, tree, q, k_tree, v_tree, \
                     B, Hq, Hkv, plan.G, plan.chunks, Rpad, sl2, part_o, part_ml, out)
  const bool un = Hq % 4 == 0;
  if (is_bf16) {                                    // the prefix pass took the tree keys
    if (un) TR_COMBINE(true, true, false); else TR_COMBINE(true, false, false);
  } else {
    if (un) TR_COMBINE(false, true, true); else TR_COMBINE(false, false, true);
  }
#undef TR_COMBINE
  prof_end(s);
  return hipGetLastError();
}

}  // namespace tr
