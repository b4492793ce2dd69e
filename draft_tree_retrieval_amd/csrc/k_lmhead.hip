// LM head fused with the top-k of its logits: z = h W^T (h [R][H] hidden
// states of the tree nodes, W [V][H] the output embedding, both bfloat16,
// float32 accumulation), and for every row the k best ids of z, selected as
// the top-k step selects them (value descending, ties to the lower id), so
// the logits never reach HBM.  The update M[x~_i] = argtopk(p~_{i+1}) only
// needs those ids (Chinese summary of "Token Recycling", section Method);
// softmax is increasing, so selecting on z is selecting on p.
//
// Decode-sized R makes this a skinny product bound by streaming W once:
// each block owns 128 vocabulary rows and 96 query rows with 8 waves.
// Four consumer waves own two 16-row vocabulary tiles each.  A consumer
// loads its W tiles straight from HBM into registers: per 128-k
// super-step, 256 contiguous bytes of each row, from four loads issued
// back to back that each read 64 contiguous bytes of the tile's 16 rows
// (the A operand of one v_mfma_f32_16x16x32_bf16 step), with four
// super-steps in flight.  Four producer waves copy the
// h chunk of each super-step HBM/L2 -> LDS with the LDS DMA
// (global_load_lds_dwordx4), three chunks ahead, in an XOR-swizzled layout
// that keeps the B operand reads (16 rows, one 16-byte column chunk)
// conflict-free; each B operand read serves both of a consumer's tiles.  A
// wave's load counter completes in issue order, so keeping the h copies in
// waves of their own means no consumer ever waits for an h chunk behind its
// W loads.
//
// Epilogue, per query row: a consumer lane holds 8 of the block's 128
// logits (a holder; 16 holders per row).  The threshold T is the 8th
// largest of the 16 holder maxima: at least eight holders reach it, so
// nothing below it is among the row's 8 best.  The values reaching T (10
// on average for random logits, at most 128) go to a per-row LDS list as
// 64-bit keys (order code, then the complemented id); a thread per
// candidate counts the row's larger keys and writes ranks 0..7, so the
// block's 8 best per row land descending.  The block's super-steps start at
// a chunk that differs between the blocks an XCD runs at once.  A second
// kernel (one block per row) merges the slices.
#include "dev_common.h"

namespace tr {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kLhRows = 96;     // query rows per block (6 tiles of 16)
constexpr int kLhTiles = kLhRows / 16;
constexpr int kLhCons = 4;      // consumer waves: two 16-row vocabulary tiles each
constexpr int kLhVtW = 2;
constexpr int kLhProd = 4;      // producer waves: the h chunk DMA
constexpr int kLhDmaPerProd = kLhRows * 16 / 64 / kLhProd;    // 6 DMA loads per chunk each
constexpr int kLhKc = 128;      // k per super-step (one staged h chunk)
constexpr int kLhWRing = 8;     // W k-steps (32 k) held per consumer wave, seven in flight
constexpr int kLhUnroll = 4;    // steps per loop round
constexpr int kLhHBuf = 4;      // staged h chunks (three in flight ahead of the one in use)
constexpr int kLhChunkBytes = kLhRows * kLhKc * 2;      // 24 KB
constexpr int kLhCand = 128;    // candidate slots per row (every logit of the block)
constexpr int kLhRowsPerBuf = kLhChunkBytes / (kLhCand * 8);   // candidate lists per h buffer
static_assert(kLhRowsPerBuf * kLhHBuf >= kLhRows, "the candidate lists fit the h buffers");

}  // namespace

__global__ __launch_bounds__(512) void lmhead_topk_kernel(const uint16_t* __restrict__ h,
                                                           const uint16_t* W, int R, int H,
                                                           int64_t V, int nvs,
                                                           uint64_t* __restrict__ part) {
  // Four separate h buffers (the unrolled loops name each one statically):
  // with one array the compiler could not tell an LDS read from DMA writes
  // still in flight elsewhere in it.  After the loop they hold the
  // candidate lists.
  __shared__ __attribute__((aligned(16))) uint8_t hbuf0[kLhChunkBytes];
  __shared__ __attribute__((aligned(16))) uint8_t hbuf1[kLhChunkBytes];
  __shared__ __attribute__((aligned(16))) uint8_t hbuf2[kLhChunkBytes];
  __shared__ __attribute__((aligned(16))) uint8_t hbuf3[kLhChunkBytes];
  __shared__ __attribute__((aligned(16))) uint32_t s_hm[kLhRows][16];   // holder maxima
  __shared__ uint32_t s_thr[kLhRows];
  __shared__ __attribute__((aligned(16))) uint32_t s_cnt[kLhRows];
  static_assert(kLhHBuf == 4 && kLhUnroll % kLhHBuf == 0 && (4 * kLhUnroll) % kLhWRing == 0,
                "a static buffer and ring slot per unrolled step");
  auto hbuf = [&](int i) -> uint8_t* {
    return i == 0 ? hbuf0 : i == 1 ? hbuf1 : i == 2 ? hbuf2 : hbuf3;
  };
  constexpr int kThreads = 64 * (kLhCons + kLhProd);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, g = lane >> 4;
  const int vs = blockIdx.x;
  const int row0 = blockIdx.y * kLhRows;
  const int nsteps = H / kLhKc;
  // Super-step c of this block covers chunk (c + rot) mod nsteps: the 32
  // blocks an XCD runs at once read different h chunks (its L2 serves them
  // from different channels) instead of all reading the same one.
  const int rot = (vs / 8) % nsteps;
  auto chunk = [&](int c) { const int cc = c + rot; return cc >= nsteps ? cc - nsteps : cc; };
  // every wave passes the same number of barriers: whole loop rounds
  const int nround = (nsteps + kLhUnroll - 1) / kLhUnroll * kLhUnroll;
  if (tid < kLhRows) s_cnt[tid] = 0;

  // Waves kLhCons.. are producers: they alone DMA the h chunks, so the
  // consumers' in-order load counters hold W loads only and their W ring
  // never waits behind an h chunk.  Step c's barrier releases chunk c: the
  // producers reach it once their part of chunk c has landed, the
  // consumers once they are done with chunk c-1, whose buffer the
  // producers then refill with chunk c+3.
  if (w >= kLhCons) {
    const int pw = w - kLhCons;
    // chunk c into buffer b: 1536 16-byte slots, slot p = row p/16,
    // position p%16 holding column chunk (p%16) ^ (row & 15)
    auto stage_h = [&](int c, int b) {
#pragma unroll
      for (int q = 0; q < kLhDmaPerProd; ++q) {
        const int base = (q * kLhProd + pw) * 64;              // wave-uniform first slot
        const int p = base + lane;
        const int r = p >> 4, pos = p & 15, cc = pos ^ (r & 15);
        const int hr = min(row0 + r, R - 1);
        const uint16_t* src = h + int64_t(hr) * H + chunk(c) * kLhKc + cc * 8;
        __builtin_amdgcn_global_load_lds(src, hbuf(b) + base * 16, 16, 0, 0);
      }
      asm volatile("" ::: "memory");
    };
#pragma unroll
    for (int c = 0; c < kLhHBuf - 1; ++c) stage_h(min(c, nsteps - 1), c);
    for (int c0 = 0; c0 < nround; c0 += kLhUnroll) {
#pragma unroll
      for (int j = 0; j < kLhUnroll; ++j) {
        const int c = c0 + j;
        // chunks c+1 and c+2 (kLhDmaPerProd loads each) may still fly
        static_assert(2 * kLhDmaPerProd == 12, "vmcnt below");
        __builtin_amdgcn_s_waitcnt(0x0F7C);        // vmcnt(12), lgkm/exp not waited
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        stage_h(min(c + kLhHBuf - 1, nsteps - 1), (j + kLhHBuf - 1) % kLhHBuf);
      }
    }
  }

  floatx4 acc[kLhVtW][kLhTiles];
#pragma unroll
  for (int j = 0; j < kLhVtW; ++j)
#pragma unroll
    for (int t = 0; t < kLhTiles; ++t) acc[j][t] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int64_t v0 = int64_t(vs) * (kLhCons * kLhVtW * 16) + w * (kLhVtW * 16);   // this wave's tiles
  if (w < kLhCons) {
    // W rows past V repeat the last row (their keys are dropped below)
    const uint16_t* wp[kLhVtW];
#pragma unroll
    for (int j = 0; j < kLhVtW; ++j) {
      const int64_t vrow = v0 + 16 * j + li < V ? v0 + 16 * j + li : V - 1;
      wp[j] = W + vrow * H + 8 * g;
    }
    // k-step q (32 k, the A operand of one MFMA step): 64 contiguous bytes of
    // each of the tile's 16 rows (lane group g the g-th 16 bytes); k-steps
    // past the end repeat the last one
    const int nq = 4 * nsteps;
    auto load_w = [&](u32x4 (&r)[kLhVtW], int q) __attribute__((always_inline)) {
      q = min(q, nq - 1);
#pragma unroll
      for (int j = 0; j < kLhVtW; ++j)
        r[j] = *reinterpret_cast<const u32x4*>(wp[j] + chunk(q >> 2) * kLhKc + 32 * (q & 3));
      // (keeps the ring in issue order, so each wait below leaves exactly
      // the younger k-steps in flight)
      asm volatile("" ::: "memory");
    };
    u32x4 wr[kLhWRing][kLhVtW];
#pragma unroll
    for (int q = 0; q < kLhWRing; ++q) load_w(wr[q], q);
    for (int c0 = 0; c0 < nround; c0 += kLhUnroll) {
#pragma unroll
      for (int j = 0; j < kLhUnroll; ++j) {
        const int c = c0 + j;                       // steps past the end only wait
        const uint8_t* hb = hbuf(j % kLhHBuf);
        // row 16 t + li sits at byte (16 t + li) * 256, its column chunk
        // 4 s + g at position (4 s + g) ^ li (row & 15 == li).  The B
        // operands of MFMA step s + 1 are read while step s multiplies.
        bf16x8 bv[2][kLhTiles];
        auto read_b = [&](bf16x8 (&b)[kLhTiles], int s) __attribute__((always_inline)) {
          const uint8_t* hs = hb + li * 256 + (((4 * s + g) ^ li) << 4);
#pragma unroll
          for (int t = 0; t < kLhTiles; ++t) b[t] = *reinterpret_cast<const bf16x8*>(hs + t * 4096);
        };
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          constexpr int kYoung = (kLhWRing - 1) * kLhVtW;   // loads of the younger k-steps
          static_assert(kYoung == 14, "vmcnt below");
          // k-step 4c + s landed; only the younger ones' loads may still fly.
          // Written out: the compiler's own count is lost across the loop's
          // back edge and would drain every load at the first step of a round.
          __builtin_amdgcn_s_waitcnt(0x0F7E);      // vmcnt(14), lgkm/exp not waited
          asm volatile("" ::: "memory");
          if (s == 0) {                             // h chunk c is in and its buffer free
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            if (c < nsteps) read_b(bv[0], 0);
          }
          if (c < nsteps) {
            if (s < 3) read_b(bv[(s + 1) & 1], s + 1);
            __builtin_amdgcn_sched_barrier(0);      // keep the reads ahead of the products
            const int slot = (4 * j + s) % kLhWRing;
#pragma unroll
            for (int t = 0; t < kLhTiles; ++t)
#pragma unroll
              for (int vj = 0; vj < kLhVtW; ++vj)
                acc[vj][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, wr[slot][vj]), bv[s & 1][t], acc[vj][t], 0, 0, 0);
          }
          if (s == 3) {
            // the LDS reads of this chunk are done before the next barrier
            __builtin_amdgcn_s_waitcnt(0xC07F);    // lgkmcnt(0), vm/exp not waited
            asm volatile("" ::: "memory");
          }
          load_w(wr[(4 * j + s) % kLhWRing], 4 * c + s + kLhWRing);
        }
      }
    }
  }

  // ---- epilogue.  Lane (li, g) of consumer w holds z for vocabulary id
  // v0 + 16 j + 4 g + e (tile j of the wave) and query row 16 t + li.
  uint32_t code[kLhVtW][kLhTiles][4];
  if (w < kLhCons) {
#pragma unroll
    for (int j = 0; j < kLhVtW; ++j)
#pragma unroll
      for (int t = 0; t < kLhTiles; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t vid = v0 + 16 * j + 4 * g + e;
          code[j][t][e] = vid < V ? ord32(__float_as_uint(acc[j][t][e])) : 0u;   // 0: no id
        }
#pragma unroll
    for (int t = 0; t < kLhTiles; ++t) {
      uint32_t m = code[0][t][0];
#pragma unroll
      for (int j = 0; j < kLhVtW; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) m = max(m, code[j][t][e]);
      s_hm[16 * t + li][4 * w + g] = m;
    }
  }
  __syncthreads();                                // the h buffers are free from here

  // ---- the row's threshold: the 8th largest of its 16 holder maxima (at
  // least eight holders reach it, so nothing below it is among the 8 best).
  // Thread (row, i) writes it when maximum i is that value.
  for (int idx = tid; idx < kLhRows * 16; idx += kThreads) {
    const int row = idx >> 4, i = idx & 15;
    const uint32_t mi = s_hm[row][i];
    int gt = 0, ge = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 mq = *reinterpret_cast<const u32x4*>(&s_hm[row][4 * q]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gt += mq[e] > mi;
        ge += mq[e] >= mi;
      }
    }
    if (gt < 8 && ge >= 8) s_thr[row] = mi;
  }
  __syncthreads();

  // ---- candidates: the values reaching the row's threshold
  // slot s of row r sits at position s ^ (r & 15) of the row's list, so the
  // same slot of 16 consecutive rows lies in 16 different banks
  auto cand = [&](int row) -> uint64_t* {
    return reinterpret_cast<uint64_t*>(hbuf(row / kLhRowsPerBuf)) + (row % kLhRowsPerBuf) * kLhCand;
  };
  if (w < kLhCons) {
    // one slot reservation per lane and row (all six in flight at once),
    // then plain stores
    uint32_t T[kLhTiles], n[kLhTiles], slot[kLhTiles];
#pragma unroll
    for (int t = 0; t < kLhTiles; ++t) T[t] = s_thr[16 * t + li];
#pragma unroll
    for (int t = 0; t < kLhTiles; ++t) {
      n[t] = 0;
#pragma unroll
      for (int j = 0; j < kLhVtW; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) n[t] += code[j][t][e] >= T[t];
    }
#pragma unroll
    for (int t = 0; t < kLhTiles; ++t) slot[t] = n[t] ? atomicAdd(&s_cnt[16 * t + li], n[t]) : 0u;
#pragma unroll
    for (int t = 0; t < kLhTiles; ++t) {
      uint64_t* list = cand(16 * t + li);
#pragma unroll
      for (int j = 0; j < kLhVtW; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t c = code[j][t][e];
          if (c >= T[t]) list[(slot[t]++) ^ li] = key_of(c, uint32_t(v0 + 16 * j + 4 * g + e));
        }
    }
  }
  __syncthreads();

  // ---- lane (row, slot): the candidate's rank among the row's (all keys
  // differ: distinct ids), ranks 0..7 written (code 0, ids past V, as key 0),
  // so the block's 8 best per row land descending (a row has at least 8
  // candidates).  A wave takes 4 rows at a time, 16 lanes per row; the keys
  // are read 4 at a time over the aligned 16-position blocks that hold
  // slots 0 .. n-1, the positions of slots past n skipped.
  for (int rg = w; rg < kLhRows / 4; rg += kThreads / 64) {
    const int row = 4 * rg + g;
    const int n = int(s_cnt[row]);
    const uint64_t* list = cand(row);
    const int sw = row & 15;
    for (int slot = li; slot < n; slot += 16) {
      const uint64_t x = list[slot ^ sw];
      int rank = 0;
      for (int p0 = 0; p0 < ((n + 15) & ~15); p0 += 4) {   // the swizzle stays within 16
        const u64x2 a = *reinterpret_cast<const u64x2*>(list + p0);
        const u64x2 b = *reinterpret_cast<const u64x2*>(list + p0 + 2);
        const uint64_t y[4] = {a[0], a[1], b[0], b[1]};
#pragma unroll
        for (int q = 0; q < 4; ++q) rank += (((p0 + q) ^ sw) < n) & (y[q] > x);
      }
      if (rank < 8 && row0 + row < R)
        part[(int64_t(row0 + row) * nvs + vs) * 8 + rank] = (x >> 32) ? x : 0ull;
    }
  }
}

hipError_t launch_lmhead(const void* h, const void* W, int32_t R, int32_t H, int64_t V,
                         uint64_t* part, int32_t nvs, hipStream_t s) {
  dim3 grid(unsigned(nvs), unsigned((R + kLhRows - 1) / kLhRows));
  prof_begin(s, TR_KERNEL_LMHEAD);
  hipLaunchKernelGGL(lmhead_topk_kernel, grid, dim3(64 * (kLhCons + kLhProd)), 0, s,
                     reinterpret_cast<const uint16_t*>(h), reinterpret_cast<const uint16_t*>(W),
                     R, H, V, nvs, part);
  prof_end(s);
  return hipGetLastError();
}

}  // namespace tr
