// LM head fused with the top-k of its logits: z = h W^T (h [R][H] hidden
// states of the tree nodes, W [V][H] the output embedding, both bfloat16,
// float32 accumulation), and for every row the k best ids of z, selected as
// the top-k step selects them (value descending, ties to the lower id), so
// the logits never reach HBM.  The update M[x~_i] = argtopk(p~_{i+1}) only
// needs those ids (Chinese summary of "Token Recycling", section Method);
// softmax is increasing, so selecting on z is selecting on p.
//
// Decode-sized R makes this a skinny product bound by streaming W once:
// each block owns 128 vocabulary rows and 96 query rows with 12 waves.
// Eight consumer waves own one 16-row vocabulary tile each; a consumer
// loads its W tile straight from HBM into registers, 64 contiguous bytes
// per lane per 128-k super-step, four super-steps in flight, and uses it as
// the A operand of v_mfma_f32_16x16x32_bf16.  Four producer waves copy the
// h chunk of each super-step HBM/L2 -> LDS with the LDS DMA
// (global_load_lds_dwordx4), three chunks ahead, in an XOR-swizzled layout
// that keeps the B operand reads (16 rows, one 16-byte column chunk)
// conflict-free.  A wave's load counter completes in issue order, so
// keeping the h copies in waves of their own means no consumer ever waits
// for an h chunk behind its W loads.  The contraction index is permuted
// consistently on both operands: MFMA step s of a super-step, lane group
// g, element e stands for k = 32 g + 8 s + e, so a lane's 64 loaded bytes
// feed its four steps.
//
// Epilogue: a consumer lane holds 4 vocabulary ids x 1 query row per row
// tile.  The 16 keys of a query row in a wave are sorted and merged across
// the four lane groups down to the wave's 8 best; the eight lists of a row
// are merged pairwise in three rounds by all threads, and the block writes
// its 8 best keys per row.  A second kernel (one block per row) merges the
// slices.
#include "dev_common.h"

namespace tr {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kLhRows = 96;     // query rows per block (6 tiles of 16)
constexpr int kLhTiles = kLhRows / 16;
constexpr int kLhCons = 8;      // consumer waves: one 16-row vocabulary tile each
constexpr int kLhProd = 4;      // producer waves: the h chunk DMA
constexpr int kLhDmaPerProd = kLhRows * 16 / 64 / kLhProd;    // 6 DMA loads per chunk each
constexpr int kLhKc = 128;      // k per super-step (one staged h chunk)
constexpr int kLhRing = 4;      // W super-steps in flight per consumer wave
constexpr int kLhUnroll = 4;    // steps per loop round
constexpr int kLhHBuf = 4;      // staged h chunks (three in flight ahead of the one in use)
constexpr int kLhChunkBytes = kLhRows * kLhKc * 2;      // 24 KB

__device__ __forceinline__ void ce(uint64_t& a, uint64_t& b) {   // a >= b afterwards
  const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
  a = hi;
  b = lo;
}

// The 8 best of two descending lists of 8, descending.
__device__ __forceinline__ void merge8(uint64_t (&a)[8], const uint64_t (&b)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = a[i] > b[7 - i] ? a[i] : b[7 - i];   // bitonic
#pragma unroll
  for (int j = 4; j > 0; j >>= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((i & j) == 0) ce(a[i], a[i + j]);
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) { return shfl_xor_u64(v, m); }

}  // namespace

__global__ __launch_bounds__(768) void lmhead_topk_kernel(const uint16_t* __restrict__ h,
                                                           const uint16_t* W, int R, int H,
                                                           int64_t V, int nvs,
                                                           uint64_t* __restrict__ part) {
  // Four separate h buffers (the unrolled loops name each one statically)
  // and a separate key table: with one array the compiler could not tell
  // an LDS read from DMA writes still in flight elsewhere in it.
  __shared__ __attribute__((aligned(16))) uint8_t hbuf0[kLhChunkBytes];
  __shared__ __attribute__((aligned(16))) uint8_t hbuf1[kLhChunkBytes];
  __shared__ __attribute__((aligned(16))) uint8_t hbuf2[kLhChunkBytes];
  __shared__ __attribute__((aligned(16))) uint8_t hbuf3[kLhChunkBytes];
  __shared__ uint64_t s_top[kLhRows * 64];                              // 48 KB
  static_assert(kLhHBuf == 4 && kLhUnroll % kLhHBuf == 0 && kLhUnroll % kLhRing == 0,
                "a static buffer and ring slot per unrolled step");
  auto hbuf = [&](int i) -> uint8_t* {
    return i == 0 ? hbuf0 : i == 1 ? hbuf1 : i == 2 ? hbuf2 : hbuf3;
  };
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, g = lane >> 4;
  const int vs = blockIdx.x;
  const int row0 = blockIdx.y * kLhRows;
  const int nsteps = H / kLhKc;
  // every wave passes the same number of barriers: whole loop rounds
  const int nround = (nsteps + kLhUnroll - 1) / kLhUnroll * kLhUnroll;

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
        const uint16_t* src = h + int64_t(hr) * H + c * kLhKc + cc * 8;
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

  floatx4 acc[kLhTiles];
#pragma unroll
  for (int t = 0; t < kLhTiles; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int64_t v0 = int64_t(vs) * (kLhCons * 16) + w * 16;     // this wave's vocabulary tile
  if (w < kLhCons) {
    // W rows past V repeat the last row (their keys are dropped below)
    const int64_t vrow = v0 + li < V ? v0 + li : V - 1;
    const uint16_t* wp = W + vrow * H + 32 * g;
    auto load_w = [&](u32x4 (&r)[4], int c) {
      const u32x4* p = reinterpret_cast<const u32x4*>(wp + c * kLhKc);
#pragma unroll
      for (int s = 0; s < 4; ++s) r[s] = p[s];
    };
    // (compiler memory barriers keep the ring in issue order, so the wait
    // before a slot's first use leaves the younger slots in flight)
    u32x4 wr[kLhRing][4];
#pragma unroll
    for (int j = 0; j < kLhRing; ++j) {
      load_w(wr[j], min(j, nsteps - 1));
      asm volatile("" ::: "memory");
    }
    for (int c0 = 0; c0 < nround; c0 += kLhUnroll) {
#pragma unroll
      for (int j = 0; j < kLhUnroll; ++j) {
        const int c = c0 + j;                       // steps past the end only wait
        // W(c): the younger ring slots (3 x 4 loads) may stay in flight.
        // Written out: the compiler's own count is lost across the loop's
        // back edge and would drain every load at the first step of a round.
        static_assert((kLhRing - 1) * 4 == 12, "vmcnt below");
        __builtin_amdgcn_s_waitcnt(0x0F7C);        // vmcnt(12), lgkm/exp not waited
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (c < nsteps) {
          const uint8_t* hb = hbuf(j % kLhHBuf);
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, wr[j % kLhRing][s]);
            // row 16 t + li sits at byte (16 t + li) * 256, its column chunk
            // 4 g + s at position (4 g + s) ^ li (row & 15 == li)
            const uint8_t* hs = hb + li * 256 + (((4 * g + s) ^ li) << 4);
#pragma unroll
            for (int t = 0; t < kLhTiles; ++t) {
              const bf16x8 bv = *reinterpret_cast<const bf16x8*>(hs + t * 4096);
              acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv, acc[t], 0, 0, 0);
            }
          }
        }
        // the LDS reads of this step are done before the next barrier
        __builtin_amdgcn_s_waitcnt(0xC07F);        // lgkmcnt(0), vm/exp not waited
        asm volatile("" ::: "memory");
        load_w(wr[j % kLhRing], min(c + kLhRing, nsteps - 1));
        asm volatile("" ::: "memory");
      }
    }
  }

  // ---- epilogue: per query row 16 t + li, a consumer lane's keys are
  // vocabulary ids v0 + 4 g + e
  __syncthreads();
  if (w < kLhCons) {
#pragma unroll
    for (int t = 0; t < kLhTiles; ++t) {
      uint64_t kk[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t vid = v0 + 4 * g + e;
        kk[e] = vid < V ? make_key(__float_as_uint(acc[t][e]), uint32_t(vid)) : 0ull;
      }
      ce(kk[0], kk[1]);
      ce(kk[2], kk[3]);
      ce(kk[0], kk[2]);
      ce(kk[1], kk[3]);
      ce(kk[1], kk[2]);
      // with lane group g ^ 1: the 8 keys of both, descending
#pragma unroll
      for (int e = 0; e < 4; ++e) kk[4 + e] = shfl_xor64(kk[3 - e], 16);   // partner's, ascending
#pragma unroll
      for (int j = 4; j > 0; j >>= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if ((i & j) == 0) ce(kk[i], kk[i + j]);
      // with lane group g ^ 2: the 8 best of the 16
      uint64_t other[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) other[e] = shfl_xor64(kk[e], 32);
      merge8(kk, other);
      // lanes of group g write keys 2 g, 2 g + 1 of the wave's 8
      const int row = t * 16 + li;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if ((e >> 1) == g) s_top[row * 64 + w * 8 + e] = kk[e];
    }
  }
  __syncthreads();
  // The block's 8 best of each row: the 8 descending lists of a row (one
  // per consumer wave) merged pairwise in three rounds, one thread per
  // pair; list i of row r sits at s_top[r * 64 + 8 i].
  constexpr int kThreads = 64 * (kLhCons + kLhProd);
#pragma unroll
  for (int span = 1; span < kLhCons; span <<= 1) {
    const int pairs = kLhCons / (2 * span);
    for (int task = tid; task < kLhRows * pairs; task += kThreads) {
      const int row = task / pairs, pr = task - row * pairs;
      uint64_t* a = s_top + row * 64 + 8 * (2 * pr * span);
      const uint64_t* b = a + 8 * span;
      uint64_t x[8], y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = a[e];
        y[e] = b[e];
      }
      merge8(x, y);
      if (span * 2 < kLhCons) {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = x[e];
      } else if (row0 + row < R) {
#pragma unroll
        for (int e = 0; e < 8; ++e) part[(int64_t(row0 + row) * nvs + vs) * 8 + e] = x[e];
      }
    }
    __syncthreads();
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
