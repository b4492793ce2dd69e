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

constexpr int kSub = 64;          // keys per staged sub-block (bf16)
constexpr int kKsStride = 136;    // bf16 per staged K row: 272 bytes, conflict-free b128 reads
constexpr int kSpw = 2;           // 16-row strips per wave
constexpr int kRowsPerTile = 4 * kSpw * 16;
constexpr float kLog2e = 1.4426950408889634f;

AttnPlan plan_attn(int32_t T, int32_t B, int32_t Hq, int32_t Hkv, int64_t cap) {
  AttnPlan p{};
  p.G = Hq / Hkv;
  p.R = T * p.G;
  p.row_tiles = (p.R + kRowsPerTile - 1) / kRowsPerTile;
  int64_t base = int64_t(B) * Hkv * p.row_tiles;
  int64_t chunks = (256 + base - 1) / base;
  int64_t by_cap = (cap + kSub - 1) / kSub;
  if (chunks > by_cap) chunks = by_cap;
  if (chunks > 64) chunks = 64;
  if (chunks < 1) chunks = 1;
  p.chunks = int32_t(chunks);
  const size_t rpad = size_t(p.row_tiles) * kRowsPerTile;
  const size_t units = size_t(B) * Hkv * p.chunks * rpad;
  size_t off = kDataOff;
  p.o_off = off;
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

__device__ __forceinline__ int vt_swz(int row) { return (row + (row >> 4)) & 15; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- bf16 prefix
__global__ __launch_bounds__(256) void attn_prefix_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int64_t cap, const int32_t* __restrict__ prefix_len, int T,
    int Hq, int Hkv, int G, int R, int chunks, float sl2, float* __restrict__ part_o,
    float2* __restrict__ part_ml, uint8_t* ws) {
  const int c = blockIdx.x, rt = blockIdx.y, z = blockIdx.z;
  const int b = z / Hkv, kvh = z - b * Hkv;
  const int P = clamp_prefix(prefix_len[b], cap, ws, c == 0 && rt == 0 && kvh == 0 && threadIdx.x == 0);
  const int cs = chunk_len(P, chunks, kSub);
  const int k0 = c * cs;
  const int k1 = min(P, k0 + cs);
  if (k0 >= k1) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, g = lane >> 4;
  const int Rpad = gridDim.y * kRowsPerTile;

  __shared__ __attribute__((aligned(16))) uint16_t Ks[kSub * kKsStride];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kHeadDim * kSub];

  bf16x8 qb[kSpw][4];
#pragma unroll
  for (int s = 0; s < kSpw; ++s) {
    const int r = rt * kRowsPerTile + (w * kSpw + s) * 16 + li;
    if (r < R) {
      const int n = r / G, gq = r - n * G;
      const uint16_t* qp = q + ((int64_t(b) * T + n) * Hq + kvh * G + gq) * kHeadDim;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qb[s][ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32 + g * 8);
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qb[s][ks] = bf16x8{};
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
  const uint16_t* kbase = kc + head_off;
  const uint16_t* vbase = vc + head_off;
  const int cch = tid & 15;     // 16-byte column chunk of a 256-byte row
  const int rq = tid >> 4;      // 0..15

  u32x4 kreg[4], vreg[4];
  auto load_sub = [&](int kb) {
    const int nk = min(kSub, k1 - kb);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rk = rq + 16 * j;
      kreg[j] = rk < nk ? *reinterpret_cast<const u32x4*>(kbase + int64_t(kb + rk) * kHeadDim + cch * 8)
                        : u32x4{0, 0, 0, 0};
      const int rv = 4 * rq + j;
      vreg[j] = rv < nk ? *reinterpret_cast<const u32x4*>(vbase + int64_t(kb + rv) * kHeadDim + cch * 8)
                        : u32x4{0, 0, 0, 0};
    }
  };
  load_sub(k0);

  for (int kb = k0; kb < k1; kb += kSub) {
    const int nk = min(kSub, k1 - kb);
    __syncthreads();
    // stage K rows and V transposed (4 keys x 8 d per thread)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x4*>(&Ks[(rq + 16 * j) * kKsStride + cch * 8]) = kreg[j];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = cch * 8 + e;
      const int hw = e >> 1;
      uint32_t x0, x1;
      if (e & 1) {
        x0 = (vreg[0][hw] >> 16) | (vreg[1][hw] & 0xFFFF0000u);
        x1 = (vreg[2][hw] >> 16) | (vreg[3][hw] & 0xFFFF0000u);
      } else {
        x0 = (vreg[0][hw] & 0xFFFFu) | (vreg[1][hw] << 16);
        x1 = (vreg[2][hw] & 0xFFFFu) | (vreg[3][hw] << 16);
      }
      *reinterpret_cast<u32x2*>(&Vt[d * kSub + ((rq ^ vt_swz(d)) * 4)]) = u32x2{x0, x1};
    }
    __syncthreads();
    if (kb + kSub < k1) load_sub(kb + kSub);

    // S^T = K Q^T for 4 tiles of 16 keys
    floatx4 sacc[kSpw][4];
#pragma unroll
    for (int s = 0; s < kSpw; ++s)
#pragma unroll
      for (int t = 0; t < 4; ++t) sacc[s][t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[(t * 16 + li) * kKsStride + ks * 32 + g * 8]);
#pragma unroll
        for (int s = 0; s < kSpw; ++s)
          sacc[s][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[s][ks], sacc[s][t], 0, 0, 0);
      }
    }

    // online softmax per query row (the lane's column)
    bf16x8 pb[kSpw][2];
#pragma unroll
    for (int s = 0; s < kSpw; ++s) {
      float x[4][4];
      float mloc = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = t * 16 + 4 * g + i;
          x[t][i] = key < nk ? sacc[s][t][i] * sl2 : -INFINITY;
          mloc = fmaxf(mloc, x[t][i]);
        }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
      const float mnew = fmaxf(mrow[s], mloc);
      const float alpha = fast_exp2(mrow[s] - mnew);
      float psum = 0.f;
      uint16_t ph[4][4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pr = fast_exp2(x[t][i] - mnew);
          psum += pr;
          ph[t][i] = f32_to_bf16(pr);
        }
      psum += __shfl_xor(psum, 16, 64);
      psum += __shfl_xor(psum, 32, 64);
      lrow[s] = lrow[s] * alpha + psum;
      mrow[s] = mnew;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc[s][dt] *= alpha;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        u32x4 u;
        u[0] = uint32_t(ph[2 * pp][0]) | (uint32_t(ph[2 * pp][1]) << 16);
        u[1] = uint32_t(ph[2 * pp][2]) | (uint32_t(ph[2 * pp][3]) << 16);
        u[2] = uint32_t(ph[2 * pp + 1][0]) | (uint32_t(ph[2 * pp + 1][1]) << 16);
        u[3] = uint32_t(ph[2 * pp + 1][2]) | (uint32_t(ph[2 * pp + 1][3]) << 16);
        pb[s][pp] = __builtin_bit_cast(bf16x8, u);
      }
    }

    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int row = dt * 16 + li;
      const int sw = vt_swz(row);
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const u32x2 lo = *reinterpret_cast<const u32x2*>(&Vt[row * kSub + (((8 * pp + g) ^ sw) * 4)]);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(&Vt[row * kSub + (((8 * pp + 4 + g) ^ sw) * 4)]);
        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
        for (int s = 0; s < kSpw; ++s)
          acc[s][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[s][pp], acc[s][dt], 0, 0, 0);
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
  if (k0 >= k1) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, g = lane >> 4;
  const int Rpad = gridDim.y * kRowsPerTile;

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
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
        const float mnew = fmaxf(mrow[s], mloc);
        const float alpha = fast_exp2(mrow[s] - mnew);
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = fast_exp2(x[i] - mnew);
          psum += x[i];
        }
        psum += __shfl_xor(psum, 16, 64);
        psum += __shfl_xor(psum, 32, 64);
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
// One wave per output row (b, n, h); lane l owns d = 2l, 2l+1.  Merges the
// prefix chunk partials (chunks in order) and then the tree keys of n's
// path (n, its parent, ..., the root), all with an online softmax.
template <bool BF16>
__global__ __launch_bounds__(256) void attn_combine(
    TreeDev tree, const void* __restrict__ q, const void* __restrict__ kt,
    const void* __restrict__ vt, const int32_t* __restrict__ prefix_len, int B, int Hq, int Hkv,
    int G, int chunks, int Rpad, float sl2, const float* __restrict__ part_o,
    const float2* __restrict__ part_ml, void* __restrict__ out, int64_t cap) {
  const int T = tree.T;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= int64_t(B) * T * Hq) return;
  const int lane = threadIdx.x & 63;
  const int h = int(row % Hq);
  const int n = int((row / Hq) % T);
  const int b = int(row / (int64_t(Hq) * T));
  const int kvh = h / G, gq = h - kvh * G;
  const int r = n * G + gq;
  const int z = b * Hkv + kvh;

  auto ld2 = [&](const void* base, int64_t elem) -> float2 {
    if (BF16) {
      const uint32_t u = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(base) + elem);
      return make_float2(bf16_to_f32(uint16_t(u & 0xFFFFu)), bf16_to_f32(uint16_t(u >> 16)));
    } else {
      return *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(base) + elem);
    }
  };

  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  const int P = clamp_prefix(prefix_len[b], cap, nullptr, false);
  const int cs = chunk_len(P, chunks, kSub);
  for (int c = 0; c < chunks; ++c) {
    if (int64_t(c) * cs >= P) break;
    const int64_t unit = (int64_t(z) * chunks + c) * Rpad + r;
    const float2 ml = part_ml[unit];
    const float2 ov = *reinterpret_cast<const float2*>(part_o + unit * kHeadDim + 2 * lane);
    const float mn = fmaxf(m, ml.x);
    const float a = fast_exp2(m - mn), e = fast_exp2(ml.x - mn);
    l = l * a + ml.y * e;
    o0 = o0 * a + ov.x * e;
    o1 = o1 * a + ov.y * e;
    m = mn;
  }
  const float2 qv = ld2(q, ((int64_t(b) * T + n) * Hq + h) * kHeadDim + 2 * lane);
  int j = n;
  while (true) {
    const int64_t kv_elem = ((int64_t(b) * T + j) * Hkv + kvh) * kHeadDim + 2 * lane;
    const float2 kx = ld2(kt, kv_elem);
    const float s = wave_sum_f32(qv.x * kx.x + qv.y * kx.y) * sl2;
    const float2 vx = ld2(vt, kv_elem);
    const float mn = fmaxf(m, s);
    const float a = fast_exp2(m - mn), e = fast_exp2(s - mn);
    l = l * a + e;
    o0 = o0 * a + e * vx.x;
    o1 = o1 * a + e * vx.y;
    m = mn;
    if (j == 0) break;
    j = tree.parent[j];
  }
  const float inv = 1.f / l;
  const int64_t oe = ((int64_t(b) * T + n) * Hq + h) * kHeadDim + 2 * lane;
  if (BF16) {
    const uint32_t u = uint32_t(f32_to_bf16(o0 * inv)) | (uint32_t(f32_to_bf16(o1 * inv)) << 16);
    *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(out) + oe) = u;
  } else {
    *reinterpret_cast<float2*>(reinterpret_cast<float*>(out) + oe) = make_float2(o0 * inv, o1 * inv);
  }
}

hipError_t launch_attn(const TreeDev& tree, int32_t B, int32_t Hq, int32_t Hkv, int is_bf16,
                       const void* q, const void* k_tree, const void* v_tree, const void* k_cache,
                       const void* v_cache, int64_t cap, const int32_t* prefix_len, float scale,
                       void* out, uint8_t* ws, const AttnPlan& plan, hipStream_t s) {
  float* part_o = reinterpret_cast<float*>(ws + plan.o_off);
  float2* part_ml = reinterpret_cast<float2*>(ws + plan.ml_off);
  const float sl2 = scale * kLog2e;
  dim3 grid(plan.chunks, plan.row_tiles, B * Hkv);
  if (is_bf16)
    hipLaunchKernelGGL(attn_prefix_bf16, grid, dim3(256), 0, s,
                       reinterpret_cast<const uint16_t*>(q), reinterpret_cast<const uint16_t*>(k_cache),
                       reinterpret_cast<const uint16_t*>(v_cache), cap, prefix_len, tree.T, Hq, Hkv,
                       plan.G, plan.R, plan.chunks, sl2, part_o, part_ml, ws);
  else
    hipLaunchKernelGGL(attn_prefix_f32, grid, dim3(256), 0, s, reinterpret_cast<const float*>(q),
                       reinterpret_cast<const float*>(k_cache), reinterpret_cast<const float*>(v_cache),
                       cap, prefix_len, tree.T, Hq, Hkv, plan.G, plan.R, plan.chunks, sl2, part_o,
                       part_ml, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = int64_t(B) * tree.T * Hq;
  dim3 cgrid(unsigned((rows + 3) / 4));
  const int Rpad = plan.row_tiles * kRowsPerTile;
  if (is_bf16)
    hipLaunchKernelGGL(attn_combine<true>, cgrid, dim3(256), 0, s, tree, q, k_tree, v_tree,
                       prefix_len, B, Hq, Hkv, plan.G, plan.chunks, Rpad, sl2, part_o, part_ml, out, cap);
  else
    hipLaunchKernelGGL(attn_combine<false>, cgrid, dim3(256), 0, s, tree, q, k_tree, v_tree,
                       prefix_len, B, Hq, Hkv, plan.G, plan.chunks, Rpad, sl2, part_o, part_ml, out, cap);
  return hipGetLastError();
}

}  // namespace tr
