// Initial contents of the recycling matrix M ([B][V][k] token ids): all
// zero, random ids, or a prior matrix copied into every sequence's slot
// (Token Recycling, Method, first module: the hot start inherits a matrix
// from earlier inference; Experiment, initialisation ablation: all-zero,
// random, and fixed / shuffled / inherited prior matrices).
//
// A pure streaming write (plus a streaming read of the prior): the grid's
// y dimension walks sequences, x walks the V*k ids of one sequence in
// groups of four, so a group is one 16-byte store for int32 ids (two for
// int64) whenever V*k is a multiple of 4; otherwise every id is stored on
// its own.  No division: the flat index is b*V*k + i.
#include "tr_internal.h"

namespace tr {
namespace {

// SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014; the finaliser constants of Vigna's published
// splitmix64), used as a counter-based generator: output e of the stream
// seeded with s mixes s + (e + 1) * golden-ratio increment.
__device__ __forceinline__ uint64_t splitmix64(uint64_t seed, uint64_t e) {
  uint64_t z = seed + (e + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

struct InitArgs {
  void* M;
  const void* prior;
  uint64_t VK;        // ids per sequence
  uint64_t V;
  uint64_t seed;
  int32_t B;
  int32_t prior_bcast;  // prior has one matrix for every sequence
};

template <int MODE, typename PT>
__device__ __forceinline__ int64_t init_value(const InitArgs& a, uint64_t row, uint64_t i) {
  if constexpr (MODE == INIT_ZERO) {
    return 0;
  } else if constexpr (MODE == INIT_RANDOM) {
    // floor(u * V) with u = the high 32 bits of the draw over 2^32
    return int64_t(((splitmix64(a.seed, row * a.VK + i) >> 32) * a.V) >> 32);
  } else {
    const uint64_t src = (a.prior_bcast ? 0 : row * a.VK) + i;
    return int64_t(reinterpret_cast<const PT*>(a.prior)[src]);
  }
}

template <typename T>
__device__ __forceinline__ void load4(const void* p, uint64_t idx, int64_t v[4]) {
  if constexpr (sizeof(T) == 4) {
    const int4 x = *reinterpret_cast<const int4*>(reinterpret_cast<const int32_t*>(p) + idx);
    v[0] = x.x, v[1] = x.y, v[2] = x.z, v[3] = x.w;
  } else {
    const longlong2* q = reinterpret_cast<const longlong2*>(reinterpret_cast<const int64_t*>(p) + idx);
    const longlong2 x = q[0], y = q[1];
    v[0] = x.x, v[1] = x.y, v[2] = y.x, v[3] = y.y;
  }
}

template <typename T>
__device__ __forceinline__ void store4(void* p, uint64_t idx, const int64_t v[4]) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<int4*>(reinterpret_cast<int32_t*>(p) + idx) =
        make_int4(int32_t(v[0]), int32_t(v[1]), int32_t(v[2]), int32_t(v[3]));
  } else {
    longlong2* q = reinterpret_cast<longlong2*>(reinterpret_cast<int64_t*>(p) + idx);
    q[0] = make_longlong2(v[0], v[1]);
    q[1] = make_longlong2(v[2], v[3]);
  }
}

// VEC: V*k is a multiple of 4 (and M, prior are 16-byte aligned), so every
// group of four starts 16-byte aligned in every row.
template <int MODE, typename MT, typename PT, bool VEC>
__global__ __launch_bounds__(256) void init_m_kernel(InitArgs a) {
  const uint64_t stride = uint64_t(gridDim.x) * 256;
  for (int32_t b = blockIdx.y; b < a.B; b += gridDim.y) {
    const uint64_t row = uint64_t(b);
    if constexpr (VEC) {
      const uint64_t groups = a.VK / 4;
      for (uint64_t g = uint64_t(blockIdx.x) * 256 + threadIdx.x; g < groups; g += stride) {
        int64_t v[4];
        if constexpr (MODE == INIT_PRIOR) {
          load4<PT>(a.prior, (a.prior_bcast ? 0 : row * a.VK) + 4 * g, v);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = init_value<MODE, PT>(a, row, 4 * g + j);
        }
        store4<MT>(a.M, row * a.VK + 4 * g, v);
      }
    } else {
      for (uint64_t i = uint64_t(blockIdx.x) * 256 + threadIdx.x; i < a.VK; i += stride)
        reinterpret_cast<MT*>(a.M)[row * a.VK + i] = MT(init_value<MODE, PT>(a, row, i));
    }
  }
}

template <int MODE, typename MT, typename PT>
hipError_t launch_one(const InitArgs& a, bool vec, hipStream_t s) {
  const uint64_t units = vec ? a.VK / 4 : a.VK;
  const uint64_t bx = (units + 255) / 256;
  const dim3 grid(unsigned(bx < 2048 ? (bx ? bx : 1) : 2048), unsigned(a.B < 65535 ? a.B : 65535));
  if (vec)
    hipLaunchKernelGGL((init_m_kernel<MODE, MT, PT, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((init_m_kernel<MODE, MT, PT, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename MT>
hipError_t launch_mt(int mode, const InitArgs& a, int prior_is64, bool vec, hipStream_t s) {
  if (mode == INIT_ZERO) return launch_one<INIT_ZERO, MT, int32_t>(a, vec, s);
  if (mode == INIT_RANDOM) return launch_one<INIT_RANDOM, MT, int32_t>(a, vec, s);
  return prior_is64 ? launch_one<INIT_PRIOR, MT, int64_t>(a, vec, s)
                    : launch_one<INIT_PRIOR, MT, int32_t>(a, vec, s);
}

}  // namespace

hipError_t launch_init_m(int mode, void* M, int m_is64, int32_t B, int64_t V, int32_t k,
                         const void* prior, int prior_is64, int prior_bcast, uint64_t seed,
                         hipStream_t s) {
  InitArgs a{};
  a.M = M;
  a.prior = prior;
  a.VK = uint64_t(V) * uint64_t(k);
  a.V = uint64_t(V);
  a.seed = seed;
  a.B = B;
  a.prior_bcast = prior_bcast;
  const bool vec = a.VK % 4 == 0;
  prof_begin(s, TR_KERNEL_INIT);
  const hipError_t e = m_is64 ? launch_mt<int64_t>(mode, a, prior_is64, vec, s)
                              : launch_mt<int32_t>(mode, a, prior_is64, vec, s);
  prof_end(s);
  return e;
}

}  // namespace tr
