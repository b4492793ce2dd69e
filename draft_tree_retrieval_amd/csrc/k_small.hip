// Stand-alone retrieval and verification kernels (one workgroup per
// sequence) and the workspace fill.  Retrieval is a chain of dependent
// gathers, one per tree layer ("Token Recycling" summary, Method, second
// module: a BFS-like expansion of the last token's candidates); it is
// latency-bound, so one workgroup per sequence walks the layers with a
// barrier between them and one lane per node.
#include "tail.h"

namespace tr {

__global__ __launch_bounds__(128) void retrieve_kernel(TreeDev tree, const void* __restrict__ M,
                                                       int m_is64, int64_t V, int32_t k,
                                                       const int32_t* __restrict__ root_tok,
                                                       int32_t* __restrict__ tree_tok, uint8_t* ws) {
  __shared__ TailShared S;
  const int b = blockIdx.x;
  tail_tree(S, tree);
  __syncthreads();
  if (threadIdx.x >= 64) return;      // one wave walks the tree
  int32_t* out_b = tree_tok + int64_t(b) * tree.T;
  if (m_is64)
    tail_retrieve<int64_t>(S, tree, root_tok[b], reinterpret_cast<const int64_t*>(M) + int64_t(b) * V * k,
                           V, k, out_b, ws, false);
  else
    tail_retrieve<int32_t>(S, tree, root_tok[b], reinterpret_cast<const int32_t*>(M) + int64_t(b) * V * k,
                           V, k, out_b, ws, false);
}

__global__ __launch_bounds__(256) void verify_kernel(TreeDev tree, const int32_t* __restrict__ topk,
                                                     int32_t k, const int32_t* __restrict__ tree_tok,
                                                     int32_t* accept_len, int32_t* accept_path,
                                                     int32_t* bonus, int32_t* emitted) {
  __shared__ TailShared S;
  const int b = blockIdx.x;
  tail_load<256>(S, tree, tree_tok + int64_t(b) * tree.T, topk + int64_t(b) * tree.T * k, k);
  tail_verify(S, tree, k);
  tail_write_verdict(S, tree, b, accept_len, accept_path, bonus, emitted);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* p, size_t n16) {
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += size_t(gridDim.x) * 256)
    p[i] = make_uint4(0, 0, 0, 0);
}

// Read-bandwidth probe (a profiling aid, not a TR step): every 16-byte word
// of the buffer is read once with non-temporal loads, four independent
// loads in flight per thread, folded into one word per block and written to
// sink[block] so the loads cannot be elided.
constexpr int kProbeThreads = 512;
constexpr int kProbeBlocks = 2048;
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ p,
                                                                 size_t n16, uint32_t* sink) {
  const size_t stride = size_t(gridDim.x) * kProbeThreads;
  size_t i = size_t(blockIdx.x) * kProbeThreads + threadIdx.x;
  u32x4 acc = {0, 0, 0, 0};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    const u32x4 b = __builtin_nontemporal_load(p + i + stride);
    const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  x = wave_max_u32(x);
  if ((threadIdx.x & 63) == 0) atomicXor(sink + blockIdx.x, x);
}

hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t s) {
  const size_t n16 = bytes / 16;
  prof_begin(s, TR_KERNEL_READ_PROBE);
  hipLaunchKernelGGL(read_probe_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, s,
                     reinterpret_cast<const u32x4*>(src), n16, sink);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_retrieve(const TreeDev& tree, int32_t B, const void* M, int m_is64, int64_t V,
                           int32_t k, const int32_t* root_tok, int32_t* tree_tok, uint8_t* ws,
                           hipStream_t s) {
  prof_begin(s, TR_KERNEL_RETRIEVE);
  hipLaunchKernelGGL(retrieve_kernel, dim3(B), dim3(128), 0, s, tree, M, m_is64, V, k, root_tok,
                     tree_tok, ws);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_verify(const TreeDev& tree, int32_t B, const int32_t* topk, int32_t k,
                         const int32_t* tree_tok, int32_t* accept_len, int32_t* accept_path,
                         int32_t* bonus, int32_t* emitted, hipStream_t s) {
  prof_begin(s, TR_KERNEL_VERIFY);
  hipLaunchKernelGGL(verify_kernel, dim3(B), dim3(256), 0, s, tree, topk, k, tree_tok, accept_len,
                     accept_path, bonus, emitted);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  prof_begin(s, TR_KERNEL_FILL);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(unsigned(blocks)), dim3(256), 0, s,
                     reinterpret_cast<uint4*>(p), n16);
  prof_end(s);
  return hipGetLastError();
}

}  // namespace tr
