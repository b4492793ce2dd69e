// Allocation-free tree attention: tr_tree_attn with the call's scratch (the
// prefix partials, merge records and status word) in a fixed array of device
// memory that the library holds on every GPU it runs on, for callers that
// cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Nothing here allocates: the array is part
// of the code object, loaded with it, and held until the process ends.
#include <mutex>

#include "tr_internal.h"

namespace tr {

constexpr size_t kNoAllocScratchBytes = size_t(48) << 20;   // 48 MiB per GPU

// The array itself.  In host code its name is a host-side stand-in, not a
// device address: only the address hipGetSymbolAddress returns for the
// current device is passed to kernels.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
uint8_t* g_scratch[kMaxDevices];   // device address of scratch per device (null: not looked up yet)

// This GPU's copy of scratch: looked up once per device, with that device
// current, on the first call there.
tr_status scratch_of_current_device(uint8_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_error(e, "tr_tree_attn_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(TR_ERR_UNSUPPORTED, "tr_tree_attn_noalloc: device index outside 0..63");
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_error(e, "tr_tree_attn_noalloc: hipGetSymbolAddress");
    if (p == nullptr) return set_error(TR_ERR_HIP, "tr_tree_attn_noalloc: no device address for the scratch");
    g_scratch[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch[dev];
  return TR_OK;
}

}  // namespace
}  // namespace tr

extern "C" tr_status tr_tree_attn_noalloc(const tr_tree* t, int32_t B, int32_t Hq, int32_t Hkv,
                                          int32_t d, tr_dtype dt, const void* q,
                                          const void* k_tree, const void* v_tree,
                                          const void* k_cache, const void* v_cache, int64_t cap,
                                          const int32_t* prefix_len, float scale, void* out,
                                          uint32_t* flags, void* stream) {
  tr::AttnPlan plan;
  tr_status st = tr::attn_prepare(t, B, Hq, Hkv, d, dt, q, k_tree, v_tree, k_cache, v_cache, cap,
                                  prefix_len, scale, out, &plan);
  if (st != TR_OK) return st;
  if (plan.end > tr::kNoAllocScratchBytes)
    return tr::set_error(TR_ERR_UNSUPPORTED,
                         "tr_tree_attn_noalloc: the call needs more scratch than the 48 MiB the "
                         "library holds per GPU (use tr_tree_attn with a workspace)");
  if (flags && (reinterpret_cast<uintptr_t>(flags) & 3))
    return tr::set_error(TR_ERR_INVALID_ARGUMENT, "tr_tree_attn_noalloc: flags must be 4-byte aligned");
  uint8_t* ws = nullptr;
  st = tr::scratch_of_current_device(&ws);
  if (st != TR_OK) return st;
  return tr::hip_error(tr::launch_attn(t->dev, B, Hq, Hkv, dt == TR_BFLOAT16, q, k_tree, v_tree,
                                       k_cache, v_cache, cap, prefix_len, scale, out, ws, plan,
                                       hipStream_t(stream), nullptr,
                                       reinterpret_cast<uint8_t*>(flags)),
                       "tr_tree_attn_noalloc");
}
