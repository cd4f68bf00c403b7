// moe_permute_noalloc: moe_permute for callers that cannot allocate (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// allocation). The counting sort's per-chunk histogram lives in a fixed
// device array instead of a caller workspace; everything else is
// moe_permute's launch sequence, kernels and results.
//
// The array is a file-scope __device__ symbol: in host code its name is only
// a stand-in, so its device address is looked up once per device with
// hipGetSymbolAddress (each GPU holds its own copy) and that address is what
// the kernels receive. Every call on one device shares that device's array;
// calls that overlap on one device (different streams) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"
#include "libmoe.h"

namespace moe {
namespace {

// 1 MiB: the histogram of up to 262144 (chunk, expert) pairs, i.e. T*K up to
// 4,194,304 (token, slot) pairs at E = 256 (more at smaller E).
constexpr size_t kScratchBytes = size_t(1) << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up on the
// first call per device, then cached), or nullptr with *err set.
void* scratch_of_current_device(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_permute_noalloc(const moe_config* c, const int32_t* topk_idx, const void* x,
                                   int32_t* expert_offsets, int32_t* perm_slot, void* x_perm,
                                   void* stream) {
  int st = moe_validate(c);
  if (st != MOE_OK) return st;
  if (!expert_offsets) return MOE_ERR_NULL;
  if (c->num_tokens > 0 && (!topk_idx || !perm_slot || (x_perm && !x))) return MOE_ERR_NULL;
  for (const void* p : {static_cast<const void*>(topk_idx), x, static_cast<const void*>(expert_offsets),
                        static_cast<const void*>(perm_slot), static_cast<const void*>(x_perm)})
    if (reinterpret_cast<uintptr_t>(p) & 15u) return MOE_ERR_SHAPE;
  const size_t need = moe_workspace_size(c, MOE_WS_PERMUTE);
  if (need > kScratchBytes) return MOE_ERR_SCRATCH;
  void* ws = nullptr;
  if (c->num_tokens > 0) {
    hipError_t err;
    ws = scratch_of_current_device(&err);
    if (!ws) return MOE_ERR_HIP;
  }
  (void)hipGetLastError();
  const hipError_t err = launch_permute(*c, topk_idx, x, expert_offsets, perm_slot, x_perm, ws,
                                        reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
