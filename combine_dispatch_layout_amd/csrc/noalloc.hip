// moe_dispatch_layout_noalloc: the layout call with its workspace in a static device
// array instead of a caller-supplied buffer, for callers that cannot allocate (code
// under HIP graph capture, serving loops that must not call hipMalloc, harnesses that
// forbid it).
//
// `scratch` is zero when the code object loads, which is the state the layout's
// workspace must start in (the one-launch layout leaves it that way after every call),
// and each GPU the library runs on holds its own copy until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: the device address is
// taken once per device with hipGetSymbolAddress (with that device current) and only
// that address is passed to the kernels.  Calls that overlap in time on one GPU share
// the array and race; calls on one stream, or otherwise ordered, do not.
#include <atomic>
#include <mutex>

#include "moe_internal.h"

static __device__ __align__(256) unsigned char scratch[MOE_LAYOUT_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];  // device address of `scratch`, per device
std::mutex g_scratch_mu;

// The device address of the current device's copy of `scratch`, looked up on the
// device's first call.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" moe_status moe_dispatch_layout_noalloc(
    const int32_t* topk_idx, int64_t M, int32_t k, const int32_t* expert_bucket, int32_t G,
    int32_t B, int32_t dedup, int32_t* expert_count, int32_t* expert_offset,
    int32_t* bucket_count, int32_t* bucket_offset, int32_t* slot, int32_t* send_row,
    int32_t* send_token, int32_t* status, hipStream_t stream) {
  // the same checks as moe_dispatch_layout, all before any HIP call
  if (M < 0 || k < 1 || G < 1 || B < 1 || k > G) return MOE_ERR_INVALID_ARGUMENT;
  if (G > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || B > MOE_MAX_BUCKETS) return MOE_ERR_UNSUPPORTED;
  if (M * (int64_t)k >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if (!expert_bucket || !expert_count || !expert_offset || !bucket_count || !bucket_offset ||
      !status)
    return MOE_ERR_INVALID_ARGUMENT;
  if (M > 0 && (!topk_idx || !slot || !send_row || !send_token)) return MOE_ERR_INVALID_ARGUMENT;
  if (dedup != 0 && dedup != 1) return MOE_ERR_INVALID_ARGUMENT;
  if (moedl::layout_workspace_bytes(M, G, B) > (size_t)MOE_LAYOUT_SCRATCH_BYTES)
    return MOE_ERR_WORKSPACE;
  void* base = nullptr;
  if (scratch_address(&base) != hipSuccess) return MOE_ERR_LAUNCH;
  const moedl::LayoutWorkspace ws = moedl::carve_layout_workspace(base, M, G, B);
  const hipError_t e = moedl::launch_layout(topk_idx, M, k, expert_bucket, G, B, dedup,
                                            expert_count, expert_offset, bucket_count,
                                            bucket_offset, slot, send_row, send_token, status,
                                            ws, stream);
  return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}
