// The whole layer for callers that cannot allocate: moe_layer_forward with
// its workspace in a device array the library owns.
//
// `scratch` is a file-scope device array of kScratchBytes on every GPU the
// library runs on (each device holds its own copy at its own address, kept
// until the process ends).  In host code the name `scratch` is only a
// host-side handle: its device address on a given device comes from
// hipGetSymbolAddress, called once per device with that device current and
// cached here; only that address is ever handed to kernels.
#include <mutex>

#include "common.h"

namespace {
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the device that `stream` belongs to (the
// current device for the null stream).
moe_status scratch_address(hipStream_t stream, void** out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return MOE_ERR_HIP;
  int dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess)
    return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return MOE_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) hipSetDevice(cur);
    if (e != hipSuccess || !ptr) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_layer_forward_noalloc(const moe_problem* p, const float* logits,
                                     const float* bias, const void* x,
                                     const moe_weights* w, const int32_t* l2p,
                                     const int32_t* replica_count, void* out,
                                     int32_t* expert_counts, void* stream) {
  moe_status st = moe_check_problem(p);
  if (st != MOE_OK) return st;
  size_t need = 0;
  moe_layer_workspace_size(p, &need);
  if (need > kScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (p->T > 0) {           // T = 0 enqueues no work that needs scratch
    st = scratch_address((hipStream_t)stream, &ws);
    if (st != MOE_OK) return st;
  }
  return moe_layer_forward(p, logits, bias, x, w, l2p, replica_count, out,
                           expert_counts, ws, ws ? kScratchBytes : 0, stream);
}

}  // extern "C"
