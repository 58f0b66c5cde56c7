// csa2_layer_group_noalloc: the layer-group entry point with its scratch in a
// device array of the library instead of a caller workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// The array is defined here and only here.  In host code its name stands for
// a host-side shadow, not a device address, so host code never passes the
// name to a kernel or a copy: the first call on each device looks up that
// device's copy with hipGetSymbolAddress and keeps the address per device.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "csa2.h"
#include "launch.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(CSA2_NOALLOC_SCRATCH_BYTES);

// One copy per GPU, held until the process ends.  Nothing in it has to start
// at zero: every kernel writes the scratch it reads within the same call.
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch` on each device, once looked up

// This device's copy of the array (looked up on the first call on the device).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return csa2::set_error(CSA2_ERR_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return csa2::set_error(CSA2_ERR_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char msg[256];
      snprintf(msg, sizeof(msg), "hipGetSymbolAddress(scratch) on device %d: %s", dev,
               e != hipSuccess ? hipGetErrorString(e) : "null address");
      return csa2::set_error(CSA2_ERR_HIP, msg);
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return CSA2_OK;
}

}  // namespace

extern "C" int csa2_layer_group_noalloc(const csa2_dims* dims, const csa2_kv_cache* cache, int32_t n_layers,
                                        const csa2_layer* layers, const int32_t* q_pos, int32_t n_q,
                                        const csa2_compress_args* compress, void* stream) {
  csa2::set_error(CSA2_OK, "");
  try {
    return csa2::layer_group_run(dims, cache, n_layers, layers, q_pos, n_q, compress,
                                 [](size_t need, void** ws) -> int {
                                   if (need > kScratchBytes) {
                                     char msg[256];
                                     snprintf(msg, sizeof(msg),
                                              "this call needs %zu bytes of scratch, beyond the %zu of "
                                              "csa2_layer_group_noalloc: use csa2_layer_group with a workspace",
                                              need, kScratchBytes);
                                     return csa2::set_error(CSA2_ERR_WORKSPACE, msg);
                                   }
                                   return scratch_address(ws);
                                 },
                                 stream, false);
  } catch (...) {
    return csa2::set_error(CSA2_ERR_HIP, "internal exception");
  }
}
