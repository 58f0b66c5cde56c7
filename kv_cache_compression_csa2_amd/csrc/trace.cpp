// Kernel trace: optional start/stop HIP events attached to each kernel launch
// (see csa2_trace_enable in csa2.h).  The runtime stamps them with the
// kernel's own start and end times.  The events are created when tracing is
// enabled, never on a call path; slot bookkeeping is guarded by one mutex.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "csa2.h"
#include "launch.hpp"

namespace {

struct Slot {
  hipEvent_t begin = nullptr, end = nullptr;
  int32_t kernel = 0;
  bool ok = false;  // the launch carrying the events was enqueued
};

std::mutex g_mu;
std::vector<Slot> g_slots;
int g_used = 0;      // slots handed out since the last read
int g_dropped = 0;   // launches not recorded since the last read
int g_device = -1;   // device the events belong to
std::atomic<bool> g_on{false};

void free_events() {
  for (Slot& s : g_slots) {
    if (s.begin) (void)hipEventDestroy(s.begin);
    if (s.end) (void)hipEventDestroy(s.end);
  }
  g_slots.clear();
  g_used = g_dropped = 0;
  g_on = false;
  g_device = -1;
}

}  // namespace

namespace csa2 {

TraceSlot trace_begin(int32_t kernel) {
  TraceSlot t{-1, nullptr, nullptr};
  if (!g_on) return t;  // unsynchronised fast path: tracing is switched only between calls
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_on) return t;
  int dev = -1;
  if (g_used >= int(g_slots.size()) || hipGetDevice(&dev) != hipSuccess || dev != g_device) {
    ++g_dropped;
    return t;
  }
  const int i = g_used++;
  Slot& s = g_slots[i];
  s.kernel = kernel;
  s.ok = false;
  t.slot = i;
  t.start = s.begin;
  t.stop = s.end;
  return t;
}

void trace_end(int slot, bool launched) {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lock(g_mu);
  if (slot < g_used) g_slots[slot].ok = launched;
}

}  // namespace csa2

extern "C" {

int csa2_trace_enable(int32_t max_kernels) {
  std::lock_guard<std::mutex> lock(g_mu);
  free_events();
  if (max_kernels < 0 || max_kernels > (1 << 20)) return CSA2_ERR_INVALID_ARG;
  if (max_kernels == 0) return CSA2_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return CSA2_ERR_HIP;
  g_slots.resize(size_t(max_kernels));
  for (Slot& s : g_slots) {
    if (hipEventCreate(&s.begin) != hipSuccess || hipEventCreate(&s.end) != hipSuccess) {
      free_events();
      return CSA2_ERR_HIP;
    }
  }
  g_device = dev;
  g_on = true;
  return CSA2_OK;
}

int csa2_trace_read(csa2_trace_record* out, int32_t max, int32_t* n_dropped) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (max < 0 || (max > 0 && !out)) return CSA2_ERR_INVALID_ARG;
  int n = 0, dropped = g_dropped;
  int status = CSA2_OK;
  for (int i = 0; i < g_used; ++i) {
    Slot& s = g_slots[i];
    if (!s.ok || n >= max) {
      ++dropped;
      continue;
    }
    float ms = 0.0f;
    if (hipEventSynchronize(s.end) != hipSuccess || hipEventElapsedTime(&ms, s.begin, s.end) != hipSuccess) {
      status = CSA2_ERR_HIP;
      ++dropped;
      continue;
    }
    out[n].kernel = s.kernel;
    out[n].ms = ms;
    ++n;
  }
  g_used = 0;
  g_dropped = 0;
  if (n_dropped) *n_dropped = dropped;
  return n > 0 || status == CSA2_OK ? n : status;
}

const char* csa2_kernel_name(int32_t kernel) {
  switch (kernel) {
    case CSA2_KERNEL_COMPRESS: return "compress_kernel";
    case CSA2_KERNEL_SCAN_GENERIC: return "scan_generic_kernel";
    case CSA2_KERNEL_SCAN_BF16: return "scan_mfma_bf16_kernel";
    case CSA2_KERNEL_SCAN_FP4: return "scan_mfma_fp4_kernel";
    case CSA2_KERNEL_SELECT: return "select_kernel";
    case CSA2_KERNEL_ATTN_GENERIC: return "attn_generic_kernel";
    case CSA2_KERNEL_ATTN_BF16: return "attn_mfma_kernel<false, 32>";
    case CSA2_KERNEL_ATTN_FP4: return "attn_mfma_kernel<true, 32>";
    case CSA2_KERNEL_ATTN_MERGE: return "attn_merge_kernel";
    case CSA2_KERNEL_ATTN_FP4_G16: return "attn_mfma_kernel<true, 16>";
    case CSA2_KERNEL_SCAN_PREFILL: return "scan_prefill_kernel";
    case CSA2_KERNEL_OPROJ_MFMA: return "oproj_mfma_kernel";
    case CSA2_KERNEL_OPROJ_GENERIC: return "oproj_generic_kernel";
    case CSA2_KERNEL_OPROJ_MFMA16: return "oproj_mfma16_kernel";
    case CSA2_KERNEL_OPROJ_LDS: return "oproj_lds_kernel";
    case CSA2_KERNEL_READ_PROBE: return "read_probe_kernel";
    case CSA2_KERNEL_MFMA_PROBE: return "mfma_probe_kernel";
    case CSA2_KERNEL_SCAN_BF16_FUSED: return "scan_fused_bf16_kernel";
    case CSA2_KERNEL_SCAN_FP4_FUSED: return "scan_fused_fp4_kernel";
    default: return "unknown";
  }
}

}  // extern "C"
