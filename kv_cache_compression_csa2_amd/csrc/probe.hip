// Measurement probes, not steps of the method: a streaming read of a device
// buffer (the read bandwidth this GPU reaches for a working set of a given
// size) and a dense loop of bf16 matrix products (the matrix-core rate it
// sustains under load), the measured denominators reported next to the
// published HBM and bf16 peaks.
#include "launch.hpp"

namespace csa2 {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // 16-byte loads in flight per lane

// Each lane reads kUnroll 16-byte words a workgroup stride apart per
// iteration (a workgroup covers 32 KB contiguous per iteration), grid-strided
// over the buffer.  Out-of-range slots of the last iteration re-read the last
// word (in bounds).  The XOR of every word goes to `sink` only if it equals a
// fixed constant, which keeps the loads live without a store per lane.
__global__ __launch_bounds__(kThreads) void read_probe_kernel(const uint4* __restrict__ p, int64_t n16,
                                                               uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t step = int64_t(gridDim.x) * kThreads * kUnroll;
  for (int64_t base = int64_t(blockIdx.x) * kThreads * kUnroll + threadIdx.x; base < n16; base += step) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + int64_t(u) * kThreads;
      v[u] = p[i < n16 ? i : n16 - 1];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

typedef __bf16 probe_bf16x8 __attribute__((__vector_size__(16)));
typedef float probe_f32x16 __attribute__((__vector_size__(64)));
constexpr int kMfmaChains = 8;  // independent accumulator chains per wave

// Each wave runs kMfmaChains independent chains of v_mfma_f32_32x32x16_bf16
// for `iters` iterations on register operands (derived from the lane, so
// nothing folds; the sums stay far below the float range), then adds its
// accumulators into one value stored to `sink` only if it equals a fixed
// constant (keeps the products live).  Two workgroups per compute unit, as
// the query-blocked indexer scan runs.
__global__ __launch_bounds__(kThreads, 2) void mfma_probe_kernel(int64_t iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  probe_bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(1.0f + float(lane + i) * (1.0f / 1024.0f));
    b[i] = static_cast<__bf16>(0.5f - float(3 * lane + i) * (1.0f / 4096.0f));
  }
  probe_f32x16 acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) acc[c] = probe_f32x16{};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if (s == 1234.5f) sink[0] = s;
}

}  // namespace

hipError_t launch_mfma_probe(int64_t iters, int32_t workgroups, float* sink, hipStream_t stream) {
  return launch_kernel(CSA2_KERNEL_MFMA_PROBE, mfma_probe_kernel, dim3(unsigned(workgroups)), dim3(kThreads), 0,
                       stream, iters, sink);
}

hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  const int64_t per_wg = int64_t(kThreads) * kUnroll;
  const int64_t blocks = std::min<int64_t>((n16 + per_wg - 1) / per_wg, 4096);
  return launch_kernel(CSA2_KERNEL_READ_PROBE, read_probe_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                       static_cast<const uint4*>(buf), n16, sink);
}

}  // namespace csa2
