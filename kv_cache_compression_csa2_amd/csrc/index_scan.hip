// Indexer score scan: s_j = sum_h w_h * max(0, q_h . K_j) over a query's
// domain, plus the maximum of every aligned block of 8 and super-block of 64
// domain slots (the inputs of the hierarchical selection).
//
// Pages: zartbot walkthrough (hn.213312.xyz) section 2.3.1 (lightweight
// indexer scores main-KV entries with indexer Q and K; 32 heads x 128 in
// section 1.2) and section 2.3.4 (HSI: block maximum over blocks of 8; a
// Reindex layer scores only the pool).
//
// Domain slot i maps to entry j = i (all visible entries) or, with a pool,
// j = 8 * pool[i / 8] + i % 8.  Slots whose entry is not visible hold -inf.
#include "device_common.hpp"
#include "launch.hpp"

namespace csa2 {
namespace {

constexpr int kThreads = 256;

// Generic path: one thread per domain slot, float32 accumulation.  Serves
// every shape and storage type; the wide bf16/FP4 shapes use the MFMA scan.
__global__ __launch_bounds__(kThreads) void scan_generic_kernel(
    int Hi, int di, int act_bf16, int kv_dtype, int idx_group, int ratio, int64_t capacity,
    const void* __restrict__ idx_q, const float* __restrict__ head_w, const int32_t* __restrict__ q_pos, int n_q,
    const int32_t* __restrict__ pool_in, int cand_blocks, const void* __restrict__ idx_k,
    const uint8_t* __restrict__ idx_scale, const int32_t* __restrict__ n_entries, float* __restrict__ scores,
    float* __restrict__ bmax, float* __restrict__ sbmax, int64_t dom_cap) {
  extern __shared__ float sh[];
  float* qs = sh;             // [Hi * di]
  float* ws = qs + Hi * di;   // [Hi]
  float* ss = ws + Hi;        // [kThreads]
  const int qi = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int64_t row = int64_t(b) * n_q + qi;
  for (int x = tid; x < Hi * di; x += kThreads) qs[x] = act_load(idx_q, row * Hi * di + x, act_bf16);
  for (int x = tid; x < Hi; x += kThreads) ws[x] = head_w[row * Hi + x];
  __syncthreads();

  const int64_t n = clamp_entries(n_entries, b, capacity);
  const int64_t n_vis = visible_count(n, q_pos[row], ratio);
  const int64_t i = int64_t(blockIdx.x) * kThreads + tid;
  int64_t j = -1;
  if (pool_in) {
    if (i < int64_t(cand_blocks) * 8) {
      const int64_t blk = pool_in[row * cand_blocks + i / 8];
      if (blk >= 0) j = blk * 8 + (i & 7);
    }
  } else {
    j = i;
  }
  if (j >= n_vis) j = -1;

  float s = -INFINITY;
  if (j >= 0) {
    const int64_t crow = int64_t(b) * capacity + j;
    s = 0.0f;
    for (int h = 0; h < Hi; ++h) {
      float dot = 0.0f;
      for (int e = 0; e < di; ++e) dot += qs[h * di + e] * cache_load(idx_k, idx_scale, kv_dtype, crow, di, idx_group, e);
      s += ws[h] * fmaxf(dot, 0.0f);
    }
  }
  ss[tid] = s;
  if (i < dom_cap) scores[row * dom_cap + i] = s;
  __syncthreads();
  if (tid < kThreads / 8) {
    float m = ss[tid * 8];
    for (int x = 1; x < 8; ++x) m = fmaxf(m, ss[tid * 8 + x]);
    const int64_t bi = int64_t(blockIdx.x) * (kThreads / 8) + tid;
    if (bi < dom_cap / 8) bmax[row * (dom_cap / 8) + bi] = m;
  }
  if (tid < kThreads / 64) {
    float m = ss[tid * 64];
    for (int x = 1; x < 64; ++x) m = fmaxf(m, ss[tid * 64 + x]);
    const int64_t si = int64_t(blockIdx.x) * (kThreads / 64) + tid;
    if (si < dom_cap / 64) sbmax[row * (dom_cap / 64) + si] = m;
  }
}

}  // namespace

hipError_t launch_scan(const csa2_dims& dims, const csa2_kv_cache& cache, const void* idx_q, const float* head_w,
                       const int32_t* q_pos, int32_t n_q, const int32_t* pool_in, const ScanScratch& ss,
                       hipStream_t stream) {
  const dim3 grid(unsigned(ss.dom_cap / kThreads), n_q, cache.batch);
  const size_t lds = sizeof(float) * size_t(dims.n_idx_heads * dims.d_idx + dims.n_idx_heads + kThreads);
  hipLaunchKernelGGL(scan_generic_kernel, grid, dim3(kThreads), lds, stream, dims.n_idx_heads, dims.d_idx,
                     int(dims.act_dtype == CSA2_BF16), cache.kv_dtype, cache.idx_group, cache.ratio, cache.capacity,
                     idx_q, head_w, q_pos, n_q, pool_in, dims.cand_blocks, cache.idx_k, cache.idx_scale,
                     cache.n_entries, ss.scores, ss.bmax, ss.sbmax, ss.dom_cap);
  return hipGetLastError();
}

}  // namespace csa2
