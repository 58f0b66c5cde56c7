// Sparse attention over the kept main-KV entries concatenated with the
// sliding window, one softmax over both, key = value.
//
// Pages: zartbot walkthrough (hn.213312.xyz) section 2.2.2 (global KV from the
// sparse branch and local KV from the window are concatenated and scored with
// Q), section 1.2 (64 heads of width 512 sharing one 512-d latent, 64 rotary
// dims, window 128) and section 3.3.1 (key equals value; the output is a
// convex combination of the read rows).
#include "device_common.hpp"
#include "launch.hpp"

namespace csa2 {
namespace {

constexpr int kThreads = 256;

// Generic path: one workgroup per (head, query, sequence), float32 math.
__global__ __launch_bounds__(kThreads) void attn_generic_kernel(
    int d, int d_rope, int H, int topk, int window, int act_bf16, int kv_dtype, int main_group, double theta,
    int64_t capacity, const void* __restrict__ q, const int32_t* __restrict__ q_pos, int n_q,
    const int32_t* __restrict__ topk_ids, const void* __restrict__ swa, const int32_t* __restrict__ swa_first,
    int n_swa, const void* __restrict__ main, const uint8_t* __restrict__ main_scale, void* __restrict__ out,
    float* __restrict__ lse) {
  extern __shared__ float sh[];
  float* qh = sh;           // [d]
  float* lg = qh + d;       // [topk + window]
  float* red = lg + topk + window;  // [kThreads / 64 + 2]
  const int h = blockIdx.x, qi = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int64_t row = int64_t(b) * n_q + qi;
  const int64_t t = q_pos[row];
  const int64_t qoff = (row * H + h) * d;

  // rotated query
  const int c0 = d - d_rope;
  for (int c = tid; c < c0; c += kThreads) qh[c] = act_load(q, qoff + c, act_bf16);
  for (int m = tid; m < d_rope / 2; m += kThreads) {
    const double freq = pow(theta, -2.0 * m / d_rope);
    double sn, cs;
    sincos(double(t) * freq, &sn, &cs);
    const double x = act_load(q, qoff + c0 + 2 * m, act_bf16), y = act_load(q, qoff + c0 + 2 * m + 1, act_bf16);
    qh[c0 + 2 * m] = float(x * cs - y * sn);
    qh[c0 + 2 * m + 1] = float(x * sn + y * cs);
  }
  __syncthreads();

  const int64_t win0 = t - window + 1 > 0 ? t - window + 1 : 0;
  const int64_t sfirst = swa_first[b];
  const int n_rows = topk + window;
  const float scale = 1.0f / sqrtf(float(d));

  // row r < topk: main-KV entry topk_ids[r]; r >= topk: window position win0 + r - topk
  auto row_src = [&](int r, int64_t& crow, int64_t& srow) {
    crow = -1;
    srow = -1;
    if (r < topk) {
      const int64_t j = topk_ids[row * topk + r];
      if (j >= 0 && j < capacity) crow = int64_t(b) * capacity + j;
    } else {
      const int64_t p = win0 + (r - topk);
      const int64_t s = p - sfirst;
      if (p <= t && s >= 0 && s < n_swa) srow = int64_t(b) * n_swa + s;
    }
  };

  for (int r = wid; r < n_rows; r += kThreads / 64) {
    int64_t crow, srow;
    row_src(r, crow, srow);
    float v = -INFINITY;
    if (crow >= 0 || srow >= 0) {
      float part = 0.0f;
      for (int c = lane; c < d; c += 64) {
        const float x = crow >= 0 ? cache_load(main, main_scale, kv_dtype, crow, d, main_group, c)
                                  : act_load(swa, srow * d + c, act_bf16);
        part += qh[c] * x;
      }
      v = wave_sum(part) * scale;
    }
    if (lane == 0) lg[r] = v;
  }
  __syncthreads();

  // max and denominator
  float mx = -INFINITY;
  for (int r = tid; r < n_rows; r += kThreads) mx = fmaxf(mx, lg[r]);
  mx = wave_max(mx);
  if (lane == 0) red[wid] = mx;
  __syncthreads();
  mx = red[0];
  for (int x = 1; x < kThreads / 64; ++x) mx = fmaxf(mx, red[x]);
  __syncthreads();
  float den = 0.0f;
  for (int r = tid; r < n_rows; r += kThreads) den += lg[r] == -INFINITY ? 0.0f : expf(lg[r] - mx);
  den = wave_sum(den);
  if (lane == 0) red[wid] = den;
  __syncthreads();
  den = 0.0f;
  for (int x = 0; x < kThreads / 64; ++x) den += red[x];
  for (int r = tid; r < n_rows; r += kThreads) lg[r] = lg[r] == -INFINITY ? 0.0f : expf(lg[r] - mx) / den;
  __syncthreads();

  // out = P . rows
  for (int c = tid; c < d; c += kThreads) {
    float acc = 0.0f;
    for (int r = 0; r < n_rows; ++r) {
      const float p = lg[r];
      if (p == 0.0f) continue;
      int64_t crow, srow;
      row_src(r, crow, srow);
      const float x = crow >= 0 ? cache_load(main, main_scale, kv_dtype, crow, d, main_group, c)
                                : act_load(swa, srow * d + c, act_bf16);
      acc += p * x;
    }
    if (!(mx > -INFINITY)) acc = 0.0f;
    if (act_bf16) reinterpret_cast<uint16_t*>(out)[qoff + c] = f32_to_bf16(acc);
    else reinterpret_cast<float*>(out)[qoff + c] = acc;
  }
  if (lse && tid == 0) lse[row * H + h] = mx > -INFINITY ? mx + logf(den) : -INFINITY;
}

}  // namespace

size_t attn_workspace_bytes(const csa2_dims&, const csa2_kv_cache&, int32_t) { return 0; }

hipError_t launch_attn(const csa2_dims& dims, const csa2_kv_cache& cache, const void* q, const int32_t* q_pos,
                       int32_t n_q, const int32_t* topk, const void* swa_kv, const int32_t* swa_first_pos,
                       int32_t n_swa, void* out, float* lse, void*, size_t, hipStream_t stream) {
  const dim3 grid(dims.n_heads, n_q, cache.batch);
  const size_t lds = sizeof(float) * size_t(dims.d + dims.topk + dims.window + kThreads / 64 + 2);
  hipLaunchKernelGGL(attn_generic_kernel, grid, dim3(kThreads), lds, stream, dims.d, dims.d_rope, dims.n_heads,
                     dims.topk, dims.window, int(dims.act_dtype == CSA2_BF16), cache.kv_dtype, cache.main_group,
                     dims.rope_theta, cache.capacity, q, q_pos, n_q, topk, swa_kv, swa_first_pos, n_swa, cache.main,
                     cache.main_scale, out, lse);
  return hipGetLastError();
}

}  // namespace csa2
