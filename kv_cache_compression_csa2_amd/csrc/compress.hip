// Compressor: merge latent rows into cache entries, rotate, store main KV,
// project and store the indexer K.
//
// Pages: zartbot walkthrough (hn.213312.xyz) section 2.3.1 (ratio 2 in the
// encoder with channel-wise learned weights, ratio 1 in the decoder, no
// overlap; indexer K projected from the main KV) and section 2.4.4 (the cache
// is quantised after RoPE, FP4 main KV).
//
// One workgroup writes one entry.  Everything before the stores runs in
// float64: the merge, the rotation (angles and sin/cos) and the 512 -> 128
// projection, so each stored value is the single rounding of the exact value
// and agrees bit-for-bit with an independent float64 computation except when
// that value sits within float64 noise of a rounding boundary.  The kernel is
// a negligible share of a decode step (one row per sequence) and of a prefill
// chunk (2048 rows), so float64 costs nothing that matters.
#include "device_common.hpp"
#include "launch.hpp"

namespace csa2 {
namespace {

constexpr int kThreads = 1024;

// Store `n` float64 values as one cache row of the given format.
__device__ void store_row(const double* v, int n, int dtype, int group, void* base, uint8_t* scale_base, int64_t row) {
  const int tid = threadIdx.x;
  if (dtype == CSA2_F32) {
    float* dst = reinterpret_cast<float*>(base) + row * n;
    for (int c = tid; c < n; c += kThreads) dst[c] = __double2float_rn(v[c]);
  } else if (dtype == CSA2_BF16) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(base) + row * n;
    for (int c = tid; c < n; c += kThreads) dst[c] = f64_to_bf16(v[c]);
  } else {
    uint8_t* dst = reinterpret_cast<uint8_t*>(base) + row * (n / 2);
    uint8_t* sdst = scale_base + row * (n / group);
    for (int g = tid; g < n / group; g += kThreads) {
      const double* x = v + g * group;
      double amax = 0.0;
      for (int i = 0; i < group; ++i) amax = fmax(amax, fabs(x[i]));
      const uint32_t sc = e4m3_scale_code(amax);
      const double s = e4m3_to_f64(sc);
      sdst[g] = uint8_t(sc);
      for (int i = 0; i < group; i += 2) {
        uint32_t lo = 0u, hi = 0u;
        if (s > 0.0) {
          lo = e2m1_code(x[i], s);
          hi = e2m1_code(x[i + 1], s);
        }
        dst[(g * group + i) / 2] = uint8_t(lo | (hi << 4));
      }
    }
  }
}

// ACT_BF16 is a template parameter: a runtime dtype branch inside the
// unrolled W_ik loop would make the compiler wait for every load in turn.
template <bool ACT_BF16>
__global__ __launch_bounds__(kThreads) void compress_kernel(
    int d, int d_rope, int d_idx, int kv_dtype, int main_group, int idx_group, int ratio,
    int64_t capacity, RopeTable rope, const void* __restrict__ latent, const int32_t* __restrict__ first_pos,
    int n_pos, const float* __restrict__ pair_logits, const void* __restrict__ w_ik, void* main,
    uint8_t* main_scale, void* idx_k, uint8_t* idx_scale) {
  extern __shared__ double sh[];
  double* e = sh;       // [d]  merged, then rotated entry
  double* kap = sh + d;  // [d_idx] projection
  constexpr int act_bf16 = ACT_BF16 ? 1 : 0;
  const int m = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int64_t fp = first_pos[b];
  if (fp < 0 || fp % ratio) return;
  const int64_t j = fp / ratio + m;
  if (j < 0 || j >= capacity) return;
  const int64_t row = int64_t(b) * capacity + j;

  // 1. merge the ratio adjacent rows with the per-channel softmax weights
  for (int c = tid; c < d; c += kThreads) {
    double acc;
    if (ratio == 1) {
      acc = double(act_load(latent, (int64_t(b) * n_pos + m) * d + c, act_bf16));
    } else {
      double mx = -INFINITY;
      for (int i = 0; i < ratio; ++i) mx = fmax(mx, double(pair_logits[i * d + c]));
      double den = 0.0;
      for (int i = 0; i < ratio; ++i) den += exp(double(pair_logits[i * d + c]) - mx);
      acc = 0.0;
      for (int i = 0; i < ratio; ++i) {
        const double a = exp(double(pair_logits[i * d + c]) - mx) / den;
        acc += a * double(act_load(latent, (int64_t(b) * n_pos + int64_t(ratio) * m + i) * d + c, act_bf16));
      }
    }
    e[c] = acc;
  }
  __syncthreads();

  // 2. rotate the trailing d_rope channels at the entry's last position
  const double p = double(int64_t(ratio) * j + ratio - 1);
  const int c0 = d - d_rope;
  for (int mm = tid; mm < d_rope / 2; mm += kThreads) {
    const double freq = rope.inv_freq[mm];
    double sn, cs;
    sincos(p * freq, &sn, &cs);
    const double x = e[c0 + 2 * mm], y = e[c0 + 2 * mm + 1];
    e[c0 + 2 * mm] = x * cs - y * sn;
    e[c0 + 2 * mm + 1] = x * sn + y * cs;
  }
  __syncthreads();

  // 3. main KV row
  store_row(e, d, kv_dtype, main_group, main, main_scale, row);

  // 4. indexer K = e_hat . W_ik, from the unrounded rotated entry.  Thread
  // (part, pair) sums output channels 2*pair, 2*pair+1 over a slice of the
  // input channels; W_ik rows are read as contiguous pairs, 32 loads in
  // flight before the FMAs (this kernel is latency-bound, not
  // bandwidth-bound); the float64 partials are added through LDS.
  {
    const int pairs = d_idx / 2;
    const int parts = kThreads / pairs > 0 ? kThreads / pairs : 1;
    const int pair = tid % pairs, part = tid / pairs;
    const int span = (d + parts - 1) / parts;
    double* red = kap + d_idx;  // [parts][d_idx]
    if (part < parts) {
      double a0 = 0.0, a1 = 0.0;
      const int c_lo = part * span, c_hi = min(d, c_lo + span);
      for (int p0 = pair; p0 < pairs; p0 += kThreads) {
        a0 = a1 = 0.0;
        int c = c_lo;
        for (; c + 32 <= c_hi; c += 32) {
          float w0[32], w1[32];
#pragma unroll
          for (int u = 0; u < 32; ++u) {
            const int64_t off = int64_t(c + u) * d_idx + 2 * p0;
            if constexpr (ACT_BF16) {
              const uint32_t two = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(w_ik) + off);
              w0[u] = bf16_to_f32(uint16_t(two & 0xFFFFu));
              w1[u] = bf16_to_f32(uint16_t(two >> 16));
            } else {
              const float2 two = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(w_ik) + off);
              w0[u] = two.x;
              w1[u] = two.y;
            }
          }
#pragma unroll
          for (int u = 0; u < 32; ++u) {
            a0 += e[c + u] * double(w0[u]);
            a1 += e[c + u] * double(w1[u]);
          }
        }
        for (; c < c_hi; ++c) {
          a0 += e[c] * double(act_load(w_ik, int64_t(c) * d_idx + 2 * p0, act_bf16));
          a1 += e[c] * double(act_load(w_ik, int64_t(c) * d_idx + 2 * p0 + 1, act_bf16));
        }
        red[part * d_idx + 2 * p0] = a0;
        red[part * d_idx + 2 * p0 + 1] = a1;
      }
    }
    __syncthreads();
    for (int o = tid; o < d_idx; o += kThreads) {
      double acc = 0.0;
      for (int x = 0; x < parts; ++x) acc += red[x * d_idx + o];
      kap[o] = acc;
    }
  }
  __syncthreads();
  store_row(kap, d_idx, kv_dtype, idx_group, idx_k, idx_scale, row);
}

}  // namespace

hipError_t launch_compress(const csa2_dims& dims, const csa2_kv_cache& cache, const void* latent,
                           const int32_t* first_pos, int32_t n_pos, const float* pair_logits, const void* w_ik,
                           hipStream_t stream) {
  const dim3 grid(n_pos / cache.ratio, cache.batch);
  const int parts = kThreads / (dims.d_idx / 2) > 0 ? kThreads / (dims.d_idx / 2) : 1;
  const size_t lds = sizeof(double) * size_t(dims.d + dims.d_idx + parts * dims.d_idx);
  auto kern = dims.act_dtype == CSA2_BF16 ? compress_kernel<true> : compress_kernel<false>;
  const hipError_t err = launch_kernel(CSA2_KERNEL_COMPRESS, kern, grid, dim3(kThreads), lds, stream, dims.d, dims.d_rope, dims.d_idx, cache.kv_dtype, cache.main_group, cache.idx_group, cache.ratio,
                     cache.capacity, make_rope_table(dims), latent, first_pos, n_pos, pair_logits, w_ik, cache.main,
                     cache.main_scale, cache.idx_k, cache.idx_scale);
  return err;
}

}  // namespace csa2
