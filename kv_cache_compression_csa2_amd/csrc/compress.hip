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
constexpr int kPre = 32;  // input channels of W_ik a thread loads per batch

// Store `n` float64 values (n <= kThreads) as one cache row of the given
// format; thread c stores channel c.  FP4: the `group` channels of one scale
// are `group` consecutive lanes of one wave (group is 16 or 32 and channel
// groups start at multiples of it), so the group's largest magnitude comes
// from a butterfly over those lanes, every lane derives the same scale code,
// encodes its own value, and the even lane of each pair writes the byte.
// `tiled`: the row goes to indexer K tile storage at data row `drow`; the
// FP4 scales always go row-major to row `row`.
__device__ void store_row(const double* v, int n, int dtype, int group, void* base, uint8_t* scale_base, int64_t row,
                          bool tiled, int64_t drow) {
  const int c = threadIdx.x;
  const bool on = c < n;
  uint8_t* bytes = reinterpret_cast<uint8_t*>(base);
  if (dtype == CSA2_F32) {
    if (on) *reinterpret_cast<float*>(bytes + (tiled ? idx_byte(drow, 4 * n, 4 * c) : (row * n + c) * 4)) = __double2float_rn(v[c]);
  } else if (dtype == CSA2_BF16) {
    if (on) *reinterpret_cast<uint16_t*>(bytes + (tiled ? idx_byte(drow, 2 * n, 2 * c) : (row * n + c) * 2)) = f64_to_bf16(v[c]);
  } else {
    const double x = on ? v[c] : 0.0;
    double amax = fabs(x);
    for (int o = 1; o < group; o <<= 1) amax = fmax(amax, __shfl_xor(amax, o));
    const uint32_t sc = e4m3_scale_code(amax);
    const double s = e4m3_to_f64(sc);
    const uint32_t code = s > 0.0 ? e2m1_code(x, s) : 0u;
    const uint32_t odd = uint32_t(__shfl_xor(int(code), 1));
    if (on && (c & 1) == 0) bytes[tiled ? idx_byte(drow, n / 2, c / 2) : row * (n / 2) + c / 2] = uint8_t(code | (odd << 4));
    if (on && c % group == 0) scale_base[row * (n / group) + c / group] = uint8_t(sc);
  }
}

// W_ik[c .. c+kPre) x columns (2 pair, 2 pair + 1), rows past c_hi read row c_hi - 1.
template <bool ACT_BF16>
__device__ __forceinline__ void load_w(const void* __restrict__ w_ik, int d_idx, int pair, int c, int c_hi,
                                       float (&w0)[kPre], float (&w1)[kPre]) {
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const int64_t off = int64_t(min(c + u, c_hi - 1)) * d_idx + 2 * pair;
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
}

// ACT_BF16 is a template parameter: a runtime dtype branch inside the
// unrolled W_ik loop would make the compiler wait for every load in turn.
//
// The kernel is latency-bound (one entry per sequence in decode), so the
// reads that do not depend on the entry - this thread's first batch of W_ik
// (bf16) and its rotation angle - are issued or computed while the latent
// rows are still on their way.  d <= kThreads: thread c owns channel c.
template <bool ACT_BF16>
__global__ __launch_bounds__(kThreads) void compress_kernel(
    int d, int d_rope, int d_idx, int kv_dtype, int main_group, int idx_group, int ratio,
    int64_t capacity, RopeTable rope, const void* __restrict__ latent, const int32_t* __restrict__ first_pos,
    int n_pos, const float* __restrict__ pair_logits, const void* __restrict__ w_ik, void* main,
    uint8_t* main_scale, void* idx_k, uint8_t* idx_scale) {
  extern __shared__ double sh[];
  double* e = sh;       // [d]  merged, then rotated entry
  double* kap = sh + d;  // [d_idx] projection
  double* red = kap + d_idx;  // [parts][d_idx] partial projections
  constexpr int act_bf16 = ACT_BF16 ? 1 : 0;
  const int m = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int64_t fp = first_pos[b];
  if (fp < 0 || fp % ratio) return;
  const int64_t j = fp / ratio + m;
  if (j < 0 || j >= capacity) return;
  const int64_t row = int64_t(b) * capacity + j;

  // Projection layout: thread (part, pair) sums output channels 2 pair and
  // 2 pair + 1 over the input channels [c_lo, c_hi); d_idx <= 512 gives
  // pairs <= 256 and parts >= 4, so every thread has one pair.
  const int pairs = d_idx / 2;
  const int parts = kThreads / pairs;
  const int pair = tid % pairs, part = tid / pairs;
  const int span = (d + parts - 1) / parts;
  const int c_lo = min(d, part * span), c_hi = min(d, c_lo + span);  // empty for a trailing part
  const bool proj = part < parts;
  // (bf16 weights only: 64 float32 weights held this long would not fit the
  // 128 registers of a 1024-thread workgroup next to the float64 work)
  float w0[kPre], w1[kPre];
  if (ACT_BF16 && proj && c_lo < c_hi) load_w<ACT_BF16>(w_ik, d_idx, pair, c_lo, c_hi, w0, w1);

  // 1. merge the ratio adjacent rows with the per-channel softmax weights
  double acc = 0.0;
  if (tid < d) {
    const int c = tid;
    if (ratio == 1) {
      acc = double(act_load(latent, (int64_t(b) * n_pos + m) * d + c, act_bf16));
    } else {
      double mx = -INFINITY;
      for (int i = 0; i < ratio; ++i) mx = fmax(mx, double(pair_logits[i * d + c]));
      double den = 0.0;
      for (int i = 0; i < ratio; ++i) den += exp(double(pair_logits[i * d + c]) - mx);
      // the weights sum to 1: the last row plus the weighted differences of
      // the others (exact when the merged rows agree)
      const int64_t row0 = (int64_t(b) * n_pos + int64_t(ratio) * m) * d + c;
      const double last = double(act_load(latent, row0 + int64_t(ratio - 1) * d, act_bf16));
      double dsum = 0.0;
      for (int i = 0; i < ratio - 1; ++i) {
        const double a = exp(double(pair_logits[i * d + c]) - mx) / den;
        dsum += a * (double(act_load(latent, row0 + int64_t(i) * d, act_bf16)) - last);
      }
      acc = dsum + last;
    }
  }

  // 2. rotation of the trailing d_rope channels at the entry's last position
  const int c0 = d - d_rope;
  double sn = 0.0, cs = 1.0;
  if (tid < d_rope / 2) sincos(double(int64_t(ratio) * j + ratio - 1) * rope.inv_freq[tid], &sn, &cs);
  if (tid < d) e[tid] = acc;
  __syncthreads();
  if (tid < d_rope / 2) {
    const double x = e[c0 + 2 * tid], y = e[c0 + 2 * tid + 1];
    e[c0 + 2 * tid] = x * cs - y * sn;
    e[c0 + 2 * tid + 1] = x * sn + y * cs;
  }
  __syncthreads();

  // 3. main KV row
  store_row(e, d, kv_dtype, main_group, main, main_scale, row, false, row);

  // 4. indexer K = e_hat . W_ik, from the unrounded rotated entry, summed
  // over the input channels in order; the float64 partials of the parts are
  // added through LDS.
  if (proj) {
    double a0 = 0.0, a1 = 0.0;
    for (int c = c_lo; c < c_hi; c += kPre) {
      if (!ACT_BF16 || c != c_lo) load_w<ACT_BF16>(w_ik, d_idx, pair, c, c_hi, w0, w1);
      const int cnt = min(kPre, c_hi - c);
#pragma unroll
      for (int u = 0; u < kPre; ++u) {
        if (u < cnt) {
          a0 += e[c + u] * double(w0[u]);
          a1 += e[c + u] * double(w1[u]);
        }
      }
    }
    red[part * d_idx + 2 * pair] = a0;
    red[part * d_idx + 2 * pair + 1] = a1;
  }
  __syncthreads();
  if (tid < d_idx) {
    double s = 0.0;
    for (int x = 0; x < parts; ++x) s += red[x * d_idx + tid];
    kap[tid] = s;
  }
  __syncthreads();
  store_row(kap, d_idx, kv_dtype, idx_group, idx_k, idx_scale, row, true, int64_t(b) * idx_rows_padded(capacity) + j);
}

}  // namespace

hipError_t launch_compress(const csa2_dims& dims, const csa2_kv_cache& cache, const void* latent,
                           const int32_t* first_pos, int32_t n_pos, const float* pair_logits, const void* w_ik,
                           hipStream_t stream) {
  const dim3 grid(n_pos / cache.ratio, cache.batch);
  const int parts = kThreads / (dims.d_idx / 2);
  const size_t lds = sizeof(double) * size_t(dims.d + dims.d_idx + parts * dims.d_idx);
  auto kern = dims.act_dtype == CSA2_BF16 ? compress_kernel<true> : compress_kernel<false>;
  const hipError_t err = launch_kernel(CSA2_KERNEL_COMPRESS, kern, grid, dim3(kThreads), lds, stream, dims.d, dims.d_rope, dims.d_idx, cache.kv_dtype, cache.main_group, cache.idx_group, cache.ratio,
                     cache.capacity, make_rope_table(dims), latent, first_pos, n_pos, pair_logits, w_ik, cache.main,
                     cache.main_scale, cache.idx_k, cache.idx_scale);
  return err;
}

}  // namespace csa2
