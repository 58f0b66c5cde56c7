// Compressor arithmetic for one cache entry, shared by the compress kernel
// and the decode scan that writes the step's entry itself.
//
// Pages: zartbot walkthrough (hn.213312.xyz) section 2.3.1 (ratio 2 in the
// encoder with channel-wise learned weights, ratio 1 in the decoder, no
// overlap; indexer K projected from the main KV) and section 2.4.4 (the cache
// is quantised after RoPE, FP4 main KV).
//
// Everything before the stores runs in float64: the merge, the rotation
// (angles and sin/cos) and the 512 -> 128 projection, so each stored value is
// the single rounding of the exact value and agrees bit-for-bit with an
// independent float64 computation except when that value sits within float64
// noise of a rounding boundary.
//
// The compress kernel runs an entry on 1024 threads: thread c owns channel c
// of the merge, the rotation and the row stores, and thread (part, pair)
// sums projection outputs 2 pair and 2 pair + 1 over its part's slice of
// input channels; the parts' partial sums are then added in part order.  The
// decode scan's compressing workgroup runs the same entry on 256 threads
// (d = 512, d_idx = 128): thread t owns channels t and t + 256, and in the
// projection sums outputs 8 (t % 16) .. 8 (t % 16) + 7 over part t / 16.
// Each output's sum over a part's channels, and over the parts, is formed in
// the same order in both, so both store the same bits.
#pragma once

#include "device_common.hpp"
#include "launch.hpp"

namespace csa2 {

constexpr int kCompressVirtual = 1024;
constexpr int kCompressPre = 32;  // input channels of W_ik loaded per batch

// LDS doubles an entry needs: the entry, the projection, the projection
// partials of every part.
__host__ __device__ constexpr int compress_lds_doubles(int d, int d_idx) {
  return d + d_idx + (kCompressVirtual / (d_idx / 2)) * d_idx;
}

// Store channel c (on: c < n) of a row of float64 values in the given format.
// FP4: the `group` channels of one scale are `group` consecutive lanes of one
// wave (group is 16 or 32 and channel groups start at multiples of it), so
// the group's largest magnitude comes from a butterfly over those lanes,
// every lane derives the same scale code, encodes its own value, and the even
// lane of each pair writes the byte.  Every lane of the wave must call it (the
// butterflies), with consecutive channels on consecutive lanes.  `tiled`: the
// row goes to indexer K tile storage at data row `drow`; the FP4 scales always
// go row-major to row `row`.  `mirror` (LDS, or NULL): the stored bytes of
// the row again, row-major (bf16: 2 n bytes; FP4: n / 2 code bytes, then the
// n / group scale bytes).
__device__ __forceinline__ void store_channel(double x_in, int c, int n, int dtype, int group, void* base,
                                              uint8_t* scale_base, int64_t row, bool tiled, int64_t drow,
                                              uint8_t* mirror = nullptr) {
  const bool on = c < n;
  uint8_t* bytes = reinterpret_cast<uint8_t*>(base);
  if (dtype == CSA2_F32) {
    if (on) *reinterpret_cast<float*>(bytes + (tiled ? idx_byte(drow, 4 * n, 4 * c) : (row * n + c) * 4)) = __double2float_rn(x_in);
  } else if (dtype == CSA2_BF16) {
    const uint16_t v = f64_to_bf16(x_in);
    if (on) *reinterpret_cast<uint16_t*>(bytes + (tiled ? idx_byte(drow, 2 * n, 2 * c) : (row * n + c) * 2)) = v;
    if (on && mirror) reinterpret_cast<uint16_t*>(mirror)[c] = v;
  } else {
    const double x = on ? x_in : 0.0;
    double amax = fabs(x);
    for (int o = 1; o < group; o <<= 1) amax = fmax(amax, __shfl_xor(amax, o));
    const uint32_t sc = e4m3_scale_code(amax);
    const double s = e4m3_to_f64(sc);
    const uint32_t code = s > 0.0 ? e2m1_code(x, s) : 0u;
    const uint32_t odd = uint32_t(__shfl_xor(int(code), 1));
    if (on && (c & 1) == 0) bytes[tiled ? idx_byte(drow, n / 2, c / 2) : row * (n / 2) + c / 2] = uint8_t(code | (odd << 4));
    if (on && c % group == 0) scale_base[row * (n / group) + c / group] = uint8_t(sc);
    if (on && mirror && (c & 1) == 0) mirror[c / 2] = uint8_t(code | (odd << 4));
    if (on && mirror && c % group == 0) mirror[n / 2 + c / group] = uint8_t(sc);
  }
}

// A batch of W_ik as loaded: rows c .. c+kCompressPre, columns 2 pair and
// 2 pair + 1 (bf16: one 32-bit word per row; float32: two).  Converted at use,
// so a batch in flight costs kCompressPre (bf16) registers.
template <bool ACT_BF16>
struct WBatch {
  uint32_t v[kCompressPre][ACT_BF16 ? 1 : 2];
};

// Issue the loads of a W_ik batch; rows past c_hi read row c_hi - 1.
template <bool ACT_BF16>
__device__ __forceinline__ void load_w(const void* __restrict__ w_ik, int d_idx, int pair, int c, int c_hi,
                                       WBatch<ACT_BF16>& W) {
  const bool whole = c + kCompressPre <= c_hi;  // (no clamping: plain strided addresses)
#pragma unroll
  for (int u = 0; u < kCompressPre; ++u) {
    const int64_t off = int64_t(whole ? c + u : min(c + u, c_hi - 1)) * d_idx + 2 * pair;
    if constexpr (ACT_BF16) {
      W.v[u][0] = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(w_ik) + off);
    } else {
      const uint2 two = *reinterpret_cast<const uint2*>(reinterpret_cast<const float*>(w_ik) + off);
      W.v[u][0] = two.x;
      W.v[u][1] = two.y;
    }
  }
}

template <bool ACT_BF16>
__device__ __forceinline__ float w_col0(const WBatch<ACT_BF16>& W, int u) {
  if constexpr (ACT_BF16) return bf16_to_f32(uint16_t(W.v[u][0] & 0xFFFFu));
  else return __uint_as_float(W.v[u][0]);
}
template <bool ACT_BF16>
__device__ __forceinline__ float w_col1(const WBatch<ACT_BF16>& W, int u) {
  if constexpr (ACT_BF16) return bf16_to_f32(uint16_t(W.v[u][0] >> 16));
  else return __uint_as_float(W.v[u][1]);
}

// The projection of a 256-thread block (d = 512, d_idx = 128, bf16 W_ik):
// thread t sums output channels 8 (t % 16) .. 8 (t % 16) + 7 over the 32
// input channels of part t / 16 - the 16 parts and spans of the 1024-thread
// layout, and each output's sum formed in the same order, so the same bits -
// reading W_ik 16 bytes (8 columns) at a time, WR rows per batch.
template <int WR>
struct WideBatch {
  uint4 v[WR];
};
template <int WR>
__device__ __forceinline__ void load_w_wide(const void* __restrict__ w_ik, int col, int c, WideBatch<WR>& W) {
#pragma unroll
  for (int u = 0; u < WR; ++u)
    W.v[u] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(w_ik) + int64_t(c + u) * 128 + col);
}

// Write entry m of sequence b (the entry at first_pos[b] / ratio + m) with a
// block of NT threads: 1024 (any shape), or 256 for d = 512, d_idx = 128,
// bf16 activations (fixed at compile time, so every load is unconditional and
// unrolled: a load under a branch makes the compiler wait for it where the
// branch joins).  Returns the entry's index, or -1 when first_pos[b] is not
// a whole entry or the entry lies outside the cache (nothing written).
// `sh`: LDS of compress_lds_doubles(d, d_idx) doubles.  `mirror` (LDS or
// NULL): receives the stored indexer K row (see store_channel), complete
// after the block's next barrier.  Every thread of the block calls it.
// ACT_BF16 is a template parameter: a runtime dtype branch inside the
// unrolled W_ik loop would make the compiler wait for every load in turn.
//
// The loads that do not depend on the entry's position - the latent rows,
// then the first PRE batches of W_ik - are issued before first_pos[b] is
// known, so one round trip to memory brings them all (the latent first, so
// the merge need not wait for W_ik), and the rotation's sines and cosines are
// computed while they are in flight; each later batch of W_ik is issued when
// the batch PRE places before it has been used.  WR: rows of W_ik per batch of
// the 256-thread projection.
template <bool ACT_BF16, int NT, int PRE = 1, int WR = 16>
__device__ int64_t compress_entry(const CompressParams& P, int m, int b, double* sh, uint8_t* mirror = nullptr) {
  constexpr bool kWide = NT == 256;
  static_assert(NT == kCompressVirtual || (kWide && ACT_BF16), "1024 threads, or 256 for the fixed shape");
  constexpr int R = kWide ? 2 : 1;  // latent channels per thread
  constexpr int kWideSpan = 32;     // 512 input channels / 16 parts
  constexpr int kBatches = kWide ? kWideSpan / WR : 1;
  static_assert(!kWide || (kWideSpan % WR == 0 && PRE >= 1 && PRE <= kBatches), "W_ik batches");
  static_assert(kWide || PRE == 1, "one batch in flight at 1024 threads");
  const int d = kWide ? 512 : P.d, d_idx = kWide ? 128 : P.d_idx;
  double* e = sh;                 // [d]  merged, then rotated entry
  double* kap = sh + d;           // [d_idx] projection
  double* red = kap + d_idx;      // [parts][d_idx] partial projections
  constexpr int act_bf16 = ACT_BF16 ? 1 : 0;
  const int tid = threadIdx.x;
  const int ratio = P.ratio;

  // 1024-thread projection layout: thread (part, pair) sums output channels
  // 2 pair and 2 pair + 1 over the input channels [c_lo, c_hi); d_idx <= 512
  // gives pairs <= 256 and parts >= 4, so every thread has one pair.
  const int pairs = d_idx / 2;
  const int parts = kCompressVirtual / pairs;
  const int span = (d + parts - 1) / parts;
  const int pair = tid % pairs, part = tid / pairs;
  const int c_lo = min(d, part * span), c_hi = min(d, c_lo + span);
  // 256-thread layout
  const int w_col = 8 * (tid & 15), w_part = tid >> 4, w_lo = w_part * kWideSpan;

  // 1a. the latent row as stored (used when one position makes an entry;
  // loaded whatever the ratio - row m exists - and converted at use, so
  // nothing waits for it here)
  uint32_t lat[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t off = (int64_t(b) * P.n_pos + m) * d + min(tid + NT * r, d - 1);
    if constexpr (ACT_BF16) lat[r] = reinterpret_cast<const uint16_t*>(P.latent)[off];
    else lat[r] = reinterpret_cast<const uint32_t*>(P.latent)[off];
  }
  // 1b. the first batches of W_ik
  WBatch<ACT_BF16> wb;
  WideBatch<WR> ww[kBatches];
  if constexpr (kWide) {
#pragma unroll
    for (int q = 0; q < PRE; ++q) load_w_wide<WR>(P.w_ik, w_col, w_lo + q * WR, ww[q]);
  } else {
    if (part < parts && c_lo < c_hi) load_w<ACT_BF16>(P.w_ik, d_idx, pair, c_lo, c_hi, wb);
  }

  // the entry's place (uniform over the block: nothing is written when it
  // has none, and every thread returns here), and the rotation angle's sine
  // and cosine for thread i < d_rope / 2, computed while the loads are in
  // flight
  const int64_t fp = P.first_pos[b];
  if (fp < 0 || fp % P.ratio) return -1;
  const int64_t j = fp / P.ratio + m;
  if (j < 0 || j >= P.capacity) return -1;
  const int64_t row = int64_t(b) * P.capacity + j;
  double sn = 0.0, cs = 1.0;
  if (tid < P.d_rope / 2) sincos(double(int64_t(ratio) * j + ratio - 1) * P.rope.inv_freq[tid], &sn, &cs);

  // 1c. merge the ratio adjacent rows with the per-channel softmax weights
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = tid + NT * r;
    if (c >= d) continue;
    double acc;
    if (ratio == 1) {
      acc = double(ACT_BF16 ? bf16_to_f32(uint16_t(lat[r])) : __uint_as_float(lat[r]));
    } else {
      double mx = -INFINITY;
      for (int i = 0; i < ratio; ++i) mx = fmax(mx, double(P.pair_logits[i * d + c]));
      double den = 0.0;
      for (int i = 0; i < ratio; ++i) den += exp(double(P.pair_logits[i * d + c]) - mx);
      // the weights sum to 1: the last row plus the weighted differences of
      // the others (exact when the merged rows agree)
      const int64_t row0 = (int64_t(b) * P.n_pos + int64_t(ratio) * m) * d + c;
      const double last = double(act_load(P.latent, row0 + int64_t(ratio - 1) * d, act_bf16));
      double dsum = 0.0;
      for (int i = 0; i < ratio - 1; ++i) {
        const double a = exp(double(P.pair_logits[i * d + c]) - mx) / den;
        dsum += a * (double(act_load(P.latent, row0 + int64_t(i) * d, act_bf16)) - last);
      }
      acc = dsum + last;
    }
    e[c] = acc;
  }

  // 2. rotation of the trailing d_rope channels at the entry's last position
  const int c0 = d - P.d_rope;
  __syncthreads();
  if (tid < P.d_rope / 2) {
    const double x = e[c0 + 2 * tid], y = e[c0 + 2 * tid + 1];
    e[c0 + 2 * tid] = x * cs - y * sn;
    e[c0 + 2 * tid + 1] = x * sn + y * cs;
  }
  __syncthreads();

  // 3. main KV row
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = tid + NT * r;
    store_channel(c < d ? e[c] : 0.0, c, d, P.kv_dtype, P.main_group, P.main, P.main_scale, row, false, row);
  }

  // 4. indexer K = e_hat . W_ik, from the unrounded rotated entry, summed
  // over the input channels in order; the float64 partials of the parts are
  // added through LDS.
  if constexpr (kWide) {
    double acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.0;
#pragma unroll
    for (int q = 0; q < kBatches; ++q) {
      WideBatch<WR>& W = ww[q];
#pragma unroll
      for (int u = 0; u < WR; ++u) {
        const double ev = e[w_lo + q * WR + u];
        const uint32_t w4[4] = {W.v[u].x, W.v[u].y, W.v[u].z, W.v[u].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[2 * k] += ev * double(bf16_to_f32(uint16_t(w4[k] & 0xFFFFu)));
          acc[2 * k + 1] += ev * double(bf16_to_f32(uint16_t(w4[k] >> 16)));
        }
      }
      // the batch PRE places on, once this one is used
      if (q + PRE < kBatches) load_w_wide<WR>(P.w_ik, w_col, w_lo + (q + PRE) * WR, ww[q + PRE]);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) red[w_part * 128 + w_col + k] = acc[k];
  } else if (part < parts) {
    double a0 = 0.0, a1 = 0.0;
    for (int c = c_lo; c < c_hi; c += kCompressPre) {
      if (c != c_lo) load_w<ACT_BF16>(P.w_ik, d_idx, pair, c, c_hi, wb);
      const int cnt = min(kCompressPre, c_hi - c);
      if (cnt == kCompressPre) {
        // a whole batch: no per-element branches, so the entry's values are
        // read from LDS ahead of the two dependent sums
#pragma unroll
        for (int u = 0; u < kCompressPre; ++u) {
          a0 += e[c + u] * double(w_col0(wb, u));
          a1 += e[c + u] * double(w_col1(wb, u));
        }
      } else {
#pragma unroll
        for (int u = 0; u < kCompressPre; ++u) {
          if (u < cnt) {
            a0 += e[c + u] * double(w_col0(wb, u));
            a1 += e[c + u] * double(w_col1(wb, u));
          }
        }
      }
    }
    red[part * d_idx + 2 * pair] = a0;
    red[part * d_idx + 2 * pair + 1] = a1;
  }
  __syncthreads();
  if (tid < d_idx) {
    // (in order over the parts, the loads of four issued together)
    double s = 0.0;
    int x = 0;
    for (; x + 4 <= parts; x += 4) {
      const double r0 = red[x * d_idx + tid], r1 = red[(x + 1) * d_idx + tid];
      const double r2 = red[(x + 2) * d_idx + tid], r3 = red[(x + 3) * d_idx + tid];
      s += r0;
      s += r1;
      s += r2;
      s += r3;
    }
    for (; x < parts; ++x) s += red[x * d_idx + tid];
    kap[tid] = s;
  }
  __syncthreads();
  // (d_idx <= 512 channels: one per thread at 1024 threads, 128 at 256)
  const int c = tid;
  store_channel(c < d_idx ? kap[min(c, d_idx - 1)] : 0.0, c, d_idx, P.kv_dtype, P.idx_group, P.idx_k, P.idx_scale, row,
                true, int64_t(b) * idx_rows_padded(P.capacity) + j, mirror);
  return j;
}

}  // namespace csa2
