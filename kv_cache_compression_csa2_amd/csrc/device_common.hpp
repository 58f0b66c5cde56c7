// Device helpers shared by the CSA2 kernels: storage formats, score keys,
// block-wide scans.  gfx950 (CDNA4), wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

constexpr int kWave = 64;

// Pointer into LDS that keeps its address space through structs and calls, so
// accesses compile to ds_* instructions instead of generic (flat) ones.
typedef __attribute__((address_space(3))) uint32_t lds_u32;

__device__ __forceinline__ void lds_inc(lds_u32* p) {
  __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// ---------------------------------------------------------------- bfloat16 --

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// float32 -> bfloat16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// float64 -> bfloat16 with a single rounding to nearest even: first round to
// odd into float32 (truncate, then set the last bit if anything was lost),
// then round float32 to bfloat16.  Rounding to odd into a format with at
// least two more significand bits than the target makes the second rounding
// exact (Boldo & Melquiond, "When double rounding is odd").
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  float f = __double2float_rz(x);
  if (double(f) != x) f = __uint_as_float(__float_as_uint(f) | 1u);
  return f32_to_bf16(f);
}

// ------------------------------------------------------------- E4M3 / E2M1 --

// Value of an E4M3 (FN) code: bias 7, subnormals below exponent field 1.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : float(m) * (1.0f / 512.0f);
  return (c & 0x80u) ? -v : v;
}

__device__ __forceinline__ double e4m3_to_f64(uint32_t c) { return double(e4m3_to_f32(c)); }

// Magnitudes of the E2M1 codes 0..7.
__device__ __forceinline__ float e2m1_mag(uint32_t i) {
  // 0, 0.5, 1, 1.5, 2, 3, 4, 6
  const uint32_t e = (i >> 1) & 3u, m = i & 1u;
  return e ? __uint_as_float(((e + 126u) << 23) | (m << 22)) : 0.5f * float(m);
}

__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const float v = e2m1_mag(c & 7u);
  return (c & 8u) ? -v : v;
}

// E4M3 code of the value nearest to amax/6 (ties to the even code),
// saturating at 448.  Decided by exact comparisons of amax against 6x the
// candidate values and midpoints, so no rounded quotient decides it.
__device__ __forceinline__ uint32_t e4m3_scale_code(double amax) {
  if (!(amax > 0.0)) return 0u;
  if (amax >= 6.0 * 448.0) return 0x7Eu;
  // c = the largest code in [0, 0x7E] with 6*value(c) <= amax (values
  // increase with the code).  First the largest code whose value is at most
  // the rounded quotient x = amax / 6, read off x's exponent and leading
  // significand bits (below 2^-6: the subnormal codes m 2^-9); x lies within
  // half an ulp of amax / 6 and neighbouring E4M3 values differ by more than
  // 1/16 of the larger, so no more than one value lies between them and one
  // exact comparison each way corrects the estimate.
  const double x = amax / 6.0;
  uint32_t c;
  if (x < 0.015625) {
    c = uint32_t(x * 512.0);  // floor, 0..7
  } else {
    const uint64_t u = uint64_t(__double_as_longlong(x));
    const int ex = int((u >> 52) & 0x7FFu) - 1023;  // -6 .. 8
    c = min((uint32_t(ex + 7) << 3) | (uint32_t(u >> 49) & 7u), 0x7Eu);
  }
  if (c > 0u && 6.0 * e4m3_to_f64(c) > amax) --c;
  else if (c < 0x7Eu && 6.0 * e4m3_to_f64(c + 1u) <= amax) ++c;
  if (c == 0x7Eu) return c;
  const double m6 = 3.0 * (e4m3_to_f64(c) + e4m3_to_f64(c + 1u));  // 6 * midpoint, exact
  if (amax > m6) return c + 1u;
  if (amax == m6) return (c & 1u) ? c + 1u : c;
  return c;
}

// E2M1 code of the value v whose v*scale is nearest to x (ties to the even
// code), saturating at 6; zero magnitude is code 0.  scale > 0.
__device__ __forceinline__ uint32_t e2m1_code(double x, double scale) {
  const double a = fabs(x);
  uint32_t idx = 0u;
  // midpoints between consecutive magnitudes; each product is exact
  const double mids[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
#pragma unroll
  for (int i = 0; i < 7; ++i) {
    const double m = mids[i] * scale;
    idx += (a > m) || (a == m && ((i + 1) & 1) == 0);
  }
  return (signbit(x) && idx) ? (idx | 8u) : idx;
}

// ------------------------------------------------------------- score keys --

// Order-preserving map of a float score to uint32 (larger score -> larger
// key).  -0 is folded onto +0 so that equal scores compare equal.  -inf (an
// invalid slot) maps below every finite score.
__device__ __forceinline__ uint32_t score_key(float s) {
  if (s == 0.0f) s = 0.0f;
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr uint32_t kKeyNegInf = 0x007FFFFFu;  // score_key(-inf)
constexpr uint32_t kKeyForced = 0xFFFFFFFFu;  // above every finite score

// ------------------------------------------------------------ block scans --

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

// Exclusive prefix sum over the threads of a block of NT threads (NT a
// multiple of 64).  `total` receives the block total.  `scratch` holds
// NT/64 + 1 words of LDS.  Contains barriers: call from all threads.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scratch, uint32_t& total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const uint32_t inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) scratch[wid] = inc;
  __syncthreads();
  if (wid == 0) {
    uint32_t w = lane < NW ? scratch[lane] : 0u;
    const uint32_t wi = wave_inclusive_scan(w);
    if (lane < NW) scratch[lane] = wi - w;
    if (lane == NW - 1) scratch[NW] = wi;
  }
  __syncthreads();
  const uint32_t out = scratch[wid] + inc - v;
  total = scratch[NW];
  __syncthreads();
  return out;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// ------------------------------------------------------------ row readers --

// Visible entries of a query at position t: entry j is visible iff
// ratio*j + ratio - 1 <= t, and j < n (n already clamped to capacity).
__device__ __forceinline__ int64_t visible_count(int64_t n, int64_t t, int ratio) {
  if (t + 1 <= 0) return 0;
  const int64_t v = (t + 1) / ratio;
  return v < n ? v : n;
}

__device__ __forceinline__ int64_t clamp_entries(const int32_t* n_entries, int b, int64_t capacity) {
  int64_t n = n_entries[b];
  return n < 0 ? 0 : (n > capacity ? capacity : n);
}

// Element c of an activation row (float32 or bfloat16 bits).
__device__ __forceinline__ float act_load(const void* base, int64_t off, int act_bf16) {
  return act_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[off])
                  : reinterpret_cast<const float*>(base)[off];
}

// Indexer K layout.  Each sequence's rows are padded to a multiple of 32 and
// stored in tiles of 32 rows; inside a tile the rows' 16-byte chunks are
// transposed: chunk c of row r lies at byte (32 c + r % 32) * 16 of tile
// r / 32, so chunk c of the tile's 32 rows is 512 contiguous bytes.  A load in
// the MFMA operand layout (one lane per row, 16 bytes each) is then one
// contiguous run per 32 lanes.  FP4 scales stay row-major.
__host__ __device__ constexpr int64_t idx_rows_padded(int64_t capacity) { return (capacity + 31) / 32 * 32; }

// Byte x of indexer K row `row` (row counted over all sequences, each padded
// to idx_rows_padded(capacity) rows; row_bytes a multiple of 16).
__device__ __forceinline__ int64_t idx_byte(int64_t row, int row_bytes, int x) {
  return (row >> 5) * (int64_t(row_bytes) << 5) + ((int64_t(x >> 4) << 5) + (row & 31)) * 16 + (x & 15);
}

// Element c of indexer K row `row` (tiled as above; FP4 scales of the same
// entry at row-major row `srow`).
__device__ __forceinline__ float idx_load(const void* data, const uint8_t* scale, int dtype, int64_t row, int64_t srow,
                                          int width, int group, int c) {
  const uint8_t* d = reinterpret_cast<const uint8_t*>(data);
  if (dtype == 0) return *reinterpret_cast<const float*>(d + idx_byte(row, 4 * width, 4 * c));
  if (dtype == 1) return bf16_to_f32(*reinterpret_cast<const uint16_t*>(d + idx_byte(row, 2 * width, 2 * c)));
  const uint8_t byte = d[idx_byte(row, width / 2, c >> 1)];
  const uint32_t code = (c & 1) ? (byte >> 4) : (byte & 0xF);
  return e2m1_to_f32(code) * e4m3_to_f32(scale[srow * (width / group) + c / group]);
}

// Element c of cache row `row` (F32 = 0, BF16 = 1, FP4 = 2).
__device__ __forceinline__ float cache_load(const void* data, const uint8_t* scale, int dtype, int64_t row,
                                            int width, int group, int c) {
  if (dtype == 0) return reinterpret_cast<const float*>(data)[row * width + c];
  if (dtype == 1) return bf16_to_f32(reinterpret_cast<const uint16_t*>(data)[row * width + c]);
  const uint8_t byte = reinterpret_cast<const uint8_t*>(data)[row * (width / 2) + (c >> 1)];
  const uint32_t code = (c & 1) ? (byte >> 4) : (byte & 0xF);
  return e2m1_to_f32(code) * e4m3_to_f32(scale[row * (width / group) + c / group]);
}

}  // namespace csa2
