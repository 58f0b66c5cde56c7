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
    int d, int d_rope, int H, int topk, int window, int act_bf16, int kv_dtype, int main_group, RopeTable rope,
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
    const double freq = rope.inv_freq[m];
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


// ------------------------------------------------------------------ MFMA ---
//
// Production shape: d = 512, heads in groups of 32, bf16 queries, bf16 or FP4
// main KV.  A workgroup (4 waves) owns one (query, head group of 32, run of
// 32-row tiles); the rows of a query are the kept entries followed by the
// window rows, padded to whole tiles.  Per tile:
//   1. the 32 rows are staged in LDS as bf16 (FP4 rows are dequantised on the
//      way: codes converted exactly, then scaled in float32, exact);
//   2. logits L^T[row][head] = R . Q^T: wave w contracts its quarter of the
//      512 channels (8 x v_mfma_f32_32x32x16_bf16) and the four partial sums
//      are added through LDS;
//   3. online softmax per head (running max and denominator);
//   4. O[head][c] += P . R, where P comes straight from the logit registers
//      (the 32x32 accumulator layout - lane = one column, 16 rows - is the
//      operand layout of the next product) and R is put in that same layout
//      by multiplying the staged rows with a 0/1 selection matrix on the
//      MFMA unit, so no LDS transpose is needed.  Wave w owns channels
//      [128w, 128w+128) of the output.
// With several workgroups per (query, head group) each writes its
// unnormalised partial output and (max, denominator); attn_merge_kernel
// combines them by log-sum-exp weights.

typedef __bf16 bf16x8_t __attribute__((__vector_size__(16)));
typedef __bf16 bf16x2_t __attribute__((__vector_size__(4)));
typedef float f32x16_t __attribute__((__vector_size__(64)));

constexpr int kD = 512;
constexpr int kRowPitch = kD * 2 + 16;  // bytes per staged row; the pad spreads rows over LDS banks

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// 16 FP4 code bytes (32 values) -> 32 bf16 values times their E4M3 scales
// (s0 for the first 16 values, s1 for the rest); all products are exact.
__device__ __forceinline__ void dequant_fp4_32(uint4 codes, float s0, float s1, uint4* out) {
  const uint32_t w[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float sc = q < 2 ? s0 : s1;
    bf16x2_t pr[4] = {__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], 1.0f, 0),
                      __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], 1.0f, 1),
                      __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], 1.0f, 2),
                      __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], 1.0f, 3)};
    bf16x8_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = static_cast<__bf16>(static_cast<float>(pr[i][0]) * sc);
      v[2 * i + 1] = static_cast<__bf16>(static_cast<float>(pr[i][1]) * sc);
    }
    out[q] = __builtin_bit_cast(uint4, v);
  }
}

__device__ __forceinline__ int acc_row(int i, int half) { return 8 * (i >> 2) + 4 * half + (i & 3); }

// Value of v held by lane src (lower half) or src + 4 (upper half): the head
// of accumulator row acc_row(i, half).  Two uniform readlanes and a select
// instead of a cross-lane LDS permute.
__device__ __forceinline__ float lane_value(float v, int src, int half) {
  const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
  const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src + 4));
  return half ? hi : lo;
}

template <bool FP4>
__global__ __launch_bounds__(256) void attn_mfma_kernel(
    int H, int topk, int window, int main_group, int d_rope, int64_t capacity, RopeTable rope,
    const uint16_t* __restrict__ q, const int32_t* __restrict__ q_pos, int n_q, const int32_t* __restrict__ topk_ids,
    const uint16_t* __restrict__ swa, const int32_t* __restrict__ swa_first, int n_swa,
    const uint8_t* __restrict__ main, const uint8_t* __restrict__ main_scale, int n_tiles, int tiles_per_split,
    int n_splits, uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  __shared__ __align__(16) uint8_t rt[32 * kRowPitch];
  __shared__ float lpart[4][16][64];
  __shared__ int rvalid[32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 31, h = lane >> 5;
  const int split = blockIdx.x, hg = blockIdx.y;
  const int64_t bq = blockIdx.z, b = bq / n_q;
  const int64_t t = q_pos[bq];

  // B operand of the logits: the rotated query, lane = head, this wave's channel quarter
  bf16x8_t qop[8];
  {
    const uint16_t* qrow = q + (bq * H + hg * 32 + n) * kD;
    const int c_rot0 = kD - d_rope;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c0 = 128 * wave + 16 * s + 8 * h;
      bf16x8_t v = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + c0));
      if (c0 + 8 > c_rot0) {
#pragma unroll
        for (int pi = 0; pi < 4; ++pi) {
          const int c = c0 + 2 * pi;
          if (c >= c_rot0) {
            const double phi = double(t) * rope.inv_freq[(c - c_rot0) / 2];
            const double two_pi = 6.283185307179586476925, inv_two_pi = 0.15915494309189533577;
            const float red = float(phi - two_pi * rint(phi * inv_two_pi));  // angle reduced in float64
            float sn, cs;
            sincosf(red, &sn, &cs);
            const float x = static_cast<float>(v[2 * pi]), y = static_cast<float>(v[2 * pi + 1]);
            v[2 * pi] = static_cast<__bf16>(x * cs - y * sn);
            v[2 * pi + 1] = static_cast<__bf16>(x * sn + y * cs);
          }
        }
      }
      qop[s] = v;
    }
  }
  // 0/1 selection operands that turn staged rows into the P.R operand layout
  bf16x8_t eop[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int i = 0; i < 8; ++i) eop[e][i] = static_cast<__bf16>(n == 16 * e + 8 * h + i ? 1.0f : 0.0f);

  const float scale = 0.044194173824159216f;  // 1/sqrt(512)
  float m_run = -INFINITY, l_run = 0.0f;
  f32x16_t oacc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) oacc[cb] = f32x16_t{};
  const int64_t win0 = t - window + 1 > 0 ? t - window + 1 : 0;
  const int64_t sfirst = swa ? swa_first[b] : 0;
  const int tile_lo = split * tiles_per_split;
  const int tile_hi = min(n_tiles, tile_lo + tiles_per_split);

  for (int tile = tile_lo; tile < tile_hi; ++tile) {
    // ---- 1. stage 32 rows (8 threads per row, 16-byte chunks interleaved) ----
    {
      const int rr = tid >> 3, p = tid & 7;
      const int64_t r = int64_t(tile) * 32 + rr;
      int64_t crow = -1, srow = -1;
      if (r < topk) {
        const int64_t j = topk_ids[bq * topk + r];
        if (j >= 0 && j < capacity) crow = b * capacity + j;
      } else if (r < topk + window) {
        const int64_t pp = win0 + (r - topk), sidx = pp - sfirst;
        if (swa && pp <= t && sidx >= 0 && sidx < n_swa) srow = b * n_swa + sidx;
      }
      uint8_t* dst = rt + rr * kRowPitch;
      if (FP4 && crow >= 0) {
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          const int ch = p + 8 * v;  // 32-value chunk of the row
          const uint4 codes = *reinterpret_cast<const uint4*>(main + crow * (kD / 2) + 16 * ch);
          float s0, s1;
          if (main_group == 32) {
            s0 = s1 = e4m3_to_f32(main_scale[crow * (kD / 32) + ch]);
          } else {
            s0 = e4m3_to_f32(main_scale[crow * (kD / 16) + 2 * ch]);
            s1 = e4m3_to_f32(main_scale[crow * (kD / 16) + 2 * ch + 1]);
          }
          uint4 o[4];
          dequant_fp4_32(codes, s0, s1, o);
#pragma unroll
          for (int u = 0; u < 4; ++u) *reinterpret_cast<uint4*>(dst + (4 * ch + u) * 16) = o[u];
        }
      } else if (crow >= 0 || srow >= 0) {
        const uint4* src = crow >= 0 ? reinterpret_cast<const uint4*>(main + crow * (kD * 2))
                                     : reinterpret_cast<const uint4*>(swa + srow * kD);
#pragma unroll
        for (int v = 0; v < 8; ++v) *reinterpret_cast<uint4*>(dst + (p + 8 * v) * 16) = src[p + 8 * v];
      } else {
#pragma unroll
        for (int v = 0; v < 8; ++v) *reinterpret_cast<uint4*>(dst + (p + 8 * v) * 16) = make_uint4(0, 0, 0, 0);
      }
      if (p == 0) rvalid[rr] = (crow >= 0 || srow >= 0);
    }
    __syncthreads();

    // ---- 2. logits over this wave's channel quarter, summed across waves ----
    bf16x8_t aop[8];
    f32x16_t lacc = f32x16_t{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c0 = 128 * wave + 16 * s + 8 * h;
      aop[s] = *reinterpret_cast<const bf16x8_t*>(rt + n * kRowPitch + c0 * 2);
      lacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[s], qop[s], lacc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) lpart[wave][i][lane] = lacc[i];
    __syncthreads();
    float lg[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float v = (lpart[0][i][lane] + lpart[1][i][lane] + lpart[2][i][lane] + lpart[3][i][lane]) * scale;
      lg[i] = rvalid[acc_row(i, h)] ? v : -INFINITY;
      tmax = fmaxf(tmax, lg[i]);
    }

    // ---- 3. online softmax for head n (rows split between lanes n and n+32) ----
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = m_new == -INFINITY ? 1.0f : __expf(m_run - m_new);
    float psum = 0.0f;
    bf16x8_t pop[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pv = lg[i] == -INFINITY ? 0.0f : __expf(lg[i] - m_new);
      psum += pv;
      pop[i >> 3][i & 7] = static_cast<__bf16>(pv);
    }
    psum += __shfl_xor(psum, 32, kWave);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float a = lane_value(alpha, acc_row(i, 0), h);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) oacc[cb][i] *= a;
    }

    // ---- 4. rows into operand layout, then O += P . R for this wave's channels ----
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      f32x16_t ct = f32x16_t{};
      ct = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[2 * cb], eop[0], ct, 0, 0, 0);
      ct = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[2 * cb + 1], eop[1], ct, 0, 0, 0);
      bf16x8_t rop[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) rop[i >> 3][i & 7] = static_cast<__bf16>(ct[i]);
      oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pop[0], rop[0], oacc[cb], 0, 0, 0);
      oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pop[1], rop[1], oacc[cb], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- outputs: lane holds channel 128w + 32cb + n of heads acc_row(i, h) ----
  if (n_splits == 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int hh = acc_row(i, h);
      const float lh = lane_value(l_run, acc_row(i, 0), h);
      const float inv = lh > 0.0f ? 1.0f / lh : 0.0f;
      uint16_t* orow = out + (bq * H + hg * 32 + hh) * kD + 128 * wave + n;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) orow[32 * cb] = f32_to_bf16(oacc[cb][i] * inv);
    }
    if (lse && wave == 0 && h == 0) lse[bq * H + hg * 32 + n] = l_run > 0.0f ? m_run + logf(l_run) : -INFINITY;
  } else {
    const int64_t prow = (bq * n_splits + split) * H + hg * 32;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float* orow = part_o + (prow + acc_row(i, h)) * kD + 128 * wave + n;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) orow[32 * cb] = oacc[cb][i];
    }
    if (wave == 0 && h == 0) {
      part_ml[(prow + n) * 2] = m_run;
      part_ml[(prow + n) * 2 + 1] = l_run;
    }
  }
}

// Combine the split partials of one (query, head): weights exp(m_s - M) / L,
// computed once by one wave, then each thread adds four channels of every
// split with 16-byte loads.
extern "C" __device__ float __ockl_wfred_max_f32(float);
extern "C" __device__ float __ockl_wfred_add_f32(float);

constexpr int kMaxSplits = 64;

__global__ __launch_bounds__(128) void attn_merge_kernel(int H, int n_splits, const float* __restrict__ part_o,
                                                         const float* __restrict__ part_ml,
                                                         uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ float wgt[kMaxSplits];
  const int head = blockIdx.x, tid = threadIdx.x;
  const int64_t bq = blockIdx.y;
  if (tid < kWave) {
    const int64_t at = ((bq * n_splits + tid) * H + head) * 2;
    const float m = tid < n_splits ? part_ml[at] : -INFINITY;
    const float l = tid < n_splits ? part_ml[at + 1] : 0.0f;
    const float M = __ockl_wfred_max_f32(m);
    const float e = m > -INFINITY ? __expf(m - M) : 0.0f;
    const float L = __ockl_wfred_add_f32(e * l);
    if (tid < n_splits) wgt[tid] = L > 0.0f ? e / L : 0.0f;
    if (lse && tid == 0) lse[bq * H + head] = L > 0.0f ? M + logf(L) : -INFINITY;
  }
  __syncthreads();
  const int c = 4 * tid;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int sp = 0; sp < n_splits; ++sp) {
    const float wv = wgt[sp];
    const float4 v = *reinterpret_cast<const float4*>(part_o + ((bq * n_splits + sp) * H + head) * kD + c);
    acc.x += wv * v.x;
    acc.y += wv * v.y;
    acc.z += wv * v.z;
    acc.w += wv * v.w;
  }
  uint2 packed;
  packed.x = uint32_t(f32_to_bf16(acc.x)) | (uint32_t(f32_to_bf16(acc.y)) << 16);
  packed.y = uint32_t(f32_to_bf16(acc.z)) | (uint32_t(f32_to_bf16(acc.w)) << 16);
  *reinterpret_cast<uint2*>(out + (bq * H + head) * kD + c) = packed;
}

struct AttnPlan {
  bool mfma;
  int n_tiles, tiles_per_split, n_splits;
};

AttnPlan plan_attn(const csa2_dims& dims, const csa2_kv_cache& cache, int32_t n_q) {
  AttnPlan p{};
  p.mfma = dims.d == kD && dims.n_heads % 32 == 0 && dims.act_dtype == CSA2_BF16 &&
           (cache.kv_dtype == CSA2_BF16 || cache.kv_dtype == CSA2_FP4);
  p.n_tiles = (dims.topk + dims.window + 31) / 32;
  p.tiles_per_split = p.n_tiles;
  p.n_splits = 1;
  if (!p.mfma || n_q <= 0) return p;
  const int64_t units = int64_t(cache.batch) * n_q * (dims.n_heads / 32);
  int splits = int(units >= 512 ? 1 : (512 + units - 1) / units);
  splits = splits < 1 ? 1 : (splits > p.n_tiles ? p.n_tiles : splits);
  splits = splits > kMaxSplits ? kMaxSplits : splits;
  p.tiles_per_split = (p.n_tiles + splits - 1) / splits;
  p.n_splits = (p.n_tiles + p.tiles_per_split - 1) / p.tiles_per_split;
  return p;
}

}  // namespace

size_t attn_workspace_bytes(const csa2_dims& dims, const csa2_kv_cache& cache, int32_t n_q) {
  const AttnPlan p = plan_attn(dims, cache, n_q);
  if (!p.mfma || p.n_splits == 1) return 0;
  const size_t rows = size_t(cache.batch) * n_q * p.n_splits * dims.n_heads;
  const size_t o_bytes = (rows * kD * 4 + 255) / 256 * 256;
  return o_bytes + rows * 2 * 4;
}

hipError_t launch_attn(const csa2_dims& dims, const csa2_kv_cache& cache, const void* q, const int32_t* q_pos,
                       int32_t n_q, const int32_t* topk, const void* swa_kv, const int32_t* swa_first_pos,
                       int32_t n_swa, void* out, float* lse, void* ws, size_t, hipStream_t stream) {
  const AttnPlan p = plan_attn(dims, cache, n_q);
  if (p.mfma) {
    float* part_o = nullptr;
    float* part_ml = nullptr;
    if (p.n_splits > 1) {
      const size_t rows = size_t(cache.batch) * n_q * p.n_splits * dims.n_heads;
      part_o = static_cast<float*>(ws);
      part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + (rows * kD * 4 + 255) / 256 * 256);
    }
    const dim3 grid(p.n_splits, dims.n_heads / 32, unsigned(int64_t(cache.batch) * n_q));
    auto kern = cache.kv_dtype == CSA2_FP4 ? attn_mfma_kernel<true> : attn_mfma_kernel<false>;
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, dims.n_heads, dims.topk, dims.window, cache.main_group,
                       dims.d_rope, cache.capacity, make_rope_table(dims), static_cast<const uint16_t*>(q), q_pos, n_q, topk,
                       static_cast<const uint16_t*>(swa_kv), swa_first_pos, n_swa,
                       static_cast<const uint8_t*>(cache.main), cache.main_scale, p.n_tiles, p.tiles_per_split,
                       p.n_splits, static_cast<uint16_t*>(out), lse, part_o, part_ml);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_splits == 1) return e;
    hipLaunchKernelGGL(attn_merge_kernel, dim3(dims.n_heads, unsigned(int64_t(cache.batch) * n_q)), dim3(128), 0,
                       stream, dims.n_heads, p.n_splits, part_o, part_ml, static_cast<uint16_t*>(out), lse);
    return hipGetLastError();
  }
  const dim3 grid(dims.n_heads, n_q, cache.batch);
  const size_t lds = sizeof(float) * size_t(dims.d + dims.topk + dims.window + kThreads / 64 + 2);
  hipLaunchKernelGGL(attn_generic_kernel, grid, dim3(kThreads), lds, stream, dims.d, dims.d_rope, dims.n_heads,
                     dims.topk, dims.window, int(dims.act_dtype == CSA2_BF16), cache.kv_dtype, cache.main_group,
                     make_rope_table(dims), cache.capacity, q, q_pos, n_q, topk, swa_kv, swa_first_pos, n_swa, cache.main,
                     cache.main_scale, out, lse);
  return hipGetLastError();
}

}  // namespace csa2
