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
    int d, int d_rope, int H, int topk, int window, int act_bf16, int swa_fp8, int kv_dtype, int main_group, RopeTable rope,
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
  // no window buffer (n_swa == 0): swa_first may be NULL and no window row is read
  const int64_t sfirst = (swa && n_swa > 0) ? swa_first[b] : 0;
  const int n_rows = topk + window;
  const float scale = rope.logit_scale;

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

  // window element: activation type, or one E4M3 (FN) byte
  auto swa_load = [&](int64_t srow, int c) -> float {
    return swa_fp8 ? e4m3_to_f32(static_cast<const uint8_t*>(swa)[srow * d + c]) : act_load(swa, srow * d + c, act_bf16);
  };

  for (int r = wid; r < n_rows; r += kThreads / 64) {
    int64_t crow, srow;
    row_src(r, crow, srow);
    float v = -INFINITY;
    if (crow >= 0 || srow >= 0) {
      float part = 0.0f;
      for (int c = lane; c < d; c += 64) {
        const float x = crow >= 0 ? cache_load(main, main_scale, kv_dtype, crow, d, main_group, c) : swa_load(srow, c);
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
      const float x = crow >= 0 ? cache_load(main, main_scale, kv_dtype, crow, d, main_group, c) : swa_load(srow, c);
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
// Production shape: d = 512, heads in groups of 16, bf16 queries, bf16 or FP4
// main KV.  A workgroup (4 waves) owns one (query, group of 16 heads, run of
// 16-row tiles); the rows of a query are the kept entries followed by the
// window rows.  Each wave takes every fourth tile and runs it alone - no
// workgroup barrier inside the loop - double-buffering its tiles in two LDS
// slabs of its own:
//   1. a tile's 16 rows are copied global -> LDS with global_load_lds_dwordx4
//      (one 1 KB row per instruction, lane i -> bytes 16i..16i+15), issued a
//      tile ahead from inline assembly: the compiler's wait insertion would
//      drain such copies before every LDS read, so the kernel waits for them
//      itself.  Every tile issues exactly 16 copies so one wait count covers
//      it: a row that names no source copies the head group's first query row
//      (finite data) and is masked out of the softmax.  FP4 rows arrive in
//      registers (codes and scales, a tile ahead) and are dequantised into
//      the slab (E2M1 codes converted exactly, times the E4M3 scale in
//      float32 - exact in bf16);
//   2. logits L[row][head] = R . Q^T over the 512 channels (16 products of
//      v_mfma_f32_16x16x32_bf16; rows read from the slab, lane = row; the 16
//      heads' rotated queries held in registers, lane = head);
//   3. online softmax per head against a reference max that is raised (with
//      the output rescaled) only when a logit exceeds it by more than
//      kRescaleGap; each lane sums only its own rows, reduced once at the end;
//   4. O^T[channel][head] += R^T . P: the slab is read transposed with
//      ds_read_b64_tr_b16 (within each 16 lanes,
//      lane j's element i is element j%4 of the 8 bytes that lane 4i+j/4
//      addresses), giving lane = channel and 4 consecutive rows - the A
//      operand of v_mfma_f32_16x16x16_bf16; P is the B operand exactly as the
//      logits left it, and each lane keeps the head of its softmax state.
// At the end the four waves' (reference max, sum, O) are combined through LDS
// in a fixed order.  The head groups of one (query, row split) are placed on
// one XCD (workgroups are dealt to the 8 XCDs in turn) so they share those
// rows in that L2, and the (query, split) pairs go round all 8 XCDs.  With
// several row splits per (query, head group) each workgroup writes its
// unnormalised output and (reference max, sum); attn_merge_kernel
// combines them.

typedef __bf16 bf16x8_t __attribute__((__vector_size__(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kD = 512;
constexpr int kPitch = kD * 2 + 32;  // LDS bytes per row: the pad puts the 4 rows of a transposed read on distinct banks
constexpr int kSlab = 16 * kPitch;   // one 16-row tile
constexpr int kLdsLoop = 4 * 2 * kSlab;  // two slabs per wave
constexpr int kLdsSlabs = 4 * 16 * kD * 4;  // the four waves' fp32 outputs at the end, reusing the loop space
constexpr int kLdsMl = kLdsLoop > kLdsSlabs ? kLdsLoop : kLdsSlabs;  // (max, sum) of the four waves
constexpr int kLdsRope = kLdsMl + 2 * 4 * 16 * 4;                     // (cos, sin) per rotary pair
constexpr int kLdsIds = kLdsRope + 2 * 64 * 4;                        // kept-entry ids of the workgroup's rows
constexpr int kMaxIds = 2048 + 16;                                    // topk <= 2048, plus a straddling tile
constexpr int kAttnLds = kLdsIds + kMaxIds * 4;
// SHARE needs only its ring of two slabs, the rotation table and the ids, so
// two workgroups fit a compute unit; with bf16 rows the kernel also fits the
// registers of two waves per SIMD (FP4's dequantisation registers would spill)
constexpr int kShareRope = 2 * kSlab;
constexpr int kShareIds = kShareRope + 2 * 64 * 4;
constexpr int kShareLds = kShareIds + kMaxIds * 4;
// Softmax reference: logits are exponentiated against a per-head reference
// max that is raised (and the output rescaled) only when a logit exceeds it
// by more than this, so P stays below e^8 and the sums far from overflow.
constexpr float kRescaleGap = 8.0f;

// Copy 16 bytes per lane from global address `src` to LDS byte address
// `lds_addr` + 16 * lane (global_load_lds_dwordx4; the LDS base goes in M0).
// Its completion is tracked only by the caller's s_waitcnt vmcnt.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved; naming it tells the compiler it changes
__device__ __forceinline__ void copy_row_to_lds(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_addr), "v"(src) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// First channel of k-chunk k (8 channels) held by lane group g in the operands
// of the logit products.  bf16 caches: chunk k covers channels [32k, 32k+32)
// so each load instruction reads 64 contiguous bytes per row.  FP4 caches:
// lane group g covers channels [128g, 128g+128), so its codes are 64
// contiguous bytes.  The contraction may run in any channel order as long as
// both operands use the same one.
template <bool FP4>
__device__ __forceinline__ int chan0(int g, int k) { return FP4 ? 128 * g + 8 * k : 32 * k + 8 * g; }

// 8 E2M1 codes (one 32-bit word, low nibble first) times scale s -> 8 bf16.
__device__ __forceinline__ uint4 dequant8(uint32_t w, float s) {
  const f32x2 f[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0),
                      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1),
                      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2),
                      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3)};
  bf16x8_t v;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    v[2 * p] = static_cast<__bf16>(f[p][0] * s);
    v[2 * p + 1] = static_cast<__bf16>(f[p][1] * s);
  }
  return __builtin_bit_cast(uint4, v);
}

// FP4 codes of a lane's part of its row (channels 128g .. 128g+127) and the
// row's scales (all 16 bytes for groups of 32; for groups of 16 the 16 bytes
// holding this lane's 8).
struct Fp4Regs {
  uint4 c[4];
  uint4 sc;
};

// Per-tile facts, uniform across the wave: bit i = row i of the tile.
struct TileMask {
  uint32_t valid;  // the row has a source
  uint32_t fp4;    // the row is an FP4 cache row
  uint32_t w8;     // the row is an FP8 window row (copied as 512 bytes, widened in LDS)
};

// FP4: the cache is FP4 with one E4M3 scale per MG channels (MG = 16 or 32).
// SHARE (64 heads, many queries): one workgroup per (query, row split), wave
// w owns heads 16w .. 16w+15, and the four waves run every row tile together
// from a shared ring of two slabs, each wave copying (and for FP4
// dequantising) four of the tile's 16 rows: a row is gathered once per query
// instead of once per head group.  No cross-wave combine; with row splits
// each wave stores its heads' unnormalised output for attn_merge_kernel.
// W8: window rows are E4M3 (FN) bytes, copied as they are and widened to
// bf16 in the slab (exact) before the tile is used.
template <bool FP4, int MG, bool SHARE, bool W8>
__global__ __launch_bounds__(256, SHARE && !FP4 ? 2 : 1) void attn_mfma_kernel(
    int H, int topk, int window, int d_rope, int64_t capacity, RopeTable rope,
    const uint16_t* __restrict__ q, const int32_t* __restrict__ q_pos, int n_q, int64_t n_bq,
    const int32_t* __restrict__ topk_ids, const uint16_t* __restrict__ swa, const int32_t* __restrict__ swa_first,
    int n_swa, const uint8_t* __restrict__ main, const uint8_t* __restrict__ main_scale, int n_tiles,
    int tiles_per_split, int n_splits, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t wg = blockIdx.x, x8 = wg & 7, rest = wg >> 3;
  int hg, split;
  int64_t bq;
  if constexpr (SHARE) {
    // workgroup -> (query, row split): consecutive queries (which share
    // window rows) on one XCD
    hg = wave;
    const int64_t n_pairs = n_bq * n_splits;
    const int64_t pair = x8 * ((n_pairs + 7) / 8) + rest;
    if (pair >= n_pairs) return;  // padding workgroup (uniform)
    bq = pair / n_splits;
    split = int(pair % n_splits);
  } else {
    // workgroup -> (query, split, head group): the G head groups of one
    // (query, split) pair share an XCD (id % 8), the pairs go round the XCDs
    const int G = H / 16;
    hg = int(rest % G);
    const int64_t pair = (rest / G) * 8 + x8;
    if (pair >= n_bq * n_splits) return;  // padding workgroup (uniform)
    bq = pair / n_splits;
    split = int(pair % n_splits);
  }
  const int64_t b = bq / n_q, t = q_pos[bq];
  uint8_t* rs = SHARE ? lds : lds + wave * 2 * kSlab;

  const int tile_lo = split * tiles_per_split;
  const int tile_hi = min(n_tiles, tile_lo + tiles_per_split);
  const int64_t win0 = t - window + 1 > 0 ? t - window + 1 : 0;
  const int64_t sfirst = swa ? swa_first[b] : 0;
  const uint16_t* qrow0 = q + (bq * H + hg * 16) * kD;  // finite stand-in for rows with no source

  // The workgroup's loads that do not depend on each other go out together,
  // at addresses that are always valid, with no branch around them (a load
  // under a branch made the compiler wait for it where the branch joined,
  // and this prologue took three round trips to memory: 3.5 us of a 12 us
  // 32K decode workgroup): the query, the rotary frequencies, the kept-entry
  // ids of the workgroup's rows.
  // B operand of the logits: head l16's query, chunk k = channels chan0(g, k) .. +8
  bf16x8_t qtmp[16];
  {
    const uint16_t* qrow = qrow0 + l16 * kD;
#pragma unroll
    for (int k = 0; k < 16; ++k) qtmp[k] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + chan0<FP4>(g, k)));
  }
  const double inv_freq = rope.inv_freq[min(tid, kMaxRopePairs - 1)];  // used where tid < d_rope / 2
  int32_t* ids_lds = reinterpret_cast<int32_t*>(lds + (SHARE ? kShareIds : kLdsIds));
  const int row_lo = tile_lo * 16;
  const int r_end = min(tile_hi * 16, topk);
  int32_t idv[(kMaxIds + 255) / 256];
#pragma unroll
  for (int i = 0; i < (kMaxIds + 255) / 256; ++i) {
    const int r = row_lo + tid + 256 * i;
    // used only where r < r_end; past it, every lane reads the last id it needs
    idv[i] = topk_ids[bq * topk + min(r, r_end - 1)];
  }
  // kept-entry ids of this workgroup's rows, and the rotation of this query's
  // position for each rotary pair, once per workgroup
#pragma unroll
  for (int i = 0; i < (kMaxIds + 255) / 256; ++i) {
    const int r = row_lo + tid + 256 * i;
    if (r < r_end) ids_lds[r - row_lo] = idv[i];
  }
  float* rtab = reinterpret_cast<float*>(lds + (SHARE ? kShareRope : kLdsRope));
  if (tid < d_rope / 2) {
    const double phi = double(t) * inv_freq;
    const double two_pi = 6.283185307179586476925, inv_two_pi = 0.15915494309189533577;
    const float red = float(phi - two_pi * rint(phi * inv_two_pi));  // angle reduced in float64
    float sn, cs;
    sincosf(red, &sn, &cs);
    rtab[2 * tid] = cs;
    rtab[2 * tid + 1] = sn;
  }
  // Complete every load so far with a wait the compiler sees: its own waits
  // count only the loads it knows of, and inside the loop the row copies it
  // does not know of would make any vmcnt it inserts drain them too.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  {
    const int c_rot0 = kD - d_rope;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (!FP4 && 32 * k + 32 <= c_rot0) continue;  // no rotary channel in this chunk (uniform)
#pragma unroll
      for (int pi = 0; pi < 4; ++pi) {
        const int c = chan0<FP4>(g, k) + 2 * pi;
        const int m = c >= c_rot0 ? (c - c_rot0) / 2 : 0;
        const float cs = rtab[2 * m], sn = rtab[2 * m + 1];
        const float x = static_cast<float>(qtmp[k][2 * pi]), y = static_cast<float>(qtmp[k][2 * pi + 1]);
        if (c >= c_rot0) {
          qtmp[k][2 * pi] = static_cast<__bf16>(x * cs - y * sn);
          qtmp[k][2 * pi + 1] = static_cast<__bf16>(x * sn + y * cs);
        }
      }
    }
  }
  const bf16x8_t* qreg = qtmp;

  // Issue the copies of `tile` into slab `buf`: for FP4 caches this lane's
  // codes and scales into `fr` first (5 loads), then the 16 row copies.
  // Returns uniform row masks.
  auto issue = [&](int tile, int buf, Fp4Regs& fr) -> TileMask {
    // lanes 0..15 (and their copies in the other lane groups) work out rows 0..15
    const int64_t r = int64_t(tile) * 16 + l16;
    const uint8_t* src = reinterpret_cast<const uint8_t*>(qrow0);
    int64_t crow = 0;
    bool valid = false, fp4 = false;
    if (r < topk) {
      const int64_t j = ids_lds[r - row_lo];
      if (j >= 0 && j < capacity) {
        valid = true;
        crow = b * capacity + j;
        if (FP4) fp4 = true;
        else src = main + crow * (kD * 2);
      }
    } else if (r < topk + window) {
      const int64_t pp = win0 + (r - topk), sidx = pp - sfirst;
      if (swa && pp <= t && sidx >= 0 && sidx < n_swa) {
        valid = true;
        src = W8 ? reinterpret_cast<const uint8_t*>(swa) + (b * n_swa + sidx) * kD
                 : reinterpret_cast<const uint8_t*>(swa + (b * n_swa + sidx) * kD);
      }
    }
    TileMask m;
    m.valid = uint32_t(__ballot(valid)) & 0xFFFFu;  // lanes 0..15 hold rows 0..15
    m.fp4 = uint32_t(__ballot(fp4)) & 0xFFFFu;
    m.w8 = W8 ? uint32_t(__ballot(valid && r >= topk)) & 0xFFFFu : 0u;
    if constexpr (FP4) {
      if (!SHARE || (l16 >> 2) == wave) {  // SHARE: this wave's four rows
        const uint8_t* codes = main + crow * (kD / 2) + 64 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) fr.c[i] = reinterpret_cast<const uint4*>(codes)[i];
        fr.sc = *reinterpret_cast<const uint4*>(main_scale + crow * (kD / MG) + (MG == 16 ? 16 * (g >> 1) : 0));
      }
    }
    const uint32_t slab = __builtin_amdgcn_readfirstlane(
        uint32_t(reinterpret_cast<uintptr_t>((lds_void*)(rs + buf * kSlab))));
    const uint64_t src_u = reinterpret_cast<uint64_t>(src);
#pragma unroll
    for (int ii = 0; ii < (SHARE ? 4 : 16); ++ii) {
      const int i = SHARE ? 4 * wave + ii : ii;  // uniform
      const uint64_t row = (uint64_t(uint32_t(__builtin_amdgcn_readlane(int(src_u >> 32), i))) << 32) |
                           uint32_t(__builtin_amdgcn_readlane(int(uint32_t(src_u)), i));
      // an FP8 window row is 512 bytes: the upper half-wave copies it again
      // into the slab row's upper half, which the widening overwrites
      const uint32_t off = (W8 && (m.w8 >> i) & 1u) ? 16 * (lane & 31) : 16 * lane;
      copy_row_to_lds(reinterpret_cast<const void*>(row + off), slab + i * kPitch);
    }
    return m;
  };

  const float scale = rope.logit_scale;  // 1/sqrt(512), times the YaRN temperature
  float m_ref = -INFINITY, l_part = 0.0f;  // l_part: this lane's rows only
  f32x4 oacc[32];
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) oacc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // FP4 rows of a tile into its slab, from `fr`: waits for everything issued
  // so far (this tile's loads are the youngest).
  auto dequant_tile = [&](int buf, const TileMask m, const Fp4Regs& fr) {
    uint8_t* slab = rs + buf * kSlab;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (((m.fp4 >> l16) & 1u) && (!SHARE || (l16 >> 2) == wave)) {
      const uint32_t w4[16] = {fr.c[0].x, fr.c[0].y, fr.c[0].z, fr.c[0].w, fr.c[1].x, fr.c[1].y,
                               fr.c[1].z, fr.c[1].w, fr.c[2].x, fr.c[2].y, fr.c[2].z, fr.c[2].w,
                               fr.c[3].x, fr.c[3].y, fr.c[3].z, fr.c[3].w};
      // this lane's scales: scales 4g .. 4g+3 of the row (groups of 32), or
      // 8g .. 8g+7 (groups of 16: bytes 8(g&1) .. of the 16 loaded)
      const uint32_t scw[4] = {fr.sc.x, fr.sc.y, fr.sc.z, fr.sc.w};
      uint32_t sw[2];
      if constexpr (MG == 32) {
        sw[0] = scw[g];
        sw[1] = 0u;
      } else {
        sw[0] = scw[2 * (g & 1)];
        sw[1] = scw[2 * (g & 1) + 1];
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        // channels 128g + 8k: scale (8k)/MG among this lane's 128/MG
        const int si = (8 * k) / MG;
        *reinterpret_cast<uint4*>(slab + l16 * kPitch + (128 * g + 8 * k) * 2) =
            dequant8(w4[k], e4m3_to_f32((sw[si >> 2] >> (8 * (si & 3))) & 0xFFu));
      }
    }
  };

  // Widen the FP8 window rows this wave copied into slab `buf` (their copies
  // have landed): one 8-byte read per lane takes the whole row before the
  // 16-byte writes replace it with its bf16 values (E4M3 values are exact in
  // bf16: at most 4 significant bits, exponents within range).
  auto widen_w8 = [&](int buf, const TileMask m) {
    uint8_t* slab = rs + buf * kSlab;
#pragma unroll
    for (int ii = 0; ii < (SHARE ? 4 : 16); ++ii) {
      const int i = SHARE ? 4 * wave + ii : ii;  // uniform
      if (!((m.w8 >> i) & 1u)) continue;
      const uint2 v = *reinterpret_cast<const uint2*>(slab + i * kPitch + 8 * lane);
      const uint32_t w2[2] = {v.x, v.y};
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(w2[k]), false);  // bytes 0, 1
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(w2[k]), true);   // bytes 2, 3
        o[2 * k] = (__float_as_uint(lo[0]) >> 16) | (__float_as_uint(lo[1]) & 0xFFFF0000u);
        o[2 * k + 1] = (__float_as_uint(hi[0]) >> 16) | (__float_as_uint(hi[1]) & 0xFFFF0000u);
      }
      *reinterpret_cast<uint4*>(slab + i * kPitch + 16 * lane) = uint4{o[0], o[1], o[2], o[3]};
    }
  };

  // Compute the tile in slab `buf`.  `more`: the next tile's 16 copies were
  // issued after this tile's and may stay in flight (bf16 caches; for FP4 the
  // wait happened in dequant_tile).
  auto compute = [&](int buf, const TileMask m, bool more) {
    const uint8_t* slab = rs + buf * kSlab;
    if constexpr (!FP4 && !SHARE) {
      if (more) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    if constexpr (W8 && !SHARE) widen_w8(buf, m);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // ---- logits: lane holds head l16, rows 4g + r of the tile ----
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(slab + l16 * kPitch + chan0<FP4>(g, k) * 2);
      const bf16x8_t qb = qreg[k];
      if (k & 1) acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb, acc1, 0, 0, 0);
      else acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb, acc0, 0, 0, 0);
    }

    // ---- online softmax for head l16: reference max m_ref, per-lane partial sums ----
    float lg[4], mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      lg[r] = ((m.valid >> (4 * g + r)) & 1u) ? (acc0[r] + acc1[r]) * scale : -INFINITY;
      mx = fmaxf(mx, lg[r]);
    }
    if (__ballot(mx > m_ref + kRescaleGap)) {  // rare: raise the reference to the head's max
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float m_new = fmaxf(m_ref, mx);
      if (m_ref != -INFINITY && __ballot(m_new != m_ref)) {
        const float alpha = __expf(m_ref - m_new);
        l_part *= alpha;
#pragma unroll
        for (int cb = 0; cb < 32; ++cb) oacc[cb] *= alpha;
      }
      m_ref = m_new;
    }
    s16x4 pop;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = lg[r] == -INFINITY ? 0.0f : __expf(lg[r] - m_ref);
      l_part += p;
      pop[r] = __builtin_bit_cast(short, static_cast<__bf16>(p));
    }

    // ---- O^T += R^T . P, rows read transposed from the slab ----
    const uint8_t* tr_base = slab + (4 * g + (l16 >> 2)) * kPitch + 4 * (l16 & 3) * 2;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      const s16x4 at = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tr_base + 32 * cb));
      oacc[cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(at, pop, oacc[cb], 0, 0, 0);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // slab reads done before it is refilled
  };

  Fp4Regs fa{}, fb{};
  TileMask ma{0u, 0u, 0u}, mb{0u, 0u, 0u};
  if constexpr (SHARE) {
    // every wave runs every tile; tile t is in slab t % 2 (deeper rings
    // measured no faster: four slabs at one workgroup per compute unit, and
    // three slabs at two, 0.570 against 0.561 ms for a 4096-query prefill:
    // each wave's own chain of logits, softmax and P.V per tile bounds it,
    // not the copies in flight)
    int tile = tile_lo;
    if (tile < tile_hi) ma = issue(tile, 0, fa);
    while (tile < tile_hi) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's copies and loads of `tile`
      if constexpr (FP4) dequant_tile(0, ma, fa);
      if constexpr (W8) widen_w8(0, ma);
      __syncthreads();  // the whole tile is in slab 0; every wave is done with slab 1
      if (tile + 1 < tile_hi) mb = issue(tile + 1, 1, fb);
      compute(0, ma, false);
      if (++tile >= tile_hi) break;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if constexpr (FP4) dequant_tile(1, mb, fb);
      if constexpr (W8) widen_w8(1, mb);
      __syncthreads();
      if (tile + 1 < tile_hi) ma = issue(tile + 1, 0, fa);
      compute(1, mb, false);
      ++tile;
    }
    // each wave owns its heads: no combine; normalise and store, or with
    // row splits store the unnormalised output and (reference max, sum)
    l_part += __shfl_xor(l_part, 16, kWave);
    l_part += __shfl_xor(l_part, 32, kWave);
    const int64_t head = int64_t(wave) * 16 + l16;
    if (n_splits > 1) {
      const int64_t prow = (bq * n_splits + split) * H + head;
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) *reinterpret_cast<f32x4*>(part_o + prow * kD + 16 * cb + 4 * g) = oacc[cb];
      if (g == 0) {
        part_ml[prow * 2] = m_ref;
        part_ml[prow * 2 + 1] = l_part;
      }
      return;
    }
    const float inv = l_part > 0.0f ? 1.0f / l_part : 0.0f;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      uint2 pk;
      pk.x = uint32_t(f32_to_bf16(oacc[cb][0] * inv)) | (uint32_t(f32_to_bf16(oacc[cb][1] * inv)) << 16);
      pk.y = uint32_t(f32_to_bf16(oacc[cb][2] * inv)) | (uint32_t(f32_to_bf16(oacc[cb][3] * inv)) << 16);
      *reinterpret_cast<uint2*>(out + (bq * H + head) * kD + 16 * cb + 4 * g) = pk;
    }
    if (lse && g == 0) lse[bq * H + head] = l_part > 0.0f ? m_ref + logf(l_part) : -INFINITY;
    return;
  }
  int tile = tile_lo + wave;
  if (tile < tile_hi) ma = issue(tile, 0, fa);
  while (tile < tile_hi) {
    const bool more_a = tile + 4 < tile_hi;
    if constexpr (FP4) dequant_tile(0, ma, fa);
    if (more_a) mb = issue(tile + 4, 1, fb);
    compute(0, ma, more_a);
    tile += 4;
    if (tile >= tile_hi) break;
    const bool more_b = tile + 4 < tile_hi;
    if constexpr (FP4) dequant_tile(1, mb, fb);
    if (more_b) ma = issue(tile + 4, 0, fa);
    compute(1, mb, more_b);
    tile += 4;
  }

  // ---- combine the four waves (fixed order), then store ----
  __syncthreads();  // every wave is done with its slabs
  float* slabs = reinterpret_cast<float*>(lds);
  float* mls = reinterpret_cast<float*>(lds + kLdsMl);
  l_part += __shfl_xor(l_part, 16, kWave);
  l_part += __shfl_xor(l_part, 32, kWave);
  if (g == 0) {
    mls[wave * 16 + l16] = m_ref;
    mls[64 + wave * 16 + l16] = l_part;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, mls[w * 16 + l16]);
  float L = 0.0f, f_own = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float mw = mls[w * 16 + l16];
    const float f = mw == -INFINITY ? 0.0f : __expf(mw - M);
    L += f * mls[64 + w * 16 + l16];
    if (w == wave) f_own = f;
  }
  float* my = slabs + wave * (16 * kD);
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) *reinterpret_cast<f32x4*>(my + (cb * 64 + lane) * 4) = oacc[cb] * f_own;
  __syncthreads();
  const int64_t head = int64_t(hg) * 16 + l16;
  if (n_splits == 1) {
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int cb = wave * 8 + i;
      f32x4 s = *reinterpret_cast<const f32x4*>(slabs + (cb * 64 + lane) * 4);
#pragma unroll
      for (int w = 1; w < 4; ++w) s += *reinterpret_cast<const f32x4*>(slabs + w * (16 * kD) + (cb * 64 + lane) * 4);
      uint2 pk;
      pk.x = uint32_t(f32_to_bf16(s[0] * inv)) | (uint32_t(f32_to_bf16(s[1] * inv)) << 16);
      pk.y = uint32_t(f32_to_bf16(s[2] * inv)) | (uint32_t(f32_to_bf16(s[3] * inv)) << 16);
      *reinterpret_cast<uint2*>(out + (bq * H + head) * kD + 16 * cb + 4 * g) = pk;
    }
    if (lse && wave == 0 && g == 0) lse[bq * H + head] = L > 0.0f ? M + logf(L) : -INFINITY;
  } else {
    const int64_t prow = (bq * n_splits + split) * H + head;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int cb = wave * 8 + i;
      f32x4 s = *reinterpret_cast<const f32x4*>(slabs + (cb * 64 + lane) * 4);
#pragma unroll
      for (int w = 1; w < 4; ++w) s += *reinterpret_cast<const f32x4*>(slabs + w * (16 * kD) + (cb * 64 + lane) * 4);
      *reinterpret_cast<f32x4*>(part_o + prow * kD + 16 * cb + 4 * g) = s;
    }
    if (wave == 0 && g == 0) {
      part_ml[prow * 2] = M;
      part_ml[prow * 2 + 1] = L;
    }
  }
}

// Combine the split partials of one (query, head): weights exp(m_s - M) / L,
// computed once by one wave, then each thread adds four channels of every
// split with 16-byte loads.  blockIdx.z picks one of up to two merges (two
// layers of a group whose merges share a launch).
extern "C" __device__ float __ockl_wfred_max_f32(float);
extern "C" __device__ float __ockl_wfred_add_f32(float);

constexpr int kMaxSplits = 64;

struct MergeJobs {
  const float* part_o[2];
  const float* part_ml[2];
  uint16_t* out[2];
  float* lse[2];
};

__global__ __launch_bounds__(128) void attn_merge_kernel(int H, int n_splits, MergeJobs jobs) {
  __shared__ float wgt[kMaxSplits];
  const int head = blockIdx.x, tid = threadIdx.x, job = blockIdx.z;
  const int64_t bq = blockIdx.y;
  const float* __restrict__ part_o = jobs.part_o[job];
  const float* __restrict__ part_ml = jobs.part_ml[job];
  uint16_t* __restrict__ out = jobs.out[job];
  float* __restrict__ lse = jobs.lse[job];
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
  bool share;  // one workgroup per query, waves = head groups (64 heads, many queries)
  int n_tiles, tiles_per_split, n_splits;
  int64_t n_blocks;  // 1-D grid of the MFMA kernel
};

// Queries of 64 heads from kShareMinQueries up take one workgroup per query
// whose waves share each row tile (SHARE), with row splits while the queries
// alone do not fill the compute units; fewer queries (decode) take a
// workgroup per (query, head group), with row splits up to about 256
// workgroups.  Each wave's tile
// stream is latency-bound, so more workgroups in flight beat the cost of
// merging the splits.
constexpr int64_t kShareMinQueries = 128;  // 64 queries: per head group 24.6 us, shared 28.7 us
AttnPlan plan_attn(const csa2_dims& dims, const csa2_kv_cache& cache, int32_t n_q) {
  AttnPlan p{};
  p.mfma = dims.d == kD && dims.n_heads % 16 == 0 && dims.act_dtype == CSA2_BF16 &&
           (cache.kv_dtype == CSA2_BF16 || cache.kv_dtype == CSA2_FP4);
  p.n_tiles = (dims.topk + dims.window + 15) / 16;
  p.tiles_per_split = p.n_tiles;
  p.n_splits = 1;
  if (!p.mfma || n_q <= 0) return p;
  const int64_t n_bq = int64_t(cache.batch) * n_q, G = dims.n_heads / 16;
  auto set_splits = [&](int64_t units, int64_t target) {
    int splits = int(units >= target ? 1 : (target + units - 1) / units);
    splits = splits < 1 ? 1 : (splits > p.n_tiles ? p.n_tiles : splits);
    splits = splits > kMaxSplits ? kMaxSplits : splits;
    p.tiles_per_split = (p.n_tiles + splits - 1) / splits;
    p.n_splits = (p.n_tiles + p.tiles_per_split - 1) / p.tiles_per_split;
  };
  if (dims.n_heads == 64 && n_bq >= kShareMinQueries) {
    // one workgroup per (query, row split): bf16 rows split up to about 256
    // workgroups (a 128-query replay segment: 2 splits, 47 -> 41 us per
    // layer with the merge; 4 splits 46 us, their partials cost more than
    // the parallelism gains); FP4 rows never split (a 200-query chunk: 103
    // us unsplit, 120-123 us + merge split, 142 us per head group)
    p.share = true;
    set_splits(n_bq, cache.kv_dtype == CSA2_FP4 ? 128 : 256);
    p.n_blocks = 8 * ((n_bq * p.n_splits + 7) / 8);
    return p;
  }
  // about 256 workgroups; with fewer than 64 (query, head group) units,
  // about 128: the splits' partials and their merge then cost more than the
  // extra parallelism gains (4 x 256K group: 184 -> 180 us; 32K x 16 keeps
  // 256: 128 took 17.2 against 14.6 us)
  set_splits(n_bq * G, n_bq * G >= 64 ? 256 : 128);
  p.n_blocks = 8 * G * ((n_bq * p.n_splits + 7) / 8);
  return p;
}

}  // namespace

bool attn_shares_tiles(const csa2_dims& dims, const csa2_kv_cache& cache, int32_t n_q) {
  return plan_attn(dims, cache, n_q).share;
}

size_t attn_workspace_bytes(const csa2_dims& dims, const csa2_kv_cache& cache, int32_t n_q) {
  const AttnPlan p = plan_attn(dims, cache, n_q);
  if (!p.mfma || p.n_splits == 1) return 0;
  const size_t rows = size_t(cache.batch) * n_q * p.n_splits * dims.n_heads;
  const size_t o_bytes = (rows * kD * 4 + 255) / 256 * 256;
  return o_bytes + rows * 2 * 4;
}

hipError_t launch_attn_merge(const AttnMerge* jobs, int n_jobs, hipStream_t stream) {
  if (n_jobs < 1 || n_jobs > 2) return hipErrorInvalidValue;
  MergeJobs mj{};
  for (int j = 0; j < n_jobs; ++j) {
    const AttnMerge& m = jobs[j];
    if (m.n_splits < 2 || m.n_splits > kMaxSplits || m.n_heads != jobs[0].n_heads ||
        m.n_splits != jobs[0].n_splits || m.n_bq != jobs[0].n_bq)
      return hipErrorInvalidValue;
    mj.part_o[j] = m.part_o;
    mj.part_ml[j] = m.part_ml;
    mj.out[j] = m.out;
    mj.lse[j] = m.lse;
  }
  return launch_kernel(CSA2_KERNEL_ATTN_MERGE, attn_merge_kernel,
                       dim3(unsigned(jobs[0].n_heads), unsigned(jobs[0].n_bq), unsigned(n_jobs)), dim3(128), 0, stream,
                       jobs[0].n_heads, jobs[0].n_splits, mj);
}

hipError_t launch_attn(const csa2_dims& dims, const csa2_kv_cache& cache, const void* q, const int32_t* q_pos,
                       int32_t n_q, const int32_t* topk, const void* swa_kv, const int32_t* swa_first_pos,
                       int32_t n_swa, void* out, float* lse, void* ws, size_t, hipStream_t stream,
                       AttnMerge* merge) {
  if (merge) *merge = AttnMerge{};
  const AttnPlan p = plan_attn(dims, cache, n_q);
  if (p.mfma) {
    float* part_o = nullptr;
    float* part_ml = nullptr;
    if (p.n_splits > 1) {
      const size_t rows = size_t(cache.batch) * n_q * p.n_splits * dims.n_heads;
      part_o = static_cast<float*>(ws);
      part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + (rows * kD * 4 + 255) / 256 * 256);
    }
    if (p.n_blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    static bool attr_set = false;
    if (!attr_set) {
      for (const void* f : {reinterpret_cast<const void*>(attn_mfma_kernel<false, 32, false, false>),
                            reinterpret_cast<const void*>(attn_mfma_kernel<true, 32, false, false>),
                            reinterpret_cast<const void*>(attn_mfma_kernel<true, 16, false, false>),
                            reinterpret_cast<const void*>(attn_mfma_kernel<false, 32, true, false>),
                            reinterpret_cast<const void*>(attn_mfma_kernel<true, 32, true, false>),
                            reinterpret_cast<const void*>(attn_mfma_kernel<true, 16, true, false>),
                            reinterpret_cast<const void*>(attn_mfma_kernel<false, 32, false, true>),
                            reinterpret_cast<const void*>(attn_mfma_kernel<true, 32, false, true>),
                            reinterpret_cast<const void*>(attn_mfma_kernel<true, 16, false, true>),
                            reinterpret_cast<const void*>(attn_mfma_kernel<false, 32, true, true>),
                            reinterpret_cast<const void*>(attn_mfma_kernel<true, 32, true, true>),
                            reinterpret_cast<const void*>(attn_mfma_kernel<true, 16, true, true>)}) {
        const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kAttnLds);
        if (e != hipSuccess) return e;
      }
      attr_set = true;
    }
    const bool w8 = dims.swa_dtype == CSA2_FP8;
    auto pick = [&](auto k_bf16, auto k_fp4_32, auto k_fp4_16) {
      return cache.kv_dtype != CSA2_FP4 ? k_bf16 : (cache.main_group == 32 ? k_fp4_32 : k_fp4_16);
    };
    auto kern = p.share ? (w8 ? pick(attn_mfma_kernel<false, 32, true, true>, attn_mfma_kernel<true, 32, true, true>,
                                     attn_mfma_kernel<true, 16, true, true>)
                              : pick(attn_mfma_kernel<false, 32, true, false>, attn_mfma_kernel<true, 32, true, false>,
                                     attn_mfma_kernel<true, 16, true, false>))
                        : (w8 ? pick(attn_mfma_kernel<false, 32, false, true>, attn_mfma_kernel<true, 32, false, true>,
                                     attn_mfma_kernel<true, 16, false, true>)
                              : pick(attn_mfma_kernel<false, 32, false, false>, attn_mfma_kernel<true, 32, false, false>,
                                     attn_mfma_kernel<true, 16, false, false>));
    const int32_t kid = cache.kv_dtype != CSA2_FP4 ? CSA2_KERNEL_ATTN_BF16
                        : (cache.main_group == 32 ? CSA2_KERNEL_ATTN_FP4 : CSA2_KERNEL_ATTN_FP4_G16);
    hipError_t e = launch_kernel(kid, kern,
                                 dim3(unsigned(p.n_blocks)), dim3(256), p.share ? kShareLds : kAttnLds, stream,
                                 dims.n_heads, dims.topk,
                                 dims.window, dims.d_rope, cache.capacity, make_rope_table(dims),
                                 static_cast<const uint16_t*>(q), q_pos, n_q, int64_t(cache.batch) * n_q, topk,
                                 static_cast<const uint16_t*>(swa_kv), swa_first_pos, n_swa,
                                 static_cast<const uint8_t*>(cache.main), cache.main_scale, p.n_tiles,
                                 p.tiles_per_split, p.n_splits, static_cast<uint16_t*>(out), lse, part_o, part_ml);
    if (e != hipSuccess || p.n_splits == 1) return e;
    AttnMerge m;
    m.part_o = part_o;
    m.part_ml = part_ml;
    m.out = static_cast<uint16_t*>(out);
    m.lse = lse;
    m.n_heads = dims.n_heads;
    m.n_splits = p.n_splits;
    m.n_bq = int64_t(cache.batch) * n_q;
    if (merge) {
      *merge = m;
      return hipSuccess;
    }
    return launch_attn_merge(&m, 1, stream);
  }
  const dim3 grid(dims.n_heads, n_q, cache.batch);
  const size_t lds = sizeof(float) * size_t(dims.d + dims.topk + dims.window + kThreads / 64 + 2);
  const hipError_t err = launch_kernel(CSA2_KERNEL_ATTN_GENERIC, attn_generic_kernel, grid, dim3(kThreads), lds, stream, dims.d, dims.d_rope, dims.n_heads,
                     dims.topk, dims.window, int(dims.act_dtype == CSA2_BF16), int(dims.swa_dtype == CSA2_FP8), cache.kv_dtype, cache.main_group,
                     make_rope_table(dims), cache.capacity, q, q_pos, n_q, topk, swa_kv, swa_first_pos, n_swa, cache.main,
                     cache.main_scale, out, lse);
  return err;
}

}  // namespace csa2
