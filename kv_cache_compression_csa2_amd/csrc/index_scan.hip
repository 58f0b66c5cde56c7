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
#include <atomic>

#include "compress_entry.hpp"

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
    const int64_t crow = int64_t(b) * idx_rows_padded(capacity) + j, srow = int64_t(b) * capacity + j;
    s = 0.0f;
    for (int h = 0; h < Hi; ++h) {
      float dot = 0.0f;
      for (int e = 0; e < di; ++e) dot += qs[h * di + e] * idx_load(idx_k, idx_scale, kv_dtype, crow, srow, di, idx_group, e);
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


// ------------------------------------------------------------------ MFMA ---
//
// Production shape: 32 indexer heads x 128, bf16 queries, bf16 or FP4 (one
// E4M3 scale per 32 channels) indexer K.  The per-tile contraction
// S[head][entry] = Q[32 x 128] . K^T[128 x 32] runs as eight 32x32x16 MFMAs.
// Operands come straight from memory in MFMA layout: lane l supplies row
// (l % 32) with eight consecutive k of its half (l / 32); the order in which
// k is visited is free, so it is chosen to make each lane's K bytes
// contiguous: bf16, one 128-byte run per lane; FP4, two 16-byte runs, each
// one whole scale group (lane half h takes groups h and 2 + h, so the two
// halves of one k-step may belong to different groups, which the exact
// per-element dequantisation below allows).  Accumulator lane l register r holds head
// 8*(r/4) + 4*(l/32) + r%4 of entry l % 32; the head sum w_h * ReLU(.) runs in
// registers, then one cross-half shuffle completes the entry score.
//
// FP4 runs on the fp16 MFMA with every K element dequantised exactly: an
// E2M1 value times an E4M3 scale has at most 6 significant bits and lies in
// [2^-10, 2688], so it is an fp16 normal.  The scaled FP4 convert applies
// the scale's power of two (it reads only the exponent of its scale
// operand), and one packed fp16 multiply by the scale's significand (1.mmm)
// finishes each pair exactly.  The query goes to fp16 times 2^k, with k
// chosen from the query's largest magnitude so that it lands in [2^14, 2^15)
// (exact for every element down to 2^-28 of that magnitude; smaller ones
// fall to fp16 subnormals, whose rounding, at most 2^-24 of 2^k, is far below
// the float32 accumulation error); ReLU commutes with the positive factor,
// so the score is multiplied by 2^-k at the end, exactly.
//
// A workgroup (4 waves) covers 4 kSbW super-blocks of 64 domain slots; wave
// w takes super-blocks w, w+4, ... (two 32-entry tiles each), kBatch at a
// time, with the loads of the next batch issued before the current one is
// contracted.  The batches are fully unrolled so the two load buffers are
// fixed registers.  POOL: the domain is a block pool (slot -> pool entry).

extern "C" __device__ uint32_t __ockl_wfred_max_u32(uint32_t);

typedef __bf16 bf16x8_t __attribute__((__vector_size__(16)));
typedef _Float16 f16x8_t __attribute__((__vector_size__(16)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((__vector_size__(64)));

constexpr int kSbPerWave = 4;
constexpr int kFp4Ahead = 1;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Eight E2M1 codes (one dword, low nibble first) times the E4M3 scale s ->
// eight exact fp16 values; mpair holds s's significand twice (fp16).
__device__ __forceinline__ f16x8_t fp4x8_to_f16(uint32_t w, float s, uint32_t mpair) {
  const f16x2_t m = __builtin_bit_cast(f16x2_t, mpair);
  uint4 v;
  v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 0) * m);
  v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 1) * m);
  v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 2) * m);
  v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 3) * m);
  return __builtin_bit_cast(f16x8_t, v);
}

// The significand 1.mmm of a positive float (its value over its power of
// two) as a pair of fp16 values; exact for the E4M3 scale values.
__device__ __forceinline__ uint32_t significand_pair(float s) {
  const uint32_t h = ((__float_as_uint(s) >> 13) & 0x3FFu) | 0x3C00u;
  return h | (h << 16);
}

// max(x, 0) as an integer max on the bits (fmaxf adds a canonicalising max)
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Signed-integer image of a float that orders like the float (negative
// values have their magnitude bits flipped); its own inverse.  Maxima of
// scores are taken on these, so each step is one integer max (a float max
// would first canonicalise the exchanged operand).
__device__ __forceinline__ int ord_int(int b) { return b ^ int(uint32_t(b >> 31) >> 1); }

// Maximum with the value of another lane of the same 16-lane row, by DPP.
// Every pattern used reads a lane inside the row, so bound_ctrl changes
// nothing but lets the compiler fold the move into one v_max_i32_dpp.
template <int CTRL>
__device__ __forceinline__ int max_dpp(int k) { return max(k, __builtin_amdgcn_mov_dpp(k, CTRL, 0xF, 0xF, true)); }
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // lane i of each 8 <- lane 7 - i
constexpr int kDppMirror = 0x140;     // lane i of each 16 <- lane 15 - i

// x of this lane plus x of the lane 32 away (the two halves swap through
// v_permlane32_swap; whichever half each result holds, their sum is the pair's)
__device__ __forceinline__ float add_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Maximum over the two 16-lane rows of each 32-lane half (rows 0 and 1, 2 and 3).
__device__ __forceinline__ int max_row_pairs(int k) {
  const auto r = __builtin_amdgcn_permlane16_swap(uint32_t(k), uint32_t(k), false, false);
  return max(int(r[0]), int(r[1]));
}

// FP4 scans: the indexer query as the fp16 A operand, times 2^k so its
// largest magnitude sits just below 2^15 (k undone on the score by
// `unscale`).  The operand is the same for the workgroup's four waves: each
// converts two of the eight operand chunks of every lane, after one shared
// maximum fixes k, and all read the whole operand back from LDS
// ([chunk][lane]).  Every thread of the workgroup calls it.
// (in two steps: the loads, then the rest, so that a caller can issue the
// loads early)
__device__ __forceinline__ void fp4_query_load(const uint16_t* qrow, int h, int wave, uint4 (&qraw)[2]) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int q = 2 * wave + c;
    qraw[c] = *reinterpret_cast<const uint4*>(qrow + 64 * (q >> 2) + 32 * h + 8 * (q & 3));
  }
}
__device__ __forceinline__ const uint4* fp4_query_finish(const uint4 (&qraw)[2], int wave, int lane, float& unscale) {
  __shared__ uint32_t q_amax[4];
  __shared__ uint4 q_op[8][64];  // [chunk][lane]
  uint32_t amax = 0;  // largest |q| (bits of a non-negative float)
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const uint32_t w4[4] = {qraw[c].x, qraw[c].y, qraw[c].z, qraw[c].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) amax = max(amax, max((w4[i] << 16) & 0x7FFF0000u, w4[i] & 0x7FFF0000u));
  }
  amax = __ockl_wfred_max_u32(amax);
  if (lane == 0) q_amax[wave] = amax;
  __syncthreads();
  amax = max(max(q_amax[0], q_amax[1]), max(q_amax[2], q_amax[3]));
  const int e = amax ? int(amax >> 23) - 127 : 0;  // floor(log2 max|q|)
  const int k = min(100, max(-100, 14 - e));
  const float up = __uint_as_float(uint32_t(127 + k) << 23);
  unscale = __uint_as_float(uint32_t(127 - k) << 23);
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const uint32_t w4[4] = {qraw[c].x, qraw[c].y, qraw[c].z, qraw[c].w};
    uint4 v;
    uint32_t* vv = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x2_t pr = {_Float16(__uint_as_float(w4[i] << 16) * up), _Float16(__uint_as_float(w4[i] & 0xFFFF0000u) * up)};
      vv[i] = __builtin_bit_cast(uint32_t, pr);
    }
    q_op[2 * wave + c][lane] = v;
  }
  __syncthreads();
  return &q_op[0][0];
}
__device__ __forceinline__ const uint4* fp4_query_lds(const uint16_t* qrow, int h, int wave, int lane,
                                                      float& unscale) {
  uint4 qraw[2];
  fp4_query_load(qrow, h, wave, qraw);
  return fp4_query_finish(qraw, wave, lane, unscale);
}

// The score of a tile's entry from its products: the lane's 16 heads'
// w_h * max(0, logit) in two partial sums (half the dependent chain), plus
// the other half's 16 (both halves hold the same sum), times `unscale`.
__device__ __forceinline__ float tile_score(const f32x16_t& acc, const float (&wreg)[16], float unscale) {
  float part = 0.0f, part1 = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    part = fmaf(wreg[r], relu(acc[r]), part);
    part1 = fmaf(wreg[r + 1], relu(acc[r + 1]), part1);
  }
  part += part1;
  return add_halves(part) * unscale;
}

// Tile loads of one batch (kBatch super-blocks = 2 kBatch tiles of 32 entries).
template <bool FP4, int kBatch>
struct ScanBatch {
  int32_t slot[2 * kBatch];
  bool valid[2 * kBatch];
  uint4 kb[FP4 ? 1 : 2 * kBatch][8];
  uint4 kf[FP4 ? 2 * kBatch : 1][2];
  uint32_t ks[FP4 ? 2 * kBatch : 1];
};

// bx: this workgroup's block of super-blocks, b: its sequence (query
// blockIdx.y); j_skip: an entry left out of
// the scores and maxima (the step's entry of a fused decode scan; read only
// when SKIP), or -1.
template <bool FP4, bool POOL, int kBatch, int kSbW, int kAhead, bool SKIP = false>
__device__ __forceinline__ void scan_mfma_body(
    int ratio, int64_t capacity, const uint16_t* __restrict__ idx_q, const float* __restrict__ head_w,
    const int32_t* __restrict__ q_pos, int n_q, const int32_t* __restrict__ pool_in, int cand_blocks,
    const uint8_t* __restrict__ idx_k, const uint8_t* __restrict__ idx_scale, const int32_t* __restrict__ n_entries,
    float* __restrict__ scores, float* __restrict__ bmax, float* __restrict__ sbmax, int64_t dom_cap, int bx, int b,
    int j_skip) {
  constexpr int kTiles = 2 * kBatch;
  constexpr int kIters = kSbW / kBatch;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, h = lane >> 5;
  const int qi = blockIdx.y;
  const int64_t row = int64_t(b) * n_q + qi;
  const int nsb = int(dom_cap / 64);
  const int n_vis = int(visible_count(clamp_entries(n_entries, b, capacity), q_pos[row], ratio));
  const int sb0 = bx * (4 * kSbW) + wave;
  const int last_tile = int(idx_rows_padded(capacity) / 32) - 1;
  // this lane's bytes inside a tile: row n, and its half's first chunk
  const uint32_t lane_off = uint32_t(n) * 16u + uint32_t(h) * (FP4 ? 512u : 4096u);
  // this sequence's rows (bf16: 256 bytes, FP4: 64 code bytes + 4 scale bytes)
  const uint8_t* kseq = idx_k + int64_t(b) * idx_rows_padded(capacity) * (FP4 ? 64 : 256);
  const uint8_t* sseq = FP4 ? idx_scale + int64_t(b) * capacity * 4 : nullptr;
  const int32_t* prow = POOL ? pool_in + row * cand_blocks : nullptr;
  float* srow = scores + row * dom_cap;
  float* brow = bmax + row * (dom_cap / 8);
  float* sbrow = sbmax + row * nsb;

  // The loads and stores are issued unconditionally (slots past the visible
  // entries read a valid row and are masked; every lane stores, the domain
  // being whole workgroups of super-blocks): a load or a store under a
  // branch makes the compiler's wait counts assume the branch was skipped,
  // so each batch waited for the loads of the batch issued after it and the
  // prefetch was void (FP4 1M scan 40.5 -> 35.5 us, 32K bf16 scan 26.7 ->
  // 25.2 us).
  auto issue = [&](int it, ScanBatch<FP4, kBatch>& B) {
    const int sb_first = sb0 + 4 * kBatch * it;
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      const int sb = sb_first + 4 * (t >> 1);  // wave-uniform
      B.slot[t] = sb * 64 + 32 * (t & 1) + n;
      int j = B.slot[t];
      if constexpr (POOL) {
        const int blk = sb < nsb && B.slot[t] / 8 < cand_blocks ? prow[B.slot[t] / 8] : -1;
        j = blk >= 0 ? blk * 8 + (B.slot[t] & 7) : -1;
      }
      B.valid[t] = sb < nsb && j >= 0 && j < n_vis && (!SKIP || j != j_skip);
      const uint8_t* tile;
      int jj;  // the entry whose scales are read
      if constexpr (POOL) {
        jj = B.valid[t] ? j : 0;
        // tile jj / 32, row jj % 32: chunk c at (32 c + jj % 32) * 16
        tile = kseq + int64_t(jj >> 5) * (FP4 ? 2048 : 8192) + (jj & 31) * 16 + h * (FP4 ? 512 : 4096);
      } else {
        // slot = entry: the tile is the same for the whole wave (clamped to
        // the sequence's last padded tile; rows past the visible ones are
        // masked), so the address is a wave-uniform base plus the lane's
        // fixed 32-bit offset and costs no per-lane arithmetic
        const int tu = min(2 * sb + (t & 1), last_tile);
        tile = kseq + int64_t(tu) * (FP4 ? 2048 : 8192) + lane_off;
        jj = min(32 * tu + n, int(capacity) - 1);
      }
      if constexpr (FP4) {
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) B.kf[t][g2] = *reinterpret_cast<const uint4*>(tile + g2 * 1024);
        // the entry's four scale bytes as loaded: shifting them here would
        // wait for the load at issue time and void the prefetch
        B.ks[t] = *reinterpret_cast<const uint32_t*>(sseq + int64_t(jj) * 4);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) B.kb[t][q] = *reinterpret_cast<const uint4*>(tile + q * 512);
      }
    }
    // keep the loads here, a batch ahead of their use (the scheduler would
    // otherwise sink each next to its product)
    __builtin_amdgcn_sched_barrier(0);
  };

  // kAhead batches' loads fly while one is contracted
  ScanBatch<FP4, kBatch> buf[kAhead + 1];
#pragma unroll
  for (int a = 0; a < kAhead; ++a)
    if (a < kIters) issue(a, buf[a]);

  // A operand (indexer query) and the lane's 16 head weights, held for the whole scan
  const uint16_t* qrow = idx_q + (row * 32 + n) * 128;
  float wreg[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) wreg[r] = head_w[row * 32 + 8 * (r >> 2) + 4 * h + (r & 3)];
  bf16x8_t qop[FP4 ? 1 : 8];
  // FP4: the fp16 operand stays in LDS ([chunk][lane]) and is read at each
  // product: 32 registers fewer than holding it (30.5 against 31.9 us for
  // the 1M FP4 scan)
  const uint4* q_lds = nullptr;
  float unscale = 1.0f;
  if constexpr (FP4) {
    q_lds = fp4_query_lds(qrow, h, wave, lane, unscale);
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) qop[q] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 64 * h + 8 * q));
  }

#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    if (it + kAhead < kIters) issue(it + kAhead, buf[(it + kAhead) % (kAhead + 1)]);
    ScanBatch<FP4, kBatch>& B = buf[it % (kAhead + 1)];
    int tmax[kTiles];
    // the tiles' products first, interleaved (independent accumulator
    // chains keep the matrix pipe busy), then each tile's epilogue
    f32x16_t acc[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) acc[t] = f32x16_t{};
    {
      if constexpr (FP4) {
        // this lane's groups: h (first 16 bytes) and 2 + h (second)
        float sg[kTiles][2];
        uint32_t mp[kTiles][2];
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
          const uint32_t ks = B.ks[t] >> (8 * h);  // scales h and 2 + h in bytes 0 and 2
          sg[t][0] = __builtin_amdgcn_cvt_f32_fp8(int(ks), 0);
          sg[t][1] = __builtin_amdgcn_cvt_f32_fp8(int(ks), 2);
          mp[t][0] = significand_pair(sg[t][0]);
          mp[t][1] = significand_pair(sg[t][1]);
        }
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
#pragma unroll
          for (int sub = 0; sub < 4; ++sub) {
#pragma unroll
            for (int t = 0; t < kTiles; ++t) {
              const uint32_t w4[4] = {B.kf[t][g2].x, B.kf[t][g2].y, B.kf[t][g2].z, B.kf[t][g2].w};
              acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, q_lds[(4 * g2 + sub) * 64 + lane]),
                                                              fp4x8_to_f16(w4[sub], sg[t][g2], mp[t][g2]), acc[t], 0, 0, 0);
            }
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
          for (int t = 0; t < kTiles; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qop[q], as_bf16x8(B.kb[t][q]), acc[t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      float sc = tile_score(acc[t], wreg, unscale);
      if (!B.valid[t]) sc = -INFINITY;
      // block (8 lanes) and tile (32 lanes) maxima, as ordered integers; the
      // butterflies leave each maximum in every lane it covers
      int m = ord_int(__float_as_int(sc));
      m = max_dpp<kDppXor1>(m);
      m = max_dpp<kDppXor2>(m);
      m = max_dpp<kDppHalfMirror>(m);
      const float bmx = __int_as_float(ord_int(m));
      m = max_dpp<kDppMirror>(m);
      tmax[t] = max_row_pairs(m);
      // every lane stores (lanes holding the same value write the same
      // address), so no store sits under a branch: the domain is whole
      // workgroups of super-blocks, every slot of this wave lies in it
      const int slot = (sb0 + 4 * kBatch * it + 4 * (t >> 1)) * 64 + 32 * (t & 1) + n;
      srow[slot] = sc;
      brow[slot >> 3] = bmx;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) sbrow[sb0 + 4 * kBatch * it + 4 * u] = __int_as_float(ord_int(max(tmax[2 * u], tmax[2 * u + 1])));
  }
}

#define SCAN_ARGS                                                                                                     \
  int ratio, int64_t capacity, const uint16_t *__restrict__ idx_q, const float *__restrict__ head_w,                 \
      const int32_t *__restrict__ q_pos, int n_q, const int32_t *__restrict__ pool_in, int cand_blocks,               \
      const uint8_t *__restrict__ idx_k, const uint8_t *__restrict__ idx_scale,                                       \
      const int32_t *__restrict__ n_entries, float *__restrict__ scores, float *__restrict__ bmax,                    \
      float *__restrict__ sbmax, int64_t dom_cap
#define SCAN_PASS \
  ratio, capacity, idx_q, head_w, q_pos, n_q, pool_in, cand_blocks, idx_k, idx_scale, n_entries, scores, bmax, sbmax, dom_cap

// bf16: one super-block pair per batch, 2 waves per SIMD (the double load
// buffer takes the registers of a third); FP4: one pair per batch at 3.
// SBW: super-blocks per wave (kSbPerWave; 2 or 1 when the scan has too few
// workgroups to cover the compute units, see launch_scan)
template <bool POOL, int SBW>
__global__ __launch_bounds__(256, 2) void scan_mfma_bf16_kernel(SCAN_ARGS) {
  scan_mfma_body<false, POOL, 1, SBW, 1>(SCAN_PASS, int(blockIdx.x), int(blockIdx.z), -1);
}
template <bool POOL, int SBW>
__global__ __launch_bounds__(256, 3) void scan_mfma_fp4_kernel(SCAN_ARGS) {
  scan_mfma_body<true, POOL, 1, SBW, kFp4Ahead>(SCAN_PASS, int(blockIdx.x), int(blockIdx.z), -1);
}

// The step's entry of sequence b in a fused decode scan (the compressor's
// entry 0 at first_pos[b]), or -1 when it writes none.
__device__ __forceinline__ int fused_entry(const CompressParams& P, int b) {
  const int64_t fp = P.first_pos[b];
  if (fp < 0 || fp % P.ratio) return -1;
  const int64_t j = fp / P.ratio;
  return j < P.capacity ? int(j) : -1;
}

// The compressing workgroup of a fused decode scan (sequence b, one query): writes the step's entry with the compressor's arithmetic (256
// threads standing for the compress kernel's 1024: the same bits), then
// scores it as the scan scores any entry - the same operands, products in
// the same order and the same fold - and leaves the score and the entry's id
// for the selection (fix_score / fix_id: -inf / -1 when the entry is not
// visible to the query).  The other workgroups leave the entry out.
//
// It runs beside a scan that keeps memory busy, where each dependent round
// trip to memory is slow, so its chain holds as few as it can: the query, the
// head weights, the latent row and W_ik (all of it for bf16 caches; half,
// within the FP4 scan's register budget) are requested together up front, the
// entry is scored from the LDS copy of the stored indexer row (no reload),
// and its waves take issue priority over the scan's on the compute unit.
template <bool FP4>
__device__ void scan_fused_entry(const ScanFuse& fz, int ratio, int64_t capacity, const uint16_t* __restrict__ idx_q,
                                 const float* __restrict__ head_w, const int32_t* __restrict__ q_pos, int n_q,
                                 const int32_t* __restrict__ n_entries, int b) {
  extern __shared__ double csh[];
  __builtin_amdgcn_s_setprio(2);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;
  const int64_t row = int64_t(b) * n_q;
  // the query operand and head weights, as the scan holds them, requested first
  const uint16_t* qrow = idx_q + (row * 32 + n) * 128;
  float wreg[16];
  auto load_wreg = [&]() {
#pragma unroll
    for (int r = 0; r < 16; ++r) wreg[r] = head_w[row * 32 + 8 * (r >> 2) + 4 * h + (r & 3)];
  };
  if constexpr (!FP4) load_wreg();  // (FP4: after the entry, within the register budget)
  bf16x8_t qop[FP4 ? 1 : 8];
  uint4 qraw[2];
  if constexpr (FP4) {
    fp4_query_load(qrow, h, wave, qraw);
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) qop[q] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 64 * h + 8 * q));
  }
  const int64_t n_vis = visible_count(clamp_entries(n_entries, b, capacity), q_pos[row], ratio);
  uint8_t* mirror = reinterpret_cast<uint8_t*>(csh + compress_lds_doubles(fz.cp.d, fz.cp.d_idx));
  const int64_t j = compress_entry<true, 256, FP4 ? 1 : 2, FP4 ? 8 : 16>(fz.cp, 0, b, csh, mirror);
  float unscale = 1.0f;
  const uint4* q_lds = nullptr;
  if constexpr (FP4) load_wreg();
  if constexpr (FP4) q_lds = fp4_query_finish(qraw, wave, lane, unscale);  // its barrier also publishes mirror
  else __syncthreads();                                                     // mirror is complete
  const bool live = j >= 0 && j < n_vis;  // uniform
  if (live && wave == 0) {
    // every lane takes the entry's row (column j % 32 is the one kept)
    f32x16_t acc = f32x16_t{};
    if constexpr (FP4) {
      uint4 kf[2];
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) kf[g2] = *reinterpret_cast<const uint4*>(mirror + 16 * (2 * g2 + h));
      const uint32_t ks = *reinterpret_cast<const uint32_t*>(mirror + 64) >> (8 * h);
      float sg[2];
      uint32_t mp[2];
      sg[0] = __builtin_amdgcn_cvt_f32_fp8(int(ks), 0);
      sg[1] = __builtin_amdgcn_cvt_f32_fp8(int(ks), 2);
      mp[0] = significand_pair(sg[0]);
      mp[1] = significand_pair(sg[1]);
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        const uint32_t w4[4] = {kf[g2].x, kf[g2].y, kf[g2].z, kf[g2].w};
#pragma unroll
        for (int sub = 0; sub < 4; ++sub)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, q_lds[(4 * g2 + sub) * 64 + lane]),
                                                       fp4x8_to_f16(w4[sub], sg[g2], mp[g2]), acc, 0, 0, 0);
      }
    } else {
      uint4 kb[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) kb[q] = *reinterpret_cast<const uint4*>(mirror + 2 * (64 * h + 8 * q));
#pragma unroll
      for (int q = 0; q < 8; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qop[q], as_bf16x8(kb[q]), acc, 0, 0, 0);
    }
    const float sc = tile_score(acc, wreg, unscale);
    if (lane == int(j & 31)) fz.fix_score[row] = sc;
  }
  if (tid == 0) {
    fz.fix_id[row] = live ? int32_t(j) : -1;
    if (!live) fz.fix_score[row] = -INFINITY;
  }
}

// Decode scan that writes the step's entry, on a one-dimensional grid of
// batch * (nx + 1) workgroups for one query per sequence: workgroup L <
// batch compresses and scores sequence L's entry (scan_fused_entry), and
// workgroup batch + i scans block i % nx of sequence i / nx, as
// scan_mfma_*_kernel's (x, z), leaving the entry out.  The compressing
// workgroups come first in dispatch order, so that they start with the scan
// (placed last, they started only as the first scan workgroups finished and
// ended after them).  kSbW: super-blocks per scan wave.
template <bool FP4, int kSbW>
__device__ __forceinline__ void scan_fused_body(SCAN_ARGS, const ScanFuse& fz) {
  const int nx = int((dom_cap / 64 + 4 * kSbW - 1) / (4 * kSbW));
  const int batch = int(gridDim.x) / (nx + 1);
  const int L = int(blockIdx.x);
  if (L < batch) {
    scan_fused_entry<FP4>(fz, ratio, capacity, idx_q, head_w, q_pos, n_q, n_entries, L);
    return;
  }
  const int b = (L - batch) / nx;
  scan_mfma_body<FP4, false, 1, kSbW, FP4 ? kFp4Ahead : 1, true>(SCAN_PASS, L - batch - b * nx, b,
                                                                 fused_entry(fz.cp, b));
}
// bf16: half-size scan blocks.  The compressing workgroups hold slots that
// the scan's first wave would use (32K x 16 decode: 512 full-size blocks
// for 512 resident workgroups), which pushes scan blocks into a later wave;
// a half-size block ends sooner (32K x 16: 29.3 -> 27.9 us; 256K x 4, which
// needs several waves anyway: 52.4 against 52.9 us).  One kernel choosing
// the block size at run time compiled slower than either (29.3 us at 32K).
constexpr int kFusedSbBf16 = 2;
constexpr int kFusedSbFp4 = kSbPerWave;
__global__ __launch_bounds__(256, 2) void scan_fused_bf16_kernel(SCAN_ARGS, ScanFuse fz) {
  scan_fused_body<false, kFusedSbBf16>(SCAN_PASS, fz);
}
__global__ __launch_bounds__(256, 3) void scan_fused_fp4_kernel(SCAN_ARGS, ScanFuse fz) {
  scan_fused_body<true, kFusedSbFp4>(SCAN_PASS, fz);
}

// ------------------------------------------------------- query-blocked scan --
//
// Many queries per sequence (chunked prefill): the score contraction is a
// GEMM per head, S_h = Q_h . K^T, whose K operand is shared by all 32 heads.
// A workgroup (4 waves) owns 32 queries of one sequence and 256 entries; wave
// w owns entries [64w, 64w+64).  Each wave loads its entries' indexer K
// once, in registers, as the A operand of v_mfma_f32_32x32x16_bf16 (lane =
// entry, 8 channels per lane and k-step; 2 blocks of 32 entries x 8 k-steps),
// which keeps every operand and accumulator in the 256 architected registers
// (with 128 entries per wave part of K went to AGPRs and came back by a copy
// before every product) and lets two workgroups share a compute unit,
// so the products are logits^T[entry][query]: a lane then holds one query and
// runs of 4 consecutive entries, which makes the head weight one value per
// lane, the score stores 16 bytes wide and a block maximum one exchange.
// The heads then stream through LDS two at a time: the 32 queries' rows of
// heads 2p and 2p+1 (2 x 8 KB) are copied global -> LDS (global_load_lds_dwordx4,
// from inline assembly so the compiler does not drain them before LDS reads)
// two pairs ahead into three LDS stages, and every wave contracts each head
// against its resident K (8 k-steps x 4 blocks), then adds w_h * max(0, logit)
// into its 32 x 128 scores - one head's additions run under the next head's
// products (two accumulator sets).  One workgroup barrier per head pair.  The
// query rows sit in LDS XOR-swizzled by 16-byte chunk so the B-operand reads
// of 32 rows spread over the banks.
// Scores, block maxima and super-block maxima are then written in the same
// layout as the per-query scan.  The workgroups of one query block run on one
// XCD (workgroups are dealt to the 8 XCDs in turn), entry blocks in order, so
// the block's query rows stay in that L2 while K streams.

constexpr int kPQ = 32;               // queries per query block
constexpr int kQB = 1;                // query blocks per workgroup, in turn, sharing its resident K
                                      // (more than one overflows the register file at this tile size)
constexpr int kEB = 2;                // 32-entry blocks per wave (its resident K: 32 kEB registers)
constexpr int kPE = 4 * 32 * kEB;     // entries per workgroup
constexpr int kQTile = kPQ * 256;     // one head's query rows (bytes)
constexpr int kHPS = 4;               // heads per LDS stage (even): one workgroup barrier per stage
constexpr int kStages = 2;            // stages in LDS: kStages - 1 stages' copies fly
constexpr int kNStage = 32 / kHPS;    // stages per query block

typedef float f32x16_t_ __attribute__((__vector_size__(64)));

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved; naming it tells the compiler it changes
// Copy 16 bytes per lane from global `src` to LDS byte address `lds_addr` +
// 16 * lane.  Completion is tracked only by the caller's s_waitcnt vmcnt.
__device__ __forceinline__ void copy16_to_lds(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_addr), "v"(src) : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS slot (16 bytes) of chunk c (0..15) of query row q (0..31) in a head tile.
__device__ __forceinline__ int qslot(int q, int c) { return q * 16 + (c ^ (q & 15)); }

__global__ __launch_bounds__(256, 2) void scan_prefill_kernel(
    int ratio, int64_t capacity, const uint16_t* __restrict__ idx_q, const float* __restrict__ head_w,
    const int32_t* __restrict__ q_pos, int n_q, const uint8_t* __restrict__ idx_k,
    const int32_t* __restrict__ n_entries, float* __restrict__ scores, float* __restrict__ bmax,
    float* __restrict__ sbmax, int64_t dom_cap, int nqs, int neb, int groups) {
  __shared__ __align__(16) uint8_t qtile[kHPS * kStages][kQTile];  // kStages stages x kHPS heads
  __shared__ __align__(16) float wl[32][kPQ];  // head weights [head][query]
  __shared__ int nvis[kPQ];
  __shared__ int vis_max;

  // workgroup -> (sequence, kQB query blocks, entry block): the entry blocks
  // of one query group share an XCD (id % 8) and follow each other
  const int64_t wg = blockIdx.x, x8 = wg & 7, rest = wg >> 3;
  const int64_t grp = x8 + 8 * (rest / neb);
  if (grp >= groups) return;  // padding workgroup (uniform)
  const int eb = int(rest % neb);
  const int b = int(grp / nqs), qbase = int(grp % nqs) * (kQB * kPQ);
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 31, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t e_wg = int64_t(eb) * kPE, e0 = e_wg + 32 * kEB * wave;
  const int64_t n_ent = clamp_entries(n_entries, b, capacity);

  // ---- issue first, independent of the bookkeeping below: this wave's
  // entries' indexer K (the A operand, resident for all heads) and the query
  // tiles of heads 0 and 1 ----
  uint4 kreg[kEB][8];
#pragma unroll
  for (int blk = 0; blk < kEB; ++blk) {
    int64_t e = e0 + 32 * blk + n;
    e = e < capacity ? e : capacity - 1;  // slots past the cache: any valid row (masked below)
    // tile e / 32 of this sequence, row e % 32: chunk c at (32 c + e % 32) * 16
    const uint8_t* tile = idx_k + (int64_t(b) * idx_rows_padded(capacity) + (e & ~int64_t(31))) * 256 + (e & 31) * 16;
#pragma unroll
    for (int s = 0; s < 8; ++s) kreg[blk][s] = *reinterpret_cast<const uint4*>(tile + (2 * s + hl) * 512);  // channels 16s + 8hl .. +8
  }
  // copies of the query tiles of heads kHPS p .. kHPS p + kHPS - 1 into stage
  // p % kStages: 8 kHPS instructions of 1 KB (4 query rows each); wave w
  // issues 2 kHPS of them
  auto issue_pair = [&](int p, int q0) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(
        uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void*)qtile[kHPS * (p % kStages)])));
#pragma unroll
    for (int m4 = 0; m4 < 2 * kHPS; ++m4) {
      const int m = 2 * kHPS * wave + m4;   // head kHPS p + m / 8, instruction m % 8
      const int hh = kHPS * p + (m >> 3);
      const int slot = (m & 7) * 64 + lane;  // destination slot in that head's tile
      const int q = slot >> 4;               // query row of the slot
      const int c = (slot & 15) ^ (q & 15);  // its chunk (inverse of qslot)
      const int qg = min(q0 + q, n_q - 1);   // rows past the last query: any valid row (never stored)
      const uint16_t* src = idx_q + ((int64_t(b) * n_q + qg) * 32 + hh) * 128 + 8 * c;
      copy16_to_lds(src, base + m * 1024);
    }
  };
#pragma unroll 1
  for (int qs = 0; qs < kQB; ++qs) {
    const int q0 = qbase + qs * kPQ;
    if (q0 >= n_q) break;  // uniform
    issue_pair(0, q0);

    // ---- per-query visibility and head weights ----
    __syncthreads();  // the previous block's readers of vis_max, nvis and wl are done
    if (tid == 0) vis_max = 0;
    __syncthreads();
    if (tid < kPQ) {
      const int q = q0 + tid;
      const int v = q < n_q ? int(visible_count(n_ent, q_pos[int64_t(b) * n_q + q], ratio)) : 0;
      nvis[tid] = v;
      atomicMax(&vis_max, v);
    }
    for (int x = tid; x < 32 * kPQ; x += 256) {
      const int hh = x / kPQ, qq = x % kPQ;
      wl[hh][qq] = q0 + qq < n_q ? head_w[(int64_t(b) * n_q + q0 + qq) * 32 + hh] : 0.0f;
    }
    // every load so far (K included) complete, with a wait the compiler sees:
    // from here on the kernel's own vmcnt waits count only head copies
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    for (int pp = 1; pp < kStages - 1; ++pp) issue_pair(pp, q0);
    __syncthreads();
    const int64_t vmax = vis_max;
    const bool wave_live = e0 < vmax;  // some query sees some entry of this wave's range

    f32x16_t_ sacc[kEB];
#pragma unroll
    for (int blk = 0; blk < kEB; ++blk) sacc[blk] = f32x16_t_{};

    if (e_wg < vmax) {
      // Software pipeline over the heads: each k-step's query operand of
      // head h+1 is read from LDS into the register of head h's operand as
      // soon as head h's two products have taken it (eight operands live, a
      // head of products to arrive), and head h-1's ReLU.w fold is
      // interleaved with head h's products (a product, then four VALU
      // instructions), so one wave keeps the matrix pipe fed while its VALU
      // and LDS work proceed.  Head h-1's logits are complete by then (its
      // last product issued one product earlier).  The stage barrier sits
      // before a stage's last head, during which the next stage's first
      // head is read.
      // head products into acc, reading the next head's operands from tile
      // `nqt` into op, interleaved with fold(w_prev, prev): scores +=
      // w_prev * max(0, logit) (ReLU as an integer max on the bits)
      auto head_step = [&](bf16x8_t (&op)[8], f32x16_t_* acc, const uint8_t* nqt, float w_prev,
                           const f32x16_t_* prev) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
#pragma unroll
          for (int blk = 0; blk < kEB; ++blk)
            acc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kreg[blk][s]), op[s],
                                                               s == 0 ? f32x16_t_{} : acc[blk], 0, 0, 0);
          op[s] = *reinterpret_cast<const bf16x8_t*>(nqt + 16 * qslot(n, 2 * s + hl));
        }
#pragma unroll
        for (int blk = 0; blk < kEB; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sacc[blk][r] += w_prev * __int_as_float(max(__float_as_int(prev[blk][r]), 0));
        // per k-step: a product, four VALU, the other product, the operand read, four VALU
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
      };
      // this wave's copies of stage p landed (those of the stages after it,
      // at most kStages - 2 of 2 kHPS instructions each, may still fly);
      // after the barrier every wave's copies are visible and the slot of
      // stage p - 1 is free for stage p + kStages - 1
      auto stage_ready = [&](int p) {
        const int ahead = min(kStages - 2, kNStage - 1 - p) * 2 * kHPS;
        if (ahead >= 16)
          asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
        else if (ahead >= 8)
          asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else if (ahead >= 4)
          asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        else
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (p + kStages - 1 < kNStage) issue_pair(p + kStages - 1, q0);
      };
      bf16x8_t op[8];
      f32x16_t_ acc0[kEB], acc1[kEB];
#pragma unroll
      for (int blk = 0; blk < kEB; ++blk) acc1[blk] = f32x16_t_{};  // "head -1": folds nothing
      stage_ready(0);
      if (wave_live) {
#pragma unroll
        for (int s = 0; s < 8; ++s) op[s] = *reinterpret_cast<const bf16x8_t*>(qtile[0] + 16 * qslot(n, 2 * s + hl));
      }
      for (int p = 0; p < kNStage; ++p) {  // heads kHPS p + j: even j into acc0, odd into acc1
        const uint8_t* qt = qtile[kHPS * (p % kStages)];
#pragma unroll
        for (int j = 0; j < kHPS; ++j) {
          const int h = kHPS * p + j;
          const uint8_t* nqt;  // the tile of head h + 1
          if (j + 1 < kHPS) {
            nqt = qt + (j + 1) * kQTile;
          } else {
            if (p + 1 < kNStage) stage_ready(p + 1);
            // after the last stage the reads re-read this stage (never used)
            nqt = qtile[kHPS * ((p + 1 < kNStage ? p + 1 : p) % kStages)];
          }
          if (wave_live) {
            const float w_prev = h > 0 ? wl[h - 1][n] : 0.0f;
            if (j % 2 == 0)
              head_step(op, acc0, nqt, w_prev, acc1);
            else
              head_step(op, acc1, nqt, w_prev, acc0);
          }
        }
      }
      if (wave_live) {
        const float w = wl[31][n];
#pragma unroll
        for (int blk = 0; blk < kEB; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[blk][r] += w * __int_as_float(max(__float_as_int(acc1[blk][r]), 0));
      }
    }

    // ---- mask, store scores and maxima ----
    // lane: query n, entries e0 + 32 blk + 8j + 4hl + i (i < 4) in sacc[blk][4j + i]
    if (e0 >= dom_cap) continue;  // uniform per wave
    const int q = q0 + n;
    const int64_t row = int64_t(b) * n_q + q;
    const int64_t vis = nvis[n];
    const int64_t nsb = dom_cap / 64;
    float m_sb[(kEB + 1) / 2];
#pragma unroll
    for (int i = 0; i < (kEB + 1) / 2; ++i) m_sb[i] = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < kEB; ++blk) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t e = e0 + 32 * blk + 8 * j + 4 * hl;
        float4 v;
        v.x = e < vis ? sacc[blk][4 * j] : -INFINITY;
        v.y = e + 1 < vis ? sacc[blk][4 * j + 1] : -INFINITY;
        v.z = e + 2 < vis ? sacc[blk][4 * j + 2] : -INFINITY;
        v.w = e + 3 < vis ? sacc[blk][4 * j + 3] : -INFINITY;
        if (q < n_q) *reinterpret_cast<float4*>(scores + row * dom_cap + e) = v;
        float m = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
        m = fmaxf(m, __shfl_xor(m, 32, kWave));  // the block's other 4 entries
        if (q < n_q && hl == 0) bmax[row * (dom_cap / 8) + (e0 + 32 * blk + 8 * j) / 8] = m;
        m_sb[blk >> 1] = fmaxf(m_sb[blk >> 1], m);
      }
    }
#pragma unroll
    for (int p2 = 0; p2 < (kEB + 1) / 2; ++p2) {
      const int64_t sb = (e0 + 64 * p2) / 64;
      if (q < n_q && hl == 0 && sb < nsb) sbmax[row * nsb + sb] = m_sb[p2];
    }
  }
}


// Compute units of the current device (looked up once per device).
hipError_t compute_units(int* cus) {
  static std::atomic<int> known[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && (*cus = known[dev].load(std::memory_order_relaxed)) > 0) return hipSuccess;
  e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess && dev >= 0 && dev < 64) known[dev].store(*cus, std::memory_order_relaxed);
  return e;
}

template <bool FP4, bool POOL>
auto scan_kernel_for(int sbw) {
  if constexpr (FP4) return sbw == 1 ? scan_mfma_fp4_kernel<POOL, 1> : sbw == 2 ? scan_mfma_fp4_kernel<POOL, 2>
                                                                              : scan_mfma_fp4_kernel<POOL, kSbPerWave>;
  else return sbw == 1 ? scan_mfma_bf16_kernel<POOL, 1> : sbw == 2 ? scan_mfma_bf16_kernel<POOL, 2>
                                                                  : scan_mfma_bf16_kernel<POOL, kSbPerWave>;
}

}  // namespace

hipError_t launch_scan(const csa2_dims& dims, const csa2_kv_cache& cache, const void* idx_q, const float* head_w,
                       const int32_t* q_pos, int32_t n_q, const int32_t* pool_in, const ScanScratch& ss,
                       hipStream_t stream) {
  const bool mfma_shape = dims.n_idx_heads == 32 && dims.d_idx == 128 && dims.act_dtype == CSA2_BF16 &&
                          (cache.kv_dtype == CSA2_BF16 || (cache.kv_dtype == CSA2_FP4 && cache.idx_group == 32));
  if (mfma_shape && cache.kv_dtype == CSA2_BF16 && !pool_in && n_q >= 8) {
    // many queries per sequence: query-blocked MFMA scan
    const int nqs = (n_q + kQB * kPQ - 1) / (kQB * kPQ);
    const int neb = int((ss.dom_cap + kPE - 1) / kPE);
    const int64_t groups = int64_t(cache.batch) * nqs;
    const int64_t blocks = 8 * int64_t(neb) * ((groups + 7) / 8);
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    return launch_kernel(CSA2_KERNEL_SCAN_PREFILL, scan_prefill_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream,
                         cache.ratio, cache.capacity, static_cast<const uint16_t*>(idx_q), head_w, q_pos, n_q,
                         static_cast<const uint8_t*>(cache.idx_k), cache.n_entries, ss.scores, ss.bmax, ss.sbmax,
                         ss.dom_cap, nqs, neb, int(groups));
  }
  if (mfma_shape) {
    const int64_t nsb = ss.dom_cap / 64;
    if (nsb > (int64_t(1) << 24) || cache.capacity > (int64_t(1) << 24)) return hipErrorInvalidConfiguration;  // 32-bit slots
    const bool fp4 = cache.kv_dtype == CSA2_FP4;
    if (ss.fuse) {  // one query per sequence, flat domain (checked by the caller)
      if (pool_in || n_q != 1) return hipErrorInvalidValue;
      // the entry's workspace, then the LDS copy of its indexer row
      const size_t lds = sizeof(double) * size_t(compress_lds_doubles(dims.d, dims.d_idx)) + 2 * size_t(dims.d_idx);
      if (lds > 64 * 1024) return hipErrorInvalidConfiguration;
      const int sbw = fp4 ? kFusedSbFp4 : kFusedSbBf16;
      const int64_t nx = (nsb + 4 * sbw - 1) / (4 * sbw);
      if ((nx + 1) * cache.batch > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
      const dim3 grid(unsigned((nx + 1) * cache.batch), 1, 1);
      return launch_kernel(fp4 ? CSA2_KERNEL_SCAN_FP4_FUSED : CSA2_KERNEL_SCAN_BF16_FUSED,
                           fp4 ? scan_fused_fp4_kernel : scan_fused_bf16_kernel, grid, dim3(256), lds, stream,
                           cache.ratio, cache.capacity, static_cast<const uint16_t*>(idx_q), head_w, q_pos, n_q,
                           pool_in, dims.cand_blocks, static_cast<const uint8_t*>(cache.idx_k), cache.idx_scale,
                           cache.n_entries, ss.scores, ss.bmax, ss.sbmax, ss.dom_cap, *ss.fuse);
    }
    // Few rows (a decode step's pool-domain Reindex scan: 16384 slots per
    // query, 16 workgroups each) leave most compute units idle and each
    // workgroup's chain of loads sets the time: smaller blocks, so that the
    // workgroups at least cover the compute units (4 x 256K Reindex scans
    // 11.2 / 8.8 -> 5.9 / 4.5 us with 1 super-block per wave); with many
    // rows (replay segments, prefill chunks) smaller blocks cost more than
    // they spread (a 128-query replay segment's scans 53-62 -> 71-80 us).
    int cus = 0;
    const hipError_t ce = compute_units(&cus);
    if (ce != hipSuccess) return ce;
    const int64_t wgs = (nsb + 4 * kSbPerWave - 1) / (4 * kSbPerWave) * n_q * cache.batch;
    const int sbw = wgs >= cus ? kSbPerWave : (2 * wgs >= cus ? 2 : 1);
    auto kern = fp4 ? (pool_in ? scan_kernel_for<true, true>(sbw) : scan_kernel_for<true, false>(sbw))
                    : (pool_in ? scan_kernel_for<false, true>(sbw) : scan_kernel_for<false, false>(sbw));
    const dim3 grid(unsigned((nsb + 4 * sbw - 1) / (4 * sbw)), n_q, cache.batch);
    const hipError_t err = launch_kernel(cache.kv_dtype == CSA2_FP4 ? CSA2_KERNEL_SCAN_FP4 : CSA2_KERNEL_SCAN_BF16, kern, grid, dim3(256), 0, stream, cache.ratio, cache.capacity,
                       static_cast<const uint16_t*>(idx_q), head_w, q_pos, n_q, pool_in, dims.cand_blocks,
                       static_cast<const uint8_t*>(cache.idx_k), cache.idx_scale, cache.n_entries, ss.scores, ss.bmax,
                       ss.sbmax, ss.dom_cap);
    return err;
  }
  const dim3 grid(unsigned(ss.dom_cap / kThreads), n_q, cache.batch);
  const size_t lds = sizeof(float) * size_t(dims.n_idx_heads * dims.d_idx + dims.n_idx_heads + kThreads);
  const hipError_t err = launch_kernel(CSA2_KERNEL_SCAN_GENERIC, scan_generic_kernel, grid, dim3(kThreads), lds, stream, dims.n_idx_heads, dims.d_idx,
                     int(dims.act_dtype == CSA2_BF16), cache.kv_dtype, cache.idx_group, cache.ratio, cache.capacity,
                     idx_q, head_w, q_pos, n_q, pool_in, dims.cand_blocks, cache.idx_k, cache.idx_scale,
                     cache.n_entries, ss.scores, ss.bmax, ss.sbmax, ss.dom_cap);
  return err;
}

}  // namespace csa2
