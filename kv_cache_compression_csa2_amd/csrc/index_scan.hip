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


// ------------------------------------------------------------------ MFMA ---
//
// Production shape: 32 indexer heads x 128, bf16 queries, bf16 or FP4 (one
// E4M3 scale per 32 channels) indexer K.  The per-tile contraction
// S[head][entry] = Q[32 x 128] . K^T[128 x 32] runs as eight
// v_mfma_f32_32x32x16_bf16.  Operands come straight from memory in MFMA
// layout: lane l supplies row (l % 32) with eight consecutive k of its half
// (l / 32); the order in which k is visited is free, so it is chosen to make
// each lane's K bytes contiguous (bf16: one 128-byte run per lane) or to keep
// every step inside one FP4 scale group (FP4: the group scale is applied to
// the step-group's partial sum after the MFMA, because the hardware's scaled
// FP4 convert honours only the exponent of its scale).  Accumulator lane l
// register r holds head 8*(r/4) + 4*(l/32) + r%4 of entry l % 32; the head
// sum w_h * ReLU(.) runs in registers, then one cross-half shuffle completes
// the entry score.
//
// A workgroup (4 waves) covers 16 super-blocks of 64 domain slots; wave w
// takes super-blocks w, w+4, w+8, w+12, two 32-entry tiles each.

typedef __bf16 bf16x8_t __attribute__((__vector_size__(16)));
typedef __bf16 bf16x2_t __attribute__((__vector_size__(4)));
typedef float f32x16_t __attribute__((__vector_size__(64)));

constexpr int kSbPerWave = 4;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Eight E2M1 codes (one dword, low nibble first) -> eight exact bf16 values.
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16(uint32_t w) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
  uint4 v;
  v.x = __builtin_bit_cast(uint32_t, a);
  v.y = __builtin_bit_cast(uint32_t, b);
  v.z = __builtin_bit_cast(uint32_t, c);
  v.w = __builtin_bit_cast(uint32_t, d);
  return as_bf16x8(v);
}

template <bool FP4>
__device__ __forceinline__ void scan_mfma_body(
    int ratio, int64_t capacity, const uint16_t* __restrict__ idx_q, const float* __restrict__ head_w,
    const int32_t* __restrict__ q_pos, int n_q, const int32_t* __restrict__ pool_in, int cand_blocks,
    const uint8_t* __restrict__ idx_k, const uint8_t* __restrict__ idx_scale, const int32_t* __restrict__ n_entries,
    float* __restrict__ scores, float* __restrict__ bmax, float* __restrict__ sbmax, int64_t dom_cap) {
  constexpr int kBatch = FP4 ? 4 : 1;  // super-blocks whose loads are issued together
  constexpr int kTiles = 2 * kBatch;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int qi = blockIdx.y, b = blockIdx.z;
  const int64_t row = int64_t(b) * n_q + qi;
  const int64_t nsb = dom_cap / 64;
  const int64_t n_vis = visible_count(clamp_entries(n_entries, b, capacity), q_pos[row], ratio);

  // A operand (indexer query) and the lane's 16 head weights, held for the whole scan
  bf16x8_t qop[8];
  const uint16_t* qrow = idx_q + (row * 32 + n) * 128;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int k0 = FP4 ? 32 * (s >> 1) + 16 * h + 8 * (s & 1) : 64 * h + 8 * s;
    qop[s] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + k0));
  }
  float wreg[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) wreg[r] = head_w[row * 32 + 8 * (r >> 2) + 4 * h + (r & 3)];

  const int64_t sb0 = int64_t(blockIdx.x) * (4 * kSbPerWave) + wave;
  for (int it = 0; it < kSbPerWave; it += kBatch) {
    const int64_t sb_first = sb0 + 4 * it;
    if (sb_first >= nsb) break;
    const bool any_visible = pool_in || sb_first * 64 < n_vis;

    // ---- issue the loads of kTiles tiles ----
    int64_t slot[kTiles];
    bool valid[kTiles];
    uint4 kb[FP4 ? 1 : kTiles][8];
    uint2 kf[FP4 ? kTiles : 1][4];
    uint32_t ks[FP4 ? kTiles : 1];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      const int64_t sb = sb_first + 4 * (t >> 1);
      slot[t] = sb * 64 + 32 * (t & 1) + n;
      int64_t j = -1;
      if (sb < nsb && any_visible) {
        if (pool_in) {
          const int64_t blk = slot[t] / 8 < cand_blocks ? pool_in[row * cand_blocks + slot[t] / 8] : -1;
          if (blk >= 0) j = blk * 8 + (slot[t] & 7);
        } else {
          j = slot[t];
        }
      }
      valid[t] = j >= 0 && j < n_vis;
      const int64_t crow = int64_t(b) * capacity + (valid[t] ? j : 0);
      if (any_visible) {
        if (FP4) {
          const uint8_t* p = idx_k + crow * 64 + 8 * h;
#pragma unroll
          for (int g = 0; g < 4; ++g) kf[t][g] = *reinterpret_cast<const uint2*>(p + 16 * g);
          ks[t] = *reinterpret_cast<const uint32_t*>(idx_scale + crow * 4);
        } else {
          const uint4* p = reinterpret_cast<const uint4*>(idx_k + (crow * 128 + 64 * h) * 2);
#pragma unroll
          for (int s = 0; s < 8; ++s) kb[t][s] = p[s];
        }
      }
    }

    // ---- contract, reduce over heads, write scores and maxima ----
    float tmax[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      float part = 0.0f;
      if (any_visible) {
        if (FP4) {
          f32x16_t acc[4];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            acc[g] = f32x16_t{};
            acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qop[2 * g], fp4x8_to_bf16(kf[t][g].x), acc[g], 0, 0, 0);
            acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qop[2 * g + 1], fp4x8_to_bf16(kf[t][g].y), acc[g], 0, 0, 0);
          }
          const float s0 = e4m3_to_f32(ks[t] & 0xFF), s1 = e4m3_to_f32((ks[t] >> 8) & 0xFF);
          const float s2 = e4m3_to_f32((ks[t] >> 16) & 0xFF), s3 = e4m3_to_f32(ks[t] >> 24);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float dot = s0 * acc[0][r] + s1 * acc[1][r] + s2 * acc[2][r] + s3 * acc[3][r];
            part += wreg[r] * fmaxf(dot, 0.0f);
          }
        } else {
          f32x16_t acc = f32x16_t{};
#pragma unroll
          for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qop[s], as_bf16x8(kb[t][s]), acc, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 16; ++r) part += wreg[r] * fmaxf(acc[r], 0.0f);
        }
      }
      float sc = part + __shfl_xor(part, 32, kWave);
      if (!valid[t]) sc = -INFINITY;
      const int64_t sb = sb_first + 4 * (t >> 1);
      if (sb < nsb && h == 0) scores[row * dom_cap + slot[t]] = sc;
      float m = fmaxf(sc, __shfl_xor(sc, 1, kWave));
      m = fmaxf(m, __shfl_xor(m, 2, kWave));
      m = fmaxf(m, __shfl_xor(m, 4, kWave));
      if (sb < nsb && h == 0 && (n & 7) == 0) bmax[row * (dom_cap / 8) + slot[t] / 8] = m;
      m = fmaxf(m, __shfl_xor(m, 8, kWave));
      m = fmaxf(m, __shfl_xor(m, 16, kWave));
      tmax[t] = m;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t sb = sb_first + 4 * u;
      if (sb < nsb && lane == 0) sbmax[row * nsb + sb] = fmaxf(tmax[2 * u], tmax[2 * u + 1]);
    }
  }
}

// bf16 keeps one tile pair in flight per wave and fits 3 waves per SIMD;
// FP4 keeps four pairs in flight (its rows are a quarter the size) at 2.
__global__ __launch_bounds__(256, 3) void scan_mfma_bf16_kernel(
    int ratio, int64_t capacity, const uint16_t* __restrict__ idx_q, const float* __restrict__ head_w,
    const int32_t* __restrict__ q_pos, int n_q, const int32_t* __restrict__ pool_in, int cand_blocks,
    const uint8_t* __restrict__ idx_k, const uint8_t* __restrict__ idx_scale, const int32_t* __restrict__ n_entries,
    float* __restrict__ scores, float* __restrict__ bmax, float* __restrict__ sbmax, int64_t dom_cap) {
  scan_mfma_body<false>(ratio, capacity, idx_q, head_w, q_pos, n_q, pool_in, cand_blocks, idx_k, idx_scale, n_entries,
                        scores, bmax, sbmax, dom_cap);
}

__global__ __launch_bounds__(256, 2) void scan_mfma_fp4_kernel(
    int ratio, int64_t capacity, const uint16_t* __restrict__ idx_q, const float* __restrict__ head_w,
    const int32_t* __restrict__ q_pos, int n_q, const int32_t* __restrict__ pool_in, int cand_blocks,
    const uint8_t* __restrict__ idx_k, const uint8_t* __restrict__ idx_scale, const int32_t* __restrict__ n_entries,
    float* __restrict__ scores, float* __restrict__ bmax, float* __restrict__ sbmax, int64_t dom_cap) {
  scan_mfma_body<true>(ratio, capacity, idx_q, head_w, q_pos, n_q, pool_in, cand_blocks, idx_k, idx_scale, n_entries,
                       scores, bmax, sbmax, dom_cap);
}

// ------------------------------------------------------- query-blocked scan --
//
// Many queries per sequence (chunked prefill): the score contraction is a
// GEMM per head, S_h = Q_h . K^T, whose K operand is shared by all 32 heads.
// A workgroup (4 waves) owns 32 queries of one sequence and 512 entries; wave
// w owns entries [128w, 128w+128).  Each wave loads its entries' indexer K
// once, in registers, as the A operand of v_mfma_f32_32x32x16_bf16 (lane =
// entry, 8 channels per lane and k-step; 4 blocks of 32 entries x 8 k-steps),
// so the products are logits^T[entry][query]: a lane then holds one query and
// runs of 4 consecutive entries, which makes the head weight one value per
// lane, the score stores 16 bytes wide and a block maximum one exchange.
// The heads then stream through LDS two at a time: the 32 queries' rows of
// heads 2p and 2p+1 (2 x 8 KB) are copied global -> LDS (global_load_lds_dwordx4,
// from inline assembly so the compiler does not drain them before LDS reads)
// one pair ahead into a double buffer, and every wave contracts each head
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
constexpr int kPE = 512;              // entries per workgroup
constexpr int kQTile = kPQ * 256;     // one head's query rows (bytes)

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

__global__ __launch_bounds__(256, 1) void scan_prefill_kernel(
    int ratio, int64_t capacity, const uint16_t* __restrict__ idx_q, const float* __restrict__ head_w,
    const int32_t* __restrict__ q_pos, int n_q, const uint8_t* __restrict__ idx_k,
    const int32_t* __restrict__ n_entries, float* __restrict__ scores, float* __restrict__ bmax,
    float* __restrict__ sbmax, int64_t dom_cap, int nqs, int neb, int groups) {
  __shared__ __align__(16) uint8_t qtile[4][kQTile];  // 2 stages x 2 heads
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
  const int64_t e_wg = int64_t(eb) * kPE, e0 = e_wg + 128 * wave;
  const int64_t n_ent = clamp_entries(n_entries, b, capacity);

  // ---- issue first, independent of the bookkeeping below: this wave's
  // entries' indexer K (the A operand, resident for all heads) and the query
  // tiles of heads 0 and 1 ----
  uint4 kreg[4][8];
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    int64_t e = e0 + 32 * blk + n;
    e = e < capacity ? e : capacity - 1;  // slots past the cache: any valid row (masked below)
    const uint4* p = reinterpret_cast<const uint4*>(idx_k + ((int64_t(b) * capacity + e) * 128 + 8 * hl) * 2);
#pragma unroll
    for (int s = 0; s < 8; ++s) kreg[blk][s] = p[2 * s];  // channels 16s + 8hl .. +8
  }
  // copies of the query tiles of heads 2p and 2p+1 into stage p & 1: 16
  // instructions of 1 KB (4 query rows each); wave w issues 4 of them
  auto issue_pair = [&](int p, int q0) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(
        uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void*)qtile[2 * (p & 1)])));
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4) {
      const int m = 4 * wave + m4;          // 0..15: head 2p + m / 8, instruction m % 8
      const int hh = 2 * p + (m >> 3);
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
    __syncthreads();
    const int64_t vmax = vis_max;
    const bool wave_live = e0 < vmax;  // some query sees some entry of this wave's range

    f32x16_t_ sacc[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) sacc[blk] = f32x16_t_{};

    if (e_wg < vmax) {
      // logits of head hh from tile `qt` into acc
      auto contract = [&](const uint8_t* qt, f32x16_t_* acc) {
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) acc[blk] = f32x16_t_{};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(qt + 16 * qslot(n, 2 * s + hl));
#pragma unroll
          for (int blk = 0; blk < 4; ++blk)
            acc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kreg[blk][s]), a, acc[blk], 0, 0, 0);
        }
      };
      // scores += w_hh * max(0, logit); max(0, x) as an integer max on the bits
      auto fold = [&](int hh, const f32x16_t_* acc) {
        const float w = wl[hh][n];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sacc[blk][r] += w * __int_as_float(max(__float_as_int(acc[blk][r]), 0));
      };
      f32x16_t_ acc_a[4], acc_b[4];
      for (int p = 0; p < 16; ++p) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's copies of heads 2p, 2p+1
        __syncthreads();  // every wave's copies landed; the other stage is free
        if (p + 1 < 16) issue_pair(p + 1, q0);
        if (!wave_live) continue;
        const uint8_t* qt = qtile[2 * (p & 1)];
        contract(qt, acc_a);                       // head 2p
        if (p > 0) fold(2 * p - 1, acc_b);         // head 2p-1, under head 2p's products
        contract(qt + kQTile, acc_b);              // head 2p+1
        fold(2 * p, acc_a);                        // head 2p, under head 2p+1's products
      }
      if (wave_live) fold(31, acc_b);
    }

    // ---- mask, store scores and maxima ----
    // lane: query n, entries e0 + 32 blk + 8j + 4hl + i (i < 4) in sacc[blk][4j + i]
    if (e0 >= dom_cap) continue;  // uniform per wave
    const int q = q0 + n;
    const int64_t row = int64_t(b) * n_q + q;
    const int64_t vis = nvis[n];
    const int64_t nsb = dom_cap / 64;
    float m_sb[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
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
    for (int p2 = 0; p2 < 2; ++p2) {
      const int64_t sb = (e0 + 64 * p2) / 64;
      if (q < n_q && hl == 0 && sb < nsb) sbmax[row * nsb + sb] = m_sb[p2];
    }
  }
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
    const dim3 grid(unsigned((nsb + 4 * kSbPerWave - 1) / (4 * kSbPerWave)), n_q, cache.batch);
    auto kern = cache.kv_dtype == CSA2_FP4 ? scan_mfma_fp4_kernel : scan_mfma_bf16_kernel;
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
