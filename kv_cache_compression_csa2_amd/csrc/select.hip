// Top-k and HSI pool selection over the scan's scores, block maxima and
// super-block maxima.
//
// Pages: zartbot walkthrough (hn.213312.xyz) section 1.2 (index_topk 512,
// candidate_topk_blocks 2048, candidate_block_size 8) and section 2.3.4 (the
// Full layer keeps its own top-k from its full scores; the pool is the best
// 2048 blocks by block maximum, the newest visible block forced in, expanded
// into a fixed-size pool; the pool is the prior stage of a two-level search).
//
// Exact hierarchical selection.  Order candidates by (score desc, id asc).
// Claim: the best m items all lie inside the best m groups, groups ranked by
// (group max desc, group id asc), when groups are aligned runs of ids.  If an
// item x of group G is among the best m but G is not among the best m groups,
// each of the m groups ranked above G holds its own maximum item, and that
// item ranks above x (higher score, or equal score and lower id because the
// whole group lies below G) - m items above x, a contradiction.  So the top-k
// entries are found by: top-k super-blocks (64 slots) -> top-k blocks (8
// slots) inside them -> top-k slots inside those blocks.  The pool is found
// the same way with the forced block and its super-block given a key above
// every score (the argument then runs over the remaining kappa-1 places).
//
// Each level is a radix select over at most 16384 keys held in LDS: three
// histogram passes (11, 11, 10 bits of the order-preserving key) find the
// threshold key and how many ties to keep; after the first pass only the keys
// of the threshold bin are revisited (gathered into a short list when they
// fit); one wave scans each histogram; ties go to the lowest positions; an
// order-preserving compaction (wave ballots + a scan over waves) emits the
// chosen positions ascending.  One 1024-thread workgroup per (sequence, query).
#include "device_common.hpp"
#include "launch.hpp"

namespace csa2 {
namespace {

constexpr int kNT = 1024;
constexpr int kNW = kNT / kWave;
constexpr int kMaxCand = 16384;
constexpr int kMaxList = 2048;
// Histogram bin b lives at word b + b/32: the single wave that scans the bins
// reads 32 consecutive bins per lane, and the pad puts the lanes on distinct
// LDS banks.
constexpr int kHistWords = 2048 + 2048 / 32;
__device__ __forceinline__ int hbin(int b) { return b + (b >> 5); }

struct SelLds {
  uint32_t* keys;  // [kMaxCand]
  uint32_t* la;    // [kMaxList]
  uint32_t* lb;    // [kMaxList]
  uint32_t* cand;  // [kMaxList] keys sharing the threshold prefix (unordered)
  uint32_t* hist;  // [kHistWords] padded bins (see hbin), all zero between passes
  uint32_t* wsum;  // [2 * kNW]
  uint32_t* misc;  // [8]
};

__device__ __forceinline__ uint64_t lanemask_lt() { return (uint64_t(1) << (threadIdx.x & 63)) - 1; }

// Wave 0 only: find the bin holding the need-th largest key among nb bins of
// hist (digits compared from the top), write {bin, need left inside it,
// total count, bin count} to misc[0..3], and clear the bins.
__device__ __forceinline__ void find_digit(const SelLds& L, int nb, uint32_t need) {
  const int lane = threadIdx.x & 63;
  const int per = nb / kWave;
  uint32_t s = 0;
  for (int x = 0; x < per; ++x) s += L.hist[hbin(lane * per + x)];
  const uint32_t incl = wave_inclusive_scan(s);
  const uint32_t total = __shfl(incl, kWave - 1, kWave);
  uint32_t above = total - incl;  // keys in the bins of higher lanes
  if (above < need && need <= above + s) {
    for (int x = per - 1; x >= 0; --x) {
      const int bin = lane * per + x;
      const uint32_t h = L.hist[hbin(bin)];
      if (above < need && need <= above + h) {
        L.misc[0] = uint32_t(bin);
        L.misc[1] = need - above;
        L.misc[3] = h;
      }
      above += h;
    }
  }
  if (lane == 0) {
    L.misc[2] = total;
    L.misc[4] = 0;  // candidate-list fill counter
  }
  for (int x = 0; x < per; ++x) L.hist[hbin(lane * per + x)] = 0;
}

// Select the best min(m, #valid) of keys[0..n) (valid: key > kKeyNegInf),
// ties to the lower position; write the chosen positions ascending to out[].
// Returns the number chosen.  All threads of the block must call it; hist
// must be zero on entry and is zero on exit.
__device__ int select_top(const SelLds& L, int n, int m, uint32_t* out) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int seg = (((n + kNW - 1) / kNW) + 63) & ~63;
  const int lo = w * seg, hi = min(n, lo + seg);

  // pass 1 over every key: top 11 bits
  for (int p = lo + lane; p < hi; p += kWave) {
    const uint32_t k = L.keys[p];
    if (k > kKeyNegInf) atomicAdd(&L.hist[hbin(int(k >> 21))], 1u);
  }
  __syncthreads();
  if (w == 0) find_digit(L, 2048, uint32_t(m));
  __syncthreads();
  const uint32_t total = L.misc[2];
  uint32_t T = kKeyNegInf, need_eq = 0;
  if (total > uint32_t(m)) {
    uint32_t prefix = L.misc[0] << 21, mask = 0xFFE00000u, need = L.misc[1];
    const bool use_list = L.misc[3] <= uint32_t(kMaxList);
    if (use_list) {  // gather the keys of the threshold bin once; later passes read only them
      for (int p = lo + lane; p < hi; p += kWave) {
        const uint32_t k = L.keys[p];
        if (k > kKeyNegInf && (k & mask) == prefix) L.cand[atomicAdd(&L.misc[4], 1u)] = k;
      }
      __syncthreads();
    }
    const int nc = use_list ? int(L.misc[4]) : n;
    const int cseg = (((nc + kNW - 1) / kNW) + 63) & ~63;
    const int clo = w * cseg, chi = min(nc, clo + cseg);
    const int shifts[2] = {10, 0};
    const int bits[2] = {11, 10};
    for (int pass = 0; pass < 2; ++pass) {
      const int sh = shifts[pass];
      const uint32_t dmask = (1u << bits[pass]) - 1u;
      for (int p = clo + lane; p < chi; p += kWave) {
        const uint32_t k = use_list ? L.cand[p] : L.keys[p];
        if (k > kKeyNegInf && (k & mask) == prefix) atomicAdd(&L.hist[hbin(int((k >> sh) & dmask))], 1u);
      }
      __syncthreads();
      if (w == 0) find_digit(L, 1 << bits[pass], need);
      __syncthreads();
      prefix |= L.misc[0] << sh;
      mask |= dmask << sh;
      need = L.misc[1];
      __syncthreads();
    }
    T = prefix;
    need_eq = need;
  }

  // per-wave counts of keys above and equal to the threshold
  uint32_t gt = 0, eq = 0;
  for (int p = lo + lane; p < hi; p += kWave) {
    const uint32_t k = L.keys[p];
    gt += k > T;
    eq += (k == T) && (k > kKeyNegInf);
  }
  for (int off = 32; off > 0; off >>= 1) {
    gt += __shfl_xor(gt, off, kWave);
    eq += __shfl_xor(eq, off, kWave);
  }
  if (lane == 0) {
    L.wsum[w] = gt;
    L.wsum[kNW + w] = eq;
  }
  __syncthreads();
  uint32_t eq_base = 0, sel_base = 0, cum_eq = 0, chosen = 0;
  for (int x = 0; x < kNW; ++x) {
    if (x == w) {
      eq_base = cum_eq;
      sel_base = chosen;
    }
    const uint32_t e = L.wsum[kNW + x];
    const uint32_t take = need_eq > cum_eq ? min(e, need_eq - cum_eq) : 0u;
    chosen += L.wsum[x] + take;
    cum_eq += e;
  }
  // order-preserving compaction inside the wave's segment
  uint32_t run_eq = 0, run_sel = 0;
  for (int base = lo; base < lo + seg; base += kWave) {
    const int p = base + lane;
    const uint32_t k = p < hi ? L.keys[p] : 0u;
    const bool is_gt = k > T;
    const bool is_eq = (k == T) && (k > kKeyNegInf);
    const uint64_t eqm = __ballot(is_eq);
    const uint32_t eq_rank = eq_base + run_eq + __popcll(eqm & lanemask_lt());
    const bool sel = is_gt || (is_eq && eq_rank < need_eq);
    const uint64_t selm = __ballot(sel);
    if (sel) out[sel_base + run_sel + __popcll(selm & lanemask_lt())] = uint32_t(p);
    run_eq += __popcll(eqm);
    run_sel += __popcll(selm);
  }
  __syncthreads();
  return int(chosen);
}

__device__ __forceinline__ uint32_t key_at(const float* a, int64_t i) { return score_key(a[i]); }

__global__ __launch_bounds__(kNT) void select_kernel(int topk, int cand_blocks, int ratio, int64_t capacity,
                                                     const int32_t* __restrict__ q_pos, int n_q,
                                                     const int32_t* __restrict__ pool_in,
                                                     const int32_t* __restrict__ n_entries,
                                                     const float* __restrict__ scores, const float* __restrict__ bmax,
                                                     const float* __restrict__ sbmax, int64_t dom_cap,
                                                     int32_t* __restrict__ topk_out, int32_t* __restrict__ pool_out,
                                                     float* __restrict__ topk_scores) {
  extern __shared__ uint32_t lds[];
  SelLds L;
  L.keys = lds;
  L.la = L.keys + kMaxCand;
  L.lb = L.la + kMaxList;
  L.cand = L.lb + kMaxList;
  L.hist = L.cand + kMaxList;
  L.wsum = L.hist + kHistWords;
  L.misc = L.wsum + 2 * kNW;
  for (int x = threadIdx.x; x < kHistWords; x += kNT) L.hist[x] = 0;

  const int qi = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int64_t row = int64_t(b) * n_q + qi;
  const int64_t nsb = dom_cap / 64, nb = dom_cap / 8;
  const float* sc = scores + row * dom_cap;
  const float* bm = bmax + row * nb;
  const float* sbm = sbmax + row * nsb;

  // ---- HSI pool (full domain only) ----
  if (pool_out) {
    const int64_t n = clamp_entries(n_entries, b, capacity);
    const int64_t n_vis = visible_count(n, q_pos[row], ratio);
    const int64_t fb = n_vis > 0 ? (n_vis - 1) / 8 : -1;
    const int64_t fsb = fb >= 0 ? fb / 8 : -1;
    for (int64_t p = tid; p < nsb; p += kNT) L.keys[p] = p == fsb ? kKeyForced : key_at(sbm, p);
    __syncthreads();
    const int na = select_top(L, int(nsb), cand_blocks, L.la);
    for (int p = tid; p < 8 * na; p += kNT) {
      const int64_t blk = int64_t(L.la[p >> 3]) * 8 + (p & 7);
      L.keys[p] = blk == fb ? kKeyForced : key_at(bm, blk);
    }
    __syncthreads();
    const int nbsel = select_top(L, 8 * na, cand_blocks, L.lb);
    for (int x = tid; x < cand_blocks; x += kNT) {
      int32_t v = -1;
      if (x < nbsel) v = int32_t(int64_t(L.la[L.lb[x] >> 3]) * 8 + (L.lb[x] & 7));
      pool_out[row * cand_blocks + x] = v;
    }
    __syncthreads();
  }

  // ---- top-k entries ----
  for (int64_t p = tid; p < nsb; p += kNT) L.keys[p] = key_at(sbm, p);
  __syncthreads();
  const int na = select_top(L, int(nsb), topk, L.la);
  for (int p = tid; p < 8 * na; p += kNT) L.keys[p] = key_at(bm, int64_t(L.la[p >> 3]) * 8 + (p & 7));
  __syncthreads();
  const int nbsel = select_top(L, 8 * na, topk, L.lb);
  // block ids of the chosen blocks (ascending)
  for (int x = tid; x < nbsel; x += kNT) L.lb[x] = L.la[L.lb[x] >> 3] * 8 + (L.lb[x] & 7);
  __syncthreads();
  for (int p = tid; p < 8 * nbsel; p += kNT) L.keys[p] = key_at(sc, int64_t(L.lb[p >> 3]) * 8 + (p & 7));
  __syncthreads();
  const int ne = select_top(L, 8 * nbsel, topk, L.la);
  for (int x = tid; x < topk; x += kNT) {
    int32_t id = -1;
    float s = -INFINITY;
    if (x < ne) {
      const int64_t slot = int64_t(L.lb[L.la[x] >> 3]) * 8 + (L.la[x] & 7);
      s = sc[slot];
      id = pool_in ? int32_t(int64_t(pool_in[row * cand_blocks + slot / 8]) * 8 + (slot & 7)) : int32_t(slot);
    }
    topk_out[row * topk + x] = id;
    if (topk_scores) topk_scores[row * topk + x] = s;
  }
}

constexpr size_t kSelectLds = sizeof(uint32_t) * (kMaxCand + 3 * kMaxList + kHistWords + 2 * kNW + 8);

}  // namespace

hipError_t launch_select(const csa2_dims& dims, const csa2_kv_cache& cache, const int32_t* q_pos, int32_t n_q,
                         const int32_t* pool_in, const ScanScratch& ss, int32_t* topk_out, int32_t* pool_out,
                         float* topk_scores, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(select_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(kSelectLds));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(select_kernel, dim3(n_q, cache.batch), dim3(kNT), kSelectLds, stream, dims.topk,
                     dims.cand_blocks, cache.ratio, cache.capacity, q_pos, n_q, pool_in, cache.n_entries, ss.scores,
                     ss.bmax, ss.sbmax, ss.dom_cap, topk_out, pool_out, topk_scores);
  return hipGetLastError();
}

}  // namespace csa2
