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
// A level whose candidates number at most m keeps them all and is skipped.
//
// Each level selects among at most 16384 keys (see select_top).  The step is
// latency-bound (one workgroup per query), so the work of every level is
// spread over 16 waves with short rolled loops, wave reductions and scans run
// on DPP, and LDS is addressed through address-space-3 pointers so every
// access is a ds_* instruction.
#include <algorithm>

#include "device_common.hpp"
#include "launch.hpp"

extern "C" __device__ uint32_t __ockl_wfscan_add_u32(uint32_t, bool);
extern "C" __device__ uint32_t __ockl_wfred_add_u32(uint32_t);
extern "C" __device__ uint32_t __ockl_wfred_min_u32(uint32_t);
extern "C" __device__ uint32_t __ockl_wfred_max_u32(uint32_t);

namespace csa2 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int kNT = 1024;
constexpr int kNW = kNT / kWave;
constexpr int kMaxCand = 16384;
constexpr int kSmallCand = 4096;  // LDS key capacity of the 64-register variant
constexpr int kMaxList = 2048;
constexpr int kBins = 2048;
constexpr int kBinsPerWave = kBins / kNW;  // 128: two per lane

struct SelLds {
  lds_u32* keys;  // [kMaxCand] candidate keys by position
  lds_u32* la;    // [kMaxList]
  lds_u32* lb;    // [kMaxList]
  lds_u32* hist;  // [4 * kBins]: four copies, or one histogram of 4 kBins bins; all zero between passes
  lds_u32* wred;  // [4 * kNW] per-wave partial results
  lds_u32* misc;  // [8]
};

// Reduce the kNW per-wave values wred[base .. base+kNW) with lanes < kNW of
// the calling wave; op 0 = sum, 1 = min, 2 = max.
__device__ __forceinline__ uint32_t reduce_waves(const SelLds L, int base, int op) {
  const int lane = threadIdx.x & 63;
  const uint32_t ident = op == 1 ? 0xFFFFFFFFu : 0u;
  const uint32_t v = lane < kNW ? L.wred[base + lane] : ident;
  return op == 0 ? __ockl_wfred_add_u32(v) : (op == 1 ? __ockl_wfred_min_u32(v) : __ockl_wfred_max_u32(v));
}

// Exclusive prefix over waves of the kNW values wred[base ..]: the sum of the
// values of the waves before wave w.
__device__ __forceinline__ uint32_t waves_before(const SelLds L, int base, int w) {
  const int lane = threadIdx.x & 63;
  const uint32_t v = lane < kNW ? L.wred[base + lane] : 0u;
  const uint32_t incl = __ockl_wfscan_add_u32(v, true);
  return w == 0 ? 0u : uint32_t(__builtin_amdgcn_readlane(int(incl), w - 1));
}

// Select the best min(m, #valid) of keys[0..n) (valid: key > kKeyNegInf),
// ties to the lower position; write the chosen positions ascending to out[].
// Returns the number chosen.  All threads of the block must call it, after a
// barrier that follows the put_stats() of the keys' writer; the histograms
// are zero on entry and on exit.
//
// Thread t owns the run of R consecutive positions [R t, R t + R) (R a
// multiple of 4, at most KR = the LDS key capacity / 1024), read 16 bytes at
// a time into registers once: every pass and both compaction steps then work
// on registers (re-reading them from LDS made each step wait for an LDS round
// trip per 4 keys, which measured ~1.5 us per pass on 16384 keys).  Positions
// at or past n hold the invalid key, so the loops run over all KR registers
// without bounds tests.  The threshold key T
// is found by narrowing a key interval [lo, hi] that holds it: each pass
// splits the interval into at most 2048 equal bins (8192 for 2049..4096 keys
// of which at most a quarter are selected), and the interval shrinks
// to the bin that holds the need-th largest key; when that bin is taken
// whole the search stops early.  Starting from the observed [min, max] of the
// keys spreads similar scores over many bins, and four copies of the
// histogram (by wave) cut the LDS atomic collisions of clustered keys; three
// passes always suffice for 32-bit keys.  The compaction is one block-wide
// scan of packed (greater, equal) counts, then a short walk per thread.
// The count chosen and t, a key at most the m-th largest (kKeyNegInf when
// every valid key was chosen): the next level's lower bound.
struct SelResult {
  int n;
  uint32_t t;
};

// `bound`: a key known to be at most the m-th largest (kKeyNegInf: none).
// The histogram passes start from the interval [max(bound, min), max]
// instead of [min, max]; keys below it are never chosen.
template <bool FINE, int KR>
__device__ SelResult select_top_impl(const SelLds L, int n, int m, lds_u32* out, uint32_t bound) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int R = ((((n + kNT - 1) / kNT) + 3) & ~3);
  const int p0 = R * tid;
  uint32_t kr[KR];
#pragma unroll
  for (int v = 0; v < KR; v += 4) {
    // p0 + v < n <= capacity and both are multiples of 4: the 16 bytes lie inside keys[]
    const u32x4 k4 = (v < R && p0 + v < n) ? *reinterpret_cast<const lds_u32x4*>(L.keys + p0 + v)
                                           : u32x4{kKeyNegInf, kKeyNegInf, kKeyNegInf, kKeyNegInf};
    const uint32_t kk[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) kr[v + i] = (v < R && p0 + v + i < n) ? kk[i] : kKeyNegInf;
  }
  constexpr int bin_bits = FINE ? 13 : 11;
  lds_u32* const hist = FINE ? L.hist : L.hist + kBins * (w & 3);

  const uint32_t total = reduce_waves(L, 0, 0);
  uint32_t lo = max(reduce_waves(L, kNW, 1), bound), hi = reduce_waves(L, 2 * kNW, 2);
  // wred is next written by the compaction, or by a pass after its histogram
  // barrier: only the first case needs a barrier here (total is uniform)
  if (total <= uint32_t(m)) __syncthreads();

  uint32_t T = kKeyNegInf, need = 0;
  if (total > uint32_t(m)) {
    need = uint32_t(m);
    // the found bin goes to misc[0..2] on even passes and misc[4..6] on odd
    // ones, so no barrier is needed between reading it and the next pass
    // (a slot is rewritten two passes later, after two more barriers)
    for (int pass = 0;; ++pass) {
      lds_u32* const found = L.misc + 4 * (pass & 1);
      const uint64_t width = uint64_t(hi) - lo + 1;
      const int bits = 64 - __clzll(width - 1);  // bits spanned by the interval
      const int shift = bits > bin_bits ? bits - bin_bits : 0;
#pragma unroll
      for (int i = 0; i < KR; ++i) {
        const uint32_t k = kr[i];
        if (k > kKeyNegInf && k >= lo && k <= hi) lds_inc(&hist[(k - lo) >> shift]);
      }
      __syncthreads();
      // lane `lane` of wave w holds nb consecutive bins from b0 (fine: 8 of
      // one histogram; else 2, four copies summed), read and zeroed
      constexpr int nb = FINE ? 8 : 2;
      const int b0 = FINE ? 8 * (64 * w + lane) : kBinsPerWave * w + 2 * lane;
      uint32_t hb[nb];
      if constexpr (FINE) {
        lds_u32x4* hp = reinterpret_cast<lds_u32x4*>(L.hist + b0);
        const u32x4 a = hp[0], c = hp[1];
        hp[0] = u32x4{0u, 0u, 0u, 0u};
        hp[1] = u32x4{0u, 0u, 0u, 0u};
        hb[0] = a.x; hb[1] = a.y; hb[2] = a.z; hb[3] = a.w;
        hb[4] = c.x; hb[5] = c.y; hb[6] = c.z; hb[7] = c.w;
      } else {
        hb[0] = hb[1] = 0u;
#pragma unroll
        for (int cp = 0; cp < 4; ++cp) {
          hb[0] += L.hist[kBins * cp + b0];
          hb[1] += L.hist[kBins * cp + b0 + 1];
          L.hist[kBins * cp + b0] = 0;
          L.hist[kBins * cp + b0 + 1] = 0;
        }
      }
      uint32_t s = 0;
#pragma unroll
      for (int i = 0; i < nb; ++i) s += hb[i];
      const uint32_t incl = __ockl_wfscan_add_u32(s, true);
      const uint32_t wtot = uint32_t(__builtin_amdgcn_readlane(int(incl), kWave - 1));
      if (lane == 0) L.wred[w] = wtot;
      __syncthreads();
      // keys in the bins of higher waves, then of higher lanes of this wave
      const uint32_t v = lane < kNW ? L.wred[kNW - 1 - lane] : 0u;  // from the top wave down
      const uint32_t incl_rev = __ockl_wfscan_add_u32(v, true);
      const uint32_t above_w = w == kNW - 1 ? 0u : uint32_t(__builtin_amdgcn_readlane(int(incl_rev), kNW - 2 - w));
      uint32_t above = above_w + (wtot - incl);
      if (above < need && need <= above + s) {  // this lane holds the bin: walk its bins from the top
#pragma unroll
        for (int i = nb - 1; i >= 0; --i) {
          if (need > above && need <= above + hb[i]) {
            found[0] = uint32_t(b0 + i);
            found[1] = need - above;
            found[2] = hb[i];
          }
          above += hb[i];
        }
      }
      __syncthreads();
      const uint32_t bin = found[0], in_bin = found[2];
      need = found[1];
      const uint64_t new_lo = uint64_t(lo) + (uint64_t(bin) << shift);
      hi = uint32_t(min(uint64_t(hi), new_lo + (uint64_t(1) << shift) - 1));
      lo = uint32_t(new_lo);
      if (need == in_bin) {  // the whole bin is taken: every key >= lo, no ties to break
        T = lo - 1;          // lo > kKeyNegInf, so T >= kKeyNegInf
        need = 0;
        break;
      }
      if (shift == 0) {  // a single key value: the threshold
        T = lo;
        break;
      }
    }
  }

  // order-preserving compaction: (greater, equal) counts packed 16:16, one block scan
  uint32_t gt = 0, eq = 0;  // T >= kKeyNegInf, so k > T implies a valid key
#pragma unroll
  for (int i = 0; i < KR; ++i) {
    gt += kr[i] > T;
    eq += kr[i] == T && kr[i] > kKeyNegInf;
  }
  const uint32_t packed = (gt << 16) | eq;
  const uint32_t incl = __ockl_wfscan_add_u32(packed, true);
  if (lane == kWave - 1) L.wred[w] = incl;
  __syncthreads();
  const uint32_t wv = lane < kNW ? L.wred[lane] : 0u;
  const uint32_t wincl = __ockl_wfscan_add_u32(wv, true);
  const uint32_t before_w = w == 0 ? 0u : uint32_t(__builtin_amdgcn_readlane(int(wincl), w - 1));
  const uint32_t all = uint32_t(__builtin_amdgcn_readlane(int(wincl), kNW - 1));
  const uint32_t before = before_w + incl - packed;
  uint32_t gt_run = before >> 16, eq_run = before & 0xFFFFu;
  const uint32_t chosen = (all >> 16) + min(all & 0xFFFFu, need);
#pragma unroll
  for (int i = 0; i < KR; ++i) {
    const uint32_t k = kr[i];
    const bool g = k > T, e = k == T && k > kKeyNegInf;
    // a greater key goes after the equal keys taken so far, an equal key
    // is taken while fewer than `need` equal keys precede it
    if (g || (e && eq_run < need)) out[gt_run + min(eq_run, need)] = uint32_t(p0 + i);
    gt_run += g;
    eq_run += e;
  }
  __syncthreads();
  return SelResult{int(chosen), T};
}

// 2049..4096 keys with at most a quarter selected: one histogram of
// 4 kBins fine bins (few keys per bin in the upper tail, so the first pass
// usually ends on a bin taken whole).  Otherwise four copies (by wave) of
// kBins bins, which cut the atomic collisions of clustered keys; fine bins
// measured slower there (a threshold in the dense middle, or 2048 clustered
// pool maxima, still needs a second pass).
// The register count follows the level's size (4, 8 or 16 keys per thread):
// a loop over 16 registers holding 4 keys would do 4x the work per pass.
__device__ __attribute__((noinline)) SelResult select_top(const SelLds L, int n, int m, lds_u32* out, uint32_t bound) {
  if (n > 2048 && n <= 4096 && 4 * m <= n) return select_top_impl<true, 4>(L, n, m, out, bound);
  if (n <= 4 * kNT) return select_top_impl<false, 4>(L, n, m, out, bound);
  if (n <= 8 * kNT) return select_top_impl<false, 8>(L, n, m, out, bound);
  return select_top_impl<false, kMaxCand / kNT>(L, n, m, out, bound);
}
// The same, inlined: the 64-register variant of the kernel must not call a
// function that allocates beyond that (the full variant keeps the call, whose
// code measured ~2 us faster per pool selection)
__device__ __forceinline__ SelResult select_top_inl(const SelLds L, int n, int m, lds_u32* out, uint32_t bound) {
  if (n > 2048 && n <= 4096 && 4 * m <= n) return select_top_impl<true, kSmallCand / kNT>(L, n, m, out, bound);
  return select_top_impl<false, kSmallCand / kNT>(L, n, m, out, bound);
}

// Key of a[i]; an index outside [0, n) (never produced by a correct
// selection) reads nothing and counts as an invalid slot.
__device__ __forceinline__ uint32_t key_in(const float* a, int64_t i, int64_t n) {
  return (i >= 0 && i < n) ? score_key(a[i]) : kKeyNegInf;
}

// Count, min and max of the valid keys a thread wrote, summed over the block
// into wred (per wave; select_top reduces the waves after the barrier).
__device__ __forceinline__ void put_stats(const SelLds L, uint32_t cnt, uint32_t kmn, uint32_t kmx) {
  cnt = __ockl_wfred_add_u32(cnt);
  kmn = __ockl_wfred_min_u32(kmn);
  kmx = __ockl_wfred_max_u32(kmx);
  if ((threadIdx.x & 63) == 0) {
    const int w = threadIdx.x >> 6;
    L.wred[w] = cnt;
    L.wred[kNW + w] = kmn;
    L.wred[2 * kNW + w] = kmx;
  }
}

__device__ __forceinline__ void note_key(uint32_t k, uint32_t& cnt, uint32_t& kmn, uint32_t& kmx) {
  if (k > kKeyNegInf) {
    ++cnt;
    kmn = min(kmn, k);
    kmx = max(kmx, k);
  }
}

// keys[p] = key of src[idx(p)] for p in [0, cnt): kKeyForced where idx(p) is
// `forced`, kKeyNegInf where idx(p) lies outside [0, n), and at least
// fix_key where idx(p) is fix_at (a score the scan left out: see ScanFuse);
// then put_stats.  Every level gathers aligned runs: idx(p) = p, or
// idx(p) = 8 g(p / 8) + p % 8, and cnt and n are multiples of 4 - so four
// consecutive keys come from four consecutive, 16-byte aligned values, read
// with one 16-byte load.  Each thread issues kPer such loads (at clamped,
// always valid addresses) before it uses any, so a level's loads are in
// flight together (4-byte loads took two dependent batches: 2.6 us for the
// 4096 block maxima of a 32K decode row).  n >= 4.
template <int kPer = 4, class IdxFn>
__device__ __forceinline__ void gather_keys(const SelLds L, int cnt, const float* __restrict__ src, int n, int forced,
                                            int fix_at, uint32_t fix_key, IdxFn idx) {
  uint32_t c = 0, kmn = 0xFFFFFFFFu, kmx = 0u;
  const int quads = cnt >> 2;
  for (int base = 0; base < quads; base += kPer * kNT) {
    int id0[kPer];
    float4 v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = base + i * kNT + int(threadIdx.x);
      id0[i] = q < quads ? idx(4 * q) : -1;
      v[i] = *reinterpret_cast<const float4*>(src + min(max(id0[i], 0), n - 4));
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = base + i * kNT + int(threadIdx.x);
      if (q < quads) {
        const float vv[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        uint32_t k4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int id = id0[i] + e;
          uint32_t k = id == forced ? kKeyForced : ((id >= 0 && id < n) ? score_key(vv[e]) : kKeyNegInf);
          if (id == fix_at) k = max(k, fix_key);
          k4[e] = k;
          note_key(k, c, kmn, kmx);
        }
        *reinterpret_cast<lds_u32x4*>(L.keys + 4 * q) = u32x4{k4[0], k4[1], k4[2], k4[3]};
      }
    }
  }
  put_stats(L, c, kmn, kmx);
}

// KCAND: LDS key capacity of a level.  The full capacity (16384) leaves one
// workgroup per compute unit; shapes whose levels gather at most 4096 keys
// take a 66 KB variant bounded to 64 registers with its selections inlined,
// so two workgroups share a compute unit when many queries (chunked prefill)
// keep the chip busy, and a decode row's selections run without calls
// (32K decode select 14.5 -> 13.4 us).
template <int KCAND>
__device__ __forceinline__ void select_body(int topk, int cand_blocks, int ratio, int64_t capacity,
                                                     const int32_t* __restrict__ q_pos, int n_q,
                                                     const int32_t* __restrict__ pool_in,
                                                     const int32_t* __restrict__ n_entries,
                                                     const float* __restrict__ scores, const float* __restrict__ bmax,
                                                     const float* __restrict__ sbmax, int64_t dom_cap,
                                                     int32_t* __restrict__ topk_out, int32_t* __restrict__ pool_out,
                                                     float* __restrict__ topk_scores, int split,
                                                     const float* __restrict__ fix_score,
                                                     const int32_t* __restrict__ fix_id) {
  extern __shared__ uint32_t lds_raw[];
  lds_u32* lds = (lds_u32*)lds_raw;  // address-space cast into LDS
  constexpr int kGather = KCAND <= 4096 ? 1 : 4;  // 16-byte loads in flight per thread in a gather
  SelLds L;
  L.keys = lds;
  L.la = L.keys + KCAND;
  L.lb = L.la + kMaxList;
  L.hist = L.lb + kMaxList;
  L.wred = L.hist + 4 * kBins;
  L.misc = L.wred + 4 * kNW;
  // Each level's threshold bounds the next level's from below: each of the
  // m super-blocks (blocks) chosen holds a block (entry) whose key is its
  // own, at least the threshold, so the next level's m-th largest key is at
  // least that threshold too (the pool's forced block is forced at both
  // levels; the pool's top-k over its members' own keys has m <= kappa - 1
  // members that are not the forced one, each at least the pool threshold).
  // `bnd` carries it from one selection to the next.
  uint32_t bnd = kKeyNegInf;
  auto sel = [&](int n, int m, lds_u32* out) {
    SelResult r;
    if constexpr (KCAND <= 4096) r = select_top_inl(L, n, m, out, bnd);
    else r = select_top(L, n, m, out, bnd);
    bnd = r.t;
    return r.n;
  };
  for (int x = threadIdx.x; x < 4 * kBins; x += kNT) L.hist[x] = 0;

  const int qi = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int64_t row = int64_t(b) * n_q + qi;
  // split: two workgroups per row, blockIdx.z 0 builds the pool, 1 the flat top-k
  if (split) {
    if (blockIdx.z == 1) pool_out = nullptr;
  }
  const bool pool_only = split && blockIdx.z == 0;
  const int nsb = int(dom_cap / 64);
  const int nb = int(dom_cap / 8);
  const float* sc = scores + row * dom_cap;
  const float* bm = bmax + row * nb;
  const float* sbm = sbmax + row * nsb;
  // the entry a fused decode scan left out of its scores and maxima (its
  // compressing workgroup scored it): folded in at each level
  constexpr int kNoFix = -0x7FFFFFFF;
  const int fix_j = fix_id ? fix_id[row] : -1;
  const uint32_t fix_key = fix_j >= 0 ? score_key(fix_score[row]) : kKeyNegInf;
  const int fix_blk = fix_j >= 0 ? fix_j / 8 : kNoFix, fix_sb = fix_j >= 0 ? fix_j / 64 : kNoFix;
  const int fix_ent = fix_j >= 0 ? fix_j : kNoFix;

  // ---- HSI pool (full domain only) ----
  // nbsel blocks chosen for the top-k stage, their ids in lb[0 .. nbsel)
  int nbsel = -1;
  if (pool_out) {
    const int64_t n = clamp_entries(n_entries, b, capacity);
    const int64_t n_vis = visible_count(n, q_pos[row], ratio);
    const int fb = n_vis > 0 ? int((n_vis - 1) / 8) : -1;
    const int fsb = fb >= 0 ? fb / 8 : -1;
    uint32_t fkey = fb >= 0 ? score_key(bm[fb]) : kKeyNegInf;  // the forced block's own key
    if (fb >= 0 && fb == fix_blk) fkey = max(fkey, fix_key);
    int na = nsb;
    if (nsb > cand_blocks) {
      gather_keys<kGather>(L, nsb, sbm, nsb, fsb, fix_sb, fix_key, [](int p) { return p; });
      __syncthreads();
      na = sel(nsb, cand_blocks, L.la);
    } else {
      for (int p = tid; p < nsb; p += kNT) L.la[p] = uint32_t(p);
      __syncthreads();  // la is read across threads below
    }
    gather_keys<kGather>(L, 8 * na, bm, nb, fb, fix_blk, fix_key, [&](int p) { return int(L.la[p >> 3]) * 8 + (p & 7); });
    __syncthreads();
    const int npool = sel(8 * na, cand_blocks, L.lb);
    // the pool members' own keys (the forced block's real maximum in place of
    // its forced key), read before lb becomes block ids and keys is rewritten
    uint32_t pk[kMaxList / kNT];
#pragma unroll
    for (int i = 0; i < kMaxList / kNT; ++i) {
      const int x = tid + i * kNT;
      pk[i] = x < npool ? L.keys[L.lb[x]] : kKeyNegInf;
      if (pk[i] == kKeyForced) pk[i] = fkey;
    }
    // pool block ids (ascending), in place: thread x reads and writes lb[x] only
    for (int x = tid; x < npool; x += kNT) L.lb[x] = min(L.la[L.lb[x] >> 3] * 8 + (L.lb[x] & 7), uint32_t(nb - 1));
    for (int x = tid; x < cand_blocks; x += kNT) pool_out[row * cand_blocks + x] = x < npool ? int32_t(L.lb[x]) : -1;
    if (pool_only) return;  // uniform: the other workgroup of the row selects the top-k
    __syncthreads();
    // The best topk blocks by their own maxima all lie in the pool when
    // topk <= cand_blocks - 1: the pool holds the best cand_blocks - 1 blocks
    // other than the forced one.  So the top-k stage needs only the pool.
    if (topk < cand_blocks) {
      uint32_t c = 0, kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
      for (int i = 0; i < kMaxList / kNT; ++i) {
        const int x = tid + i * kNT;
        if (x < npool) {
          L.keys[x] = pk[i];
          note_key(pk[i], c, kmn, kmx);
        }
      }
      put_stats(L, c, kmn, kmx);
      __syncthreads();
      nbsel = sel(npool, topk, L.la);
      uint32_t ids[kMaxList / kNT];
#pragma unroll
      for (int i = 0; i < kMaxList / kNT; ++i) {
        const int x = tid + i * kNT;
        ids[i] = x < nbsel ? L.lb[L.la[x]] : 0u;
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kMaxList / kNT; ++i) {
        const int x = tid + i * kNT;
        if (x < nbsel) L.lb[x] = ids[i];
      }
      __syncthreads();
    }
  }

  // ---- top-k blocks over the whole domain (unless the pool gave them) ----
  if (nbsel < 0) {
    bnd = kKeyNegInf;  // (a pool's threshold, for kappa places, does not bound k >= kappa)
    if (nsb > topk) {
      gather_keys<kGather>(L, nsb, sbm, nsb, -1, fix_sb, fix_key, [](int p) { return p; });
      __syncthreads();
      const int na = sel(nsb, topk, L.la);
      gather_keys<kGather>(L, 8 * na, bm, nb, -1, fix_blk, fix_key,
                           [&](int p) { return int(L.la[p >> 3]) * 8 + (p & 7); });
      __syncthreads();
      nbsel = sel(8 * na, topk, L.lb);
      // block ids of the chosen blocks (ascending), in place
      for (int x = tid; x < nbsel; x += kNT) L.lb[x] = L.la[L.lb[x] >> 3] * 8 + (L.lb[x] & 7);
      __syncthreads();
    } else {
      // every super-block is kept: the block maxima are gathered in order and
      // the chosen positions are the block ids (no list, two barriers fewer)
      gather_keys<kGather>(L, nb, bm, nb, -1, fix_blk, fix_key, [](int p) { return p; });
      __syncthreads();
      nbsel = sel(nb, topk, L.lb);
    }
  }

  // ---- top-k entries inside the chosen blocks ----
  gather_keys<kGather>(L, 8 * nbsel, sc, int(dom_cap), -1, fix_ent, fix_key,
                       [&](int p) { return int(L.lb[p >> 3]) * 8 + (p & 7); });
  __syncthreads();
  const int ne = sel(8 * nbsel, topk, L.la);
  for (int x = tid; x < topk; x += kNT) {
    int32_t id = -1;
    float s = -INFINITY;
    if (x < ne) {
      const int64_t slot = min(int64_t(L.lb[L.la[x] >> 3]) * 8 + (L.la[x] & 7), dom_cap - 1);
      s = slot == fix_ent ? fix_score[row] : sc[slot];
      id = pool_in ? int32_t(int64_t(pool_in[row * cand_blocks + min(slot / 8, int64_t(cand_blocks) - 1)]) * 8 + (slot & 7))
                   : int32_t(slot);
    }
    topk_out[row * topk + x] = id;
    if (topk_scores) topk_scores[row * topk + x] = s;
  }
}

#define SELECT_ARGS                                                                                        \
  int topk, int cand_blocks, int ratio, int64_t capacity, const int32_t *__restrict__ q_pos, int n_q,         \
      const int32_t *__restrict__ pool_in, const int32_t *__restrict__ n_entries,                             \
      const float *__restrict__ scores, const float *__restrict__ bmax, const float *__restrict__ sbmax,       \
      int64_t dom_cap, int32_t *__restrict__ topk_out, int32_t *__restrict__ pool_out,                        \
      float *__restrict__ topk_scores, int split, const float *__restrict__ fix_score,                       \
      const int32_t *__restrict__ fix_id
#define SELECT_PASS                                                                                              \
  topk, cand_blocks, ratio, capacity, q_pos, n_q, pool_in, n_entries, scores, bmax, sbmax, dom_cap, topk_out, pool_out, \
      topk_scores, split, fix_score, fix_id

__global__ __launch_bounds__(kNT) void select_kernel(SELECT_ARGS) { select_body<kMaxCand>(SELECT_PASS); }
// two workgroups per compute unit: 32 waves, at most 64 registers each
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_num_vgpr(64))) void select_kernel_wide(SELECT_ARGS) {
  select_body<kSmallCand>(SELECT_PASS);
}

constexpr size_t select_lds(int kcand) { return sizeof(uint32_t) * (kcand + 2 * kMaxList + 4 * kBins + 4 * kNW + 8); }

}  // namespace

hipError_t launch_select(const csa2_dims& dims, const csa2_kv_cache& cache, const int32_t* q_pos, int32_t n_q,
                         const int32_t* pool_in, const ScanScratch& ss, int32_t* topk_out, int32_t* pool_out,
                         float* topk_scores, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(select_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(select_lds(kMaxCand)));
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(select_kernel_wide),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(select_lds(kSmallCand)));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  // keys each level gathers: super-block maxima (when they outnumber the
  // level's m), then 8 per chosen super-block, then 8 per chosen block
  const int64_t nsb = ss.dom_cap / 64;
  const int64_t m_max = std::max<int64_t>(dims.topk, pool_out ? dims.cand_blocks : 0);
  const int64_t most = std::max<int64_t>({nsb, 8 * std::min<int64_t>(nsb, m_max), 8 * int64_t(dims.topk)});
  const bool small = most <= kSmallCand;
  auto kern = small ? select_kernel_wide : select_kernel;
  // Few rows (decode) leave the GPU idle while a row's selection runs its
  // long chain of dependent steps: the pool and the flat top-k then take a
  // workgroup each and run side by side, instead of the top-k following the
  // pool inside one workgroup.  Many rows (prefill) keep one workgroup per
  // row, whose top-k reuses the pool's blocks (less work in total).
  const int split = pool_out && int64_t(cache.batch) * n_q <= 128 ? 1 : 0;
  const hipError_t err = launch_kernel(CSA2_KERNEL_SELECT, kern, dim3(n_q, cache.batch, split ? 2 : 1), dim3(kNT),
                                       select_lds(small ? kSmallCand : kMaxCand), stream, dims.topk,
                     dims.cand_blocks, cache.ratio, cache.capacity, q_pos, n_q, pool_in, cache.n_entries, ss.scores,
                     ss.bmax, ss.sbmax, ss.dom_cap, topk_out, pool_out, topk_scores, split, ss.fix_score,
                     ss.fix_id);
  return err;
}

}  // namespace csa2
