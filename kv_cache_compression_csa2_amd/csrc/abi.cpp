// C ABI of the CSA2 hot path: argument validation, workspace carving and the
// launch sequence of every entry point.  Every check runs on the host before
// any HIP call; no exception leaves this file.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "csa2.h"
#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int fail_hip(hipError_t e, const char* where) {
  return fail(CSA2_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxCapacity = int64_t(1) << 20;
constexpr size_t kAlign = 256;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int check_dims(const csa2_dims* d) {
  if (!d) return fail(CSA2_ERR_INVALID_ARG, "dims is NULL");
  if (d->d <= 0 || d->d % 32 || d->d > 1024) return fail(CSA2_ERR_UNSUPPORTED, "d=%d: need a multiple of 32 in [32, 1024]", d->d);
  if (d->d_rope < 0 || d->d_rope % 2 || d->d_rope > d->d) return fail(CSA2_ERR_INVALID_ARG, "d_rope=%d: need even, 0..d", d->d_rope);
  if (d->d_rope > 128) return fail(CSA2_ERR_UNSUPPORTED, "d_rope=%d: at most 128 rotary channels", d->d_rope);
  if (d->n_heads <= 0 || d->n_heads > 1024) return fail(CSA2_ERR_INVALID_ARG, "n_heads=%d out of range", d->n_heads);
  if (d->n_idx_heads <= 0 || d->d_idx <= 0 || d->d_idx % 32 || d->d_idx > 512)
    return fail(CSA2_ERR_UNSUPPORTED, "indexer heads %d x %d: need width a multiple of 32 up to 512", d->n_idx_heads, d->d_idx);
  if (int64_t(d->n_idx_heads) * d->d_idx > 8192)
    return fail(CSA2_ERR_UNSUPPORTED, "indexer query of %d x %d exceeds 8192 elements", d->n_idx_heads, d->d_idx);
  if (d->topk < 1 || d->topk > 2048) return fail(CSA2_ERR_UNSUPPORTED, "topk=%d: need 1..2048", d->topk);
  if (d->window < 0 || d->window > 4096) return fail(CSA2_ERR_UNSUPPORTED, "window=%d: need 0..4096", d->window);
  if (d->block_size != 8) return fail(CSA2_ERR_UNSUPPORTED, "block_size=%d: only 8 is implemented", d->block_size);
  if (d->cand_blocks < 1 || d->cand_blocks > 2048) return fail(CSA2_ERR_UNSUPPORTED, "cand_blocks=%d: need 1..2048", d->cand_blocks);
  if (d->act_dtype != CSA2_F32 && d->act_dtype != CSA2_BF16) return fail(CSA2_ERR_UNSUPPORTED, "act_dtype=%d", d->act_dtype);
  if (!(d->rope_theta > 0.0)) return fail(CSA2_ERR_INVALID_ARG, "rope_theta must be positive");
  if (d->swa_dtype != 0 && d->swa_dtype != CSA2_FP8)
    return fail(CSA2_ERR_UNSUPPORTED, "swa_dtype=%d: need 0 (activation type) or CSA2_FP8", d->swa_dtype);
  if (!(d->rope_factor == 0.0 || d->rope_factor >= 1.0))
    return fail(CSA2_ERR_INVALID_ARG, "rope_factor must be 0, 1 or more (YaRN factor)");
  if (d->rope_factor > 1.0 && d->rope_orig_len <= 0)
    return fail(CSA2_ERR_INVALID_ARG, "rope_orig_len must be positive with a YaRN factor above 1");
  return CSA2_OK;
}

// need_idx: the call reads or writes the indexer K.
int check_cache(const csa2_dims* d, const csa2_kv_cache* c, bool need_idx) {
  if (!c) return fail(CSA2_ERR_INVALID_ARG, "cache is NULL");
  if (c->kv_dtype != CSA2_F32 && c->kv_dtype != CSA2_BF16 && c->kv_dtype != CSA2_FP4)
    return fail(CSA2_ERR_UNSUPPORTED, "kv_dtype=%d", c->kv_dtype);
  if (c->ratio != 1 && c->ratio != 2) return fail(CSA2_ERR_UNSUPPORTED, "ratio=%d: need 1 or 2", c->ratio);
  if (c->batch <= 0 || c->batch > 65535) return fail(CSA2_ERR_INVALID_ARG, "batch=%d out of range", c->batch);
  if (c->reserved0 != 0) return fail(CSA2_ERR_INVALID_ARG, "cache reserved field must be 0");
  if (c->capacity <= 0 || c->capacity > kMaxCapacity)
    return fail(CSA2_ERR_UNSUPPORTED, "capacity=%lld: need 1..%lld", (long long)c->capacity, (long long)kMaxCapacity);
  if (!c->main || !c->n_entries) return fail(CSA2_ERR_INVALID_ARG, "cache main or n_entries is NULL");
  if (!aligned16(c->main)) return fail(CSA2_ERR_INVALID_ARG, "cache main is not 16-byte aligned");
  if (need_idx && !c->idx_k) return fail(CSA2_ERR_INVALID_ARG, "cache idx_k is NULL but this call needs the indexer K");
  if (c->idx_k && !aligned16(c->idx_k)) return fail(CSA2_ERR_INVALID_ARG, "cache idx_k is not 16-byte aligned");
  if (c->kv_dtype == CSA2_FP4) {
    if (c->main_group != 16 && c->main_group != 32) return fail(CSA2_ERR_UNSUPPORTED, "main_group=%d: need 16 or 32", c->main_group);
    if (c->idx_group != 16 && c->idx_group != 32) return fail(CSA2_ERR_UNSUPPORTED, "idx_group=%d: need 16 or 32", c->idx_group);
    if (d->d % c->main_group || d->d_idx % c->idx_group) return fail(CSA2_ERR_INVALID_ARG, "widths must be multiples of the FP4 groups");
    if (!c->main_scale) return fail(CSA2_ERR_INVALID_ARG, "FP4 cache needs main_scale");
    if (!aligned16(c->main_scale)) return fail(CSA2_ERR_INVALID_ARG, "cache main_scale is not 16-byte aligned");
    if (need_idx && !c->idx_scale) return fail(CSA2_ERR_INVALID_ARG, "FP4 cache needs idx_scale");
    if (c->idx_scale && !aligned16(c->idx_scale)) return fail(CSA2_ERR_INVALID_ARG, "cache idx_scale is not 16-byte aligned");
  }
  return CSA2_OK;
}

int check_ptr(const void* p, const char* name) {
  if (!p) return fail(CSA2_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(CSA2_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return CSA2_OK;
}

// Domain slots per (sequence, query) in the scratch: whole workgroups of the
// decode scan (16 super-blocks of 64 slots), so its stores need no bounds test.
constexpr size_t kDomAlign = 1024;
int64_t dom_cap_flat(const csa2_kv_cache* c) { return int64_t(round_up(size_t(c->capacity), kDomAlign)); }
int64_t dom_cap_pool(const csa2_dims* d) { return int64_t(round_up(size_t(d->cand_blocks) * 8, kDomAlign)); }

size_t index_ws_bytes(const csa2_dims* d, const csa2_kv_cache* c, int32_t n_q) {
  const int64_t cap = dom_cap_flat(c) > dom_cap_pool(d) ? dom_cap_flat(c) : dom_cap_pool(d);
  const size_t rows = size_t(c->batch) * size_t(n_q);
  return round_up(rows * cap * 4, kAlign) + round_up(rows * (cap / 8) * 4, kAlign) + round_up(rows * (cap / 64) * 4, kAlign) +
         2 * round_up(rows * 4, kAlign);
}

csa2::ScanScratch carve_index(void* ws, const csa2_dims* d, const csa2_kv_cache* c, int32_t n_q, bool pool_domain) {
  const int64_t cap = dom_cap_flat(c) > dom_cap_pool(d) ? dom_cap_flat(c) : dom_cap_pool(d);
  const size_t rows = size_t(c->batch) * size_t(n_q);
  csa2::ScanScratch s;
  char* p = static_cast<char*>(ws);
  s.dom_cap = pool_domain ? dom_cap_pool(d) : dom_cap_flat(c);
  s.scores = reinterpret_cast<float*>(p);
  p += round_up(rows * cap * 4, kAlign);
  s.bmax = reinterpret_cast<float*>(p);
  p += round_up(rows * (cap / 8) * 4, kAlign);
  s.sbmax = reinterpret_cast<float*>(p);
  p += round_up(rows * (cap / 64) * 4, kAlign);
  // the step entry's score and id when the decode scan writes the entry
  s.fix_score = reinterpret_cast<float*>(p);
  p += round_up(rows * 4, kAlign);
  s.fix_id = reinterpret_cast<int32_t*>(p);
  return s;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return CSA2_OK;
  if (!ws) return fail(CSA2_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", need);
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return fail(CSA2_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < need) return fail(CSA2_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, need);
  return CSA2_OK;
}

int check_compress(const csa2_dims* d, const csa2_kv_cache* c, const void* latent, const int32_t* first_pos,
                   int32_t n_pos, const float* pair_logits, const void* w_ik) {
  int st;
  if ((st = check_ptr(latent, "latent")) || (st = check_ptr(first_pos, "first_pos")) || (st = check_ptr(w_ik, "w_ik")))
    return st;
  if (n_pos <= 0 || n_pos % c->ratio) return fail(CSA2_ERR_INVALID_ARG, "n_pos=%d: need a positive multiple of ratio %d", n_pos, c->ratio);
  if (n_pos / c->ratio > 65535) return fail(CSA2_ERR_UNSUPPORTED, "n_pos=%d: at most 65535 entries per call", n_pos);
  if ((c->ratio == 1) != (pair_logits == nullptr)) return fail(CSA2_ERR_INVALID_ARG, "pair_logits must be NULL iff ratio == 1");
  if (pair_logits && !aligned16(pair_logits)) return fail(CSA2_ERR_INVALID_ARG, "pair_logits is not 16-byte aligned");
  return CSA2_OK;
}

int check_attn(const csa2_dims* dims, const void* q, const int32_t* q_pos, int32_t n_q, const int32_t* topk,
                      const void* swa_kv, const int32_t* swa_first_pos, int32_t n_swa, void* out, const float* lse) {
  int st;
  if (n_q <= 0 || n_q > 65535) return fail(CSA2_ERR_INVALID_ARG, "n_q=%d out of range", n_q);
  if ((st = check_ptr(q, "q")) || (st = check_ptr(q_pos, "q_pos")) || (st = check_ptr(topk, "topk")) ||
      (st = check_ptr(out, "out")))
    return st;
  if (n_swa < 0) return fail(CSA2_ERR_INVALID_ARG, "n_swa=%d is negative", n_swa);
  if (n_swa > 0 && ((st = check_ptr(swa_kv, "swa_kv")) || (st = check_ptr(swa_first_pos, "swa_first_pos")))) return st;
  if (lse && !aligned16(lse)) return fail(CSA2_ERR_INVALID_ARG, "lse is not 16-byte aligned");
  return CSA2_OK;
}

// hipGetLastError() is per thread and sticky across unrelated runtime calls
// (another library's probe may have left an error behind); clear it so that
// the check after our launches reports only our launches.
void clear_stale_error() { (void)hipGetLastError(); }

int run_compress(const csa2_dims* d, const csa2_kv_cache* c, const void* latent, const int32_t* first_pos,
                 int32_t n_pos, const float* pair_logits, const void* w_ik, hipStream_t s) {
  clear_stale_error();
  hipError_t e = csa2::launch_compress(*d, *c, latent, first_pos, n_pos, pair_logits, w_ik, s);
  return e == hipSuccess ? CSA2_OK : fail_hip(e, "compress launch");
}

// The decode scan writes the step's entry itself (csa2::ScanFuse) when the
// step compresses one entry per sequence and its first index step scans the
// whole cache for one query per sequence on the matrix cores: one launch and
// one pass fewer than the compress kernel followed by the scan.
bool fuse_compress(const csa2_dims* d, const csa2_kv_cache* c, const csa2_compress_args* compress, int32_t n_q,
                   const csa2_layer& first) {
  const bool mfma_shape = d->n_idx_heads == 32 && d->d_idx == 128 && d->act_dtype == CSA2_BF16 &&
                          (c->kv_dtype == CSA2_BF16 || (c->kv_dtype == CSA2_FP4 && c->idx_group == 32));
  // the compressing workgroup's 256 threads are laid out for d = 512
  return compress && compress->n_pos == c->ratio && n_q == 1 && mfma_shape && d->d == 512 &&
         (first.mode == CSA2_FULL || (first.mode == CSA2_REINDEX && first.source < 0));
}

int run_index(const csa2_dims* d, const csa2_kv_cache* c, const void* idx_q, const float* head_w,
              const int32_t* q_pos, int32_t n_q, const int32_t* pool_in, int32_t* topk_out, int32_t* pool_out,
              float* topk_scores, void* ws, hipStream_t s, const csa2_compress_args* fused = nullptr) {
  csa2::ScanScratch ss = carve_index(ws, d, c, n_q, pool_in != nullptr);
  csa2::ScanFuse fz;
  if (fused) {
    fz.cp = csa2::make_compress_params(*d, *c, fused->latent, fused->first_pos, fused->n_pos, fused->pair_logits,
                                       fused->w_ik);
    fz.fix_score = const_cast<float*>(ss.fix_score);
    fz.fix_id = const_cast<int32_t*>(ss.fix_id);
    ss.fuse = &fz;
  } else {
    ss.fix_score = nullptr;
    ss.fix_id = nullptr;
  }
  clear_stale_error();
  hipError_t e = csa2::launch_scan(*d, *c, idx_q, head_w, q_pos, n_q, pool_in, ss, s);
  if (e != hipSuccess) return fail_hip(e, "index scan launch");
  e = csa2::launch_select(*d, *c, q_pos, n_q, pool_in, ss, topk_out, pool_out, topk_scores, s);
  if (e != hipSuccess) return fail_hip(e, "top-k select launch");
  return CSA2_OK;
}

// ---- the layer group's attention streams ----
//
// In a layer group each attention launch needs only the top-k of one index
// step (its own layer's, or its Reuse source's); it does not wait for the
// index steps after it nor for the other attention launches.  The index
// steps stay in order on the caller's stream; each attention launch goes to
// one of the library's attention streams, waits for the event recorded after
// the index step that feeds it, and uses its own slice of the workspace; the
// caller's stream then waits for every attention stream.  Events and stream
// waits are captured into a HIP graph as its edges.  Measured on one MI355X:
// 16 attention launches of a 128-query replay segment took 0.67 ms on one
// stream, 0.49 ms on two, 0.52-0.54 ms on four, and the 20-layer replay
// step went from 1.214 to 0.994 ms.  The one-workgroup-per-(query, head
// group) decode launches fill the compute units alone and slowed down side
// by side (0.32 -> 0.35-0.38 ms); even on one stream of their own beside the
// index steps the cross-queue waits cost more than the overlap gained (the
// 4-layer 256K decode group 202 -> 215 us), so those groups stay on the
// caller's stream.
constexpr int kMaxDevices = 64;
constexpr int kMaxGroupLayers = 64;

struct GroupStreams {
  bool ready = false;
  hipStream_t attn[csa2::kGroupAttnStreams] = {};
  hipEvent_t indexed[kMaxGroupLayers] = {};  // after layer i's index step, on the caller's stream
  hipEvent_t done[csa2::kGroupAttnStreams] = {};  // after an attention stream's last launch of a call
};

// One lock for the streams and events of every device: a call records and
// waits on them, so two host threads must not interleave their calls.
std::mutex g_group_mu;
GroupStreams g_group[kMaxDevices];

// The current device's attention streams and events (g_group_mu held),
// created on the first call that is not being captured; nullptr when they
// do not exist and cannot be created now (the call then runs on one stream).
GroupStreams* group_streams(hipStream_t caller) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  GroupStreams& g = g_group[dev];
  if (g.ready) return &g;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(caller, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) return nullptr;
  bool ok = true;
  for (auto& st : g.attn) ok = ok && hipStreamCreateWithFlags(&st, hipStreamNonBlocking) == hipSuccess;
  for (auto& e : g.indexed) ok = ok && hipEventCreateWithFlags(&e, hipEventDisableTiming) == hipSuccess;
  for (auto& e : g.done) ok = ok && hipEventCreateWithFlags(&e, hipEventDisableTiming) == hipSuccess;
  if (!ok) {  // release what was created; the call runs on one stream
    for (auto& st : g.attn) {
      if (st) (void)hipStreamDestroy(st);
      st = nullptr;
    }
    for (auto& e : g.indexed) {
      if (e) (void)hipEventDestroy(e);
      e = nullptr;
    }
    for (auto& e : g.done) {
      if (e) (void)hipEventDestroy(e);
      e = nullptr;
    }
    (void)hipGetLastError();
    return nullptr;
  }
  g.ready = true;
  return &g;
}

// Whether the layers' buffers let their attention launches run out of
// order: no buffer a layer writes (out, lse, top-k, pool) overlaps a buffer
// another layer reads or writes (its queries, indexer queries and weights,
// window rows and positions, outputs).  A Reuse layer's read of its source's
// top-k and a Reindex layer's read of its source's pool are ordered by the
// events.  The byte ranges are sorted, so the check is O(n log n).
bool layers_independent(const csa2_dims* d, const csa2_kv_cache* c, int32_t n_layers, const csa2_layer* layers,
                        int32_t n_q) {
  struct Range {
    uintptr_t lo, hi;
    int layer;
    bool write;
  };
  const uint64_t rows = uint64_t(c->batch) * uint64_t(n_q);
  const uint64_t act = d->act_dtype == CSA2_BF16 ? 2 : 4;
  std::vector<Range> r;
  r.reserve(size_t(n_layers) * 9);
  auto add = [&](const void* p, uint64_t bytes, int layer, bool write) {
    if (p && bytes) r.push_back({reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + bytes, layer, write});
  };
  for (int i = 0; i < n_layers; ++i) {
    const csa2_layer& L = layers[i];
    add(L.out, rows * d->n_heads * d->d * act, i, true);
    add(L.lse, rows * d->n_heads * 4, i, true);
    add(L.topk, rows * d->topk * 4, i, true);
    if (L.make_pool) add(L.pool, rows * d->cand_blocks * 4, i, true);
    add(L.q, rows * d->n_heads * d->d * act, i, false);
    add(L.idx_q, rows * d->n_idx_heads * d->d_idx * act, i, false);
    add(L.head_w, rows * d->n_idx_heads * 4, i, false);
    if (L.n_swa > 0) {
      add(L.swa_kv, uint64_t(c->batch) * L.n_swa * d->d * (d->swa_dtype == CSA2_FP8 ? 1 : act), i, false);
      add(L.swa_first_pos, uint64_t(c->batch) * 4, i, false);
    }
  }
  std::sort(r.begin(), r.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t i = 0; i < r.size(); ++i)
    for (size_t j = i + 1; j < r.size() && r[j].lo < r[i].hi; ++j)
      if (r[i].layer != r[j].layer && (r[i].write || r[j].write)) return false;
  return true;
}

}  // namespace

namespace csa2 {

int set_error(int status, const char* msg) { return fail(status, "%s", msg); }

size_t layer_group_ws_bytes(const csa2_dims* dims, const csa2_kv_cache* cache, int32_t n_q, int slices) {
  return round_up(index_ws_bytes(dims, cache, n_q), kAlign) + size_t(slices) * attn_workspace_bytes(*dims, *cache, n_q);
}

int layer_group_run(const csa2_dims* dims, const csa2_kv_cache* cache, int32_t n_layers, const csa2_layer* layers,
                    const int32_t* q_pos, int32_t n_q, const csa2_compress_args* compress, const WorkspaceFn& get_ws,
                    void* stream, bool concurrent) {
  int st;
  if ((st = check_dims(dims))) return st;
  if (n_layers <= 0 || n_layers > 64) return fail(CSA2_ERR_INVALID_ARG, "n_layers=%d: need 1..64", n_layers);
  if (!layers) return fail(CSA2_ERR_INVALID_ARG, "layers is NULL");
  bool need_idx = compress != nullptr;
  for (int i = 0; i < n_layers; ++i) need_idx |= layers[i].mode != CSA2_REUSE;
  if ((st = check_cache(dims, cache, need_idx))) return st;
  if ((st = check_ptr(q_pos, "q_pos"))) return st;
  if (compress) {
    if (compress->reserved0 != 0) return fail(CSA2_ERR_INVALID_ARG, "compress reserved field must be 0");
    if ((st = check_compress(dims, cache, compress->latent, compress->first_pos, compress->n_pos,
                             compress->pair_logits, compress->w_ik)))
      return st;
  }
  for (int i = 0; i < n_layers; ++i) {
    const csa2_layer& L = layers[i];
    if (L.mode == CSA2_FULL) {
      if (L.source != -1) return fail(CSA2_ERR_MODE_ORDER, "layer %d: a Full layer has no source", i);
      if (L.make_pool && !L.pool) return fail(CSA2_ERR_INVALID_ARG, "layer %d: make_pool needs a pool buffer", i);
    } else if (L.mode == CSA2_REINDEX) {
      if (L.source != -1) {
        if (L.source < 0 || L.source >= i) return fail(CSA2_ERR_MODE_ORDER, "layer %d: Reindex source %d is not an earlier layer", i, L.source);
        const csa2_layer& S = layers[L.source];
        if (S.mode != CSA2_FULL || !S.make_pool)
          return fail(CSA2_ERR_MODE_ORDER, "layer %d: Reindex source %d is not a Full layer with a pool", i, L.source);
      }
      if (L.make_pool) return fail(CSA2_ERR_INVALID_ARG, "layer %d: only Full layers build a pool", i);
    } else if (L.mode == CSA2_REUSE) {
      if (L.source < 0 || L.source >= i) return fail(CSA2_ERR_MODE_ORDER, "layer %d: Reuse source %d is not an earlier layer", i, L.source);
      if (layers[L.source].mode == CSA2_REUSE)
        return fail(CSA2_ERR_MODE_ORDER, "layer %d: Reuse source %d must be a Full or Reindex layer", i, L.source);
      if (L.make_pool) return fail(CSA2_ERR_INVALID_ARG, "layer %d: only Full layers build a pool", i);
    } else {
      return fail(CSA2_ERR_UNSUPPORTED, "layer %d: mode %d unknown", i, L.mode);
    }
    if (L.mode != CSA2_REUSE) {
      if ((st = check_ptr(L.idx_q, "layer idx_q")) || (st = check_ptr(L.head_w, "layer head_w")) ||
          (st = check_ptr(L.topk, "layer topk")))
        return st;
    } else if (L.topk && !aligned16(L.topk)) {
      return fail(CSA2_ERR_INVALID_ARG, "layer %d: topk is not 16-byte aligned", i);
    }
    if ((st = check_attn(dims, L.q, q_pos, n_q, L.mode == CSA2_REUSE ? layers[L.source].topk : L.topk, L.swa_kv,
                         L.swa_first_pos, L.n_swa, L.out, L.lse)))
      return st;
  }
  const size_t idx_bytes = round_up(index_ws_bytes(dims, cache, n_q), kAlign);
  const size_t attn_bytes = attn_workspace_bytes(*dims, *cache, n_q);
  void* ws = nullptr;
  if ((st = get_ws(layer_group_ws_bytes(dims, cache, n_q, concurrent ? kGroupAttnStreams : 1), &ws))) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  // attention streams: for groups of more than one layer, one workgroup per
  // query in the attention, and independent buffers
  std::unique_lock<std::mutex> lock(g_group_mu, std::defer_lock);
  GroupStreams* gs = nullptr;
  if (concurrent && n_layers > 1 && attn_shares_tiles(*dims, *cache, n_q) &&
      layers_independent(dims, cache, n_layers, layers, n_q)) {
    lock.lock();
    gs = group_streams(s);
    if (!gs) lock.unlock();
  }
  const int n_attn = gs ? kGroupAttnStreams : 0;
  bool used[kGroupAttnStreams] = {};
  // On the caller's stream with the workspace's two attention slices, the
  // row-split attention of consecutive layers alternates between the slices
  // and one merge launch combines two layers (a kernel boundary and a merge
  // launch fewer per pair; the same arithmetic, so the same bits): no layer
  // reads another layer's attention output, and the layers' buffers must not
  // overlap, since the two merges run in one launch.
  const bool pair_merges = !gs && concurrent && n_layers > 1 && layers_independent(dims, cache, n_layers, layers, n_q);
  AttnMerge pending;
  bool has_pending = false;
  int slice = 0;

  const bool fused = fuse_compress(dims, cache, compress, n_q, layers[0]);
  if (compress && !fused &&
      (st = run_compress(dims, cache, compress->latent, compress->first_pos, compress->n_pos, compress->pair_logits,
                         compress->w_ik, s)))
    return st;
  char* attn_ws = static_cast<char*>(ws) + idx_bytes;
  int next_attn = 0;
  // the caller's stream waits for every attention stream used so far
  auto join = [&]() -> int {
    for (int k = 0; k < n_attn; ++k) {
      if (!used[k]) continue;
      hipError_t e = hipEventRecord(gs->done[k], gs->attn[k]);
      if (e == hipSuccess) e = hipStreamWaitEvent(s, gs->done[k], 0);
      if (e != hipSuccess) return fail_hip(e, "attention stream join");
    }
    return CSA2_OK;
  };
  // an error after work went to the attention streams: join them first (the
  // caller's stream stays ordered after everything enqueued), keep the error
  auto bail = [&](int status) -> int {
    if (gs) {
      const std::string keep = g_last_error;
      (void)join();
      g_last_error = keep;
    }
    return status;
  };
  for (int i = 0; i < n_layers; ++i) {
    const csa2_layer& L = layers[i];
    const int32_t* use_topk = L.topk;
    if (L.mode == CSA2_FULL || L.mode == CSA2_REINDEX) {
      const int32_t* pool_in = L.mode == CSA2_REINDEX && L.source >= 0 ? layers[L.source].pool : nullptr;
      st = run_index(dims, cache, L.idx_q, L.head_w, q_pos, n_q, pool_in, L.topk,
                     L.mode == CSA2_FULL && L.make_pool ? L.pool : nullptr, nullptr, ws, s,
                     i == 0 && fused ? compress : nullptr);
      if (st) return bail(st);
      if (gs) {
        const hipError_t e = hipEventRecord(gs->indexed[i], s);
        if (e != hipSuccess) return bail(fail_hip(e, "index event"));
      }
    } else {
      use_topk = layers[L.source].topk;
    }
    // the attention's stream: the caller's, or an attention stream that
    // waits for the index step feeding this layer
    hipStream_t as = s;
    char* aws = pair_merges ? attn_ws + size_t(slice) * attn_bytes : attn_ws;
    if (gs) {
      const int k = next_attn++ % n_attn;
      as = gs->attn[k];
      aws = attn_ws + size_t(k) * attn_bytes;
      used[k] = true;
      const hipError_t e = hipStreamWaitEvent(as, gs->indexed[L.mode == CSA2_REUSE ? L.source : i], 0);
      if (e != hipSuccess) return bail(fail_hip(e, "attention stream wait"));
    }
    if (L.mode == CSA2_REUSE && L.topk) {
      const hipError_t e = hipMemcpyAsync(L.topk, use_topk, sizeof(int32_t) * size_t(cache->batch) * n_q * dims->topk,
                                          hipMemcpyDeviceToDevice, as);
      if (e != hipSuccess) return bail(fail_hip(e, "reuse top-k copy"));
    }
    clear_stale_error();
    AttnMerge m;
    hipError_t e = launch_attn(*dims, *cache, L.q, q_pos, n_q, use_topk, L.n_swa ? L.swa_kv : nullptr,
                               L.n_swa ? L.swa_first_pos : nullptr, L.n_swa, L.out, L.lse, aws, attn_bytes, as,
                               pair_merges ? &m : nullptr);
    if (e != hipSuccess) return bail(fail_hip(e, "attention launch"));
    if (pair_merges && m.n_splits > 0) {
      if (has_pending) {  // this layer's partials are in the other slice
        const AttnMerge jobs[2] = {pending, m};
        e = launch_attn_merge(jobs, 2, s);
        has_pending = false;
      } else {
        pending = m;
        has_pending = true;
      }
      if (e != hipSuccess) return bail(fail_hip(e, "attention merge launch"));
      slice ^= 1;
    }
  }
  if (has_pending) {
    const hipError_t e = launch_attn_merge(&pending, 1, s);
    if (e != hipSuccess) return bail(fail_hip(e, "attention merge launch"));
  }
  if (gs && (st = join())) return st;
  return CSA2_OK;
}

}  // namespace csa2

extern "C" {

int32_t csa2_abi_version(void) { return CSA2_ABI_VERSION; }

const char* csa2_last_error(void) { return g_last_error.c_str(); }

const char* csa2_status_str(int status) {
  switch (status) {
    case CSA2_OK: return "CSA2_OK";
    case CSA2_ERR_INVALID_ARG: return "CSA2_ERR_INVALID_ARG";
    case CSA2_ERR_UNSUPPORTED: return "CSA2_ERR_UNSUPPORTED";
    case CSA2_ERR_WORKSPACE: return "CSA2_ERR_WORKSPACE";
    case CSA2_ERR_MODE_ORDER: return "CSA2_ERR_MODE_ORDER";
    case CSA2_ERR_HIP: return "CSA2_ERR_HIP";
    default: return "CSA2_ERR_UNKNOWN";
  }
}

size_t csa2_workspace_size(const csa2_dims* dims, const csa2_kv_cache* cache, int32_t entry_point, int32_t n_q) {
  g_last_error.clear();
  try {
    if (check_dims(dims) || check_cache(dims, cache, false)) return 0;
    if (n_q <= 0 || n_q > 65535) {  // the calls' range
      fail(CSA2_ERR_INVALID_ARG, "n_q=%d out of range", n_q);
      return 0;
    }
    switch (entry_point) {
      case CSA2_EP_COMPRESS: return 0;
      case CSA2_EP_INDEX_TOPK: return index_ws_bytes(dims, cache, n_q);
      case CSA2_EP_SPARSE_ATTN: return csa2::attn_workspace_bytes(*dims, *cache, n_q);
      case CSA2_EP_LAYER_GROUP:
        return csa2::layer_group_ws_bytes(dims, cache, n_q, csa2::kGroupAttnStreams);
      default:
        fail(CSA2_ERR_INVALID_ARG, "entry_point=%d unknown", entry_point);
        return 0;
    }
  } catch (...) {
    fail(CSA2_ERR_HIP, "internal exception");
    return 0;
  }
}

int csa2_compress(const csa2_dims* dims, const csa2_kv_cache* cache, const void* latent, const int32_t* first_pos,
                  int32_t n_pos, const float* pair_logits, const void* w_ik, void* stream) {
  g_last_error.clear();
  try {
    int st;
    if ((st = check_dims(dims)) || (st = check_cache(dims, cache, true))) return st;
    if ((st = check_compress(dims, cache, latent, first_pos, n_pos, pair_logits, w_ik))) return st;
    return run_compress(dims, cache, latent, first_pos, n_pos, pair_logits, w_ik, static_cast<hipStream_t>(stream));
  } catch (...) {
    return fail(CSA2_ERR_HIP, "internal exception");
  }
}

int csa2_index_topk(const csa2_dims* dims, const csa2_kv_cache* cache, const void* idx_q, const float* head_w,
                    const int32_t* q_pos, int32_t n_q, const int32_t* pool_in, int32_t* topk_out, int32_t* pool_out,
                    float* topk_scores, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  try {
    int st;
    if ((st = check_dims(dims)) || (st = check_cache(dims, cache, true))) return st;
    if (n_q <= 0 || n_q > 65535) return fail(CSA2_ERR_INVALID_ARG, "n_q=%d out of range", n_q);
    if ((st = check_ptr(idx_q, "idx_q")) || (st = check_ptr(head_w, "head_w")) || (st = check_ptr(q_pos, "q_pos")) ||
        (st = check_ptr(topk_out, "topk_out")))
      return st;
    if (pool_in && pool_out) return fail(CSA2_ERR_INVALID_ARG, "pool_in and pool_out are exclusive");
    if (pool_in && !aligned16(pool_in)) return fail(CSA2_ERR_INVALID_ARG, "pool_in is not 16-byte aligned");
    if (pool_out && !aligned16(pool_out)) return fail(CSA2_ERR_INVALID_ARG, "pool_out is not 16-byte aligned");
    if (topk_scores && !aligned16(topk_scores)) return fail(CSA2_ERR_INVALID_ARG, "topk_scores is not 16-byte aligned");
    if ((st = check_ws(ws, ws_bytes, index_ws_bytes(dims, cache, n_q)))) return st;
    return run_index(dims, cache, idx_q, head_w, q_pos, n_q, pool_in, topk_out, pool_out, topk_scores, ws,
                     static_cast<hipStream_t>(stream));
  } catch (...) {
    return fail(CSA2_ERR_HIP, "internal exception");
  }
}


int csa2_sparse_attn(const csa2_dims* dims, const csa2_kv_cache* cache, const void* q, const int32_t* q_pos,
                     int32_t n_q, const int32_t* topk, const void* swa_kv, const int32_t* swa_first_pos,
                     int32_t n_swa, void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  try {
    int st;
    if ((st = check_dims(dims)) || (st = check_cache(dims, cache, false))) return st;
    if ((st = check_attn(dims, q, q_pos, n_q, topk, swa_kv, swa_first_pos, n_swa, out, lse))) return st;
    if ((st = check_ws(ws, ws_bytes, csa2::attn_workspace_bytes(*dims, *cache, n_q)))) return st;
    clear_stale_error();
    hipError_t e = csa2::launch_attn(*dims, *cache, q, q_pos, n_q, topk, n_swa ? swa_kv : nullptr,
                                     n_swa ? swa_first_pos : nullptr, n_swa, out, lse, ws, ws_bytes,
                                     static_cast<hipStream_t>(stream));
    return e == hipSuccess ? CSA2_OK : fail_hip(e, "attention launch");
  } catch (...) {
    return fail(CSA2_ERR_HIP, "internal exception");
  }
}

int csa2_layer_group(const csa2_dims* dims, const csa2_kv_cache* cache, int32_t n_layers, const csa2_layer* layers,
                     const int32_t* q_pos, int32_t n_q, const csa2_compress_args* compress, void* ws, size_t ws_bytes,
                     void* stream) {
  g_last_error.clear();
  try {
    return csa2::layer_group_run(dims, cache, n_layers, layers, q_pos, n_q, compress,
                                 [&](size_t need, void** out) -> int {
                                   const int st = check_ws(ws, ws_bytes, need);
                                   *out = ws;
                                   return st;
                                 },
                                 stream, true);
  } catch (...) {
    return fail(CSA2_ERR_HIP, "internal exception");
  }
}


int csa2_grouped_out_proj(int32_t act_dtype, int32_t n_tok, int32_t width, int32_t n_groups, int32_t rank,
                          const void* x, const void* w, void* y, void* stream) {
  g_last_error.clear();
  try {
    if (act_dtype != CSA2_F32 && act_dtype != CSA2_BF16)
      return fail(CSA2_ERR_UNSUPPORTED, "act_dtype=%d: the projection takes F32 or BF16", act_dtype);
    if (n_tok < 0 || width <= 0 || n_groups <= 0 || rank <= 0)
      return fail(CSA2_ERR_INVALID_ARG, "n_tok=%d width=%d n_groups=%d rank=%d: n_tok must be >= 0, the rest > 0",
                  n_tok, width, n_groups, rank);
    if (width % n_groups)
      return fail(CSA2_ERR_INVALID_ARG, "width=%d is not a multiple of n_groups=%d", width, n_groups);
    if (int64_t(n_groups) * rank > (int64_t(1) << 30) || int64_t(rank) * width > (int64_t(1) << 40))
      return fail(CSA2_ERR_UNSUPPORTED, "n_groups*rank=%lld too large", (long long)(int64_t(n_groups) * rank));
    if (n_tok == 0) return CSA2_OK;
    if (!x || !w || !y) return fail(CSA2_ERR_INVALID_ARG, "x, w and y are required");
    if (!aligned16(x) || !aligned16(w) || !aligned16(y))
      return fail(CSA2_ERR_INVALID_ARG, "x, w and y must be 16-byte aligned");
    clear_stale_error();
    const hipError_t e = csa2::launch_oproj(act_dtype, n_tok, width, n_groups, rank, x, w, y,
                                            static_cast<hipStream_t>(stream));
    return e == hipSuccess ? CSA2_OK : fail_hip(e, "output projection launch");
  } catch (...) {
    return fail(CSA2_ERR_HIP, "internal exception");
  }
}

int csa2_read_probe(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  g_last_error.clear();
  try {
    if (bytes <= 0 || bytes % 16) return fail(CSA2_ERR_INVALID_ARG, "bytes=%lld: need a positive multiple of 16", (long long)bytes);
    int st;
    if ((st = check_ptr(buf, "buf"))) return st;
    if (!sink) return fail(CSA2_ERR_INVALID_ARG, "sink is NULL");
    clear_stale_error();
    const hipError_t e = csa2::launch_read_probe(buf, bytes, sink, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? CSA2_OK : fail_hip(e, "read probe launch");
  } catch (...) {
    return fail(CSA2_ERR_HIP, "internal exception");
  }
}

int csa2_mfma_probe(int64_t iters, int32_t workgroups, float* sink, void* stream) {
  g_last_error.clear();
  try {
    if (iters < 1 || iters > (int64_t(1) << 24))
      return fail(CSA2_ERR_INVALID_ARG, "iters=%lld: need 1..2^24", (long long)iters);
    if (workgroups < 1 || workgroups > 65536)
      return fail(CSA2_ERR_INVALID_ARG, "workgroups=%d: need 1..65536", workgroups);
    if (!sink) return fail(CSA2_ERR_INVALID_ARG, "sink is NULL");
    clear_stale_error();
    const hipError_t e = csa2::launch_mfma_probe(iters, workgroups, sink, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? CSA2_OK : fail_hip(e, "matrix-core probe launch");
  } catch (...) {
    return fail(CSA2_ERR_HIP, "internal exception");
  }
}

}  // extern "C"
