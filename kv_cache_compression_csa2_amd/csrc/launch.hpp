// Host-side launchers of the CSA2 kernels (internal; the public ABI is csa2.h).
// Every launcher assumes the arguments were validated by abi.cpp and returns
// the hipError_t of its launches.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <functional>

#include "csa2.h"

namespace csa2 {

// Inverse RoPE frequencies theta^(-2m/d_rope) for pair m, computed once per
// launch on the host (libm pow, float64) and passed by value to the kernels,
// so no kernel evaluates a float64 pow per element.
constexpr int kMaxRopePairs = 64;  // d_rope <= 128
struct RopeTable {
  double inv_freq[kMaxRopePairs];  // angle per position of each rotary pair
  float logit_scale;    // attention logit scale: 1/sqrt(d), times the YaRN temperature
};

// Rotary frequencies theta^(-2m/d_rope); with a YaRN factor s > 1 (the
// NTK-by-parts interpolation of the YaRN paper, Peng et al. 2023) a pair
// whose wavelength fits the original context r = L f / (2 pi) times keeps
// its frequency when r >= 32, is divided by s when r <= 1, and blends
// linearly in between; the logits get the paper's temperature
// (0.1 ln s + 1)^2.
inline RopeTable make_rope_table(const csa2_dims& d) {
  RopeTable t{};
  const bool yarn = d.rope_factor > 1.0;
  for (int m = 0; m < d.d_rope / 2 && m < 64; ++m) {
    double f = std::pow(d.rope_theta, -2.0 * m / d.d_rope);
    if (yarn) {
      const double r = double(d.rope_orig_len) * f / (2.0 * 3.14159265358979323846);
      const double g = std::min(1.0, std::max(0.0, (r - 1.0) / 31.0));
      f = (1.0 - g) * f / d.rope_factor + g * f;
    }
    t.inv_freq[m] = f;
  }
  const double ms = yarn ? 0.1 * std::log(d.rope_factor) + 1.0 : 1.0;
  t.logit_scale = float(ms * ms / std::sqrt(double(d.d)));
  return t;
}

// Everything the compressor reads and writes (kernel argument).
struct CompressParams {
  int d, d_rope, d_idx, kv_dtype, main_group, idx_group, ratio;
  int64_t capacity;
  RopeTable rope;
  const void* latent;        // [batch][n_pos][d] act
  const int32_t* first_pos;  // [batch]
  int n_pos;
  const float* pair_logits;  // [ratio][d], NULL for ratio 1
  const void* w_ik;          // [d][d_idx] act
  void* main;
  uint8_t* main_scale;
  void* idx_k;
  uint8_t* idx_scale;
};
CompressParams make_compress_params(const csa2_dims& dims, const csa2_kv_cache& cache, const void* latent,
                                    const int32_t* first_pos, int32_t n_pos, const float* pair_logits,
                                    const void* w_ik);

// A decode scan that also writes the step's cache entry (one entry per
// sequence, one query per sequence, d = 512, d_idx = 128, bf16
// activations): one extra workgroup per sequence runs the compressor, scores
// the entry and leaves the score and the entry's id in fix_score / fix_id
// ([batch]); the scan's workgroups leave the entry out, and the selection
// folds the score back in.
struct ScanFuse {
  CompressParams cp;
  float* fix_score;  // [batch*n_q]
  int32_t* fix_id;   // [batch*n_q], -1: none
};

// Scratch layout of one index_topk call (all float32, per (batch, query)).
struct ScanScratch {
  float* scores;  // [batch*n_q][dom_cap]
  float* bmax;    // [batch*n_q][dom_cap/8]
  float* sbmax;   // [batch*n_q][dom_cap/64]
  int64_t dom_cap;  // multiple of 1024: the decode scan's workgroups cover it exactly
  const ScanFuse* fuse = nullptr;  // set: the scan writes the step's entry (see ScanFuse)
  const float* fix_score = nullptr;  // the selection's fold-in of that entry's score, or NULL
  const int32_t* fix_id = nullptr;
};

hipError_t launch_compress(const csa2_dims& dims, const csa2_kv_cache& cache, const void* latent,
                           const int32_t* first_pos, int32_t n_pos, const float* pair_logits, const void* w_ik,
                           hipStream_t stream);

hipError_t launch_scan(const csa2_dims& dims, const csa2_kv_cache& cache, const void* idx_q, const float* head_w,
                       const int32_t* q_pos, int32_t n_q, const int32_t* pool_in, const ScanScratch& ss,
                       hipStream_t stream);

hipError_t launch_select(const csa2_dims& dims, const csa2_kv_cache& cache, const int32_t* q_pos, int32_t n_q,
                         const int32_t* pool_in, const ScanScratch& ss, int32_t* topk_out, int32_t* pool_out,
                         float* topk_scores, hipStream_t stream);

// The merge of a row-split attention launch: its partials (in the launch's
// workspace) and the outputs the merged rows go to.
struct AttnMerge {
  const float* part_o = nullptr;
  const float* part_ml = nullptr;
  uint16_t* out = nullptr;
  float* lse = nullptr;
  int32_t n_heads = 0;
  int32_t n_splits = 0;  // 0: the launch was not split, nothing to merge
  int64_t n_bq = 0;
};

// With `merge` null a split launch is followed by its merge on `stream`;
// otherwise the merge is described in *merge and left to the caller
// (launch_attn_merge), which must run it before the workspace is reused.
hipError_t launch_attn(const csa2_dims& dims, const csa2_kv_cache& cache, const void* q, const int32_t* q_pos,
                       int32_t n_q, const int32_t* topk, const void* swa_kv, const int32_t* swa_first_pos,
                       int32_t n_swa, void* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream,
                       AttnMerge* merge = nullptr);
// One launch that merges one or two split launches (the same head count,
// splits and rows): the merges of two layers of a group share a launch.
hipError_t launch_attn_merge(const AttnMerge* jobs, int n_jobs, hipStream_t stream);

// Kernel trace hooks (trace.cpp).  trace_begin hands out a slot with two
// events for the next launch (slot -1 and no events when tracing is off);
// trace_end marks whether that launch was enqueued.
struct TraceSlot {
  int slot;
  hipEvent_t start, stop;
};
TraceSlot trace_begin(int32_t kernel);
void trace_end(int slot, bool launched);

// Launch `kern` on `stream` and return the launch's error.  With the kernel
// trace on, the launch carries the slot's events, which the runtime stamps
// with the kernel's own start and end times (no extra queue packets).
template <typename K, typename... Args>
hipError_t launch_kernel(int32_t kernel_id, K kern, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                         Args... args) {
  const TraceSlot t = trace_begin(kernel_id);
  if (t.slot < 0) {
    hipLaunchKernelGGL(kern, grid, block, lds, stream, args...);
    return hipGetLastError();
  }
  hipExtLaunchKernelGGL(kern, grid, block, uint32_t(lds), stream, t.start, t.stop, 0u, args...);
  const hipError_t e = hipGetLastError();
  trace_end(t.slot, e == hipSuccess);
  return e;
}

size_t attn_workspace_bytes(const csa2_dims& dims, const csa2_kv_cache& cache, int32_t n_q);
// Whether the attention of n_q queries per sequence runs one workgroup per
// query whose waves share each row tile (many queries), which leaves compute
// units free for a second attention launch at the same time.
bool attn_shares_tiles(const csa2_dims& dims, const csa2_kv_cache& cache, int32_t n_q);

// csa2_layer_group's argument checks and launch sequence with the workspace
// supplied by get_ws(need, &ws), called once after every argument check
// passed and before the first launch; a nonzero status from it is returned
// unchanged.  Errors are recorded as for the entry points; the caller clears
// the last error and catches exceptions.
// concurrent: the attention launches may run on the library's own streams
// (see csa2_layer_group); false keeps every launch on `stream`.
using WorkspaceFn = std::function<int(size_t need, void** ws)>;
int layer_group_run(const csa2_dims* dims, const csa2_kv_cache* cache, int32_t n_layers, const csa2_layer* layers,
                    const int32_t* q_pos, int32_t n_q, const csa2_compress_args* compress, const WorkspaceFn& get_ws,
                    void* stream, bool concurrent);
// Workspace bytes of a layer group: the index scratch, then one attention
// workspace per attention stream (`slices`: 1 when every launch stays on
// the caller's stream, kGroupAttnStreams when they may not).
constexpr int kGroupAttnStreams = 2;
size_t layer_group_ws_bytes(const csa2_dims* dims, const csa2_kv_cache* cache, int32_t n_q, int slices);
// Record `msg` as the last error of this thread and return `status`.
int set_error(int status, const char* msg);

hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_mfma_probe(int64_t iters, int32_t workgroups, float* sink, hipStream_t stream);

hipError_t launch_oproj(int32_t act_dtype, int32_t n_tok, int32_t width, int32_t n_groups, int32_t rank,
                        const void* x, const void* w, void* y, hipStream_t stream);

}  // namespace csa2
