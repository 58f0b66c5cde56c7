// csa2_layer_plan: the cross-layer plan of a CSA2 model from its per-layer
// compress ratios and its kv-source, index-source and candidate-source
// layers.  Host logic only (no HIP call); see csa2.h for the rules.
#include <cstdio>
#include <cstring>
#include <vector>

#include "csa2.h"
#include "launch.hpp"

namespace {

bool sorted_unique_in_range(const int32_t* a, int32_t n, int32_t n_layers) {
  for (int32_t i = 0; i < n; ++i) {
    if (a[i] < 0 || a[i] >= n_layers) return false;
    if (i > 0 && a[i] <= a[i - 1]) return false;
  }
  return true;
}

int plan_error(const char* fmt, int32_t a, int32_t b = 0) {
  char msg[256];
  snprintf(msg, sizeof(msg), fmt, a, b);
  return csa2::set_error(CSA2_ERR_INVALID_ARG, msg);
}

}  // namespace

extern "C" int csa2_layer_plan(int32_t n_layers, const int32_t* ratios, int32_t n_kv, const int32_t* kv_src,
                               int32_t n_idx, const int32_t* idx_src, int32_t cand_src, csa2_plan_layer* out) {
  csa2::set_error(CSA2_OK, "");
  try {
    if (n_layers <= 0 || n_layers > 4096) return plan_error("n_layers=%d: need 1..4096", n_layers);
    if (!ratios || !out || (n_kv > 0 && !kv_src) || (n_idx > 0 && !idx_src))
      return csa2::set_error(CSA2_ERR_INVALID_ARG, "a required array is NULL");
    if (n_kv < 0 || n_idx < 0) return plan_error("list lengths must be >= 0 (%d, %d)", n_kv, n_idx);
    if (!sorted_unique_in_range(kv_src, n_kv, n_layers))
      return csa2::set_error(CSA2_ERR_INVALID_ARG, "kv_src must be ascending, distinct layer numbers");
    if (!sorted_unique_in_range(idx_src, n_idx, n_layers))
      return csa2::set_error(CSA2_ERR_INVALID_ARG, "idx_src must be ascending, distinct layer numbers");
    std::vector<char> is_kv(size_t(n_layers), 0), is_idx(size_t(n_layers), 0);
    for (int32_t i = 0; i < n_kv; ++i) is_kv[size_t(kv_src[i])] = 1;
    for (int32_t i = 0; i < n_idx; ++i) is_idx[size_t(idx_src[i])] = 1;
    for (int32_t l = 0; l < n_layers; ++l)
      if (ratios[l] != 0 && ratios[l] != 1 && ratios[l] != 2) return plan_error("layer %d: ratio %d (need 0, 1 or 2)", l, ratios[l]);
    for (int32_t i = 0; i < n_kv; ++i) {
      const int32_t l = kv_src[i];
      if (ratios[l] == 0) return plan_error("kv-source layer %d has ratio 0 (no compressed KV)", l);
      if (!is_idx[size_t(l)]) return plan_error("kv-source layer %d is not an index source (a Full layer runs the indexer)", l);
    }
    if (cand_src >= 0 && (cand_src >= n_layers || !is_kv[size_t(cand_src)]))
      return plan_error("candidate-source layer %d is not a kv-source layer", cand_src);

    int32_t group = -1, latest_idx = -1;
    for (int32_t l = 0; l < n_layers; ++l) {
      csa2_plan_layer& p = out[l];
      if (ratios[l] == 0) {  // window-only layer: no compressed KV, no top-k
        if (is_idx[size_t(l)]) return plan_error("index-source layer %d has ratio 0", l);
        p = csa2_plan_layer{-1, -1, -1, 0};
        continue;
      }
      if (is_kv[size_t(l)]) {
        group = l;
        latest_idx = l;
        p = csa2_plan_layer{l, CSA2_FULL, -1, l == cand_src ? 1 : 0};
        continue;
      }
      if (group < 0 || ratios[group] != ratios[l])
        return plan_error("layer %d (ratio %d) has no earlier kv-source layer of its ratio", l, ratios[l]);
      // layers of another ratio in between would have opened their own group
      for (int32_t m = group + 1; m < l; ++m)
        if (ratios[m] != ratios[l]) return plan_error("layer %d: its group is interrupted at layer %d", l, m);
      if (is_idx[size_t(l)]) {
        // Reindex: rescore the group's pool when its Full layer builds one, else every visible entry
        p = csa2_plan_layer{group, CSA2_REINDEX, group == cand_src ? group : -1, 0};
        latest_idx = l;
      } else {
        p = csa2_plan_layer{group, CSA2_REUSE, latest_idx, 0};
      }
    }
    return CSA2_OK;
  } catch (...) {
    return csa2::set_error(CSA2_ERR_HIP, "internal exception");
  }
}
