// Host-side check of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (see build.py,
// build_host_check): every argument-validation path, the workspace sizing,
// the layer plan and the status strings, on the CPU.  No call here reaches
// the GPU: every entry point is given arguments that its host checks reject
// before any HIP call, and fake device pointers are never dereferenced.
// Exit status 0 when every expectation holds.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "csa2.h"

namespace {

int g_failures = 0;

void expect(bool ok, const char* what, int line) {
  if (!ok) {
    ++g_failures;
    std::fprintf(stderr, "FAILED line %d: %s (last error: %s)\n", line, what, csa2_last_error());
  }
}
#define EXPECT(cond) expect((cond), #cond, __LINE__)

void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>(uintptr_t(0x100000) + off); }

csa2_dims dims() {
  csa2_dims d;
  std::memset(&d, 0, sizeof(d));
  d.d = 512;
  d.d_rope = 64;
  d.n_heads = 64;
  d.n_idx_heads = 32;
  d.d_idx = 128;
  d.topk = 512;
  d.window = 128;
  d.block_size = 8;
  d.cand_blocks = 2048;
  d.act_dtype = CSA2_BF16;
  d.rope_theta = 10000.0;
  return d;
}

csa2_kv_cache cache() {
  csa2_kv_cache c;
  std::memset(&c, 0, sizeof(c));
  c.kv_dtype = CSA2_BF16;
  c.ratio = 1;
  c.main_group = 32;
  c.idx_group = 32;
  c.batch = 2;
  c.capacity = 4096;
  c.main = fake();
  c.idx_k = fake();
  c.n_entries = static_cast<const int32_t*>(fake());
  return c;
}

csa2_layer layer(int mode, int source) {
  csa2_layer L;
  std::memset(&L, 0, sizeof(L));
  L.mode = mode;
  L.source = source;
  L.n_swa = 128;
  L.q = L.idx_q = L.swa_kv = fake();
  L.head_w = static_cast<const float*>(fake());
  L.swa_first_pos = static_cast<const int32_t*>(fake());
  L.out = fake();
  L.topk = static_cast<int32_t*>(fake());
  return L;
}

}  // namespace

int main() {
  EXPECT(csa2_abi_version() == CSA2_ABI_VERSION);
  for (int s = 1; s >= -6; --s) EXPECT(std::strlen(csa2_status_str(s)) > 0);
  EXPECT(std::strcmp(csa2_status_str(-4), "CSA2_ERR_MODE_ORDER") == 0);

  // ---- workspace sizing ----
  csa2_dims d = dims();
  csa2_kv_cache c = cache();
  for (int ep = CSA2_EP_COMPRESS; ep <= CSA2_EP_LAYER_GROUP; ++ep) {
    const size_t n = csa2_workspace_size(&d, &c, ep, 1);
    EXPECT(ep == CSA2_EP_COMPRESS ? n == 0 : n > 0);
  }
  EXPECT(csa2_workspace_size(nullptr, &c, CSA2_EP_INDEX_TOPK, 1) == 0 && std::strlen(csa2_last_error()) > 0);
  EXPECT(csa2_workspace_size(&d, &c, 99, 1) == 0);
  EXPECT(csa2_workspace_size(&d, &c, CSA2_EP_INDEX_TOPK, 0) == 0);
  {
    csa2_kv_cache big = cache();
    big.batch = 64;
    big.capacity = int64_t(1) << 20;
    EXPECT(csa2_workspace_size(&d, &big, CSA2_EP_LAYER_GROUP, 1) > (size_t(64) << 20));
  }

  // ---- dims and cache validation through csa2_index_topk ----
  auto index = [&](const csa2_dims& dd, const csa2_kv_cache& cc) {
    return csa2_index_topk(&dd, &cc, fake(), static_cast<const float*>(fake()), static_cast<const int32_t*>(fake()), 1,
                           nullptr, static_cast<int32_t*>(fake()), nullptr, nullptr, fake(), size_t(1) << 40, nullptr);
  };
  struct DimCase { int field; int value; int status; };
  const DimCase dcases[] = {{0, 100, CSA2_ERR_UNSUPPORTED}, {1, 3, CSA2_ERR_INVALID_ARG},  {7, 16, CSA2_ERR_UNSUPPORTED},
                            {5, 4096, CSA2_ERR_UNSUPPORTED}, {8, 0, CSA2_ERR_UNSUPPORTED}, {9, 7, CSA2_ERR_UNSUPPORTED},
                            {4, 48, CSA2_ERR_UNSUPPORTED},  {2, 0, CSA2_ERR_INVALID_ARG},  {6, -1, CSA2_ERR_UNSUPPORTED}};
  for (const DimCase& k : dcases) {
    csa2_dims dd = dims();
    int32_t* f[] = {&dd.d, &dd.d_rope, &dd.n_heads, &dd.n_idx_heads, &dd.d_idx, &dd.topk, &dd.window, &dd.block_size,
                    &dd.cand_blocks, &dd.act_dtype};
    *f[k.field] = k.value;
    EXPECT(index(dd, cache()) == k.status);
  }
  {
    csa2_dims dd = dims();
    dd.rope_theta = 0.0;
    EXPECT(index(dd, cache()) == CSA2_ERR_INVALID_ARG);
    dd = dims();
    dd.rope_factor = 0.5;
    EXPECT(index(dd, cache()) == CSA2_ERR_INVALID_ARG);
    dd = dims();
    dd.rope_factor = 16.0;
    dd.rope_orig_len = 0;
    EXPECT(index(dd, cache()) == CSA2_ERR_INVALID_ARG);
  }
  {
    csa2_kv_cache cc = cache();
    cc.ratio = 3;
    EXPECT(index(dims(), cc) == CSA2_ERR_UNSUPPORTED);
    cc = cache();
    cc.capacity = (int64_t(1) << 20) + 1;
    EXPECT(index(dims(), cc) == CSA2_ERR_UNSUPPORTED);
    cc = cache();
    cc.main = fake(4);
    EXPECT(index(dims(), cc) == CSA2_ERR_INVALID_ARG);
    cc = cache();
    cc.idx_k = nullptr;
    EXPECT(index(dims(), cc) == CSA2_ERR_INVALID_ARG);
    cc = cache();
    cc.kv_dtype = CSA2_FP4;
    cc.main_scale = static_cast<uint8_t*>(fake());
    cc.idx_scale = nullptr;
    EXPECT(index(dims(), cc) == CSA2_ERR_INVALID_ARG);
  }
  // workspace too small, pool in and out together
  EXPECT(csa2_index_topk(&d, &c, fake(), static_cast<const float*>(fake()), static_cast<const int32_t*>(fake()), 1, nullptr,
                         static_cast<int32_t*>(fake()), nullptr, nullptr, fake(), 16, nullptr) == CSA2_ERR_WORKSPACE);
  EXPECT(csa2_index_topk(&d, &c, fake(), static_cast<const float*>(fake()), static_cast<const int32_t*>(fake()), 1,
                         static_cast<const int32_t*>(fake()), static_cast<int32_t*>(fake()), static_cast<int32_t*>(fake()),
                         nullptr, fake(), size_t(1) << 40, nullptr) == CSA2_ERR_INVALID_ARG);

  // ---- compress, attention ----
  EXPECT(csa2_compress(&d, &c, fake(), static_cast<const int32_t*>(fake()), 4, static_cast<const float*>(fake()), fake(),
                       nullptr) == CSA2_ERR_INVALID_ARG);  // logits at ratio 1
  EXPECT(csa2_compress(&d, &c, nullptr, static_cast<const int32_t*>(fake()), 4, nullptr, fake(), nullptr) ==
         CSA2_ERR_INVALID_ARG);
  EXPECT(csa2_sparse_attn(&d, &c, fake(), static_cast<const int32_t*>(fake()), 0, static_cast<const int32_t*>(fake()),
                          fake(), static_cast<const int32_t*>(fake()), 128, fake(), nullptr, fake(), size_t(1) << 40,
                          nullptr) == CSA2_ERR_INVALID_ARG);
  EXPECT(csa2_sparse_attn(&d, &c, fake(), static_cast<const int32_t*>(fake()), 1, static_cast<const int32_t*>(fake()),
                          fake(), static_cast<const int32_t*>(fake()), -1, fake(), nullptr, fake(), size_t(1) << 40,
                          nullptr) == CSA2_ERR_INVALID_ARG);

  // ---- layer group modes, and the allocation-free variant's limit ----
  {
    const csa2_layer bad[2] = {layer(CSA2_FULL, -1), layer(CSA2_REUSE, 1)};
    EXPECT(csa2_layer_group(&d, &c, 2, bad, static_cast<const int32_t*>(fake()), 1, nullptr, fake(), size_t(1) << 40,
                            nullptr) == CSA2_ERR_MODE_ORDER);
    const csa2_layer reindex_no_pool[2] = {layer(CSA2_FULL, -1), layer(CSA2_REINDEX, 0)};
    EXPECT(csa2_layer_group(&d, &c, 2, reindex_no_pool, static_cast<const int32_t*>(fake()), 1, nullptr, fake(),
                            size_t(1) << 40, nullptr) == CSA2_ERR_MODE_ORDER);
    EXPECT(csa2_layer_group(&d, &c, 0, bad, static_cast<const int32_t*>(fake()), 1, nullptr, fake(), size_t(1) << 40,
                            nullptr) == CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_layer_group_noalloc(&d, &c, 2, bad, static_cast<const int32_t*>(fake()), 1, nullptr, nullptr) ==
           CSA2_ERR_MODE_ORDER);
    csa2_kv_cache big = cache();
    big.batch = 64;
    big.capacity = int64_t(1) << 20;
    const csa2_layer one[1] = {layer(CSA2_FULL, -1)};
    EXPECT(csa2_layer_group_noalloc(&d, &big, 1, one, static_cast<const int32_t*>(fake()), 1, nullptr, nullptr) ==
           CSA2_ERR_WORKSPACE);
    EXPECT(std::strstr(csa2_last_error(), "scratch") != nullptr);
  }

  // ---- output projection, read probe, trace ----
  EXPECT(csa2_grouped_out_proj(CSA2_FP4, 1, 32768, 8, 1024, fake(), fake(), fake(), nullptr) == CSA2_ERR_UNSUPPORTED);
  EXPECT(csa2_grouped_out_proj(CSA2_BF16, 1, 32767, 8, 1024, fake(), fake(), fake(), nullptr) == CSA2_ERR_INVALID_ARG);
  EXPECT(csa2_grouped_out_proj(CSA2_BF16, 0, 32768, 8, 1024, nullptr, nullptr, nullptr, nullptr) == CSA2_OK);
  EXPECT(csa2_read_probe(fake(), 24, static_cast<uint32_t*>(fake()), nullptr) == CSA2_ERR_INVALID_ARG);
  EXPECT(csa2_mfma_probe(0, 512, static_cast<float*>(fake()), nullptr) == CSA2_ERR_INVALID_ARG);
  EXPECT(csa2_mfma_probe(16, 65537, static_cast<float*>(fake()), nullptr) == CSA2_ERR_INVALID_ARG);
  EXPECT(csa2_mfma_probe(16, 512, nullptr, nullptr) == CSA2_ERR_INVALID_ARG);
  EXPECT(csa2_trace_read(nullptr, -1, nullptr) == CSA2_ERR_INVALID_ARG);
  EXPECT(std::strcmp(csa2_kernel_name(CSA2_KERNEL_SELECT), "select_kernel") == 0);

  // ---- the layer plan of the pages' schedule ----
  {
    std::vector<int32_t> ratios = {0, 0};
    for (int i = 0; i < 18; ++i) ratios.push_back(2);
    for (int i = 0; i < 20; ++i) ratios.push_back(1);
    const int32_t kv[] = {2, 8, 14, 20}, idx[] = {2, 8, 14, 20, 24, 28, 32, 36};
    std::vector<csa2_plan_layer> out(ratios.size());
    EXPECT(csa2_layer_plan(int32_t(ratios.size()), ratios.data(), 4, kv, 8, idx, 20, out.data()) == CSA2_OK);
    EXPECT(out[0].group == -1 && out[1].mode == -1);
    EXPECT(out[20].mode == CSA2_FULL && out[20].make_pool == 1 && out[24].mode == CSA2_REINDEX && out[24].source == 20);
    EXPECT(out[39].mode == CSA2_REUSE && out[39].source == 36 && out[7].source == 2);
    const int32_t bad_kv[] = {8, 2};
    EXPECT(csa2_layer_plan(int32_t(ratios.size()), ratios.data(), 2, bad_kv, 8, idx, 20, out.data()) ==
           CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_layer_plan(int32_t(ratios.size()), ratios.data(), 4, kv, 8, idx, 3, out.data()) == CSA2_ERR_INVALID_ARG);
    EXPECT(csa2_layer_plan(0, ratios.data(), 4, kv, 8, idx, 20, out.data()) == CSA2_ERR_INVALID_ARG);
  }

  if (g_failures == 0) std::printf("abi_host_check: all host checks passed\n");
  return g_failures == 0 ? 0 : 1;
}
