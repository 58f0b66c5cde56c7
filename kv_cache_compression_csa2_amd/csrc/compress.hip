// Compressor: merge latent rows into cache entries, rotate, store main KV,
// project and store the indexer K.
//
// Pages: zartbot walkthrough (hn.213312.xyz) section 2.3.1 (ratio 2 in the
// encoder with channel-wise learned weights, ratio 1 in the decoder, no
// overlap; indexer K projected from the main KV) and section 2.4.4 (the cache
// is quantised after RoPE, FP4 main KV).
//
// One workgroup writes one entry.  Everything before the stores runs in
// float64: the merge, the rotation (angles and sin/cos) and the 512 -> 128
// projection, so each stored value is the single rounding of the exact value
// and agrees bit-for-bit with an independent float64 computation except when
// that value sits within float64 noise of a rounding boundary.  The kernel is
// a negligible share of a decode step (one row per sequence) and of a prefill
// chunk (2048 rows), so float64 costs nothing that matters.
#include "compress_entry.hpp"

namespace csa2 {
namespace {

constexpr int kThreads = kCompressVirtual;  // one thread per virtual thread of the entry's layout

// One workgroup writes one entry (compress_entry: the float64 merge,
// rotation and projection and the exact rounding to the storage format).
// The kernel is latency-bound (one entry per sequence in decode), so the
// reads that do not depend on the entry - this thread's first batch of W_ik
// (bf16) and its rotation angle - are issued or computed while the latent
// rows are still on their way.
template <bool ACT_BF16>
__global__ __launch_bounds__(kThreads) void compress_kernel(CompressParams P) {
  extern __shared__ double sh[];
  (void)compress_entry<ACT_BF16, kThreads>(P, int(blockIdx.x), int(blockIdx.y), sh);
}

}  // namespace

CompressParams make_compress_params(const csa2_dims& dims, const csa2_kv_cache& cache, const void* latent,
                                    const int32_t* first_pos, int32_t n_pos, const float* pair_logits,
                                    const void* w_ik) {
  CompressParams P;
  P.d = dims.d;
  P.d_rope = dims.d_rope;
  P.d_idx = dims.d_idx;
  P.kv_dtype = cache.kv_dtype;
  P.main_group = cache.main_group;
  P.idx_group = cache.idx_group;
  P.ratio = cache.ratio;
  P.capacity = cache.capacity;
  P.rope = make_rope_table(dims);
  P.latent = latent;
  P.first_pos = first_pos;
  P.n_pos = n_pos;
  P.pair_logits = pair_logits;
  P.w_ik = w_ik;
  P.main = cache.main;
  P.main_scale = cache.main_scale;
  P.idx_k = cache.idx_k;
  P.idx_scale = cache.idx_scale;
  return P;
}

hipError_t launch_compress(const csa2_dims& dims, const csa2_kv_cache& cache, const void* latent,
                           const int32_t* first_pos, int32_t n_pos, const float* pair_logits, const void* w_ik,
                           hipStream_t stream) {
  const dim3 grid(n_pos / cache.ratio, cache.batch);
  const size_t lds = sizeof(double) * size_t(compress_lds_doubles(dims.d, dims.d_idx));
  auto kern = dims.act_dtype == CSA2_BF16 ? compress_kernel<true> : compress_kernel<false>;
  const hipError_t err = launch_kernel(CSA2_KERNEL_COMPRESS, kern, grid, dim3(kThreads), lds, stream,
                                       make_compress_params(dims, cache, latent, first_pos, n_pos, pair_logits, w_ik));
  return err;
}

}  // namespace csa2
