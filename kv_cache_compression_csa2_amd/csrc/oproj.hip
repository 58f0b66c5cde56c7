// Grouped low-rank output projection after the attention.
//
// Pages: zartbot walkthrough (hn.213312.xyz) section 1.2: the output
// projection is split into o_groups = 8 groups, with o_lora_rank = 1024 per
// group.  Group g takes its own contiguous slice of the concatenated head
// outputs (n_heads / o_groups heads, K = n_heads d / o_groups channels) to
// `rank` outputs:
//   y[t][g rank + r] = sum_c x[t][g K + c] * w[g][r][c]
// with float32 accumulation, stored in the activation type (bf16: round to
// nearest even).
//
// The bf16 path runs on the matrix cores in three kernels: at most 16 rows
// (decode) oproj_mfma16_kernel streams the 8 x 1024 x 4096 weights once
// (HBM-bound); many rows, with 128-output tiles, oproj_lds_kernel stages
// 128 x 128 tiles through LDS (matrix-bound); other shapes take
// oproj_mfma_kernel, whose 16 waves split K over one 32 x 32 tile.  Each is
// described at its definition.
#include "device_common.hpp"
#include "launch.hpp"

namespace csa2 {
namespace {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(16)));
typedef float f32x16_t __attribute__((__vector_size__(64)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// One 64-channel chunk of a lane's operands: A from the token row, B from
// NT weight rows.  Lane (i, h) (i = lane % 32, h = lane / 32) holds channels
// 32 h + 8 u .. 32 h + 8 u + 7 of the chunk in element u of each array, and
// product u of the chunk contracts exactly those channels on both sides.
template <int NT>
struct OpChunk {
  uint4 a[4];
  uint4 b[NT][4];
};

// NT: 32-output tiles per wave; the WAVES waves share one 32 x NT*32 tile
// and split K.
template <int NT, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void oproj_mfma_kernel(int n_tok, int width, int rank,
                                                                   const uint16_t* __restrict__ x,
                                                                   const uint16_t* __restrict__ w,
                                                                   uint16_t* __restrict__ y) {
  extern __shared__ float red[];  // [WAVES][NT][16][64]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int i = lane & 31, h = lane >> 5;
  const int g = blockIdx.z;
  const int t0 = blockIdx.x * 32, r0 = blockIdx.y * 32 * NT;
  const int n_groups = gridDim.z;
  const int K = width / n_groups, nchunk = K / 64;
  const int c_first = wv, c_step = WAVES;

  // rows past the last token repeat it; their products are never stored
  const uint16_t* xrow = x + int64_t(min(t0 + i, n_tok - 1)) * width + int64_t(g) * K + 32 * h;
  const uint16_t* wrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) wrow[t] = w + (int64_t(g) * rank + r0 + 32 * t + i) * K + 32 * h;

  auto issue = [&](int c, OpChunk<NT>& ch) {
#pragma unroll
    for (int u = 0; u < 4; ++u) ch.a[u] = *reinterpret_cast<const uint4*>(xrow + 64 * c + 8 * u);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int u = 0; u < 4; ++u) ch.b[t][u] = *reinterpret_cast<const uint4*>(wrow[t] + 64 * c + 8 * u);
    __builtin_amdgcn_sched_barrier(0);
  };

  f32x16_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;

  // keep: all ones, or zero for a chunk past the wave's range (its products
  // then add zero; a branch instead would let the compiler sink the chunk's
  // loads into it, after the other buffer's wait)
  auto contract = [&](const OpChunk<NT>& ch, uint32_t keep) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint4 a = {ch.a[u].x & keep, ch.a[u].y & keep, ch.a[u].z & keep, ch.a[u].w & keep};
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(ch.b[t][u]), acc[t], 0, 0, 0);
    }
  };

  // one chunk in flight while the other is contracted, in two fixed buffers
  // (a copy from the prefetch buffer would make the compiler wait for the
  // prefetch); the loads are unconditional (a wave past its last chunk
  // re-reads a valid one and never uses it), so the wait counts stay exact.
  // (A ring of three measured slower at K 4096: 28 against 20 us in decode.)
  OpChunk<NT> b0, b1;
  issue(min(c_first, nchunk - 1), b0);
  for (int c = c_first; c < nchunk; c += 2 * c_step) {
    issue(min(c + c_step, nchunk - 1), b1);
    contract(b0, ~0u);
    issue(min(c + 2 * c_step, nchunk - 1), b0);
    contract(b1, c + c_step < nchunk ? ~0u : 0u);
  }

  // partial tiles of the waves, summed through LDS (lane-contiguous: no bank
  // conflicts); product element r of lane l: row 8 (r / 4) + 4 (l / 32) +
  // r % 4, column l % 32
  const int out_w = n_groups * rank;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[((wv * NT + t) * 16 + r) * 64 + lane] = acc[t][r];
  __syncthreads();
  for (int o = threadIdx.x; o < NT * 1024; o += WAVES * kWave) {
    const int t = o >> 10, r = (o >> 6) & 15, l = o & 63;
    float s = 0.0f;
#pragma unroll
    for (int v = 0; v < WAVES; ++v) s += red[((v * NT + t) * 16 + r) * 64 + l];
    const int tok = t0 + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
    if (tok < n_tok) y[int64_t(tok) * out_w + int64_t(g) * rank + r0 + 32 * t + (l & 31)] = f32_to_bf16(s);
  }
}

// At most 16 tokens (decode): the 16 x 16 x 32 product, whose A operand is
// exactly the 16 token rows.  A workgroup computes the 16 tokens x 32 outputs
// of one group; its 16 waves split K as above, but each wave issues up to 4
// chunks at once (6 loads per lane per chunk), so a workgroup asks for its
// whole weight tile (32 rows x K) in one go.  Lane (j, q) (j = lane % 16,
// q = lane / 16) holds channels 16 q + 8 u .. 16 q + 8 u + 7 of a chunk for
// product u of it (u = 0, 1).
constexpr int kDecWaves = 16;
constexpr int kDecAhead = 4;
typedef float f32x4_t __attribute__((__vector_size__(16)));

__global__ __launch_bounds__(kDecWaves * kWave) void oproj_mfma16_kernel(int n_tok, int width, int rank,
                                                                          const uint16_t* __restrict__ x,
                                                                          const uint16_t* __restrict__ w,
                                                                          uint16_t* __restrict__ y) {
  __shared__ float red[kDecWaves][2][4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int j = lane & 15, q = lane >> 4;
  const int r0 = blockIdx.y * 32, g = blockIdx.z;
  const int n_groups = gridDim.z;
  const int K = width / n_groups, nchunk = K / 64;
  // rows past the last token repeat it; their products are never stored
  const uint16_t* xrow = x + int64_t(min(j, n_tok - 1)) * width + int64_t(g) * K + 16 * q;
  const uint16_t* wrow0 = w + (int64_t(g) * rank + r0 + j) * K + 16 * q;
  const uint16_t* wrow1 = wrow0 + int64_t(16) * K;

  f32x4_t acc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[t][r] = 0.0f;
  for (int c0 = wv; c0 < nchunk; c0 += kDecAhead * kDecWaves) {
    uint4 a[kDecAhead][2], b[kDecAhead][2][2];
#pragma unroll
    for (int k = 0; k < kDecAhead; ++k) {
      const int c = min(c0 + k * kDecWaves, nchunk - 1);  // unconditional: exact wait counts
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        a[k][u] = *reinterpret_cast<const uint4*>(xrow + 64 * c + 8 * u);
        b[k][0][u] = *reinterpret_cast<const uint4*>(wrow0 + 64 * c + 8 * u);
        b[k][1][u] = *reinterpret_cast<const uint4*>(wrow1 + 64 * c + 8 * u);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < kDecAhead; ++k) {
      const uint32_t keep = c0 + k * kDecWaves < nchunk ? ~0u : 0u;  // zero for a chunk past the wave's range
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint4 av = {a[k][u].x & keep, a[k][u].y & keep, a[k][u].z & keep, a[k][u].w & keep};
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(b[k][t][u]), acc[t], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wv][t][r][lane] = acc[t][r];
  __syncthreads();
  // product element r of lane l: row 4 (l / 16) + r, column l % 16
  const int o = threadIdx.x;
  if (o < 512) {
    const int t = o >> 8, r = (o >> 6) & 3, l = o & 63;
    float s = 0.0f;
#pragma unroll
    for (int v = 0; v < kDecWaves; ++v) s += red[v][t][r][l];
    const int tok = 4 * (l >> 4) + r;
    if (tok < n_tok) y[int64_t(tok) * n_groups * rank + int64_t(g) * rank + r0 + 16 * t + (l & 15)] = f32_to_bf16(s);
  }
}

// Many tokens (prefill): a workgroup computes 128 tokens x 128 outputs of one
// group with 4 waves of 64 x 64 (2 x 2 products of 32 x 32 each).  The
// 64-channel slices of its 128 token rows and 128 weight rows are copied
// global -> LDS (global_load_lds_dwordx4: no registers, and from inline
// assembly, so the compiler neither drains nor moves them) a slice ahead into
// the other of two 32 KB stages; each wave issues 8 of a slice's 32 one-KB
// copies, so one s_waitcnt vmcnt(8) and a barrier make a slice ready.  Each
// 128-byte LDS row holds its eight 16-byte chunks XOR-swizzled by (row / 2)
// % 8, so a copy instruction still reads 8 whole rows (coalesced) and the
// operand reads of 16 consecutive rows fall on distinct bank groups.  Each
// token and weight row is fetched once per workgroup and read by two waves
// from LDS: 64 flop per byte fetched.
constexpr int kTile = 128;
constexpr uint32_t kStageBytes = 2 * kTile * 128;  // A rows then B rows: 32 KB
constexpr size_t kLdsTileBytes = 2 * kStageBytes;  // two stages: 64 KB

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved; naming it tells the compiler it changes
// Copy 16 bytes per lane from global `src` to LDS byte address `lds_addr` +
// 16 * lane.  Completion is tracked only by the caller's s_waitcnt vmcnt.
__device__ __forceinline__ void copy16_to_lds(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_addr), "v"(src) : "memory", "m0");
}
#pragma clang diagnostic pop

// byte offset of 16-byte chunk c (0..7) of LDS row r inside a stage region
__device__ __forceinline__ uint32_t tile_off(int r, int c) { return uint32_t(r * 128 + 16 * (c ^ ((r >> 1) & 7))); }

__global__ __launch_bounds__(256, 2) void oproj_lds_kernel(int n_tok, int width, int rank,
                                                             const uint16_t* __restrict__ x,
                                                             const uint16_t* __restrict__ w,
                                                             uint16_t* __restrict__ y) {
  extern __shared__ __align__(16) uint8_t tile[];  // [2 stages][A 128 rows | B 128 rows][128 bytes]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 31, h = lane >> 5;
  const int wm = wv & 1, wn = wv >> 1;
  const int t0 = blockIdx.x * kTile, r0 = blockIdx.y * kTile, g = blockIdx.z;
  const int n_groups = gridDim.z;
  const int K = width / n_groups, nchunk = K / 64;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
      uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void*)tile)));

  // copy m (0..31) of a slice: rows 8 (m % 16) .. + 7 of A (m < 16) or B;
  // lane l fills physical chunk l % 8 of row 8 (m % 16) + l / 8
  auto issue = [&](int c, int stage) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = 8 * wv + j;
      const int r = 8 * (m & 15) + (lane >> 3);
      const int ch = (lane & 7) ^ ((r >> 1) & 7);  // the logical chunk that lands there
      const uint16_t* src = m < 16
          ? x + int64_t(min(t0 + r, n_tok - 1)) * width + int64_t(g) * K + 64 * c + 8 * ch  // rows past the last token repeat it
          : w + (int64_t(g) * rank + r0 + r) * K + 64 * c + 8 * ch;
      copy16_to_lds(src, lds0 + stage * kStageBytes + m * 1024);
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  issue(0, 0);
  for (int c = 0; c < nchunk; ++c) {
    // the other stage was last read before the previous iteration's closing
    // barrier; the last slice is copied again into it, unused
    issue(min(c + 1, nchunk - 1), (c + 1) & 1);
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");  // this wave's copies of slice c have landed
    __syncthreads();                                   // and every wave's
    const uint8_t* st = tile + (c & 1) * kStageBytes;
    // lane (i, h): logical chunk 2 k + h (channels 16 k + 8 h .. + 7) of its rows
    bf16x8_t av[4][2], bv[4][2];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
        av[k][a] = *reinterpret_cast<const bf16x8_t*>(st + tile_off(64 * wm + 32 * a + i, 2 * k + h));
#pragma unroll
      for (int b = 0; b < 2; ++b)
        bv[k][b] = *reinterpret_cast<const bf16x8_t*>(st + kStageBytes / 2 + tile_off(64 * wn + 32 * b + i, 2 * k + h));
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[k][a], bv[k][b], acc[a][b], 0, 0, 0);
    __syncthreads();  // stage c & 1 is free for the next iteration's copies
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no copy may land after the workgroup ends

  // product element r of lane l: row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
  const int out_w = n_groups * rank;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = t0 + 64 * wm + 32 * a + 8 * (r >> 2) + 4 * h + (r & 3);
        if (tok < n_tok)
          y[int64_t(tok) * out_w + int64_t(g) * rank + r0 + 64 * wn + 32 * b + i] = f32_to_bf16(acc[a][b][r]);
      }
}

// Any shape and either activation type: one thread per output, float32
// accumulation in channel order.
__global__ __launch_bounds__(256) void oproj_generic_kernel(int n_tok, int width, int n_groups, int rank, int act_bf16,
                                                            const void* __restrict__ x, const void* __restrict__ w,
                                                            void* __restrict__ y) {
  const int64_t out_w = int64_t(n_groups) * rank;
  const int64_t o = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (o >= int64_t(n_tok) * out_w) return;
  const int64_t tok = o / out_w, col = o % out_w;
  const int64_t g = col / rank, r = col % rank;
  const int64_t K = width / n_groups;
  const int64_t xo = tok * width + g * K, wo = (g * rank + r) * K;
  float s = 0.0f;
  for (int64_t c = 0; c < K; ++c) s = fmaf(act_load(x, xo + c, act_bf16), act_load(w, wo + c, act_bf16), s);
  if (act_bf16)
    static_cast<uint16_t*>(y)[o] = f32_to_bf16(s);
  else
    static_cast<float*>(y)[o] = s;
}

constexpr int kSplitWaves = 16;
constexpr size_t kSplitLds = sizeof(float) * kSplitWaves * 16 * 64;  // 64 KB

}  // namespace

hipError_t launch_oproj(int32_t act_dtype, int32_t n_tok, int32_t width, int32_t n_groups, int32_t rank,
                        const void* x, const void* w, void* y, hipStream_t stream) {
  if (n_tok == 0) return hipSuccess;
  const int64_t K = width / n_groups;
  if (act_dtype == CSA2_BF16 && K % 64 == 0 && rank % 32 == 0) {
    const auto* xb = static_cast<const uint16_t*>(x);
    const auto* wb = static_cast<const uint16_t*>(w);
    auto* yb = static_cast<uint16_t*>(y);
    // the 128 x 128 tiles once they cover the chip; else the K split
    const int64_t big_tiles = (int64_t(n_tok) + 127) / 128 * (rank / 128) * n_groups;
    if (rank % 128 == 0 && big_tiles >= 256) {
      static bool attr_set = false;
      if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(oproj_lds_kernel),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(kLdsTileBytes));
        if (e != hipSuccess) return e;
        attr_set = true;
      }
      const dim3 grid(uint32_t((n_tok + 127) / 128), uint32_t(rank / 128), uint32_t(n_groups));
      return launch_kernel(CSA2_KERNEL_OPROJ_LDS, oproj_lds_kernel, grid, dim3(256), kLdsTileBytes, stream, int(n_tok),
                           int(width), int(rank), xb, wb, yb);
    }
    if (n_tok <= 16)
      return launch_kernel(CSA2_KERNEL_OPROJ_MFMA16, oproj_mfma16_kernel, dim3(1, uint32_t(rank / 32), uint32_t(n_groups)),
                           dim3(kDecWaves * kWave), 0, stream, int(n_tok), int(width), int(rank), xb, wb, yb);
    const dim3 grid(uint32_t((n_tok + 31) / 32), uint32_t(rank / 32), uint32_t(n_groups));
    return launch_kernel(CSA2_KERNEL_OPROJ_MFMA, oproj_mfma_kernel<1, kSplitWaves>, grid,
                         dim3(kSplitWaves * kWave), kSplitLds, stream, int(n_tok), int(width), int(rank), xb, wb, yb);
  }
  const int64_t total = int64_t(n_tok) * n_groups * rank;
  return launch_kernel(CSA2_KERNEL_OPROJ_GENERIC, oproj_generic_kernel, dim3(uint32_t((total + 255) / 256)), dim3(256),
                       0, stream, int(n_tok), int(width), int(n_groups), int(rank), act_dtype == CSA2_BF16 ? 1 : 0, x,
                       w, y);
}

}  // namespace csa2
