/*
 * csa2.h - C ABI of the CSA2 sparse-attention hot path on AMD MI355X (gfx950).
 *
 * CSA2 is the compressed sparse attention of the DeepSeek-V4.1-Flash technical
 * report as described on the web pages this library follows:
 *   [ZB]   zartbot's walkthrough of the report (hn.213312.xyz), sections 1-3;
 *   [ELPH] elph.ru, "DeepSeek-V4.1 Flash: Squeezing the KV Cache Fourfold for
 *          Long Context";
 *   [36KR] eu.36kr.com, "What 'black technologies' does DeepSeek V4.1 Flash
 *          adopt?".
 * A layer keeps one shared latent main KV (512 channels, 64 of them rotary)
 * and an indexer K projected from it; a lightweight indexer scores the
 * entries, a top-k picks 512 of them (optionally through the hierarchical
 * sparse indexer's block pool), and attention runs over the picked rows
 * concatenated with a 128-row sliding window.  Layers share caches in Full,
 * Reindex or Reuse mode.
 *
 * Conventions for every entry point:
 *  - All array arguments are DEVICE pointers unless stated otherwise; the
 *    caller owns every buffer (inputs, outputs, caches, workspace).  The
 *    library allocates nothing on a call path and keeps no pointer after the
 *    call returns.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *    default stream).  Results are valid after the caller synchronises.
 *    csa2_layer_group may run some of its launches on streams of the
 *    library's own, ordered by events after and before work on `stream`
 *    (see there); to the caller it behaves as if all ran on `stream`.
 *  - Every argument that the host can check is checked before any HIP call;
 *    a failing check returns a negative csa2_status and enqueues nothing.
 *    Values that live on the device (positions, entry counts, indices) are
 *    clamped or skipped by the kernels, never trusted for addressing.
 *  - Errors from a kernel that faults surface at the caller's next
 *    synchronisation, as with any HIP work.
 *  - No C++ exception crosses this boundary.  csa2_last_error() returns a
 *    message for the failing call (cleared when a call starts).
 *  - Calls on different streams with different outputs and workspaces may
 *    run concurrently.
 *
 * Layouts are row-major, innermost index last.  "act" is the activation
 * element type of csa2_dims.act_dtype (float32 or bfloat16 bit patterns).
 * n_q, the queries per sequence of a call, is 1..65535.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_ABI_VERSION 7

typedef enum csa2_status {
  CSA2_OK = 0,
  CSA2_ERR_INVALID_ARG = -1, /* NULL where required, non-positive or inconsistent sizes, misalignment */
  CSA2_ERR_UNSUPPORTED = -2, /* dtype, ratio, mode or shape the kernels do not implement */
  CSA2_ERR_WORKSPACE = -3,   /* workspace missing or smaller than csa2_workspace_size() */
  CSA2_ERR_MODE_ORDER = -4,  /* Reindex/Reuse source is not a suitable earlier layer */
  CSA2_ERR_HIP = -5          /* a HIP runtime call or kernel launch failed */
} csa2_status;

typedef enum csa2_dtype {
  CSA2_F32 = 0,  /* IEEE float32 */
  CSA2_BF16 = 1, /* bfloat16 bit patterns (uint16) */
  CSA2_FP4 = 2,  /* cache only: E2M1 codes, two per byte (even channel in the low
                    nibble), plus one E4M3 (FN) scale byte per group of channels */
  CSA2_FP8 = 3   /* window rows only: one E4M3 (FN) byte per channel, no scale
                    ([ZB] 2.4.4: the window KV stays in FP8) */
} csa2_dtype;

typedef enum csa2_mode {
  CSA2_FULL = 0,    /* score all visible entries, write the top-k (and the HSI pool) */
  CSA2_REINDEX = 1, /* rescore the shared indexer K with the layer's own indexer Q */
  CSA2_REUSE = 2    /* read an earlier layer's top-k; never touches indexer K */
} csa2_mode;

typedef enum csa2_entry_point {
  CSA2_EP_COMPRESS = 0,
  CSA2_EP_INDEX_TOPK = 1,
  CSA2_EP_SPARSE_ATTN = 2,
  CSA2_EP_LAYER_GROUP = 3
} csa2_entry_point;

/* Shape of one CSA2 layer ([ZB] section 1.2 hyper-parameters). */
typedef struct csa2_dims {
  int32_t d;           /* latent width = query head width (512); a multiple of 32 in 32..1024 */
  int32_t d_rope;      /* trailing rotary channels of the latent (64); even, <= min(d, 128) */
  int32_t n_heads;     /* main query heads (64); 1..1024 */
  int32_t n_idx_heads; /* indexer heads (32); n_idx_heads * d_idx <= 8192 */
  int32_t d_idx;       /* indexer head width = indexer-K width (128); a multiple of 32 up to 512 */
  int32_t topk;        /* entries kept per query (512); 1..2048 */
  int32_t window;      /* sliding-window rows per query (128); 0..4096 */
  int32_t block_size;  /* HSI block size (8); must be 8 */
  int32_t cand_blocks; /* HSI pool size in blocks (2048); 1..2048 */
  int32_t act_dtype;   /* CSA2_F32 or CSA2_BF16 for latent, W_ik, q, idx_q, window rows, out */
  double rope_theta;   /* RoPE base (10000) */
  int32_t swa_dtype;   /* window-row elements: 0 = act_dtype, or CSA2_FP8 */
  int32_t rope_orig_len; /* YaRN: original context length (65536 in [ZB] 1.2); used when rope_factor > 1 */
  double rope_factor;  /* YaRN context-extension factor s ([ZB] 1.2: 16); 0 or 1 = plain RoPE.  With s > 1
                          rotary pair m turns at (1 - g) f_m / s + g f_m, f_m = theta^(-2m/d_rope),
                          g = clamp((L f_m / (2 pi) - 1) / 31, 0, 1) with L = rope_orig_len, and the
                          attention logits are scaled by (0.1 ln s + 1)^2 on top of 1/sqrt(d) */
} csa2_dims;

/* The shared caches of one layer group: main KV and indexer K.
 *
 * Entry j of sequence b is the merge of latent positions ratio*j ..
 * ratio*j+ratio-1, rotated at position ratio*j+ratio-1 ([ZB] 2.3.1, 2.4.4).
 * It is visible to a query at position t iff ratio*j + ratio - 1 <= t and
 * j < n_entries[b].
 *
 *  F32 / BF16:  main  [batch][capacity][d]      act-sized elements of kv_dtype
 *               idx_k tiled, rows of d_idx elements (below)
 *  FP4:         main  [batch][capacity][d/2]     bytes (E2M1 codes)
 *               main_scale [batch][capacity][d/main_group]     E4M3 bytes
 *               idx_k tiled, rows of d_idx/2 bytes (E2M1 codes)
 *               idx_scale  [batch][capacity][d_idx/idx_group]  E4M3 bytes
 *
 * Indexer K tiles: with P = capacity rounded up to a multiple of 32 and RB
 * the row's bytes (4 d_idx, 2 d_idx or d_idx/2), idx_k holds batch * P * RB
 * bytes; sequence b starts at byte b * P * RB and its rows form tiles of 32
 * (tile t = rows 32t .. 32t+31, 32 * RB bytes).  Inside a tile the rows'
 * 16-byte chunks are transposed: bytes [16c, 16c + 16) of row 32t + r lie at
 * tile byte (32c + r) * 16.  The indexer's matrix-core loads, one row per
 * lane, are then contiguous across lanes.  Padding rows are never read for
 * an entry.
 * All base pointers must be 16-byte aligned.
 */
typedef struct csa2_kv_cache {
  int32_t kv_dtype;   /* CSA2_F32, CSA2_BF16 or CSA2_FP4 */
  int32_t ratio;      /* compress ratio the entries were made with: 1 or 2 */
  int32_t main_group; /* FP4: channels per scale in main KV: 16 or 32 ([ZB] 2.4.4 says 16) */
  int32_t idx_group;  /* FP4: channels per scale in indexer K: 16 or 32 */
  int32_t batch;      /* sequences; 1..65535 */
  int32_t reserved0;  /* must be 0 */
  int64_t capacity;   /* entry slots per sequence; 1 .. 1048576 */
  void* main;
  uint8_t* main_scale;     /* FP4 only, else NULL */
  void* idx_k;             /* may be NULL for calls that never read it (Reuse attention) */
  uint8_t* idx_scale;      /* FP4 only, else NULL */
  const int32_t* n_entries; /* device [batch]; values are clamped to [0, capacity] */
} csa2_kv_cache;

/* csa2_compress - write new cache entries from latent rows (path step a1/a2/a7).
 *
 * [ZB] 2.3.1: ratio-2 layers merge two adjacent positions into one entry
 * with per-channel learned weights, ratio-1 layers keep one entry per
 * position, and the indexer K is projected from the main KV.  For each
 * sequence b and m in 0 .. n_pos/ratio-1, entry j = first_pos[b]/ratio + m:
 *   e[c]   = sum_i softmax_i(pair_logits[:, c]) * latent[b][ratio*m + i][c]
 *   e_hat  = e with its last d_rope channels rotated at position ratio*j+ratio-1
 *   main[j]  = store(e_hat)                 (round to nearest even / FP4 codec)
 *   idx_k[j] = store(e_hat . W_ik)          (from the unrounded e_hat)
 * The merge, rotation and projection run in float64, so the stored bits are
 * the single rounding of the exact value.
 *
 *  latent      [batch][n_pos][d] act
 *  first_pos   device [batch]: position of latent row 0; a multiple of ratio
 *  n_pos       rows per sequence; a positive multiple of cache->ratio
 *  pair_logits device [ratio][d] float32; NULL iff ratio == 1
 *  w_ik        device [d][d_idx] act
 * Entries that fall outside [0, capacity) are not written.  n_entries is
 * not updated: the caller owns it.
 */
int csa2_compress(const csa2_dims* dims, const csa2_kv_cache* cache, const void* latent,
                  const int32_t* first_pos, int32_t n_pos, const float* pair_logits, const void* w_ik,
                  void* stream);

/* csa2_index_topk - indexer scores and top-k selection (path steps a3/a4).
 *
 * Score of entry j for query (b, t) ([ZB] 2.3.1 lightweight indexer):
 *   s_j = sum_h head_w[h] * max(0, idx_q[h] . K_j)
 * over the domain: every visible entry (pool_in == NULL), or the visible
 * entries of the blocks listed in pool_in (Reindex, [ZB] 2.3.4).  The top-k
 * keeps the topk highest scores, ties to the lower entry id, and is written
 * in ascending entry id, padded with -1.
 * With pool_out != NULL the HSI pool is also built ([ZB] 2.3.4): the
 * per-block maximum of the full scores over aligned blocks of block_size,
 * the block of the newest visible entry forced in, then the best blocks up
 * to cand_blocks (ties to the lower block), written ascending, padded -1.
 *
 *  idx_q     [batch][n_q][n_idx_heads][d_idx] act
 *  head_w    [batch][n_q][n_idx_heads] float32
 *  q_pos     [batch][n_q] int32 token positions (>= 0)
 *  pool_in   NULL or [batch][n_q][cand_blocks] int32 block ids
 *  topk_out  [batch][n_q][topk] int32
 *  pool_out  NULL or [batch][n_q][cand_blocks] int32 (not allowed with pool_in)
 *  topk_scores NULL or [batch][n_q][topk] float32: score of each kept entry
 *  ws        workspace of at least csa2_workspace_size(..., CSA2_EP_INDEX_TOPK, n_q) bytes,
 *            256-byte aligned
 */
int csa2_index_topk(const csa2_dims* dims, const csa2_kv_cache* cache, const void* idx_q,
                    const float* head_w, const int32_t* q_pos, int32_t n_q, const int32_t* pool_in,
                    int32_t* topk_out, int32_t* pool_out, float* topk_scores, void* ws, size_t ws_bytes,
                    void* stream);

/* csa2_sparse_attn - attention over the kept entries plus the window (path step a5).
 *
 * [ZB] 2.2.2: global (sparse) KV and local (window) KV are concatenated and
 * scored together with Q; [ZB] 3.3.1: key equals value.  For query (b, t)
 * and head h, with q_hat = q rotated at t on its last d_rope channels:
 *   rows  = [main[j] for j in topk (j >= 0)] ++ [swa row of p for p in
 *            max(0, t-window+1) .. t that lies in the window buffer]
 *   out_h = softmax(q_hat . rows^T / sqrt(d)) . rows,  lse_h = log(sum exp(.))
 *
 *  q             [batch][n_q][n_heads][d] act (not rotated)
 *  q_pos         [batch][n_q] int32
 *  topk          [batch][n_q][topk] int32 entry ids or -1
 *  swa_kv        [batch][n_swa][d] act (or E4M3 bytes if dims->swa_dtype is CSA2_FP8),
 *                rows already rotated
 *  swa_first_pos [batch] int32: position of window-buffer row 0
 *  out           [batch][n_q][n_heads][d] act
 *  lse           NULL or [batch][n_q][n_heads] float32 (natural log)
 *  ws            at least csa2_workspace_size(..., CSA2_EP_SPARSE_ATTN, n_q) bytes
 * cache->idx_k may be NULL.
 */
int csa2_sparse_attn(const csa2_dims* dims, const csa2_kv_cache* cache, const void* q,
                     const int32_t* q_pos, int32_t n_q, const int32_t* topk, const void* swa_kv,
                     const int32_t* swa_first_pos, int32_t n_swa, void* out, float* lse, void* ws,
                     size_t ws_bytes, void* stream);

/* One layer of a csa2_layer_group call ([ZB] 2.3.2, 3.2 access table). */
typedef struct csa2_layer {
  int32_t mode;      /* csa2_mode */
  int32_t source;    /* REINDEX: earlier FULL layer (with make_pool) whose pool is searched,
                        or -1 to search every visible entry; REUSE: earlier FULL or REINDEX
                        layer whose top-k is read; FULL: must be -1 */
  int32_t make_pool; /* FULL: nonzero builds the HSI pool into `pool` */
  int32_t n_swa;     /* window-buffer rows */
  const void* q;     /* [batch][n_q][n_heads][d] act */
  const void* idx_q; /* FULL/REINDEX: [batch][n_q][n_idx_heads][d_idx] act; REUSE: NULL */
  const float* head_w; /* FULL/REINDEX: [batch][n_q][n_idx_heads]; REUSE: NULL */
  const void* swa_kv;  /* [batch][n_swa][d] act, or E4M3 bytes (dims->swa_dtype) */
  const int32_t* swa_first_pos; /* [batch] */
  void* out;         /* [batch][n_q][n_heads][d] act */
  float* lse;        /* NULL or [batch][n_q][n_heads] */
  int32_t* topk;     /* FULL/REINDEX: written, [batch][n_q][topk]; REUSE: NULL, or receives
                        a copy of the source's top-k */
  int32_t* pool;     /* FULL with make_pool: written, [batch][n_q][cand_blocks]; else NULL */
} csa2_layer;

/* New latent rows to compress before the group runs (Full-mode cache write). */
typedef struct csa2_compress_args {
  const void* latent;
  const int32_t* first_pos;
  int32_t n_pos;
  int32_t reserved0; /* must be 0 */
  const float* pair_logits;
  const void* w_ik;
} csa2_compress_args;

/* csa2_layer_group - run layers that share one main KV and indexer K (path step a6).
 *
 * Layers run in order on `stream`.  If `compress` is non-NULL its rows are
 * written into the cache first (csa2_compress).  Full layers score every
 * visible entry; Reindex layers rescore the pool of their source (or every
 * visible entry) with their own indexer Q; Reuse layers attend with their
 * source's top-k.  Reindex and Reuse never write the caches and Reuse
 * never reads the indexer K ([ZB] 3.2).  Sources must be earlier layers:
 * reuse flows only from earlier to later layers ([ZB] 3.3.1).
 *  q_pos  [batch][n_q] int32, shared by all layers
 *  ws     at least csa2_workspace_size(..., CSA2_EP_LAYER_GROUP, n_q) bytes
 *
 * One-entry decode steps.  When compress writes one entry per sequence
 * (n_pos = ratio), n_q = 1, d = 512 and the first layer's index step runs on
 * the matrix cores over every visible entry (32 x 128 indexer, bf16
 * activations, a bf16 cache or an FP4 cache with scales per 32), the group
 * launches no compress kernel: the first index step's scan writes the entry
 * (its extra workgroups run the compressor, with the same arithmetic and the
 * same stored bytes, and score the new entry) and the selection folds that
 * score in (kernel trace: CSA2_KERNEL_SCAN_BF16_FUSED / _FP4_FUSED).  The
 * results are those of csa2_compress followed by the layers, bit for bit.
 *
 * Attention streams.  An attention launch needs only the top-k of one index
 * step (its layer's, or its Reuse source's), not the index steps after it
 * nor the other layers' attention.  When the attention runs one workgroup
 * per query (128 or more queries per sequence, 64 heads) and the group has
 * more than one layer, the index steps run in order on `stream` and the
 * attention launches alternate between the library's two streams of this
 * device (non-blocking, default priority), each after an event recorded on
 * `stream` behind the index step that feeds it, each in its own slice of ws;
 * `stream` then waits for those streams before the call returns, so work
 * enqueued on `stream` afterwards sees every result.  The events and waits
 * are captured into a HIP graph as its edges.  Every launch stays on
 * `stream` otherwise, and also when a buffer one layer writes (out, lse,
 * topk, pool) overlaps one another layer reads or writes, or when the
 * streams do not exist yet on this device and `stream` is being captured
 * (they are created, once, by the first call that is not).  Calls from
 * several host threads are serialised while they enqueue (one lock for the
 * library's streams and events).
 *
 * Paired merges.  When every launch stays on `stream` and the layers'
 * buffers are independent (as above), a row-split attention's merge may run
 * after the next layer's attention, both layers' merges in one launch; each
 * output element is combined in the same order, so the results are the same.
 */
int csa2_layer_group(const csa2_dims* dims, const csa2_kv_cache* cache, int32_t n_layers,
                     const csa2_layer* layers, const int32_t* q_pos, int32_t n_q,
                     const csa2_compress_args* compress, void* ws, size_t ws_bytes, void* stream);

/* csa2_layer_plan - the cross-layer plan of a CSA2 model (host logic, no GPU work).
 *
 * [ZB] 1.2 gives a model's schedule as per-layer compress ratios (0 = the
 * layer keeps no compressed KV), the kv-source layers (which write a main KV
 * and indexer K: 2, 8, 14, 20), the index-source layers (which compute their
 * own top-k: 2, 8, 14, 20, 24, 28, 32, 36) and the candidate-source layer (the
 * Full layer that builds the HSI pool: 20); [ZB] 2.3.3 describes the encoder
 * blocks (a Full layer, then Reuse layers) and the decoder (a Full block, then
 * Reindex blocks searching its pool), [ZB] 3.3.1 and 3.3.3 that reuse only
 * flows from earlier to later layers.  Readings of those passages, applied per
 * layer l (0-based):
 *   ratio 0:              a window-only layer: group -1, mode -1, source -1
 *   a kv-source layer:    opens the cache group l; mode CSA2_FULL (it must be
 *                         an index source); make_pool = 1 if l is the
 *                         candidate source
 *   another index source: CSA2_REINDEX in the current group; source = the
 *                         group's Full layer if that builds the pool, else -1
 *                         (every visible entry)
 *   any other layer:      CSA2_REUSE of the latest index-source layer of its
 *                         group
 * A layer with compressed KV belongs to the latest kv-source layer, which must
 * have its ratio with no layer of another ratio in between.
 *  ratios   host [n_layers]: 0, 1 or 2
 *  kv_src   host [n_kv], idx_src host [n_idx]: ascending, distinct layer numbers
 *  cand_src a kv-source layer, or -1 (no pool)
 *  out      host [n_layers], written
 * Returns CSA2_OK or CSA2_ERR_INVALID_ARG (csa2_last_error() says why). */
typedef struct csa2_plan_layer {
  int32_t group;     /* kv-source layer whose caches the layer uses; -1: window-only */
  int32_t mode;      /* csa2_mode, or -1 for a window-only layer */
  int32_t source;    /* REINDEX: the layer whose pool is searched, or -1; REUSE: the layer whose top-k
                        is read; FULL: -1 (layer numbers, not positions in the group) */
  int32_t make_pool; /* FULL: builds the HSI pool */
} csa2_plan_layer;
int csa2_layer_plan(int32_t n_layers, const int32_t* ratios, int32_t n_kv, const int32_t* kv_src, int32_t n_idx,
                    const int32_t* idx_src, int32_t cand_src, csa2_plan_layer* out);

/* csa2_layer_group_noalloc - csa2_layer_group for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.
 *
 * Same arguments (less the workspace), checks, kernels and results as
 * csa2_layer_group, with every launch on `stream` (no attention streams).
 * The scratch the kernels need (indexer scores, block maxima, one slice of
 * attention split partials: at most csa2_workspace_size(...,
 * CSA2_EP_LAYER_GROUP, n_q) bytes) lives in a device array inside the
 * library of CSA2_NOALLOC_SCRATCH_BYTES (64 MiB), one copy per GPU, held
 * until the process ends.  That covers decode shapes (one query per
 * sequence) of up to about 12 sequences at 1M entries or 16 at 256K; a call
 * that needs more returns CSA2_ERR_WORKSPACE before any HIP work.  The first
 * call on a device looks up that device's copy (hipGetSymbolAddress); no call
 * allocates or frees memory.  Every call on one GPU uses the same array,
 * which keeps the last call's contents (nothing in it has to start at zero):
 * calls that overlap on one GPU - on different streams, or from different
 * host threads - race, and the caller must order them.  Returns a
 * csa2_status. */
#define CSA2_NOALLOC_SCRATCH_BYTES (64u << 20)
int csa2_layer_group_noalloc(const csa2_dims* dims, const csa2_kv_cache* cache, int32_t n_layers,
                             const csa2_layer* layers, const int32_t* q_pos, int32_t n_q,
                             const csa2_compress_args* compress, void* stream);

/* csa2_grouped_out_proj - the grouped low-rank output projection after the
 * attention ([ZB] 1.2: o_lora_rank 1024 in o_groups 8).
 *
 * The width = n_heads * d channels of an attention output row split into
 * n_groups contiguous slices of K = width / n_groups (the outputs of
 * n_heads / n_groups heads); group g maps its slice to `rank` outputs with its
 * own matrix:
 *   y[t][g*rank + r] = sum_c x[t][g*K + c] * w[g][r][c]
 * accumulated in float32 and stored in act_dtype (bf16: round to nearest
 * even).  The rank outputs of the groups are concatenated.
 *
 *  act_dtype  CSA2_F32 or CSA2_BF16, for x, w and y
 *  n_tok      rows of x and y (batch * n_q for a csa2_sparse_attn output); 0 does nothing
 *  x          [n_tok][width] act: the attention output, read only
 *  w          [n_groups][rank][K] act: each output's weights over its group's slice, read only
 *  y          [n_tok][n_groups*rank] act, written; must not overlap x or w
 * width must be a positive multiple of n_groups, rank positive; x, w and y
 * device pointers, 16-byte aligned.  bf16 with K a multiple of 64 and rank a
 * multiple of 32 runs on the matrix cores; other shapes run a plain kernel.
 * No workspace; nothing is allocated.  Returns a csa2_status.
 */
int csa2_grouped_out_proj(int32_t act_dtype, int32_t n_tok, int32_t width, int32_t n_groups, int32_t rank,
                          const void* x, const void* w, void* y, void* stream);

/* Bytes of workspace an entry point needs for n_q queries per sequence, or 0
 * if the arguments are invalid (csa2_last_error() then says why).  Sized
 * from cache->capacity and cache->batch.  CSA2_EP_LAYER_GROUP: the index
 * scratch and one attention slice per attention stream (two). */
size_t csa2_workspace_size(const csa2_dims* dims, const csa2_kv_cache* cache, int32_t entry_point,
                           int32_t n_q);

/* Static string naming a csa2_status. */
const char* csa2_status_str(int status);

/* Message of the last failing call on this thread; every entry point clears it
 * on entry, so it is "" after a call that succeeded. */
const char* csa2_last_error(void);

/* CSA2_ABI_VERSION of the loaded library. */
int32_t csa2_abi_version(void);

/* ---------------------------------------------------------- kernel trace --
 * Optional timing of every kernel the library launches, for profiling.  When
 * enabled, each launch carries a start and a stop HIP event that the runtime
 * stamps with the kernel's own start and end times on the device, so a
 * record's time is that kernel's duration, in launch order.  Off by default;
 * the entry points then launch plainly.  Not for use under stream capture. */
typedef enum csa2_kernel {
  CSA2_KERNEL_COMPRESS = 1,       /* compress_kernel (both activation types) */
  CSA2_KERNEL_SCAN_GENERIC = 2,   /* scan_generic_kernel */
  CSA2_KERNEL_SCAN_BF16 = 3,      /* scan_mfma_bf16_kernel */
  CSA2_KERNEL_SCAN_FP4 = 4,       /* scan_mfma_fp4_kernel */
  CSA2_KERNEL_SELECT = 5,         /* select_kernel */
  CSA2_KERNEL_ATTN_GENERIC = 6,   /* attn_generic_kernel */
  CSA2_KERNEL_ATTN_BF16 = 7,      /* attn_mfma_kernel over a bf16 cache */
  CSA2_KERNEL_ATTN_FP4 = 8,       /* attn_mfma_kernel over an FP4 cache, scales per 32 */
  CSA2_KERNEL_ATTN_MERGE = 9,     /* attn_merge_kernel */
  CSA2_KERNEL_ATTN_FP4_G16 = 10,  /* attn_mfma_kernel over an FP4 cache, scales per 16 */
  CSA2_KERNEL_SCAN_PREFILL = 11,  /* scan_prefill_kernel (many queries per sequence) */
  CSA2_KERNEL_OPROJ_MFMA = 12,    /* oproj_mfma_kernel (bf16 grouped output projection, K split) */
  CSA2_KERNEL_OPROJ_GENERIC = 13, /* oproj_generic_kernel */
  CSA2_KERNEL_OPROJ_MFMA16 = 14,  /* oproj_mfma16_kernel (bf16 grouped output projection, <= 16 rows) */
  CSA2_KERNEL_OPROJ_LDS = 15,     /* oproj_lds_kernel (bf16 grouped output projection, 128 x 128 tiles) */
  CSA2_KERNEL_READ_PROBE = 16,    /* read_probe_kernel (csa2_read_probe) */
  CSA2_KERNEL_MFMA_PROBE = 17,    /* mfma_probe_kernel (csa2_mfma_probe) */
  CSA2_KERNEL_SCAN_BF16_FUSED = 18, /* scan_fused_bf16_kernel: bf16 decode scan that writes the step's entry */
  CSA2_KERNEL_SCAN_FP4_FUSED = 19   /* scan_fused_fp4_kernel: FP4 decode scan that writes the step's entry */
} csa2_kernel;

typedef struct csa2_trace_record {
  int32_t kernel; /* csa2_kernel */
  float ms;       /* the kernel's duration on the device */
} csa2_trace_record;

/* Enable tracing of up to max_kernels launches (creating 2 * max_kernels HIP
 * events on the current device, which launches must then target), or disable
 * it and free the events when max_kernels is 0.  Drops any unread records.
 * Launches beyond max_kernels before the next read are not recorded and are
 * counted as dropped.  Returns a csa2_status. */
int csa2_trace_enable(int32_t max_kernels);

/* Wait for the recorded launches to finish and copy up to `max` records, in
 * launch order, into host array `out`; then start a new recording.  Returns
 * the number of records copied (>= 0) or a negative csa2_status.  If n_dropped
 * is not NULL it receives the number of launches not recorded (beyond the
 * capacity, or beyond `max`). */
int csa2_trace_read(csa2_trace_record* out, int32_t max, int32_t* n_dropped);

/* Static name of a csa2_kernel: the name of its __global__ function. */
const char* csa2_kernel_name(int32_t kernel);

/* csa2_read_probe - measurement utility, not a step of the method.
 *
 * Reads `bytes` bytes of device buffer `buf` once with a plain coalesced
 * streaming kernel (16-byte loads, 8 in flight per lane, 32 KB contiguous
 * per workgroup and iteration).  Its device duration, taken from the kernel
 * trace (CSA2_KERNEL_READ_PROBE), is the time this GPU needs to stream a
 * working set of that size: the measured read ceiling that a bandwidth-bound
 * kernel of the path is compared with, next to the published HBM peak.
 *  buf    device pointer, 16-byte aligned, read only
 *  bytes  a positive multiple of 16
 *  sink   device uint32, written only if the XOR of every word read equals
 *         a fixed constant (keeps the loads from being removed); may hold
 *         anything before and after
 * Enqueued on `stream`; allocates nothing.  Returns a csa2_status. */
int csa2_read_probe(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

/* csa2_mfma_probe - measurement utility, not a step of the method.
 *
 * Runs `workgroups` workgroups of 4 waves, two per compute unit, each wave
 * doing CSA2_MFMA_PROBE_CHAINS independent chains of `iters` bf16 matrix
 * products of 32 x 32 x 16 (v_mfma_f32_32x32x16_bf16, fp32 accumulation) on
 * register operands, with no memory traffic but one conditional store:
 * workgroups * CSA2_MFMA_PROBE_FLOP_PER_WG_ITER * iters flops.  Its device
 * duration, taken from the kernel trace (CSA2_KERNEL_MFMA_PROBE), gives the
 * bf16 matrix-core rate this GPU sustains under a full matrix load (at the
 * clock it holds then): the measured ceiling that the matrix-bound indexer
 * scan is compared with, next to the published peak.
 *  iters       1 .. 2^24
 *  workgroups  1 .. 65536
 *  sink        device float, written only if the accumulated sum equals a
 *              fixed constant (keeps the products from being removed)
 * Enqueued on `stream`; allocates nothing.  Returns a csa2_status. */
#define CSA2_MFMA_PROBE_CHAINS 8
#define CSA2_MFMA_PROBE_FLOP_PER_WG_ITER (4 * CSA2_MFMA_PROBE_CHAINS * 32768)
int csa2_mfma_probe(int64_t iters, int32_t workgroups, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
