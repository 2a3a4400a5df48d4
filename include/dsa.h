/*
 * dsa.h -- C ABI of libdsa: indexed sparse attention (DSA) on AMD Instinct
 * MI355X (gfx950).
 *
 * DSA, as the pages describe it ("Optimizing Next-Gen LLM Inference: Sparse
 * Attention and Mixed Parallelism in Practice" §1 and §3.1/§3.3; "Long-Context
 * LLM Inference Optimization: From Sparse Attention to System-Level
 * Co-Design", architecture section), runs three steps per query token:
 *   1. a lightweight indexer scores every visible cached position;
 *   2. a per-query Top-K keeps the K most relevant positions;
 *   3. a sparse attention kernel reads only those rows of the multi-head latent
 *      attention (MLA) cache and attends over them.
 * The entry points below expose each step and the fused pass.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers to dense, row-major arrays in the
 *    shapes given per argument.  The caller owns every buffer; the library
 *    allocates nothing (its one buffer, the fixed workspace of
 *    dsa_forward_noalloc, is a static device array), keeps no pointer after a
 *    call returns, and never synchronises: work is enqueued on `stream` (a
 *    hipStream_t; NULL is the null stream) and completes asynchronously.
 *  - Validation first: every scalar and pointer argument is checked before any
 *    HIP call.  A non-DSA_OK return enqueues nothing; dsa_last_error() then
 *    describes the problem (thread-local string).
 *  - Device-side contents are not validated (that would need a sync).  Every
 *    kernel clamps each seq_lens[b] to [0, max_seq_len] and skips index-list
 *    entries outside [0, len_b), so bad values never read out of bounds; they
 *    only give meaningless results.
 *  - Sequence b holds len_b = seq_lens[b] filled cache rows; its q_len query
 *    tokens are the last q_len of them.  Query token t sees the positions
 *    0 .. vis-1 with vis = len_b - q_len + 1 + t (causal).
 *  - Reentrant; concurrent calls on different streams must not share a
 *    workspace or an output buffer.
 *  - Workspaces of dsa_topk and dsa_forward begin with counters (one
 *    4096-bin score histogram per query) that must be zero when a call
 *    starts: the first dsa_workspace_zero_bytes(p) bytes.  Every call that
 *    returns DSA_OK leaves them zero again, so a workspace is zeroed once
 *    (dsa_workspace_init, or allocate it zeroed) and then reused without a
 *    clearing pass per call.  Zero it again after a call that failed with
 *    DSA_ERR_HIP, or before using it for a problem whose counter region is
 *    larger.  The rest of a workspace may hold anything.
 *
 * Numeric contract
 * ----------------
 *  - Index scores are accumulated in fp32 with an fp32 head reduction.  When
 *    every partial sum is an integer below 2^24 (integer-valued index queries,
 *    keys and head weights, power-of-two key scales) the scores are exact and
 *    therefore bit-identical to any exact evaluation.
 *  - Top-K ranks the fp32 scores; equal scores go to the lower position; -0
 *    equals +0.  NaN scores are not supported.
 *  - Attention logits and values are accumulated in fp32 (bf16 matrix-core
 *    products for bf16/fp8 caches), softmax uses the running-max (online)
 *    form, outputs are rounded to nearest even when out_dtype is bf16.  When
 *    the matrix-core attention splits a query's index list over several
 *    workgroups (the library's choice, for parallelism), each split's
 *    normalised output is rounded to bf16 before the fp32 merge, so an fp32
 *    out_dtype there still carries one bf16 rounding (relative 2^-9) per
 *    split; the portable kernels keep fp32 throughout.
 *
 * Workspaces
 * ----------
 *  A call whose scratch would pass 1 GiB (a long prefill chunk, a very large
 *  batch) runs as a series of launches over tiles of one sequence's query
 *  tokens, each token seeing exactly what it sees in the whole problem; the
 *  *_workspace_size functions then return one tile's scratch, which the
 *  tiles reuse in turn on `stream`.  The results are those of the whole
 *  call.  (A 4096-token chunk over 64K cached rows needs 653 MiB for
 *  dsa_forward instead of 5.1 GiB.)
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipStream_t / hipEvent_t are pointers to these opaque HIP structs. */
struct ihipStream_t;
struct ihipEvent_t;

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1,         /* bad pointer, size, dtype or scalar */
  DSA_ERR_UNSUPPORTED = 2,         /* valid but not implemented combination */
  DSA_ERR_WORKSPACE_TOO_SMALL = 3, /* ws_bytes below the *_workspace_size() value */
  DSA_ERR_HIP = 4                  /* a HIP launch reported an error */
} dsa_status;

typedef enum dsa_dtype {
  DSA_F32 = 0,       /* IEEE binary32 */
  DSA_BF16 = 1,      /* bfloat16 (upper half of binary32) */
  DSA_FP8_E4M3 = 2,  /* OCP FP8 E4M3: bias 7, no infinities, max 448, 0x7F/0xFF NaN;
                        one fp32 scale per row */
  /* Index keys only: OCP MXFP8, E4M3 elements with one E8M0 scale byte
   * (value 2^(e-127); 0xFF, NaN, must not occur) per 32 consecutive elements
   * of a row, the last group of a row shorter when idx_dim % 32 != 0: the
   * group-wise index quantisation of "Inference Acceleration for New Large
   * Model Architectures" §4.1 in the format that "Long-Context LLM Inference
   * Optimization" (Layered Quantization) names. */
  DSA_MXFP8_E4M3 = 3,
  /* Latent cache only: E4M3 elements with one fp32 scale per 128 consecutive
   * elements of a row (ceil(qk_dim / 128) scales per row), the per-token,
   * per-tile cache quantisation of "Inference Acceleration ..." §4.2. */
  DSA_FP8_E4M3_T128 = 4
} dsa_dtype;

/*
 * Problem description (host struct, read during the call only).
 *
 * Indexer ("Optimizing Next-Gen LLM Inference" §3.1; "Inference Acceleration
 * for New Large Model Architectures" §3.1): per query token, idx_heads index
 * heads of idx_dim each score every visible position s as
 *     S[s] = sum_h head_w[h] * max(0, q_idx[h,:] . k_idx[s,:] * k_scale[s])
 * (the ReLU-weighted head aggregation is this library's reading of "score,
 * then head-weight"; k_scale is 1 unless the keys are FP8_E4M3; MXFP8_E4M3
 * keys scale each group of 32 dims instead, as dsa_index_score states).
 *
 * Sparse MLA attention ("Optimization and Deployment Practices for
 * Next-Generation Sparse Attention LLMs" §1-§2): one latent row of qk_dim
 * values per cached token serves as the key of every head; its first v_dim
 * values are the value.  For head h:
 *     z_j = softmax_scale * q[h,:] . c[idx_j,:],  out[h,:] = sum_j softmax(z)_j c[idx_j, :v_dim].
 */
typedef struct dsa_problem {
  int32_t batch;        /* B >= 1 sequences */
  int32_t q_len;        /* T >= 1 query tokens per sequence (decode 1, drafts 2, prefill chunk);
                           batch * q_len <= 65535 */
  int64_t max_seq_len;  /* Lmax: rows per sequence in k_idx / kv / scores, q_len <= Lmax < 2^31 */
  int32_t idx_heads;    /* Hi >= 1 */
  int32_t idx_dim;      /* Di >= 1 */
  int32_t heads;        /* H >= 1 attention heads */
  int32_t qk_dim;       /* Dqk >= 1 latent row width (latent + rope) */
  int32_t v_dim;        /* 1 <= Dv <= Dqk: leading columns of a row used as the value */
  int32_t top_k;        /* K >= 1 */
  float softmax_scale;  /* finite, > 0 (usually 1/sqrt(qk_dim)) */
  int32_t q_idx_dtype;  /* DSA_F32 | DSA_BF16 */
  int32_t idx_key_dtype;/* DSA_F32 | DSA_BF16 | DSA_FP8_E4M3 | DSA_MXFP8_E4M3 (the last two
                           with k_scale) */
  int32_t q_dtype;      /* DSA_F32 | DSA_BF16 */
  int32_t kv_dtype;     /* DSA_F32 | DSA_BF16 | DSA_FP8_E4M3 | DSA_FP8_E4M3_T128 (the last
                           two with kv_scale) */
  int32_t out_dtype;    /* DSA_F32 | DSA_BF16 */
} dsa_problem;

#define DSA_ABI_VERSION 6
#define DSA_FORWARD_STAGES 3 /* indexer scores, Top-K, sparse attention */

int dsa_abi_version(void);
const char* dsa_status_string(dsa_status s);
/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* dsa_last_error(void);

/*
 * Indexer scores (step 1).
 *   q_idx    [B,T,Hi,Di]  q_idx_dtype (finite).  With FP8 keys the index query
 *                         is quantised to E4M3 (nearest, ties to even,
 *                         saturating at +-448) before the products, as the
 *                         pages quantise index Q and K alike ("Inference
 *                         Acceleration ..." §4.1).  With MXFP8 keys it is
 *                         quantised to MXFP8 on the fly, each head's groups of
 *                         32 on their own: shared exponent E = floor(log2 of
 *                         the group's largest magnitude) - 8, kept in
 *                         [-127, 127] (-127 for an all-zero group), elements
 *                         the nearest E4M3 values of x / 2^E, saturating (the
 *                         OCP MX v1.0 conversion); the score then uses the
 *                         dequantised query and keys.
 *   head_w   [B,T,Hi]     fp32 head weights.
 *   k_idx    [B,Lmax,Di]  idx_key_dtype index keys (E4M3 codes for both FP8 forms).
 *   k_scale  FP8_E4M3:    fp32 [B,Lmax], a positive scale per row (4-byte aligned);
 *            MXFP8_E4M3:  uint8 [B,Lmax,ceil(Di/32)] E8M0 group scales;
 *            otherwise NULL.
 *   seq_lens [B]          int32 filled rows per sequence.
 *   scores   [B,T,Lmax]   fp32 output; entries s >= vis are left unspecified
 *                         (they may be overwritten).
 * Pointers must be non-NULL (k_scale as stated); q_idx, k_idx and scores must
 * be 16-byte aligned.
 */
dsa_status dsa_index_score(const dsa_problem* p, const void* q_idx, const float* head_w,
                           const void* k_idx, const void* k_scale, const int32_t* seq_lens,
                           float* scores, struct ihipStream_t* stream);

/* Workspace bytes dsa_topk needs for problem p (0 if p is invalid). */
size_t dsa_topk_workspace_size(const dsa_problem* p);

/*
 * Leading bytes of a dsa_topk or dsa_forward workspace for problem p that
 * must be zero when a call starts (the counters; see the conventions above).
 * 0 if p is invalid.
 */
size_t dsa_workspace_zero_bytes(const dsa_problem* p);

/*
 * Zero-fills ws_bytes bytes of ws on `stream` (a kernel, so it can be
 * captured in a HIP graph).  ws: device pointer, 4-byte aligned; ws_bytes a
 * multiple of 4.  Use once on a new workspace (or after a DSA_ERR_HIP).
 */
dsa_status dsa_workspace_init(void* ws, size_t ws_bytes, struct ihipStream_t* stream);

/*
 * Per-query Top-K (step 2).
 *   scores     [B,T,Lmax] fp32 (only s < vis is read).
 *   topk_idx   [B,T,K] int32 output: the selected positions in ascending order;
 *              the last K - count entries are -1.
 *   topk_count [B,T] int32 output count = min(K, max(vis, 0)), or NULL.
 *   ws         device scratch of at least dsa_topk_workspace_size(p) bytes,
 *              16-byte aligned, whose first dsa_workspace_zero_bytes(p)
 *              bytes are zero (left zero on success).
 */
dsa_status dsa_topk(const dsa_problem* p, const float* scores, const int32_t* seq_lens,
                    int32_t* topk_idx, int32_t* topk_count, void* ws, size_t ws_bytes,
                    struct ihipStream_t* stream);

/* Workspace bytes dsa_sparse_mla_decode needs for problem p (0 if invalid). */
size_t dsa_sparse_mla_workspace_size(const dsa_problem* p);

/*
 * Sparse MLA attention over selected rows (step 3).
 *   q        [B,T,H,Dqk]  q_dtype queries (already absorbed into the latent space).
 *   kv       [B,Lmax,Dqk] kv_dtype latent cache rows.
 *   kv_scale FP8_E4M3:       fp32 [B,Lmax], a positive scale per row;
 *            FP8_E4M3_T128:  fp32 [B,Lmax,ceil(Dqk/128)], a positive scale per
 *                            128-column tile of each row;
 *            otherwise NULL.
 *                         A power-of-two scale expands its elements to bf16
 *                         exactly; any other value is applied in fp32 and the
 *                         product rounded to bf16.
 *   topk_idx [B,T,K]      int32 rows to attend over; entries outside [0, len_b)
 *                         are ignored, so -1 padding is allowed.
 *   out      [B,T,H,Dv]   out_dtype output.  No valid entry: out = 0.
 *   lse      [B,T,H]      fp32 natural-log softmax normaliser of the scaled
 *                         logits (-inf when no entry is valid), or NULL.
 *   ws       scratch of dsa_sparse_mla_workspace_size(p) bytes (any contents).
 * q, kv and out must be 16-byte aligned.
 */
dsa_status dsa_sparse_mla_decode(const dsa_problem* p, const void* q, const void* kv,
                                 const float* kv_scale, const int32_t* topk_idx,
                                 const int32_t* seq_lens, void* out, float* lse, void* ws,
                                 size_t ws_bytes, struct ihipStream_t* stream);

/* Workspace bytes dsa_forward needs for problem p (0 if invalid). */
size_t dsa_forward_workspace_size(const dsa_problem* p);

/*
 * Query tokens per tile when dsa_forward runs problem p in token tiles (see
 * Workspaces): tile (b, t0) covers tokens t0 .. min(t0 + n, T) - 1 of
 * sequence b, in order b = 0 .. B-1, t0 = 0, n, 2n, ...  Returns 0 when the
 * call runs as one pass over the whole problem, -1 for an invalid problem.
 */
int32_t dsa_forward_tile_tokens(const dsa_problem* p);

/*
 * The whole path: indexer scores -> Top-K -> sparse MLA attention, with the
 * score histogram that drives the Top-K threshold fused into the score pass.
 * Arguments as in the three calls above, plus:
 *   scores       [B,T,Lmax] fp32 output of step 1, or NULL to keep it in ws.
 *   topk_idx     [B,T,K] output of step 2, or NULL to keep it in ws.
 *   topk_count   [B,T] or NULL.
 *   ws           dsa_forward_workspace_size(p) bytes, 256-byte aligned,
 *                whose first dsa_workspace_zero_bytes(p) bytes are zero
 *                (left zero on success).
 *   stage_events NULL, or DSA_FORWARD_STAGES + 1 hipEvent_t handles: event 0
 *                is recorded on `stream` just before the score kernel, and
 *                event i after
 *                stage i (1 = scores, 2 = Top-K, 3 = attention), for per-stage
 *                timing.  With the matrix-core score kernel, events 0 and 1
 *                are taken by that kernel's dispatch at its own start and end,
 *                so they time the kernel alone.  A call that runs in token
 *                tiles (see Workspaces) records the events around every
 *                tile's stages in turn: when it returns they time the stages
 *                of its last tile.
 */
dsa_status dsa_forward(const dsa_problem* p, const void* q_idx, const float* head_w,
                       const void* k_idx, const void* k_scale, const void* q, const void* kv,
                       const float* kv_scale, const int32_t* seq_lens, float* scores,
                       int32_t* topk_idx, int32_t* topk_count, void* out, float* lse, void* ws,
                       size_t ws_bytes, struct ihipStream_t* stream,
                       struct ihipEvent_t* const* stage_events);

/*
 * Workgroup timeline, for load-balance analysis ("Inference Acceleration for
 * New Large Model Architectures" §6.3, observability).  While a buffer is
 * set, every launch of the matrix-core score kernel, the Top-K kernels and
 * the matrix-core attention kernels writes two stamps of the GPU's constant
 * 100 MHz clock per workgroup, at its start and when its first thread
 * leaves, to
 *   buf[(kind * slots + w) * 2 + 0 / 1]
 * with kind 0 scores, 1 Top-K chunk step, 2 Top-K emit step, 3 Top-K row
 * mode, 4 attention, 5 attention split merge, and w the workgroup's linear
 * index (x fastest, then y, then z).  A launch with more than `slots`
 * workgroups writes nothing; each launch overwrites its kind's entries.
 *   buf    device memory on the GPU the calls run on, at least
 *          DSA_TRACE_KINDS * slots * 2 uint64 values, 8-byte aligned, owned
 *          by the caller and kept alive while set; NULL (or slots <= 0)
 *          turns tracing off.
 * A process-wide setting, read at every launch from any thread.  Returns
 * DSA_ERR_INVALID_ARG for a misaligned buffer.
 */
#define DSA_TRACE_KINDS 6

dsa_status dsa_set_workgroup_trace(uint64_t* buf, int64_t slots);

/*
 * dsa_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * workspace is a device array the library owns, DSA_NOALLOC_WORKSPACE_BYTES
 * on each GPU it runs on, held until the process ends.  Arguments, outputs
 * and stage events are those of dsa_forward without ws / ws_bytes.
 *  - A problem whose dsa_forward_workspace_size exceeds
 *    DSA_NOALLOC_WORKSPACE_BYTES returns DSA_ERR_WORKSPACE_TOO_SMALL (nothing
 *    is enqueued); every argument is validated before any HIP call.
 *  - No hipMalloc, hipFree or allocating library call is made.  The first
 *    call on a device looks up that device's array address once.
 *  - The array keeps the last call's contents; each call first clears the
 *    counters it needs with a fill kernel on `stream`.  Every call on one GPU
 *    shares that GPU's array, so calls that overlap on one GPU (on two
 *    streams, or from two threads) race: serialise them.
 */
#define DSA_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)

dsa_status dsa_forward_noalloc(const dsa_problem* p, const void* q_idx, const float* head_w,
                               const void* k_idx, const void* k_scale, const void* q, const void* kv,
                               const float* kv_scale, const int32_t* seq_lens, float* scores,
                               int32_t* topk_idx, int32_t* topk_count, void* out, float* lse,
                               struct ihipStream_t* stream, struct ihipEvent_t* const* stage_events);

/*
 * Paged caches.  The pages have the fused indexer read the paged key cache
 * directly and the sparse attention gather its selected rows from the paged
 * KV cache, with the paged metadata prepared beside the query projection
 * ("Optimizing Next-Gen LLM Inference" §3.1; "Inference Acceleration for New
 * Large Model Architectures" §3.1 and §3.3).  Here one block table serves the
 * index-key cache and the latent cache: logical row s of sequence b is row
 * s % page_size of physical page block_table[b * max_pages + s / page_size]
 * in both, and in their per-row scales.
 *
 *   block_table  device int32 [batch, max_pages].  Entries are device data:
 *                kernels clamp them into [0, num_pages), so a bad entry gives
 *                meaningless results, never an out-of-bounds read.
 *   page_size    rows per page: a power of two, at least 64 (a page then holds
 *                whole 64-row score units).
 *   max_pages    columns of block_table; max_pages * page_size >= max_seq_len.
 *   num_pages    physical pages in each cache; num_pages * page_size * row bytes
 *                < 2^31 for each cache.
 *
 * The _paged entry points take, in place of k_idx / k_scale / kv / kv_scale,
 *   k_pages   [num_pages, page_size, idx_dim]     (idx_key_dtype)
 *   k_scales  [num_pages, page_size] fp32 (FP8_E4M3 keys),
 *             [num_pages, page_size, idx_dim/32] E8M0 (MXFP8_E4M3), else NULL
 *   kv_pages  [num_pages, page_size, qk_dim]      (kv_dtype)
 *   kv_scales [num_pages, page_size] fp32 (FP8_E4M3 cache),
 *             [num_pages, page_size, ceil(qk_dim/128)] fp32 (FP8_E4M3_T128), else NULL
 * and are otherwise the calls above (same workspaces, outputs and timing
 * events; topk_idx stays in logical positions).  They need the matrix-core
 * kernels (64 x 128 indexer, 576/512 MLA, bf16 or FP8 caches): other problems
 * return DSA_ERR_UNSUPPORTED, as does DSA_FORCE_GENERIC.
 */
typedef struct dsa_paging {
  const int32_t* block_table;
  int32_t page_size;
  int32_t max_pages;
  int64_t num_pages;
} dsa_paging;

dsa_status dsa_index_score_paged(const dsa_problem* p, const dsa_paging* pg, const void* q_idx,
                                 const float* head_w, const void* k_pages, const void* k_scales,
                                 const int32_t* seq_lens, float* scores, struct ihipStream_t* stream);
dsa_status dsa_sparse_mla_decode_paged(const dsa_problem* p, const dsa_paging* pg, const void* q,
                                       const void* kv_pages, const float* kv_scales,
                                       const int32_t* topk_idx, const int32_t* seq_lens, void* out,
                                       float* lse, void* ws, size_t ws_bytes, struct ihipStream_t* stream);
dsa_status dsa_forward_paged(const dsa_problem* p, const dsa_paging* pg, const void* q_idx,
                             const float* head_w, const void* k_pages, const void* k_scales,
                             const void* q, const void* kv_pages, const float* kv_scales,
                             const int32_t* seq_lens, float* scores, int32_t* topk_idx,
                             int32_t* topk_count, void* out, float* lse, void* ws, size_t ws_bytes,
                             struct ihipStream_t* stream, struct ihipEvent_t* const* stage_events);

/*
 * Diagnostics.  dsa_kernel_choice() names the kernels dsa_forward would launch
 * for p into buf (NUL-terminated, truncated to len): "mfma" or "generic" per
 * step, the score launch's shape and workgroup count, the Top-K mode, the
 * attention's row splits, and the token tile (0: one pass).  A call in token
 * tiles is described by its tile's launches.  Returns 0, or -1 for an invalid
 * problem or buffer.  While the environment variable DSA_FORCE_GENERIC is set
 * to a value other than "0", every call uses the portable SIMT kernels for
 * every step.
 */
int dsa_kernel_choice(const dsa_problem* p, char* buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
