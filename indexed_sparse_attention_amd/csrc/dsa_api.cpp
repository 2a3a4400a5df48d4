// Host side of libdsa: argument validation, workspace layout, kernel choice
// and launches.  Every entry point validates all of its arguments before the
// first HIP call, so a rejected call enqueues nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/dsa.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

dsa_status fail(dsa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

dsa_status ok() {
  g_last_error.clear();
  return DSA_OK;
}

// Read on every call so a process can switch paths between calls.
bool force_generic() {
  const char* e = getenv("DSA_FORCE_GENERIC");
  return e && *e && strcmp(e, "0") != 0;
}

int env_int(const char* name, int dflt) {
  const char* e = getenv(name);
  if (!e || !*e) return dflt;
  return atoi(e);
}

constexpr int64_t kAlign = 256;
int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

const int64_t kHistBins = 4096;

dsa_status validate_problem(const dsa_problem* p) {
  if (!p) return fail(DSA_ERR_INVALID_ARG, "problem is NULL");
  if (p->batch < 1) return fail(DSA_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", p->batch);
  if (p->q_len < 1) return fail(DSA_ERR_INVALID_ARG, "q_len must be >= 1 (got %d)", p->q_len);
  if (p->max_seq_len < 1 || p->max_seq_len > INT32_MAX)
    return fail(DSA_ERR_INVALID_ARG, "max_seq_len must be in [1, 2^31-1] (got %lld)",
                (long long)p->max_seq_len);
  if (p->q_len > p->max_seq_len)
    return fail(DSA_ERR_INVALID_ARG, "q_len (%d) exceeds max_seq_len (%lld)", p->q_len,
                (long long)p->max_seq_len);
  if (p->idx_heads < 1 || p->idx_dim < 1)
    return fail(DSA_ERR_INVALID_ARG, "idx_heads and idx_dim must be >= 1");
  if (p->heads < 1 || p->qk_dim < 1) return fail(DSA_ERR_INVALID_ARG, "heads and qk_dim must be >= 1");
  if (p->v_dim < 1 || p->v_dim > p->qk_dim)
    return fail(DSA_ERR_INVALID_ARG, "v_dim must be in [1, qk_dim] (got %d)", p->v_dim);
  if (p->top_k < 1) return fail(DSA_ERR_INVALID_ARG, "top_k must be >= 1 (got %d)", p->top_k);
  if (!(std::isfinite(p->softmax_scale) && p->softmax_scale > 0.0f))
    return fail(DSA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  auto in = [](int32_t d, int lo, int hi) { return d >= lo && d <= hi; };
  if (!in(p->q_idx_dtype, DSA_F32, DSA_BF16)) return fail(DSA_ERR_INVALID_ARG, "q_idx_dtype must be F32 or BF16");
  if (!in(p->idx_key_dtype, DSA_F32, DSA_MXFP8_E4M3)) return fail(DSA_ERR_INVALID_ARG, "idx_key_dtype invalid");
  if (!in(p->q_dtype, DSA_F32, DSA_BF16)) return fail(DSA_ERR_INVALID_ARG, "q_dtype must be F32 or BF16");
  if (!in(p->kv_dtype, DSA_F32, DSA_FP8_E4M3) && p->kv_dtype != DSA_FP8_E4M3_T128)
    return fail(DSA_ERR_INVALID_ARG, "kv_dtype invalid");
  if (!in(p->out_dtype, DSA_F32, DSA_BF16)) return fail(DSA_ERR_INVALID_ARG, "out_dtype must be F32 or BF16");
  // sizes must fit the int64 offsets the kernels use
  const double bt = (double)p->batch * p->q_len;
  if (bt * p->max_seq_len > 4.0e18 || (double)p->batch * p->max_seq_len * p->qk_dim > 4.0e18 ||
      bt * p->top_k > 2.0e9 || bt * p->heads > 2.0e9)
    return fail(DSA_ERR_INVALID_ARG, "problem too large");
  // (query, chunk) and (head, query) launch grids put batch * q_len on grid.y
  if (bt > 65535.0) return fail(DSA_ERR_INVALID_ARG, "batch * q_len must be <= 65535");
  if (p->heads > 65535) return fail(DSA_ERR_INVALID_ARG, "heads must be <= 65535");
  return DSA_OK;
}

// ------------------------------------------------------------------ Top-K layout
// The counters (one score-key histogram per query) come first, at offset 0
// of every workspace that holds them: they must be zero when a call starts,
// and every successful call leaves them zero again.
struct TopkLayout {
  int chunk, n_chunks;
  int64_t off_hist, zero_bytes;
  int64_t off_hdr, off_cnt, off_above, off_cand, off_blist, bytes;
};

TopkLayout topk_layout(const dsa_problem* p) {
  TopkLayout L;
  const int64_t BT = (int64_t)p->batch * p->q_len, Lmax = p->max_seq_len;
  // about 512 (query, chunk) workgroups in all, two per CU: every emit
  // workgroup resolves its query's threshold again, so more chunks than that
  // only add redundant work (at 1M positions x 8 queries, 2048 chunks of 4096
  // took twice as long as 512 of 16384)
  int64_t chunk = std::max<int64_t>(4096, (Lmax * BT + 511) / 512);
  if (env_int("DSA_SELECT_CHUNK", 0) > 0) chunk = env_int("DSA_SELECT_CHUNK", 0);  // (tuning)
  chunk = std::max<int64_t>(chunk, (Lmax + 1023) / 1024);  // at most 1024 chunks per query
  chunk = align_up(chunk, 1024);
  if (chunk > align_up(Lmax, 1024)) chunk = align_up(Lmax, 1024);
  L.chunk = (int)chunk;
  L.n_chunks = (int)((Lmax + chunk - 1) / chunk);
  L.off_hist = 0;
  L.zero_bytes = BT * kHistBins * 4;
  L.off_hdr = align_up(L.zero_bytes, kAlign);
  L.off_cnt = align_up(L.off_hdr + BT * 8, kAlign);
  L.off_above = align_up(L.off_cnt + BT * L.n_chunks * 4, kAlign);
  L.off_cand = align_up(L.off_above + BT * L.n_chunks * 4, kAlign);
  L.off_blist = align_up(L.off_cand + BT * Lmax * 8, kAlign);
  L.bytes = align_up(L.off_blist + BT * align_up(Lmax, 4) * 4, kAlign);  // rows of bin keys start 16-byte aligned
  return L;
}

// ------------------------------------------------------------------ MLA layout
struct MlaLayout {
  int splits, rows_per_split;
  int64_t off_o, off_ml, bytes;
};

bool mla_uses_mfma(const dsa_problem* p) {
  return !force_generic() && p->qk_dim == 576 && p->v_dim == 512 && p->heads % 64 == 0 &&
         (int64_t)p->top_k <= 64 * (int64_t)dsa::mla_max_rows_per_split() &&
         p->q_dtype == DSA_BF16 &&
         (p->kv_dtype == DSA_BF16 || p->kv_dtype == DSA_FP8_E4M3 || p->kv_dtype == DSA_FP8_E4M3_T128);
}

MlaLayout mla_layout(const dsa_problem* p) {
  MlaLayout L;
  const int64_t BT = (int64_t)p->batch * p->q_len;
  const int tile = dsa::mla_row_tile();
  L.splits = 1;
  L.rows_per_split = (int)align_up(p->top_k, tile);
  if (mla_uses_mfma(p)) {
    const int64_t wgs_per_split = BT * (p->heads / 64);
    int64_t target = env_int("DSA_MLA_TARGET_WGS", 256);
    int64_t s = (target + wgs_per_split - 1) / wgs_per_split;
    const int64_t max_s = std::min<int64_t>(64, (p->top_k + tile - 1) / tile);
    if (env_int("DSA_MLA_SPLITS", 0) > 0) s = env_int("DSA_MLA_SPLITS", 0);
    s = std::max<int64_t>(1, std::min(s, max_s));
    // (a workgroup stages its index list in LDS chunk after chunk, so only
    // parallelism sets the splits: many queries need none, and no merge)
    L.rows_per_split = (int)align_up((p->top_k + s - 1) / s, tile);
    L.splits = (p->top_k + L.rows_per_split - 1) / L.rows_per_split;
  }
  L.off_o = 0;
  L.off_ml = 0;
  L.bytes = 0;
  if (L.splits > 1) {
    L.off_ml = align_up((int64_t)L.splits * BT * p->heads * p->v_dim * 2, kAlign);
    L.bytes = align_up(L.off_ml + (int64_t)L.splits * BT * p->heads * 2 * 4, kAlign);
  }
  return L;
}

// ------------------------------------------------------------------ forward layout
struct FwdLayout {
  TopkLayout tk;
  MlaLayout mla;
  int64_t off_topk, off_scores, off_idx, off_mla, bytes;
};

FwdLayout fwd_layout(const dsa_problem* p) {
  FwdLayout F;
  const int64_t BT = (int64_t)p->batch * p->q_len;
  F.tk = topk_layout(p);
  F.mla = mla_layout(p);
  F.off_topk = 0;
  F.off_scores = align_up(F.tk.bytes, kAlign);
  F.off_idx = align_up(F.off_scores + BT * p->max_seq_len * 4, kAlign);
  F.off_mla = align_up(F.off_idx + BT * p->top_k * 4, kAlign);
  F.bytes = align_up(F.off_mla + F.mla.bytes, kAlign);
  return F;
}

// ------------------------------------------------------------------ token tiles
// A call whose workspace would pass 1 GiB runs as a series of launches
// over tiles of one sequence's query tokens (a long prefill chunk, or a very
// large batch): tile (b, t0, n) is the problem of sequence b alone with
// query tokens t0 .. t0+n-1, its pointers offset to them, and `len_sub` =
// T - t0 - n rows hidden from its score and Top-K kernels, so that every
// token sees exactly what it sees in the whole problem.  The workspace then
// holds one tile's scratch, reused tile after tile on the one stream.
// (DSA_TILE_BUDGET, in bytes, replaces it: tests use it to make small
// problems run in tiles)
int64_t tile_budget() {
  const char* e = getenv("DSA_TILE_BUDGET");
  if (e && *e) {
    const long long v = atoll(e);
    if (v > 0) return (int64_t)v;
  }
  return (int64_t)1 << 30;
}

dsa_problem tile_problem(const dsa_problem* p, int n) {
  dsa_problem t = *p;
  t.batch = 1;
  t.q_len = n;
  return t;
}

// query tokens per tile (0: the call runs whole), the largest power of two
// whose tile scratch fits the budget
template <class Bytes>
int tile_tokens(const dsa_problem* p, Bytes bytes) {
  const int64_t budget = tile_budget();
  if (bytes(p) <= budget) return 0;
  int n = 1;
  while (2 * (int64_t)n <= p->q_len) n *= 2;
  while (n > 1) {
    const dsa_problem t = tile_problem(p, n);
    if (bytes(&t) <= budget) break;
    n /= 2;
  }
  return n;
}

int64_t elem_bytes(int32_t dtype) { return dtype == DSA_F32 ? 4 : dtype == DSA_BF16 ? 2 : 1; }
int64_t key_row_bytes(const dsa_problem* p) { return (int64_t)p->idx_dim * elem_bytes(p->idx_key_dtype); }
int64_t key_scale_row_bytes(const dsa_problem* p) {
  if (p->idx_key_dtype == DSA_FP8_E4M3) return 4;
  if (p->idx_key_dtype == DSA_MXFP8_E4M3) return (p->idx_dim + 31) / 32;
  return 0;
}
int64_t kv_row_bytes(const dsa_problem* p) { return (int64_t)p->qk_dim * elem_bytes(p->kv_dtype); }
int64_t kv_scale_row_bytes(const dsa_problem* p) {
  if (p->kv_dtype == DSA_FP8_E4M3) return 4;
  if (p->kv_dtype == DSA_FP8_E4M3_T128) return 4 * (int64_t)((p->qk_dim + 127) / 128);
  return 0;
}

template <class T>
T* advance(T* ptr, int64_t bytes) {
  return ptr ? (T*)((const uint8_t*)ptr + bytes) : nullptr;
}

int64_t topk_bytes(const dsa_problem* p) { return topk_layout(p).bytes; }
int64_t mla_bytes(const dsa_problem* p) { return mla_layout(p).bytes; }
int64_t fwd_bytes(const dsa_problem* p) { return fwd_layout(p).bytes; }

int num_cus() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> g(mu);
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

dsa_status hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return DSA_OK;
}

#define REQUIRE(cond, ...) \
  do {                     \
    if (!(cond)) return fail(DSA_ERR_INVALID_ARG, __VA_ARGS__); \
  } while (0)

dsa_status check_index_inputs(const dsa_problem* p, const void* q_idx, const float* head_w,
                              const void* k_idx, const void* k_scale, const int32_t* seq_lens) {
  REQUIRE(q_idx && aligned(q_idx, 16), "q_idx must be non-NULL and 16-byte aligned");
  REQUIRE(head_w && aligned(head_w, 4), "head_w must be non-NULL and 4-byte aligned");
  REQUIRE(k_idx && aligned(k_idx, 16), "k_idx must be non-NULL and 16-byte aligned");
  REQUIRE(seq_lens && aligned(seq_lens, 4), "seq_lens must be non-NULL and 4-byte aligned");
  if (p->idx_key_dtype == DSA_FP8_E4M3)
    REQUIRE(k_scale && aligned(k_scale, 4), "k_scale is required (4-byte aligned) for FP8 index keys");
  else if (p->idx_key_dtype == DSA_MXFP8_E4M3)
    REQUIRE(k_scale, "k_scale (E8M0 group scales) is required for MXFP8 index keys");
  else
    REQUIRE(!k_scale, "k_scale must be NULL unless the index keys are FP8_E4M3 or MXFP8_E4M3");
  return DSA_OK;
}

dsa_status check_mla_inputs(const dsa_problem* p, const void* q, const void* kv, const float* kv_scale,
                            const int32_t* seq_lens, const void* out, const float* lse) {
  REQUIRE(q && aligned(q, 16), "q must be non-NULL and 16-byte aligned");
  REQUIRE(kv && aligned(kv, 16), "kv must be non-NULL and 16-byte aligned");
  REQUIRE(seq_lens && aligned(seq_lens, 4), "seq_lens must be non-NULL and 4-byte aligned");
  REQUIRE(out && aligned(out, 16), "out must be non-NULL and 16-byte aligned");
  REQUIRE(!lse || aligned(lse, 4), "lse must be 4-byte aligned");
  if (p->kv_dtype == DSA_FP8_E4M3 || p->kv_dtype == DSA_FP8_E4M3_T128)
    REQUIRE(kv_scale && aligned(kv_scale, 4), "kv_scale is required (4-byte aligned) for an FP8 cache");
  else
    REQUIRE(!kv_scale, "kv_scale must be NULL unless kv_dtype is FP8_E4M3 or FP8_E4M3_T128");
  if (!mla_uses_mfma(p)) {
    REQUIRE(p->qk_dim <= 2048, "qk_dim > 2048 is not supported by the portable attention kernel");
    if (p->v_dim > 1024) return fail(DSA_ERR_UNSUPPORTED, "v_dim > 1024 is not supported by the portable attention kernel");
  }
  return DSA_OK;
}

dsa::ScoreParams score_params(const dsa_problem* p, const void* q_idx, const float* head_w,
                              const void* k_idx, const void* k_scale, const int32_t* seq_lens,
                              float* scores, uint32_t* hist, int len_sub = 0) {
  dsa::ScoreParams s{};
  s.len_sub = len_sub;
  s.q_idx = q_idx;
  s.head_w = head_w;
  s.k_idx = k_idx;
  s.k_scale = k_scale;
  s.seq_lens = seq_lens;
  s.scores = scores;
  s.hist = hist;
  s.B = p->batch;
  s.T = p->q_len;
  s.Hi = p->idx_heads;
  s.Di = p->idx_dim;
  s.Lmax = p->max_seq_len;
  s.q_dtype = p->q_idx_dtype;
  s.k_dtype = p->idx_key_dtype;
  s.block_table = nullptr;
  s.num_pages = 0;
  s.max_pages = 0;
  s.page_shift = 0;
  return s;
}

dsa::TopkParams topk_params(const dsa_problem* p, const TopkLayout& L, uint8_t* ws, const float* scores,
                            const int32_t* seq_lens, int32_t* idx, int32_t* cnt, int len_sub = 0) {
  dsa::TopkParams t;
  t.len_sub = len_sub;
  t.scores = scores;
  t.seq_lens = seq_lens;
  t.hist = (uint32_t*)(ws + L.off_hist);
  t.cand = (uint2*)(ws + L.off_cand);
  t.chunk_cnt = (uint32_t*)(ws + L.off_cnt);
  t.bin_keys = (uint32_t*)(ws + L.off_blist);
  t.header = (uint2*)(ws + L.off_hdr);
  t.chunk_above = (uint32_t*)(ws + L.off_above);
  t.topk_idx = idx;
  t.topk_count = cnt;
  t.B = p->batch;
  t.T = p->q_len;
  t.K = p->top_k;
  t.Lmax = p->max_seq_len;
  t.chunk = L.chunk;
  t.n_chunks = L.n_chunks;
  return t;
}

dsa::MlaParams mla_params(const dsa_problem* p, const MlaLayout& L, uint8_t* ws, const void* q,
                          const void* kv, const float* kv_scale, const int32_t* idx,
                          const int32_t* seq_lens, void* out, float* lse) {
  dsa::MlaParams m;
  m.len_sub = 0;  // (the attention's length only bounds the index entries it accepts)
  m.q = q;
  m.kv = kv;
  m.kv_scale = kv_scale;
  m.topk_idx = idx;
  m.seq_lens = seq_lens;
  m.out = out;
  m.lse = lse;
  m.part_o = L.splits > 1 ? (uint16_t*)(ws + L.off_o) : nullptr;
  m.part_ml = L.splits > 1 ? (float*)(ws + L.off_ml) : nullptr;
  m.B = p->batch;
  m.T = p->q_len;
  m.H = p->heads;
  m.Dqk = p->qk_dim;
  m.Dv = p->v_dim;
  m.K = p->top_k;
  m.Lmax = p->max_seq_len;
  m.scale = p->softmax_scale;
  m.q_dtype = p->q_dtype;
  m.kv_dtype = p->kv_dtype;
  m.out_dtype = p->out_dtype;
  m.splits = L.splits;
  m.rows_per_split = L.rows_per_split;
  m.block_table = nullptr;
  m.num_pages = 0;
  m.max_pages = 0;
  m.page_shift = 0;
  return m;
}

int log2_exact(int64_t v) {
  int s = 0;
  while (((int64_t)1 << s) < v) ++s;
  return s;
}

bool score_uses_mfma(const dsa_problem* p);

// Paging descriptor checks; the cache-side checks for the index keys
// (index != 0) and / or the latent cache (mla != 0).
dsa_status check_paging(const dsa_problem* p, const dsa_paging* pg, bool index, bool mla) {
  REQUIRE(pg, "pg must be non-NULL");
  REQUIRE(pg->block_table && aligned(pg->block_table, 4), "block_table must be non-NULL and 4-byte aligned");
  REQUIRE(pg->page_size >= 64 && (pg->page_size & (pg->page_size - 1)) == 0,
          "page_size must be a power of two >= 64 (got %d)", pg->page_size);
  REQUIRE(pg->max_pages >= 1 && (int64_t)pg->max_pages * pg->page_size >= p->max_seq_len,
          "max_pages * page_size must cover max_seq_len (%d x %d < %d)", pg->max_pages, pg->page_size,
          p->max_seq_len);
  REQUIRE(pg->num_pages >= 1, "num_pages must be >= 1");
  REQUIRE(pg->num_pages * pg->page_size < ((int64_t)1 << 31), "num_pages * page_size must be < 2^31 rows");
  if (index) {
    if (!score_uses_mfma(p))
      return fail(DSA_ERR_UNSUPPORTED, "paged caches need the matrix-core index kernel (64 x 128, bf16 or FP8 keys)");
    const int64_t row_bytes = (int64_t)p->idx_dim * (p->idx_key_dtype == DSA_BF16 ? 2 : 1);
    REQUIRE(pg->num_pages * pg->page_size * row_bytes < ((int64_t)1 << 31),
            "the paged index-key cache must be < 2 GiB");
  }
  if (mla && !mla_uses_mfma(p))
    return fail(DSA_ERR_UNSUPPORTED, "paged caches need the matrix-core attention kernel (576/512, bf16 q)");
  return DSA_OK;
}

void apply_paging(dsa::ScoreParams& s, const dsa_paging* pg) {
  if (!pg) return;
  s.block_table = pg->block_table;
  s.num_pages = pg->num_pages;
  s.max_pages = pg->max_pages;
  s.page_shift = log2_exact(pg->page_size);
}

void apply_paging(dsa::MlaParams& m, const dsa_paging* pg) {
  if (!pg) return;
  m.block_table = pg->block_table;
  m.num_pages = pg->num_pages;
  m.max_pages = pg->max_pages;
  m.page_shift = log2_exact(pg->page_size);
}

bool score_uses_mfma(const dsa_problem* p) {
  if (force_generic()) return false;
  dsa::ScoreParams s{};
  s.Hi = p->idx_heads;
  s.Di = p->idx_dim;
  s.T = p->q_len;
  s.q_dtype = p->q_idx_dtype;
  s.k_dtype = p->idx_key_dtype;
  return dsa::score_mfma_supported(s);
}

}  // namespace

namespace dsa {

// hipFuncSetAttribute costs a runtime call per launch; it is made once per
// kernel and device instead.
hipError_t set_max_dynamic_lds(const void* kernel, int bytes) {
  static std::mutex mu;
  static std::vector<std::tuple<const void*, int, int>> done;  // (kernel, device, bytes)
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> g(mu);
  for (const auto& d : done)
    if (std::get<0>(d) == kernel && std::get<1>(d) == dev && std::get<2>(d) >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.emplace_back(kernel, dev, bytes);
  return e;
}

}  // namespace dsa

// ------------------------------------------------------------------ workgroup trace
namespace {
std::mutex g_trace_mu;
uint64_t* g_trace = nullptr;
int64_t g_trace_slots = 0;
}  // namespace

namespace dsa {
uint64_t* trace_region(int kind, int64_t grid) {
  std::lock_guard<std::mutex> g(g_trace_mu);
  if (!g_trace || grid > g_trace_slots || kind < 0 || kind >= kTraceKinds) return nullptr;
  return g_trace + (int64_t)kind * g_trace_slots * 2;
}
}  // namespace dsa

extern "C" {

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

dsa_status dsa_set_workgroup_trace(uint64_t* buf, int64_t slots) {
  static_assert(DSA_TRACE_KINDS == dsa::kTraceKinds, "trace kinds of the header and the kernels differ");
  if (buf && slots > 0) REQUIRE(aligned(buf, 8), "buf must be 8-byte aligned");
  std::lock_guard<std::mutex> g(g_trace_mu);
  g_trace = slots > 0 ? buf : nullptr;
  g_trace_slots = g_trace ? slots : 0;
  return ok();
}

const char* dsa_status_string(dsa_status s) {
  switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_WORKSPACE_TOO_SMALL: return "DSA_ERR_WORKSPACE_TOO_SMALL";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
  }
  return "DSA_UNKNOWN_STATUS";
}

const char* dsa_last_error(void) { return g_last_error.c_str(); }

static dsa_status index_score_impl(const dsa_problem* p, const dsa_paging* pg, const void* q_idx,
                                   const float* head_w, const void* k_idx, const void* k_scale,
                                   const int32_t* seq_lens, float* scores, hipStream_t stream) {
  dsa_status st = validate_problem(p);
  if (st != DSA_OK) return st;
  if ((st = check_index_inputs(p, q_idx, head_w, k_idx, k_scale, seq_lens)) != DSA_OK) return st;
  if (pg && (st = check_paging(p, pg, true, false)) != DSA_OK) return st;
  REQUIRE(scores && aligned(scores, 16), "scores must be non-NULL and 16-byte aligned");
  auto sp = score_params(p, q_idx, head_w, k_idx, k_scale, seq_lens, scores, nullptr);
  apply_paging(sp, pg);
  if ((st = hip_check(dsa::launch_score(sp, !force_generic(), num_cus(), stream), "index score launch")) != DSA_OK)
    return st;
  return ok();
}

dsa_status dsa_index_score(const dsa_problem* p, const void* q_idx, const float* head_w,
                           const void* k_idx, const void* k_scale, const int32_t* seq_lens,
                           float* scores, struct ihipStream_t* stream) {
  return index_score_impl(p, nullptr, q_idx, head_w, k_idx, k_scale, seq_lens, scores, stream);
}

dsa_status dsa_index_score_paged(const dsa_problem* p, const dsa_paging* pg, const void* q_idx,
                                 const float* head_w, const void* k_pages, const void* k_scales,
                                 const int32_t* seq_lens, float* scores, struct ihipStream_t* stream) {
  if (!pg) return fail(DSA_ERR_INVALID_ARG, "pg must be non-NULL");
  return index_score_impl(p, pg, q_idx, head_w, k_pages, k_scales, seq_lens, scores, stream);
}

static int64_t topk_ws_bytes(const dsa_problem* p) {
  const int n = tile_tokens(p, topk_bytes);
  if (!n) return topk_layout(p).bytes;
  const dsa_problem t = tile_problem(p, n);
  return topk_layout(&t).bytes;
}

size_t dsa_topk_workspace_size(const dsa_problem* p) {
  if (validate_problem(p) != DSA_OK) return 0;
  return (size_t)topk_ws_bytes(p);
}

// One launch pair (histogram, select) over problem p.
static dsa_status topk_run(const dsa_problem* p, const float* scores, const int32_t* seq_lens, int len_sub,
                           int32_t* topk_idx, int32_t* topk_count, uint8_t* w, hipStream_t s) {
  const TopkLayout L = topk_layout(p);
  dsa_status st;
  if ((st = hip_check(dsa::launch_hist(scores, seq_lens, len_sub, (uint32_t*)(w + L.off_hist), p->batch, p->q_len,
                                       p->max_seq_len, s), "histogram")) != DSA_OK) return st;
  auto tp = topk_params(p, L, w, scores, seq_lens, topk_idx, topk_count, len_sub);
  return hip_check(dsa::launch_select(tp, s), "select");
}

dsa_status dsa_topk(const dsa_problem* p, const float* scores, const int32_t* seq_lens,
                    int32_t* topk_idx, int32_t* topk_count, void* ws, size_t ws_bytes,
                    struct ihipStream_t* stream) {
  dsa_status st = validate_problem(p);
  if (st != DSA_OK) return st;
  REQUIRE(scores && aligned(scores, 4), "scores must be non-NULL and 4-byte aligned");
  REQUIRE(seq_lens && aligned(seq_lens, 4), "seq_lens must be non-NULL and 4-byte aligned");
  REQUIRE(topk_idx && aligned(topk_idx, 4), "topk_idx must be non-NULL and 4-byte aligned");
  REQUIRE(!topk_count || aligned(topk_count, 4), "topk_count must be 4-byte aligned");
  const int64_t need = topk_ws_bytes(p);
  if ((int64_t)ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "dsa_topk needs %lld workspace bytes, got %zu", (long long)need,
                ws_bytes);
  REQUIRE(ws && aligned(ws, 16), "ws must be non-NULL and 16-byte aligned");
  uint8_t* w = (uint8_t*)ws;
  const int n = tile_tokens(p, topk_bytes);
  if (!n) {
    if ((st = topk_run(p, scores, seq_lens, 0, topk_idx, topk_count, w, stream)) != DSA_OK) return st;
    return ok();
  }
  const int T = p->q_len;
  for (int b = 0; b < p->batch; ++b)
    for (int t0 = 0; t0 < T; t0 += n) {
      const int nn = std::min(n, T - t0);
      const dsa_problem t = tile_problem(p, nn);
      const int64_t q0 = (int64_t)b * T + t0;  // first query of the tile
      if ((st = topk_run(&t, scores + q0 * p->max_seq_len, seq_lens + b, T - t0 - nn, topk_idx + q0 * p->top_k,
                         topk_count ? topk_count + q0 : nullptr, w, stream)) != DSA_OK)
        return st;
    }
  return ok();
}

size_t dsa_workspace_zero_bytes(const dsa_problem* p) {
  if (validate_problem(p) != DSA_OK) return 0;
  // the counters sit at offset 0 of both workspaces, sized for the problem
  // (or the token tile) each one lays out
  int64_t z = 0;
  for (int n : {tile_tokens(p, topk_bytes), tile_tokens(p, fwd_bytes)}) {
    const dsa_problem t = n ? tile_problem(p, n) : *p;
    z = std::max<int64_t>(z, topk_layout(&t).zero_bytes);
  }
  return (size_t)z;
}

dsa_status dsa_workspace_init(void* ws, size_t ws_bytes, struct ihipStream_t* stream) {
  if (ws_bytes == 0) return ok();
  REQUIRE(ws && aligned(ws, 4), "ws must be non-NULL and 4-byte aligned");
  REQUIRE(ws_bytes % 4 == 0, "ws_bytes must be a multiple of 4 (got %zu)", ws_bytes);
  dsa_status st;
  if ((st = hip_check(dsa::launch_zero_u32((uint32_t*)ws, (int64_t)(ws_bytes / 4), stream), "zero")) != DSA_OK)
    return st;
  return ok();
}

static int64_t mla_ws_bytes(const dsa_problem* p) {
  const int n = tile_tokens(p, mla_bytes);
  if (!n) return mla_layout(p).bytes;
  const dsa_problem t = tile_problem(p, n);
  return mla_layout(&t).bytes;
}

size_t dsa_sparse_mla_workspace_size(const dsa_problem* p) {
  if (validate_problem(p) != DSA_OK) return 0;
  return (size_t)mla_ws_bytes(p);
}

// A tile's view of the paging descriptor: its sequence's row of the table.
static dsa_paging tile_paging(const dsa_paging* pg, int b) {
  dsa_paging t = *pg;
  t.block_table = pg->block_table + (int64_t)b * pg->max_pages;
  return t;
}

static dsa_status sparse_mla_impl(const dsa_problem* p, const dsa_paging* pg, const void* q, const void* kv,
                                  const float* kv_scale, const int32_t* topk_idx, const int32_t* seq_lens,
                                  void* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  dsa_status st = validate_problem(p);
  if (st != DSA_OK) return st;
  if ((st = check_mla_inputs(p, q, kv, kv_scale, seq_lens, out, lse)) != DSA_OK) return st;
  if (pg && (st = check_paging(p, pg, false, true)) != DSA_OK) return st;
  REQUIRE(topk_idx && aligned(topk_idx, 4), "topk_idx must be non-NULL and 4-byte aligned");
  const int64_t need = mla_ws_bytes(p);
  if ((int64_t)ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "dsa_sparse_mla_decode needs %lld workspace bytes, got %zu",
                (long long)need, ws_bytes);
  REQUIRE(need == 0 || (ws && aligned(ws, 16)), "ws must be non-NULL and 16-byte aligned");
  auto run = [&](const dsa_problem* t, const dsa_paging* tpg, const void* tq, const void* tkv, const float* tks,
                 const int32_t* tidx, const int32_t* tlens, void* tout, float* tlse) -> dsa_status {
    auto mp = mla_params(t, mla_layout(t), (uint8_t*)ws, tq, tkv, tks, tidx, tlens, tout, tlse);
    apply_paging(mp, tpg);
    return hip_check(dsa::launch_mla(mp, mla_uses_mfma(t), stream), "sparse attention");
  };
  const int n = tile_tokens(p, mla_bytes);
  if (!n) {
    if ((st = run(p, pg, q, kv, kv_scale, topk_idx, seq_lens, out, lse)) != DSA_OK) return st;
    return ok();
  }
  const int T = p->q_len;
  for (int b = 0; b < p->batch; ++b) {
    const dsa_paging tpg = pg ? tile_paging(pg, b) : dsa_paging{};
    const int64_t row0 = pg ? 0 : (int64_t)b * p->max_seq_len;  // first cache row of sequence b
    for (int t0 = 0; t0 < T; t0 += n) {
      const int nn = std::min(n, T - t0);
      const dsa_problem t = tile_problem(p, nn);
      const int64_t q0 = (int64_t)b * T + t0;
      if ((st = run(&t, pg ? &tpg : nullptr, advance(q, q0 * p->heads * p->qk_dim * elem_bytes(p->q_dtype)),
                    advance(kv, row0 * kv_row_bytes(p)), advance(kv_scale, row0 * kv_scale_row_bytes(p)),
                    topk_idx + q0 * p->top_k, seq_lens + b,
                    advance(out, q0 * p->heads * p->v_dim * elem_bytes(p->out_dtype)),
                    lse ? lse + q0 * p->heads : nullptr)) != DSA_OK)
        return st;
    }
  }
  return ok();
}

dsa_status dsa_sparse_mla_decode(const dsa_problem* p, const void* q, const void* kv,
                                 const float* kv_scale, const int32_t* topk_idx,
                                 const int32_t* seq_lens, void* out, float* lse, void* ws,
                                 size_t ws_bytes, struct ihipStream_t* stream) {
  return sparse_mla_impl(p, nullptr, q, kv, kv_scale, topk_idx, seq_lens, out, lse, ws, ws_bytes, stream);
}

dsa_status dsa_sparse_mla_decode_paged(const dsa_problem* p, const dsa_paging* pg, const void* q,
                                       const void* kv_pages, const float* kv_scales,
                                       const int32_t* topk_idx, const int32_t* seq_lens, void* out,
                                       float* lse, void* ws, size_t ws_bytes, struct ihipStream_t* stream) {
  if (!pg) return fail(DSA_ERR_INVALID_ARG, "pg must be non-NULL");
  return sparse_mla_impl(p, pg, q, kv_pages, kv_scales, topk_idx, seq_lens, out, lse, ws, ws_bytes, stream);
}

static int64_t fwd_ws_bytes(const dsa_problem* p) {
  const int n = tile_tokens(p, fwd_bytes);
  if (!n) return fwd_layout(p).bytes;
  const dsa_problem t = tile_problem(p, n);
  return fwd_layout(&t).bytes;
}

size_t dsa_forward_workspace_size(const dsa_problem* p) {
  if (validate_problem(p) != DSA_OK) return 0;
  return (size_t)fwd_ws_bytes(p);
}

int32_t dsa_forward_tile_tokens(const dsa_problem* p) {
  if (validate_problem(p) != DSA_OK) return -1;
  return tile_tokens(p, fwd_bytes);
}

// kValidate checks every argument but the workspace and enqueues nothing;
// kRunClearing zeroes the workspace's counters (a fill kernel) before the
// path runs, for a workspace whose contents are not known.
enum class FwdMode { kRun, kValidate, kRunClearing };

// The three stages over problem p (a whole problem or one token tile) in
// the workspace laid out for it.  With stage_events, event 0 goes before the
// scores and event i after stage i.
static dsa_status forward_run(const dsa_problem* p, const dsa_paging* pg, const void* q_idx, const float* head_w,
                              const void* k_idx, const void* k_scale, const void* q, const void* kv,
                              const float* kv_scale, const int32_t* seq_lens, int len_sub, float* scores,
                              int32_t* topk_idx, int32_t* topk_count, void* out, float* lse, uint8_t* w,
                              hipStream_t s, struct ihipEvent_t* const* stage_events) {
  dsa_status st;
  const FwdLayout F = fwd_layout(p);
  float* sc = scores ? scores : (float*)(w + F.off_scores);
  int32_t* idx = topk_idx ? topk_idx : (int32_t*)(w + F.off_idx);
  uint32_t* hist = (uint32_t*)(w + F.off_topk + F.tk.off_hist);
  auto rec = [&](int i) -> dsa_status {
    if (!stage_events) return DSA_OK;
    return hip_check(hipEventRecord((hipEvent_t)stage_events[i], s), "event record");
  };

  // the counters at the start of the workspace are zero on entry (and on return)
  // stage 1: scores (+ fused histogram when the matrix-core kernel runs, whose
  // dispatch then takes events 0 and 1 at the kernel's own start and end)
  const bool mfma_score = score_uses_mfma(p);
  auto sp = score_params(p, q_idx, head_w, k_idx, k_scale, seq_lens, sc, hist, len_sub);
  apply_paging(sp, pg);
  if (!mfma_score) {
    sp.hist = nullptr;
    if ((st = rec(0)) != DSA_OK) return st;
  }
  hipEvent_t ev0 = mfma_score && stage_events ? (hipEvent_t)stage_events[0] : nullptr;
  hipEvent_t ev1 = mfma_score && stage_events ? (hipEvent_t)stage_events[1] : nullptr;
  if ((st = hip_check(dsa::launch_score(sp, mfma_score, num_cus(), s, ev0, ev1), "index score")) != DSA_OK)
    return st;
  if (!mfma_score) {
    if ((st = hip_check(dsa::launch_hist(sc, seq_lens, len_sub, hist, p->batch, p->q_len, p->max_seq_len, s),
                        "histogram")) != DSA_OK)
      return st;
    if ((st = rec(1)) != DSA_OK) return st;
  }
  // stage 2: Top-K
  auto tp = topk_params(p, F.tk, w + F.off_topk, sc, seq_lens, idx, topk_count, len_sub);
  if ((st = hip_check(dsa::launch_select(tp, s), "select")) != DSA_OK) return st;
  if ((st = rec(2)) != DSA_OK) return st;
  // stage 3: sparse MLA attention
  auto mp = mla_params(p, F.mla, w + F.off_mla, q, kv, kv_scale, idx, seq_lens, out, lse);
  apply_paging(mp, pg);
  if ((st = hip_check(dsa::launch_mla(mp, mla_uses_mfma(p), s), "sparse attention")) != DSA_OK) return st;
  return rec(3);
}

static dsa_status forward_impl(const dsa_problem* p, const dsa_paging* pg, const void* q_idx,
                               const float* head_w, const void* k_idx, const void* k_scale, const void* q,
                               const void* kv, const float* kv_scale, const int32_t* seq_lens, float* scores,
                               int32_t* topk_idx, int32_t* topk_count, void* out, float* lse, void* ws,
                               size_t ws_bytes, hipStream_t stream, struct ihipEvent_t* const* stage_events,
                               FwdMode mode = FwdMode::kRun) {
  dsa_status st = validate_problem(p);
  if (st != DSA_OK) return st;
  if ((st = check_index_inputs(p, q_idx, head_w, k_idx, k_scale, seq_lens)) != DSA_OK) return st;
  if ((st = check_mla_inputs(p, q, kv, kv_scale, seq_lens, out, lse)) != DSA_OK) return st;
  if (pg && (st = check_paging(p, pg, true, true)) != DSA_OK) return st;
  REQUIRE(!scores || aligned(scores, 16), "scores must be 16-byte aligned");
  REQUIRE(!topk_idx || aligned(topk_idx, 4), "topk_idx must be 4-byte aligned");
  REQUIRE(!topk_count || aligned(topk_count, 4), "topk_count must be 4-byte aligned");
  if (stage_events)
    for (int i = 0; i <= DSA_FORWARD_STAGES; ++i)
      REQUIRE(stage_events[i], "stage_events[%d] is NULL", i);
  if (mode == FwdMode::kValidate) return ok();
  const int64_t need = fwd_ws_bytes(p);
  if ((int64_t)ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "dsa_forward needs %lld workspace bytes, got %zu", (long long)need,
                ws_bytes);
  REQUIRE(ws && aligned(ws, 256), "ws must be non-NULL and 256-byte aligned");

  uint8_t* w = (uint8_t*)ws;
  hipStream_t s = stream;
  const int n = tile_tokens(p, fwd_bytes);
  if (mode == FwdMode::kRunClearing) {
    const dsa_problem t = n ? tile_problem(p, n) : *p;
    if ((st = hip_check(dsa::launch_zero_u32((uint32_t*)w, topk_layout(&t).zero_bytes / 4, s),
                        "workspace counters")) != DSA_OK)
      return st;
  }
  if (!n) {
    if ((st = forward_run(p, pg, q_idx, head_w, k_idx, k_scale, q, kv, kv_scale, seq_lens, 0, scores, topk_idx,
                          topk_count, out, lse, w, s, stage_events)) != DSA_OK)
      return st;
    return ok();
  }
  // token tiles: every tile records the stage events around its own stages,
  // so on return they time the last tile's
  const int T = p->q_len;
  const int64_t H = p->heads;
  for (int b = 0; b < p->batch; ++b) {
    const dsa_paging tpg = pg ? tile_paging(pg, b) : dsa_paging{};
    const int64_t row0 = pg ? 0 : (int64_t)b * p->max_seq_len;  // first cache row of sequence b
    for (int t0 = 0; t0 < T; t0 += n) {
      const int nn = std::min(n, T - t0);
      const dsa_problem t = tile_problem(p, nn);
      const int64_t q0 = (int64_t)b * T + t0;  // first query of the tile
      if ((st = forward_run(&t, pg ? &tpg : nullptr,
                            advance(q_idx, q0 * p->idx_heads * p->idx_dim * elem_bytes(p->q_idx_dtype)),
                            head_w + q0 * p->idx_heads, advance(k_idx, row0 * key_row_bytes(p)),
                            advance(k_scale, row0 * key_scale_row_bytes(p)),
                            advance(q, q0 * H * p->qk_dim * elem_bytes(p->q_dtype)),
                            advance(kv, row0 * kv_row_bytes(p)), advance(kv_scale, row0 * kv_scale_row_bytes(p)),
                            seq_lens + b, T - t0 - nn, scores ? scores + q0 * p->max_seq_len : nullptr,
                            topk_idx ? topk_idx + q0 * p->top_k : nullptr, topk_count ? topk_count + q0 : nullptr,
                            advance(out, q0 * H * p->v_dim * elem_bytes(p->out_dtype)), lse ? lse + q0 * H : nullptr,
                            w, s, stage_events)) != DSA_OK)
        return st;
    }
  }
  return ok();
}

dsa_status dsa_forward(const dsa_problem* p, const void* q_idx, const float* head_w,
                       const void* k_idx, const void* k_scale, const void* q, const void* kv,
                       const float* kv_scale, const int32_t* seq_lens, float* scores,
                       int32_t* topk_idx, int32_t* topk_count, void* out, float* lse, void* ws,
                       size_t ws_bytes, struct ihipStream_t* stream,
                       struct ihipEvent_t* const* stage_events) {
  return forward_impl(p, nullptr, q_idx, head_w, k_idx, k_scale, q, kv, kv_scale, seq_lens, scores, topk_idx,
                      topk_count, out, lse, ws, ws_bytes, stream, stage_events);
}

dsa_status dsa_forward_noalloc(const dsa_problem* p, const void* q_idx, const float* head_w,
                               const void* k_idx, const void* k_scale, const void* q, const void* kv,
                               const float* kv_scale, const int32_t* seq_lens, float* scores,
                               int32_t* topk_idx, int32_t* topk_count, void* out, float* lse,
                               struct ihipStream_t* stream, struct ihipEvent_t* const* stage_events) {
  // every argument first (no HIP call before this), then the size bound
  dsa_status st = forward_impl(p, nullptr, q_idx, head_w, k_idx, k_scale, q, kv, kv_scale, seq_lens, scores,
                               topk_idx, topk_count, out, lse, nullptr, 0, stream, stage_events, FwdMode::kValidate);
  if (st != DSA_OK) return st;
  const int64_t need = fwd_ws_bytes(p);
  if (need > (int64_t)DSA_NOALLOC_WORKSPACE_BYTES)
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL,
                "dsa_forward_noalloc: this problem needs %lld workspace bytes, more than the %zu the library "
                "holds per GPU; use dsa_forward with a workspace of dsa_forward_workspace_size(p) bytes",
                (long long)need, (size_t)DSA_NOALLOC_WORKSPACE_BYTES);
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if ((st = hip_check(dsa::noalloc_workspace(&ws, &ws_bytes), "library workspace lookup")) != DSA_OK) return st;
  return forward_impl(p, nullptr, q_idx, head_w, k_idx, k_scale, q, kv, kv_scale, seq_lens, scores, topk_idx,
                      topk_count, out, lse, ws, ws_bytes, stream, stage_events, FwdMode::kRunClearing);
}

dsa_status dsa_forward_paged(const dsa_problem* p, const dsa_paging* pg, const void* q_idx,
                             const float* head_w, const void* k_pages, const void* k_scales,
                             const void* q, const void* kv_pages, const float* kv_scales,
                             const int32_t* seq_lens, float* scores, int32_t* topk_idx,
                             int32_t* topk_count, void* out, float* lse, void* ws, size_t ws_bytes,
                             struct ihipStream_t* stream, struct ihipEvent_t* const* stage_events) {
  if (!pg) return fail(DSA_ERR_INVALID_ARG, "pg must be non-NULL");
  return forward_impl(p, pg, q_idx, head_w, k_pages, k_scales, q, kv_pages, kv_scales, seq_lens, scores, topk_idx,
                      topk_count, out, lse, ws, ws_bytes, stream, stage_events);
}

int dsa_kernel_choice(const dsa_problem* p, char* buf, size_t len) {
  if (!buf || len == 0) return -1;
  if (validate_problem(p) != DSA_OK) {
    snprintf(buf, len, "invalid");
    return -1;
  }
  // a call in token tiles launches each stage per tile: name the tile's launches
  const int n = tile_tokens(p, fwd_bytes);
  const dsa_problem t = n ? tile_problem(p, n) : *p;
  char score[160] = "generic";
  if (score_uses_mfma(&t))
    dsa::score_launch_desc(score_params(&t, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), num_cus(),
                           score, sizeof score);
  dsa::TopkParams tk{};
  tk.B = t.batch;
  tk.T = t.q_len;
  tk.K = t.top_k;
  tk.Lmax = t.max_seq_len;
  const MlaLayout L = mla_layout(&t);
  snprintf(buf, len, "score=%s topk=%s mla=%s splits=%d rows_per_split=%d select_chunk=%d tile_tokens=%d", score,
           dsa::select_row_mode(tk) ? "radix-select, one workgroup per query" : "radix-select, chunks + emit",
           mla_uses_mfma(&t) ? "mfma" : "generic", L.splits, L.rows_per_split, topk_layout(&t).chunk, n);
  return 0;
}

}  // extern "C"
