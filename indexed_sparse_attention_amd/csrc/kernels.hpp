// Kernel parameter blocks and host-side launchers of the DSA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

struct ScoreParams {
  const void* q_idx;        // [B,T,Hi,Di] q_dtype
  const float* head_w;      // [B,T,Hi]
  const void* k_idx;        // [B,Lmax,Di] k_dtype
  const void* k_scale;      // fp32 [B,Lmax] (e4m3), E8M0 bytes [B,Lmax,Di/32] (mxfp8) or null
  const int32_t* seq_lens;  // [B]
  int len_sub;              // filled rows of sequence b: seq_lens[b] (clamped) - len_sub (see filled_rows)
  float* scores;            // [B,T,Lmax]
  uint32_t* hist;           // [B*T, 4096] (zeroed) or null
  int B, T, Hi, Di;
  int64_t Lmax;
  int q_dtype, k_dtype;
  // Paged caches (block_table non-null): k_idx [num_pages, 2^page_shift, Di]
  // and k_scale [num_pages, 2^page_shift]; row s of sequence b lives in
  // physical page block_table[b * max_pages + s >> page_shift].
  const int32_t* block_table;
  int64_t num_pages;
  int max_pages, page_shift;
  int split_mode;           // 0: by segment size; 1: every segment round-robin; 2: every segment exact (tests)
  uint64_t* wg_trace;       // null, or per-workgroup clock stamps (see trace_region)
};

struct TopkParams {
  const float* scores;      // [B,T,Lmax]
  const int32_t* seq_lens;  // [B]
  int len_sub;              // as in ScoreParams
  uint32_t* hist;           // [B*T, 4096] score-key histograms (complete on entry; cleared after use)
  uint2* cand;              // [B*T, Lmax] per-chunk ordered (key, position) candidates (bin >= threshold bin)
  uint32_t* bin_keys;       // [B*T, Lmax rounded up to 4] per-chunk ordered keys in the threshold bin
  uint2* header;            // [B*T] (threshold bin, entries above it)
  uint32_t* chunk_cnt;      // [B*T, n_chunks] candidates per chunk
  uint32_t* chunk_above;    // [B*T, n_chunks] candidates above the threshold bin per chunk
  int32_t* topk_idx;        // [B,T,K]
  int32_t* topk_count;      // [B,T] or null
  int B, T, K;
  int64_t Lmax;
  int chunk;                // positions per select workgroup
  int n_chunks;             // ceil(Lmax / chunk) <= 1024
  uint64_t* wg_trace;       // null, or per-workgroup clock stamps (see trace_region)
};

struct MlaParams {
  const void* q;            // [B,T,H,Dqk]
  const void* kv;           // [B,Lmax,Dqk]
  const float* kv_scale;    // [B,Lmax] (e4m3), [B,Lmax,ceil(Dqk/128)] (e4m3, 128-column tiles) or null
  const int32_t* topk_idx;  // [B,T,K]
  const int32_t* seq_lens;  // [B]
  int len_sub;              // as in ScoreParams
  void* out;                // [B,T,H,Dv]
  float* lse;               // [B,T,H] or null
  uint16_t* part_o;         // [splits, B*T, H, Dv] bf16, each split's output normalised by its own sum (splits > 1)
  float* part_ml;           // [splits, B*T, H, 2]  running max (base 2) and sum of each split (splits > 1)
  int B, T, H, Dqk, Dv, K;
  int64_t Lmax;
  float scale;
  int q_dtype, kv_dtype, out_dtype;
  int splits;               // row splits per query
  int rows_per_split;       // multiple of the row tile
  // Paged cache (block_table non-null): kv [num_pages, 2^page_shift, Dqk]
  // and kv_scale [num_pages, 2^page_shift], addressed as for ScoreParams.
  const int32_t* block_table;
  int64_t num_pages;
  int max_pages, page_shift;
  uint64_t* wg_trace;       // null, or per-workgroup clock stamps (see trace_region)
};

// Workgroup timeline: a kernel given a non-null wg_trace writes, from its
// first thread, the GPU's constant 100 MHz clock when workgroup w starts and
// when that thread leaves into wg_trace[2 w] and wg_trace[2 w + 1] (w the
// workgroup's linear index).  trace_region gives a launch of `kind` with
// `grid` workgroups its region of the buffer set by dsa_set_workgroup_trace,
// or null (tracing off, or the grid larger than the buffer's slots).
enum TraceKind {
  kTraceScore, kTraceSelectChunk, kTraceSelectEmit, kTraceSelectRow, kTraceMla, kTraceMlaCombine, kTraceKinds
};
uint64_t* trace_region(int kind, int64_t grid);

// Raises a kernel's dynamic LDS limit to `bytes` (once per kernel and device).
hipError_t set_max_dynamic_lds(const void* kernel, int bytes);

// index_score.hip
bool score_mfma_supported(const ScoreParams& p);
// With the matrix-core kernel, ev_start / ev_stop (either may be null) are
// recorded by the dispatch itself at the kernel's start and end.
hipError_t launch_score(const ScoreParams& p, bool allow_mfma, int num_cus, hipStream_t stream,
                        hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
// Names the matrix-core launch launch_score would make for p (snprintf's result).
int score_launch_desc(const ScoreParams& p, int num_cus, char* buf, size_t len);

// topk.hip
hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t stream);
hipError_t launch_hist(const float* scores, const int32_t* seq_lens, int len_sub, uint32_t* hist, int B, int T,
                       int64_t Lmax, hipStream_t stream);
hipError_t launch_select(const TopkParams& p, hipStream_t stream);
// Whether launch_select runs one workgroup per query (reads B, T and Lmax only).
bool select_row_mode(const TopkParams& p);

// noalloc_ws.hip: the device address (on the current device) and size of
// the library-owned workspace of dsa_forward_noalloc.
hipError_t noalloc_workspace(void** ptr, size_t* bytes);

// sparse_mla.hip
bool mla_mfma_supported(const MlaParams& p);
int mla_row_tile();
int mla_max_rows_per_split();  // index entries one MFMA-kernel workgroup stages in LDS at a time
hipError_t launch_mla(const MlaParams& p, bool allow_mfma, hipStream_t stream);

}  // namespace dsa
