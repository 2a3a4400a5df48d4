// Per-query Top-K over the indexer scores: the K largest of S[b,t,0..vis),
// ties to the lower position, emitted as a set in ascending position order
// (so the sparse attention gathers rows in address order), padded with -1
// when fewer than K positions are visible.
//
// The pages ("Optimizing Next-Gen LLM Inference" §3.1, "Inference Acceleration
// for New Large Model Architectures" §3.1) only say the indexer selects the
// Top-K positions.  Here selection is an exact radix select on the
// order-preserving 32-bit key of each fp32 score, in three parallel steps
// with no synchronisation between workgroups:
//   1. a histogram of the top 12 key bits (built inside the score pass, or by
//      hist_kernel) gives the threshold bin B: fewer than K scores lie above
//      it and at least K at or above it;
//   2. select_chunk_kernel: every chunk of every query writes, in position
//      order, the (key, position) pairs whose bin is >= B (about 2-5K per
//      query), and adds the next 12 key bits of its bin-B entries to a second
//      per-query histogram;
//   3. select_emit_kernel: every chunk again reads that second histogram and
//      its query's whole candidate list, resolves the exact K-th key tau from
//      the last 8 bits, counts the entries kept before its own chunk, and
//      writes its own kept positions: every key > tau plus, in position
//      order, the first K - #{key > tau} keys equal to tau.
// select_row_kernel does all of it in one 1024-thread workgroup per query
// (used for many short queries, where it saves two launches).
// The counters (histograms, threshold-bin count) are zero on entry and are
// cleared again by their last reader: in the emit step the query's last
// chunk to finish (an arrival ticket taken after its own reads completed),
// in row mode the query's workgroup.  The workspace is left as it was found.
#include <stdlib.h>
#include <string.h>

#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

constexpr int kSelThreads = 256;
constexpr int64_t kRowMaxLen = 262144;  // longest query range handled by one workgroup
constexpr int kSelWaves = kSelThreads / kWave;

__global__ void zero_u32_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

// Standalone histogram of the top key bits over the visible scores.
constexpr int kHistChunk = 8192;

__global__ __launch_bounds__(256) void hist_kernel(const float* scores, const int32_t* seq_lens,
                                                    uint32_t* hist, int T, int64_t Lmax) {
  __shared__ uint32_t h[kHistBins];
  const int bt = blockIdx.y, b = bt / T, t = bt % T;
  const int64_t vis = (int64_t)clamp_len(seq_lens[b], Lmax) - T + 1 + t;
  const int64_t lo = (int64_t)blockIdx.x * kHistChunk;
  const int64_t hi = min(lo + kHistChunk, vis);
  if (lo >= hi) return;
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) h[i] = 0;
  __syncthreads();
  const float* row = scores + (int64_t)bt * Lmax;
  for (int64_t s = lo + threadIdx.x; s < hi; s += blockDim.x)
    atomicAdd(&h[score_key(row[s]) >> kHistShift], 1u);
  __syncthreads();
  uint32_t* gh = hist + (int64_t)bt * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

hipError_t launch_hist(const float* scores, const int32_t* seq_lens, uint32_t* hist, int B, int T,
                       int64_t Lmax, hipStream_t stream) {
  dim3 grid((unsigned)((Lmax + kHistChunk - 1) / kHistChunk), (unsigned)(B * T));
  hipLaunchKernelGGL(hist_kernel, grid, dim3(256), 0, stream, scores, seq_lens, hist, T, Lmax);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// block-wide helpers (256 threads = 4 waves)
// --------------------------------------------------------------------------
// Inclusive prefix sum of one value per thread, in thread order; *total gets
// the block total.  s_wave: kSelWaves words of shared scratch.
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* s_wave, uint32_t* total) {
  const int wave = threadIdx.x / kWave, l = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t y = __shfl_up(v, o, kWave);
    if (l >= o) v += y;
  }
  if (l == kWave - 1) s_wave[wave] = v;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    if (w < wave) off += s_wave[w];
    tot += s_wave[w];
  }
  __syncthreads();
  *total = tot;
  return off + v;
}

// Exclusive prefix of per-element flags in (thread, element) order.
template <int V>
__device__ __forceinline__ uint32_t block_prefix_flags(const bool (&flag)[V], uint32_t* s_wave,
                                                       uint32_t* total) {
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < V; ++j) c += flag[j] ? 1u : 0u;
  return block_incl_scan(c, s_wave, total) - c;
}

// Largest bin B of the NB-bin histogram h whose suffix count sum_{i >= B} h[i]
// reaches `need`; *above = sum_{i > B} h[i].  Thread tid owns the PER bins
// just below NB - PER*tid, so an inclusive scan in thread order counts the
// entries at or above each thread's lowest bin.  All threads get the result.
template <int NB>
__device__ void find_threshold_bin(const uint32_t* h, uint32_t need, uint32_t* s_wave,
                                   uint32_t* s_res, uint32_t* bin, uint32_t* above) {
  constexpr int PER = NB / kSelThreads;
  const int tid = threadIdx.x;
  const int top = NB - 1 - PER * tid;  // this thread's highest bin
  uint32_t c[PER];
  uint32_t own = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = h[top - i];
    own += c[i];
  }
  uint32_t total;
  const uint32_t incl = block_incl_scan(own, s_wave, &total);
  const uint32_t excl = incl - own;
  if (excl < need && need <= incl) {
    uint32_t run = excl;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (run + c[i] >= need) {
        s_res[0] = (uint32_t)(top - i);
        s_res[1] = run;
        break;
      }
      run += c[i];
    }
  }
  __syncthreads();
  *bin = s_res[0];
  *above = s_res[1];
  __syncthreads();
}

constexpr int kSelV = 16;         // consecutive positions per thread per step
constexpr int kEmitCap = 6000;    // threshold-bin entries the emit step keeps in LDS
constexpr int kBinBuf = 2048;     // threshold-bin entries a chunk stages in LDS

__device__ __forceinline__ void write_all_visible(int32_t* out, int64_t c_lo, int64_t c_hi, int64_t vis, int K,
                                                  int c, int32_t* count) {
  for (int64_t s = c_lo + threadIdx.x; s < c_hi; s += blockDim.x) out[s] = (int32_t)s;
  if (c == 0) {
    for (int64_t j = vis + threadIdx.x; j < K; j += blockDim.x) out[j] = -1;
    if (threadIdx.x == 0 && count) *count = (int32_t)vis;
  }
}

// Clears the query's counters (histograms, threshold-bin count, arrivals):
// run by the last workgroup that reads them.
__device__ __forceinline__ void clear_query_counters(const TopkParams& p, int bt, int nthreads) {
  uint32_t* h = p.hist + (int64_t)bt * kHistBins;
  uint32_t* g = p.sub_hist + (int64_t)bt * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += nthreads) {
    h[i] = 0;
    g[i] = 0;
  }
  if (threadIdx.x == 0) {
    p.bin_count[bt] = 0;
    p.done[bt] = 0;
  }
}

// Step 2: candidates of one chunk + second-level histogram of the threshold bin.
__global__ __launch_bounds__(kSelThreads) void select_chunk_kernel(TopkParams p) {
  __shared__ uint32_t s_wave[kSelWaves];
  __shared__ uint32_t s_res[2];
  __shared__ uint32_t s_sub[kHistBins];
  __shared__ uint2 s_binbuf[kBinBuf + 1];
  const int tid = threadIdx.x;
  const int c = blockIdx.x;
  const int bt = blockIdx.y, b = bt / p.T, t = bt % p.T;
  const int len = clamp_len(p.seq_lens[b], p.Lmax);
  const int64_t vis = max((int64_t)0, (int64_t)len - p.T + 1 + t);
  const int K = p.K;
  int32_t* out = p.topk_idx + (int64_t)bt * K;
  const int64_t c_lo = (int64_t)c * p.chunk;
  const int64_t c_hi = min(c_lo + p.chunk, vis);
  if (vis <= K) {  // every visible position is selected; nobody reads the counters
    write_all_visible(out, c_lo, c_hi, vis, K, c, p.topk_count ? p.topk_count + bt : nullptr);
    if (c == 0) clear_query_counters(p, bt, kSelThreads);
    return;
  }
  if (c_lo >= c_hi) return;  // beyond this query's visible range

  for (int i = tid; i < kHistBins; i += kSelThreads) s_sub[i] = 0;
  uint32_t bin, above;
  find_threshold_bin<kHistBins>(p.hist + (int64_t)bt * kHistBins, (uint32_t)K, s_wave, s_res, &bin, &above);
  if (c == 0 && tid == 0) p.header[bt] = make_uint2(bin, above);

  const float* row = p.scores + (int64_t)bt * p.Lmax;
  uint2* cand = p.cand + (int64_t)bt * p.Lmax + c_lo;
  const bool vec_ok = (((uintptr_t)(row + c_lo)) & 15) == 0;
  uint32_t n_out = 0, n_bin = 0;
  for (int64_t base = c_lo; base < c_hi; base += kSelThreads * kSelV) {
    const int64_t s0 = base + (int64_t)tid * kSelV;
    float v[kSelV];
    if (vec_ok && s0 + kSelV <= c_hi) {
#pragma unroll
      for (int j = 0; j < kSelV; j += 4) {
        const f32x4 x = *(const f32x4*)(row + s0 + j);
        v[j] = x[0];
        v[j + 1] = x[1];
        v[j + 2] = x[2];
        v[j + 3] = x[3];
      }
    } else {
#pragma unroll
      for (int j = 0; j < kSelV; ++j) v[j] = (s0 + j < c_hi) ? row[s0 + j] : 0.0f;
    }
    bool f[kSelV], fb[kSelV];
    uint32_t key[kSelV];
#pragma unroll
    for (int j = 0; j < kSelV; ++j) {
      key[j] = score_key(v[j]);
      const uint32_t kb = key[j] >> kHistShift;
      f[j] = (s0 + j < c_hi) && (kb >= bin);
      fb[j] = (s0 + j < c_hi) && (kb == bin);
      if (fb[j]) atomicAdd(&s_sub[(key[j] >> 8) & 0xFFFu], 1u);
    }
    uint32_t total, total_b;
    uint32_t off = n_out + block_prefix_flags<kSelV>(f, s_wave, &total);
    uint32_t off_b = n_bin + block_prefix_flags<kSelV>(fb, s_wave, &total_b);
#pragma unroll
    for (int j = 0; j < kSelV; ++j) {
      if (f[j]) cand[off++] = make_uint2(key[j], (uint32_t)(s0 + j));
      if (fb[j]) s_binbuf[min(off_b++, (uint32_t)kBinBuf)] = make_uint2(key[j], (uint32_t)(s0 + j));
    }
    n_out += total;
    n_bin += total_b;
  }
  if (tid == 0) {
    p.chunk_cnt[(int64_t)bt * p.n_chunks + c] = n_out;
    p.chunk_above[(int64_t)bt * p.n_chunks + c] = n_out - n_bin;
    // reserve this chunk's slots in the query's list of threshold-bin entries
    s_res[0] = atomicAdd(&p.bin_count[bt], n_bin);
  }
  __syncthreads();
  {
    uint2* dst = p.bin_list + (int64_t)bt * p.Lmax + s_res[0];
    if (n_bin <= (uint32_t)kBinBuf) {
      for (uint32_t j = tid; j < n_bin; j += kSelThreads) dst[j] = s_binbuf[j];
    } else {  // more bin entries than the LDS buffer: copy them from the candidate list
      // (this workgroup wrote cand; make its stores visible to all its waves first)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __syncthreads();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      uint32_t w = 0;
      for (uint32_t j0 = 0; j0 < n_out; j0 += kSelThreads) {
        const uint32_t j = j0 + tid;
        const uint2 e = j < n_out ? cand[j] : make_uint2(0u, 0u);
        bool fl[1] = {j < n_out && (e.x >> kHistShift) == bin};
        uint32_t tot;
        const uint32_t o = w + block_prefix_flags<1>(fl, s_wave, &tot);
        if (fl[0]) dst[o] = e;
        w += tot;
      }
    }
  }
  uint32_t* gsub = p.sub_hist + (int64_t)bt * kHistBins;
  for (int i = tid; i < kHistBins; i += kSelThreads)
    if (s_sub[i]) atomicAdd(&gsub[i], s_sub[i]);
}

struct EmitShared {
  uint32_t wave[kSelWaves];
  uint32_t res[2];
  uint32_t sub[256];
  uint32_t key[kEmitCap];
  uint32_t pos[kEmitCap];
};

// Step 3: exact threshold, then this chunk's kept positions at their final slots.
// Reads only contiguous data: the query's threshold-bin entries (unordered),
// the per-chunk counts of entries above the bin, and this chunk's candidates.
__global__ __launch_bounds__(kSelThreads) void select_emit_kernel(TopkParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t emit_lds[];
  EmitShared& sh = *(EmitShared*)emit_lds;
  const int tid = threadIdx.x;
  const int c = blockIdx.x;
  const int bt = blockIdx.y, b = bt / p.T, t = bt % p.T;
  const int len = clamp_len(p.seq_lens[b], p.Lmax);
  const int64_t vis = max((int64_t)0, (int64_t)len - p.T + 1 + t);
  const int K = p.K;
  const int64_t c_lo = (int64_t)c * p.chunk;
  if (vis <= K || c_lo >= vis) return;
  int32_t* out = p.topk_idx + (int64_t)bt * K;

  const uint2 hdr = p.header[bt];
  const uint32_t bin = hdr.x, need = (uint32_t)K - hdr.y;  // entries to take from bin `bin`
  const uint32_t M = p.bin_count[bt];
  const uint2* blist = p.bin_list + (int64_t)bt * p.Lmax;
  // entries above the bin in chunks before this one
  uint32_t ab = 0;
  for (int cc = tid; cc < c; cc += kSelThreads) ab += p.chunk_above[(int64_t)bt * p.n_chunks + cc];
  uint32_t above_before;
  block_incl_scan(ab, sh.wave, &above_before);

  uint32_t bin2, above2;
  find_threshold_bin<kHistBins>(p.sub_hist + (int64_t)bt * kHistBins, need, sh.wave, sh.res, &bin2, &above2);
  const uint32_t need2 = need - above2;
  const uint32_t prefix24 = (bin << 12) | bin2;

  const bool in_lds = M <= (uint32_t)kEmitCap;
  if (in_lds) {
    for (uint32_t n = tid; n < M; n += kSelThreads) {
      const uint2 e = blist[n];
      sh.key[n] = e.x;
      sh.pos[n] = e.y;
    }
  }
  for (int i = tid; i < 256; i += kSelThreads) sh.sub[i] = 0;
  __syncthreads();
  auto key_at = [&](uint32_t n) -> uint32_t { return in_lds ? sh.key[n] : blist[n].x; };
  auto pos_at = [&](uint32_t n) -> uint32_t { return in_lds ? sh.pos[n] : blist[n].y; };

  // last 8 key bits -> exact K-th key tau
  for (uint32_t n = tid; n < M; n += kSelThreads) {
    const uint32_t k = key_at(n);
    if ((k >> 8) == prefix24) atomicAdd(&sh.sub[k & 0xFFu], 1u);
  }
  __syncthreads();
  uint32_t bin3, above3;
  find_threshold_bin<256>(sh.sub, need2, sh.wave, sh.res, &bin3, &above3);
  const uint32_t tau = (prefix24 << 8) | bin3;
  const uint32_t take_ties = need2 - above3;  // ties at tau to keep, lowest positions first

  // bin entries before this chunk: above tau, and equal to tau
  uint32_t gt = 0, eq = 0;
  for (uint32_t n = tid; n < M; n += kSelThreads) {
    if (pos_at(n) < (uint32_t)c_lo) {
      const uint32_t k = key_at(n);
      gt += k > tau ? 1u : 0u;
      eq += k == tau ? 1u : 0u;
    }
  }
  uint32_t gt_bin_before, ties_before;
  block_incl_scan(gt, sh.wave, &gt_bin_before);
  block_incl_scan(eq, sh.wave, &ties_before);

  // this chunk's candidates in order (E consecutive per thread)
  const uint2* mine = p.cand + (int64_t)bt * p.Lmax + c_lo;
  const uint32_t n_mine = p.chunk_cnt[(int64_t)bt * p.n_chunks + c];
  constexpr int E = 8;
  uint32_t gt_seen = above_before + gt_bin_before, ties_seen = ties_before;
  for (uint32_t n0 = 0; n0 < n_mine; n0 += kSelThreads * E) {
    const uint32_t nb = n0 + (uint32_t)tid * E;
    uint2 e[E];
    uint32_t g = 0, q = 0;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      e[i] = (nb + i < n_mine) ? mine[nb + i] : make_uint2(0u, 0u);
      g += (nb + i < n_mine && e[i].x > tau) ? 1u : 0u;
      q += (nb + i < n_mine && e[i].x == tau) ? 1u : 0u;
    }
    uint32_t q_tot, g_tot;
    uint32_t rank = ties_seen + block_incl_scan(q, sh.wave, &q_tot) - q;
    const uint32_t g_before = gt_seen + block_incl_scan(g, sh.wave, &g_tot) - g;
    uint32_t o = g_before + min(rank, take_ties);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      if (nb + i >= n_mine) break;
      bool sel = e[i].x > tau;
      if (e[i].x == tau) sel = rank++ < take_ties;
      if (sel) {
        if (o < (uint32_t)K) out[o] = (int32_t)e[i].y;
        ++o;
      }
    }
    gt_seen += g_tot;
    ties_seen += q_tot;
  }
  if (c == 0 && tid == 0 && p.topk_count) p.topk_count[bt] = K;

  // Arrival ticket, taken once every read of the query's counters by this
  // workgroup has completed (the fence waits for them): the last chunk of
  // the query clears them.  Nothing is published, so no cache write-back.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  if (tid == 0) {
    const uint32_t n_act = (uint32_t)((vis + p.chunk - 1) / p.chunk);
    sh.res[0] = atomicAdd(&p.done[bt], 1u) + 1u == n_act ? 1u : 0u;
  }
  __syncthreads();
  if (sh.res[0]) clear_query_counters(p, bt, kSelThreads);
}

// --------------------------------------------------------------------------
// Row mode: one 1024-thread workgroup per query streams that query's scores
// once (16 consecutive positions per thread per round, two rounds in flight),
// compacts the candidates (key bin >= threshold bin) in position order
// straight into LDS, then refines the threshold and emits there.  No global
// candidate list, no cross-workgroup synchronisation.  Used when a query's
// visible range is at most kRowMaxLen positions.
// --------------------------------------------------------------------------
constexpr int kRowThreads = 1024;
constexpr int kRowWaves = kRowThreads / kWave;
constexpr int kRowV = 16;
constexpr int kRowCap = 6000;  // candidates kept in LDS (struct < 64 KB); the rest spill to the global list

struct RowShared {
  uint32_t wave[kRowWaves];
  uint32_t res[2];
  uint32_t sub[kHistBins];
  uint32_t key[kRowCap];
  uint32_t pos[kRowCap];
};

__device__ __forceinline__ uint32_t row_incl_scan(uint32_t v, uint32_t* s_wave, uint32_t* total) {
  const int wave = threadIdx.x / kWave, l = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t y = __shfl_up(v, o, kWave);
    if (l >= o) v += y;
  }
  if (l == kWave - 1) s_wave[wave] = v;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kRowWaves; ++w) {
    if (w < wave) off += s_wave[w];
    tot += s_wave[w];
  }
  __syncthreads();
  *total = tot;
  return off + v;
}

template <int NB>
__device__ void row_threshold_bin(const uint32_t* h, uint32_t need, uint32_t* s_wave, uint32_t* s_res,
                                  uint32_t* bin, uint32_t* above) {
  constexpr int PER = NB / kRowThreads > 0 ? NB / kRowThreads : 1;
  const int tid = threadIdx.x;
  const int top = NB - 1 - PER * tid;  // this thread's highest bin (negative: none)
  uint32_t c[PER];
  uint32_t own = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = (top - i >= 0) ? h[top - i] : 0u;
    own += c[i];
  }
  uint32_t total;
  const uint32_t incl = row_incl_scan(own, s_wave, &total);
  const uint32_t excl = incl - own;
  if (excl < need && need <= incl) {
    uint32_t run = excl;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (run + c[i] >= need) {
        s_res[0] = (uint32_t)(top - i);
        s_res[1] = run;
        break;
      }
      run += c[i];
    }
  }
  __syncthreads();
  *bin = s_res[0];
  *above = s_res[1];
  __syncthreads();
}

__global__ __launch_bounds__(kRowThreads) void select_row_kernel(TopkParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t row_lds[];
  RowShared& sh = *(RowShared*)row_lds;
  const int tid = threadIdx.x;
  const int bt = blockIdx.x, b = bt / p.T, t = bt % p.T;
  const int len = clamp_len(p.seq_lens[b], p.Lmax);
  const int64_t vis = max((int64_t)0, (int64_t)len - p.T + 1 + t);
  const int K = p.K;
  int32_t* out = p.topk_idx + (int64_t)bt * K;

  if (vis <= K) {  // every visible position is selected
    for (int64_t s = tid; s < K; s += kRowThreads) out[s] = s < vis ? (int32_t)s : -1;
    if (tid == 0 && p.topk_count) p.topk_count[bt] = (int32_t)vis;
    clear_query_counters(p, bt, kRowThreads);
    return;
  }

  // 1. threshold bin from the complete histogram (then the counters are
  // cleared: this workgroup is their only reader)
  uint32_t bin, above;
  row_threshold_bin<kHistBins>(p.hist + (int64_t)bt * kHistBins, (uint32_t)K, sh.wave, sh.res, &bin, &above);
  clear_query_counters(p, bt, kRowThreads);

  // 2. one pass over the scores: candidates in position order into LDS
  const float* row = p.scores + (int64_t)bt * p.Lmax;
  uint2* spill = p.cand + (int64_t)bt * p.Lmax;  // candidates beyond kRowCap, in order
  const bool vec_ok = (((uintptr_t)row) & 15) == 0;
  constexpr int kRound = kRowThreads * kRowV;
  auto load_round = [&](int64_t base, float (&v)[kRowV]) {
    const int64_t s0 = base + (int64_t)tid * kRowV;
    if (vec_ok && s0 + kRowV <= vis) {
#pragma unroll
      for (int j = 0; j < kRowV; j += 4) {
        const f32x4 x = *(const f32x4*)(row + s0 + j);
        v[j] = x[0];
        v[j + 1] = x[1];
        v[j + 2] = x[2];
        v[j + 3] = x[3];
      }
    } else {
#pragma unroll
      for (int j = 0; j < kRowV; ++j) v[j] = (s0 + j < vis) ? row[s0 + j] : 0.0f;
    }
  };
  uint32_t N = 0;
  float cur[kRowV], nxt[kRowV];
  load_round(0, cur);
  for (int64_t base = 0; base < vis; base += kRound) {
    if (base + kRound < vis) load_round(base + kRound, nxt);
    const int64_t s0 = base + (int64_t)tid * kRowV;
    uint32_t key[kRowV];
    bool f[kRowV];
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < kRowV; ++j) {
      key[j] = score_key(cur[j]);
      f[j] = (s0 + j < vis) && ((key[j] >> kHistShift) >= bin);
      cnt += f[j] ? 1u : 0u;
    }
    uint32_t total;
    uint32_t o = N + row_incl_scan(cnt, sh.wave, &total) - cnt;
#pragma unroll
    for (int j = 0; j < kRowV; ++j) {
      if (f[j]) {
        if (o < (uint32_t)kRowCap) {
          sh.key[o] = key[j];
          sh.pos[o] = (uint32_t)(s0 + j);
        } else {
          spill[o - kRowCap] = make_uint2(key[j], (uint32_t)(s0 + j));
        }
        ++o;
      }
    }
    N += total;
#pragma unroll
    for (int j = 0; j < kRowV; ++j) cur[j] = nxt[j];
  }
  if (N > (uint32_t)kRowCap) {  // spilled candidates are read back by other waves
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  auto key_at = [&](uint32_t n) -> uint32_t { return n < (uint32_t)kRowCap ? sh.key[n] : spill[n - kRowCap].x; };
  auto pos_at = [&](uint32_t n) -> uint32_t { return n < (uint32_t)kRowCap ? sh.pos[n] : spill[n - kRowCap].y; };

  const uint32_t need = (uint32_t)K - above;
  // 3. refine: next 12 key bits among keys in `bin`, then the last 8
  for (int i = tid; i < kHistBins; i += kRowThreads) sh.sub[i] = 0;
  __syncthreads();
  for (uint32_t n = tid; n < N; n += kRowThreads) {
    const uint32_t k = key_at(n);
    if ((k >> kHistShift) == bin) atomicAdd(&sh.sub[(k >> 8) & 0xFFFu], 1u);
  }
  __syncthreads();
  uint32_t bin2, above2;
  row_threshold_bin<kHistBins>(sh.sub, need, sh.wave, sh.res, &bin2, &above2);
  const uint32_t need2 = need - above2;
  const uint32_t prefix24 = (bin << 12) | bin2;
  for (int i = tid; i < 256; i += kRowThreads) sh.sub[i] = 0;
  __syncthreads();
  for (uint32_t n = tid; n < N; n += kRowThreads) {
    const uint32_t k = key_at(n);
    if ((k >> 8) == prefix24) atomicAdd(&sh.sub[k & 0xFFu], 1u);
  }
  __syncthreads();
  uint32_t bin3, above3;
  row_threshold_bin<256>(sh.sub, need2, sh.wave, sh.res, &bin3, &above3);
  const uint32_t tau = (prefix24 << 8) | bin3;
  const uint32_t take_ties = need2 - above3;

  // 4. emit in position order (E consecutive candidates per thread)
  constexpr int E = 4;
  uint32_t gt_seen = 0, ties_seen = 0;
  for (uint32_t n0 = 0; n0 < N; n0 += kRowThreads * E) {
    const uint32_t nb = n0 + (uint32_t)tid * E;
    uint32_t k[E];
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      k[e] = (nb + e < N) ? key_at(nb + e) : 0u;
      gt += (nb + e < N && k[e] > tau) ? 1u : 0u;
      eq += (nb + e < N && k[e] == tau) ? 1u : 0u;
    }
    uint32_t eq_tot, gt_tot;
    uint32_t rank = ties_seen + row_incl_scan(eq, sh.wave, &eq_tot) - eq;
    const uint32_t gt_before = gt_seen + row_incl_scan(gt, sh.wave, &gt_tot) - gt;
    uint32_t o = gt_before + min(rank, take_ties);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (nb + e >= N) break;
      bool sel = k[e] > tau;
      if (k[e] == tau) sel = rank++ < take_ties;
      if (sel) {
        if (o < (uint32_t)K) out[o] = (int32_t)pos_at(nb + e);
        ++o;
      }
    }
    gt_seen += gt_tot;
    ties_seen += eq_tot;
  }
  if (tid == 0 && p.topk_count) p.topk_count[bt] = K;
}

// DSA_TOPK_MODE=row|chunk overrides the choice (both give identical results).
bool select_row_mode(const TopkParams& p) {
  const char* e = getenv("DSA_TOPK_MODE");
  if (e && strcmp(e, "row") == 0) return true;
  if (e && strcmp(e, "chunk") == 0) return false;
  return p.Lmax <= kRowMaxLen && (int64_t)p.B * p.T >= 512;
}

hipError_t launch_select(const TopkParams& p, hipStream_t stream) {
  if (select_row_mode(p)) {
    hipLaunchKernelGGL(select_row_kernel, dim3((unsigned)(p.B * p.T)), dim3(kRowThreads), sizeof(RowShared),
                       stream, p);
    return hipGetLastError();
  }
  dim3 grid((unsigned)p.n_chunks, (unsigned)(p.B * p.T));
  hipLaunchKernelGGL(select_chunk_kernel, grid, dim3(kSelThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_emit_kernel, grid, dim3(kSelThreads), sizeof(EmitShared), stream, p);
  return hipGetLastError();
}

}  // namespace dsa
