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
//      query) and, into a region of its own, the keys whose bin is B;
//   3. select_emit_kernel: every chunk gathers its query's bin-B keys from
//      all chunks into LDS, resolves the exact K-th key tau from two more
//      digits of 10 key bits, counts the entries kept before its own chunk,
//      and writes its own kept positions: every key > tau plus, in position
//      order, the first K - #{key > tau} keys equal to tau.
// Both steps are latency-bound (a few KB per workgroup): each issues every
// load that does not depend on another before using any, and block-wide
// prefix sums run on cross-lane (DPP) adds.
// select_row_kernel does all of it in one 1024-thread workgroup per query
// (used for many short queries, where it saves two launches).
// The only counter is the step-1 histogram: zero on entry, cleared by the
// step that follows its last reader (the emit step's chunk 0; in row mode the
// query's workgroup).  The workspace is left as it was found.
#include <stdlib.h>
#include <string.h>

#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace dsa {

constexpr int64_t kRowMaxLen = 262144;  // longest query range handled by one workgroup

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

__global__ __launch_bounds__(256) void hist_kernel(const float* scores, const int32_t* seq_lens, int len_sub,
                                                    uint32_t* hist, int T, int64_t Lmax) {
  __shared__ uint32_t h[kHistBins];
  const int bt = blockIdx.y, b = bt / T, t = bt % T;
  const int64_t vis = (int64_t)filled_rows(seq_lens[b], Lmax, len_sub) - T + 1 + t;
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

hipError_t launch_hist(const float* scores, const int32_t* seq_lens, int len_sub, uint32_t* hist, int B, int T,
                       int64_t Lmax, hipStream_t stream) {
  dim3 grid((unsigned)((Lmax + kHistChunk - 1) / kHistChunk), (unsigned)(B * T));
  hipLaunchKernelGGL(hist_kernel, grid, dim3(256), 0, stream, scores, seq_lens, len_sub, hist, T, Lmax);
  return hipGetLastError();
}

constexpr int kSelV = 16;          // consecutive positions per thread per step

__device__ __forceinline__ void write_all_visible(int32_t* out, int64_t c_lo, int64_t c_hi, int64_t vis, int K,
                                                  int c, int32_t* count) {
  for (int64_t s = c_lo + threadIdx.x; s < c_hi; s += blockDim.x) out[s] = (int32_t)s;
  if (c == 0) {
    for (int64_t j = vis + threadIdx.x; j < K; j += blockDim.x) out[j] = -1;
    if (threadIdx.x == 0 && count) *count = (int32_t)vis;
  }
}

// kSelV consecutive scores from s0; positions >= lim get arbitrary values
// (the caller masks them).  Every load is unconditional, its address clamped
// into [.., lim): with per-lane branches the compiler would drain the loads
// of one branch before issuing the other's.  VEC4: row + s0 is 16-byte
// aligned and lim - s0 is a multiple of 4 for every lane.
template <bool VEC4>
__device__ __forceinline__ void load_scores(const float* row, int64_t s0, int64_t lim, float (&v)[kSelV]) {
  if constexpr (VEC4) {
#pragma unroll
    for (int j = 0; j < kSelV; j += 4) {
      const f32x4 x = *(const f32x4*)(row + min(s0 + j, lim - 4));
      v[j] = x[0];
      v[j + 1] = x[1];
      v[j + 2] = x[2];
      v[j + 3] = x[3];
    }
  } else {
#pragma unroll
    for (int j = 0; j < kSelV; ++j) v[j] = row[min(s0 + j, lim - 1)];
  }
}

// Step 2: one chunk's candidates.  Writes, in position order, every
// (key, position) whose bin is >= B to the chunk's slots of `cand`, the keys
// whose bin is B to its slots of `bin_keys`, and the two counts.
// VEC4: the scores are 16-byte aligned and Lmax is a multiple of 4.
template <bool VEC4>
__global__ __launch_bounds__(kSelThreads) void select_chunk_kernel(TopkParams p) {
  const WgTrace wg_trace_(p.wg_trace);
  __shared__ uint32_t s_wave[2 * kSelWaves];
  __shared__ uint32_t s_res[2];
  const int tid = threadIdx.x;
  const int c = blockIdx.x;
  const int bt = blockIdx.y, b = bt / p.T, t = bt % p.T;
  const int K = p.K;
  const int64_t c_lo = (int64_t)c * p.chunk;
  const int64_t c_end = min(c_lo + (int64_t)p.chunk, p.Lmax);  // loads stay inside the query's row
  const float* row = p.scores + (int64_t)bt * p.Lmax;
  constexpr int kRound = kSelThreads * kSelV;

  // every load that depends on no other: length, histogram slice, first round of scores
  const int len = filled_rows(p.seq_lens[b], p.Lmax, p.len_sub);
  BinSlice<kHistBins> hs;
  load_bin_slice<kHistBins>(p.hist + (int64_t)bt * kHistBins, hs);
  float v[kSelV];
  load_scores<VEC4>(row, c_lo + (int64_t)tid * kSelV, c_end, v);

  const int64_t vis = max((int64_t)0, (int64_t)len - p.T + 1 + t);
  int32_t* out = p.topk_idx + (int64_t)bt * K;
  const int64_t c_hi = min(c_end, vis);
  if (vis <= K) {  // every visible position is selected; the histogram has no other reader
    write_all_visible(out, c_lo, min(c_lo + (int64_t)p.chunk, vis), vis, K, c,
                      p.topk_count ? p.topk_count + bt : nullptr);
    if (c == 0) clear_query_hist(p, bt, kSelThreads);
    return;
  }
  if (c_lo >= c_hi) return;  // beyond this query's visible range

  uint32_t bin, above;
  threshold_from_slice<kHistBins>(hs, (uint32_t)K, s_wave, s_res, &bin, &above);
  if (c == 0 && tid == 0) p.header[bt] = make_uint2(bin, above);

  uint2* cand = p.cand + (int64_t)bt * p.Lmax + c_lo;
  uint32_t* blst = p.bin_keys + (int64_t)bt * bin_key_stride(p.Lmax) + c_lo;
  uint32_t n_out = 0, n_bin = 0;
  for (int64_t base = c_lo; base < c_hi; base += kRound) {
    const int64_t s0 = base + (int64_t)tid * kSelV;
    const bool more = base + kRound < c_hi;
    float nx[kSelV];
    if (more) load_scores<VEC4>(row, s0 + kRound, c_end, nx);
    uint32_t key[kSelV];
    uint32_t cnt[2] = {0u, 0u}, tot[2];  // entries with bin >= B, with bin == B
#pragma unroll
    for (int j = 0; j < kSelV; ++j) {
      key[j] = score_key(v[j]);
      const uint32_t kb = key[j] >> kHistShift;
      const bool in = s0 + j < c_hi;
      cnt[0] += (in && kb >= bin) ? 1u : 0u;
      cnt[1] += (in && kb == bin) ? 1u : 0u;
    }
    uint32_t inc[2] = {cnt[0], cnt[1]};
    block_scan<2, kSelWaves>(inc, s_wave, tot);
    uint32_t off = n_out + inc[0] - cnt[0], off_b = n_bin + inc[1] - cnt[1];
#pragma unroll
    for (int j = 0; j < kSelV; ++j) {
      const uint32_t kb = key[j] >> kHistShift;
      const bool in = s0 + j < c_hi;
      if (in && kb >= bin) cand[off++] = make_uint2(key[j], (uint32_t)(s0 + j));
      if (in && kb == bin) blst[off_b++] = key[j];
    }
    n_out += tot[0];
    n_bin += tot[1];
    if (more) {
#pragma unroll
      for (int j = 0; j < kSelV; ++j) v[j] = nx[j];
    }
  }
  if (tid == 0) {
    p.chunk_cnt[(int64_t)bt * p.n_chunks + c] = n_out;
    p.chunk_above[(int64_t)bt * p.n_chunks + c] = n_out - n_bin;
  }
}

// Step 3: exact threshold, then this chunk's kept positions at their final
// slots.  Every load is issued before any is used: the threshold
// resolution's (all chunks' counts, the first bin-B keys of every chunk) and
// this chunk's first kSelThreads * kEmitE candidates; a typical workgroup
// waits for memory once.
__global__ __launch_bounds__(kSelThreads) void select_emit_kernel(TopkParams p) {
  const WgTrace wg_trace_(p.wg_trace);
  extern __shared__ __attribute__((aligned(16))) uint8_t emit_lds[];
  EmitShared& sh = *(EmitShared*)emit_lds;
  const int tid = threadIdx.x;
  const int c = blockIdx.x;
  const int bt = blockIdx.y, b = bt / p.T, t = bt % p.T;
  const int K = p.K;
  const int64_t chunk = p.chunk;
  const int64_t c_lo = (int64_t)c * chunk;
  const int64_t c_len = min(chunk, p.Lmax - c_lo);  // this chunk's candidate slots
  const uint2* mine = p.cand + (int64_t)bt * p.Lmax + c_lo;

  // ---- loads ----
  const int len = filled_rows(p.seq_lens[b], p.Lmax, p.len_sub);
  const uint32_t n_mine = p.chunk_cnt[(int64_t)bt * p.n_chunks + c];
  ResolveLoads rl;
  issue_resolve_loads(p, bt, rl);
  uint2 e[kEmitE];  // candidates kEmitE tid + i of the current round
#pragma unroll
  for (int i = 0; i < kEmitE; ++i) e[i] = mine[min((int64_t)(kEmitE * tid + i), c_len - 1)];

  const int64_t vis = max((int64_t)0, (int64_t)len - p.T + 1 + t);
  if (vis <= K || c_lo >= vis) return;
  int32_t* out = p.topk_idx + (int64_t)bt * K;
  const Resolved rs = resolve_threshold(p, bt, vis, rl, sh);
  const uint32_t tau = rs.tau, take_ties = rs.take_ties;

  // bin-B keys of the chunks before this one: above tau, and equal to tau
  uint32_t ge[2] = {0u, 0u}, ge_tot[2];
  for_each_bin_key(p, bt, sh, rs.in_lds, c, [&](uint32_t k) {
    ge[0] += k > tau ? 1u : 0u;
    ge[1] += k == tau ? 1u : 0u;
  });
  block_scan<2, kSelWaves>(ge, sh.wave, ge_tot);
  const uint32_t above_before = sh.aoff[c];

  // this chunk's candidates in order (kEmitE consecutive per thread)
  uint32_t gt_seen = above_before + ge_tot[0], ties_seen = ge_tot[1];
  for (uint32_t n0 = 0; n0 < n_mine; n0 += kSelThreads * kEmitE) {
    const uint32_t nbase = n0 + (uint32_t)tid * kEmitE;
    if (n0 > 0) {
#pragma unroll
      for (int i = 0; i < kEmitE; ++i) e[i] = mine[min((int64_t)(nbase + i), c_len - 1)];
    }
    uint32_t qg[2] = {0u, 0u}, qg_tot[2];  // ties, keys above tau
#pragma unroll
    for (int i = 0; i < kEmitE; ++i) {
      const bool in = nbase + i < n_mine;
      qg[0] += (in && e[i].x == tau) ? 1u : 0u;
      qg[1] += (in && e[i].x > tau) ? 1u : 0u;
    }
    uint32_t inc[2] = {qg[0], qg[1]};
    block_scan<2, kSelWaves>(inc, sh.wave, qg_tot);
    uint32_t rank = ties_seen + inc[0] - qg[0];
    const uint32_t g_before = gt_seen + inc[1] - qg[1];
    uint32_t o = g_before + min(rank, take_ties);
#pragma unroll
    for (int i = 0; i < kEmitE; ++i) {
      const bool in = nbase + i < n_mine;
      const bool tie = in && e[i].x == tau;
      const bool sel = in && (e[i].x > tau || (tie && rank < take_ties));
      rank += tie ? 1u : 0u;
      if (sel && o < (uint32_t)K) out[o] = (int32_t)e[i].y;
      o += sel ? 1u : 0u;
    }
    gt_seen += qg_tot[1];
    ties_seen += qg_tot[0];
  }
  if (c == 0) {
    if (tid == 0 && p.topk_count) p.topk_count[bt] = K;
    clear_query_hist(p, bt, kSelThreads);  // step 2, its only reader, has finished
  }
}

// --------------------------------------------------------------------------
// Row mode: one 1024-thread workgroup per query.  Each of its 16 waves
// streams one contiguous range of the query's scores (16 consecutive
// positions per lane per round, two rounds in flight) and appends its
// candidates (key bin >= threshold bin) in position order to a list of its
// own: kWaveCap entries in LDS, then a spill range in the global candidate
// list that only this wave uses (the slots of its own positions).  No
// barrier while streaming, and no other wave ever reads a wave's spill.  The
// refinement histograms and the emit then run over the 16 lists, which in
// wave order are the candidates in position order: one scan over the waves'
// counts gives each wave its output offsets.  No cross-workgroup
// synchronisation.  Used when a query's visible range is at most kRowMaxLen
// positions.  (A first version compacted each round of the whole workgroup
// with a block-wide scan, two barriers per 16K positions: 41 us for 8
// queries of 128K positions.)
// --------------------------------------------------------------------------
constexpr int kRowThreads = 1024;
constexpr int kRowWaves = kRowThreads / kWave;
constexpr int kRowV = 4;
constexpr int kRowCap = 6000;  // candidates kept in LDS (struct < 64 KB); the rest spill to the global list
constexpr int kWaveCap = kRowCap / kRowWaves;  // each wave's share of them
static_assert(kWaveCap * kRowWaves == kRowCap, "LDS list split evenly over the waves");

struct RowShared {
  uint32_t wave[kRowWaves];
  uint32_t res[2];
  uint32_t gt[kRowWaves], eq[kRowWaves];  // per wave: candidates above / equal to the K-th key
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

__global__ __launch_bounds__(kRowThreads, 8) void select_row_kernel(TopkParams p) {
  const WgTrace wg_trace_(p.wg_trace);
  extern __shared__ __attribute__((aligned(16))) uint8_t row_lds[];
  RowShared& sh = *(RowShared*)row_lds;
  const int tid = threadIdx.x, wave = tid / kWave, l = lane_id();
  const int bt = blockIdx.x, b = bt / p.T, t = bt % p.T;
  const int len = filled_rows(p.seq_lens[b], p.Lmax, p.len_sub);
  const int64_t vis = max((int64_t)0, (int64_t)len - p.T + 1 + t);
  const int K = p.K;
  int32_t* out = p.topk_idx + (int64_t)bt * K;

  if (vis <= K) {  // every visible position is selected
    for (int64_t s = tid; s < K; s += kRowThreads) out[s] = s < vis ? (int32_t)s : -1;
    if (tid == 0 && p.topk_count) p.topk_count[bt] = (int32_t)vis;
    clear_query_hist(p, bt, kRowThreads);
    return;
  }

  // 1. threshold bin from the complete histogram (then the counters are
  // cleared: this workgroup is their only reader)
  uint32_t bin, above;
  row_threshold_bin<kHistBins>(p.hist + (int64_t)bt * kHistBins, (uint32_t)K, sh.wave, sh.res, &bin, &above);
  clear_query_hist(p, bt, kRowThreads);

  // 2. each wave streams its range [lo, hi) of the scores into its own list,
  // in rounds of 1024 positions.  Ranges are multiples of 16 positions (a
  // lane's share of a round, so vector loads stay 16-byte aligned) and as
  // short as 16 equal ranges allow: a wave never holds more candidates than
  // positions, so a query that sees little more than K positions fits its
  // lists in LDS.
  constexpr int kRound = kWave * kRowV;
  const int64_t span = (vis + kRowWaves * kRowV - 1) / (kRowWaves * kRowV) * kRowV;
  const int64_t lo = min((int64_t)wave * span, vis), hi = min(lo + span, vis);
  const float* row = p.scores + (int64_t)bt * p.Lmax;
  uint32_t* lkey = sh.key + wave * kWaveCap;
  uint32_t* lpos = sh.pos + wave * kWaveCap;
  uint2* spill = p.cand + (int64_t)bt * p.Lmax + lo;  // entries kWaveCap.. of this wave's list
  const bool vec_ok = (((uintptr_t)row) & 15) == 0;
  auto load_round = [&](int64_t base, float (&v)[kRowV]) {
    const int64_t s0 = base + (int64_t)l * kRowV;
    if (vec_ok && s0 + kRowV <= hi) {
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
      for (int j = 0; j < kRowV; ++j) v[j] = (s0 + j < hi) ? row[s0 + j] : 0.0f;
    }
  };
  uint32_t n = 0;  // this wave's list length (wave-uniform)
  float cur[kRowV], nxt[kRowV];  // the round being compacted and the next one, in flight
  if (lo < hi) load_round(lo, cur);
  for (int64_t base = lo; base < hi; base += kRound) {
    if (base + kRound < hi) load_round(base + kRound, nxt);
    const int64_t s0 = base + (int64_t)l * kRowV;
    uint32_t key[kRowV];
    bool f[kRowV];
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < kRowV; ++j) {
      key[j] = score_key(cur[j]);
      f[j] = (s0 + j < hi) && ((key[j] >> kHistShift) >= bin);
      cnt += f[j] ? 1u : 0u;
    }
    const uint32_t incl = wave_incl_scan(cnt);
    uint32_t o = n + incl - cnt;
#pragma unroll
    for (int j = 0; j < kRowV; ++j) {
      if (f[j]) {
        if (o < (uint32_t)kWaveCap) {
          lkey[o] = key[j];
          lpos[o] = (uint32_t)(s0 + j);
        } else {
          spill[o - kWaveCap] = make_uint2(key[j], (uint32_t)(s0 + j));
        }
        ++o;
      }
    }
    n += __shfl(incl, kWave - 1, kWave);
#pragma unroll
    for (int j = 0; j < kRowV; ++j) cur[j] = nxt[j];
  }
  n = __builtin_amdgcn_readfirstlane(n);
  // this wave's spilled entries are read back by this wave only: its own
  // stores complete before its loads
  if (n > (uint32_t)kWaveCap) __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  auto key_at = [&](uint32_t i) -> uint32_t { return i < (uint32_t)kWaveCap ? lkey[i] : spill[i - kWaveCap].x; };
  auto pos_at = [&](uint32_t i) -> uint32_t { return i < (uint32_t)kWaveCap ? lpos[i] : spill[i - kWaveCap].y; };

  const uint32_t need = (uint32_t)K - above;
  // 3. refine: next 12 key bits among keys in `bin`, then the last 8
  for (int i = tid; i < kHistBins; i += kRowThreads) sh.sub[i] = 0;
  __syncthreads();
  for (uint32_t i = l; i < n; i += kWave) {
    const uint32_t k = key_at(i);
    if ((k >> kHistShift) == bin) atomicAdd(&sh.sub[(k >> 8) & 0xFFFu], 1u);
  }
  __syncthreads();
  uint32_t bin2, above2;
  row_threshold_bin<kHistBins>(sh.sub, need, sh.wave, sh.res, &bin2, &above2);
  const uint32_t need2 = need - above2;
  const uint32_t prefix24 = (bin << 12) | bin2;
  for (int i = tid; i < 256; i += kRowThreads) sh.sub[i] = 0;
  __syncthreads();
  for (uint32_t i = l; i < n; i += kWave) {
    const uint32_t k = key_at(i);
    if ((k >> 8) == prefix24) atomicAdd(&sh.sub[k & 0xFFu], 1u);
  }
  __syncthreads();
  uint32_t bin3, above3;
  row_threshold_bin<256>(sh.sub, need2, sh.wave, sh.res, &bin3, &above3);
  const uint32_t tau = (prefix24 << 8) | bin3;
  const uint32_t take_ties = need2 - above3;

  // 4. emit in position order: each wave's counts above / at tau, a scan
  // over the waves, then each wave writes its own entries (E consecutive
  // entries per lane) at their ranks
  uint32_t gt_w = 0, eq_w = 0;
  for (uint32_t i = l; i < n; i += kWave) {
    const uint32_t k = key_at(i);
    gt_w += k > tau ? 1u : 0u;
    eq_w += k == tau ? 1u : 0u;
  }
  for (int o = 32; o > 0; o >>= 1) {
    gt_w += __shfl_xor(gt_w, o, kWave);
    eq_w += __shfl_xor(eq_w, o, kWave);
  }
  if (l == 0) {
    sh.gt[wave] = gt_w;
    sh.eq[wave] = eq_w;
  }
  __syncthreads();
  uint32_t gt_seen = 0, ties_seen = 0;
  for (int w = 0; w < wave; ++w) {
    gt_seen += sh.gt[w];
    ties_seen += sh.eq[w];
  }
  constexpr int E = 4;
  for (uint32_t i0 = 0; i0 < n; i0 += kWave * E) {
    const uint32_t ib = i0 + (uint32_t)l * E;
    uint32_t k[E];
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      k[e] = (ib + e < n) ? key_at(ib + e) : 0u;
      gt += (ib + e < n && k[e] > tau) ? 1u : 0u;
      eq += (ib + e < n && k[e] == tau) ? 1u : 0u;
    }
    const uint32_t eq_incl = wave_incl_scan(eq), gt_incl = wave_incl_scan(gt);
    uint32_t rank = ties_seen + eq_incl - eq;
    uint32_t o = gt_seen + (gt_incl - gt) + min(rank, take_ties);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (ib + e >= n) break;
      bool sel = k[e] > tau;
      if (k[e] == tau) sel = rank++ < take_ties;
      if (sel) {
        if (o < (uint32_t)K) out[o] = (int32_t)pos_at(ib + e);
        ++o;
      }
    }
    gt_seen += __shfl(gt_incl, kWave - 1, kWave);
    ties_seen += __shfl(eq_incl, kWave - 1, kWave);
  }
  if (tid == 0 && p.topk_count) p.topk_count[bt] = K;
}

// DSA_TOPK_MODE=row|chunk overrides the choice (both give identical results).
bool select_row_mode(const TopkParams& p) {
  const char* e = getenv("DSA_TOPK_MODE");
  if (e && strcmp(e, "row") == 0) return true;
  if (e && strcmp(e, "chunk") == 0) return false;
  // one workgroup per query when the queries fill the GPU, or when they are
  // short enough that one workgroup streams a row faster than the two-kernel
  // chunked path finishes (32 queries of 8K: 15.9 against 18.0 us; 8 of
  // 128K: 30.9 against 18.0 us)
  return p.Lmax <= kRowMaxLen && ((int64_t)p.B * p.T >= 512 || p.Lmax <= 16384);
}

hipError_t launch_select(const TopkParams& p_in, hipStream_t stream) {
  TopkParams p = p_in;
  if (select_row_mode(p)) {
    p.wg_trace = trace_region(kTraceSelectRow, (int64_t)p.B * p.T);
    hipLaunchKernelGGL(select_row_kernel, dim3((unsigned)(p.B * p.T)), dim3(kRowThreads), sizeof(RowShared),
                       stream, p);
    return hipGetLastError();
  }
  dim3 grid((unsigned)p.n_chunks, (unsigned)(p.B * p.T));
  p.wg_trace = trace_region(kTraceSelectChunk, (int64_t)p.n_chunks * p.B * p.T);
  if ((((uintptr_t)p.scores) & 15) == 0 && p.Lmax % 4 == 0)
    hipLaunchKernelGGL(select_chunk_kernel<true>, grid, dim3(kSelThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(select_chunk_kernel<false>, grid, dim3(kSelThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = set_max_dynamic_lds((const void*)select_emit_kernel, (int)sizeof(EmitShared));
  if (e != hipSuccess) return e;
  p.wg_trace = trace_region(kTraceSelectEmit, (int64_t)p.n_chunks * p.B * p.T);
  hipLaunchKernelGGL(select_emit_kernel, grid, dim3(kSelThreads), sizeof(EmitShared), stream, p);
  return hipGetLastError();
}

}  // namespace dsa
