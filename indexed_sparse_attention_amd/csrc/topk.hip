// Per-query Top-K over the indexer scores: the K largest of S[b,t,0..vis),
// ties to the lower position, emitted as a set in ascending position order
// (so the sparse attention gathers rows in address order), padded with -1
// when fewer than K positions are visible.
//
// The pages ("Optimizing Next-Gen LLM Inference" §3.1, "Inference Acceleration
// for New Large Model Architectures" §3.1) only say the indexer selects the
// Top-K positions.  Here selection is an exact radix select on the
// order-preserving 32-bit key of each fp32 score:
//   1. a histogram of the top 12 key bits (built inside the score pass, or by
//      hist_kernel) gives the threshold bin B: fewer than K scores lie above
//      it and at least K at or above it;
//   2. select_kernel splits each query's positions into chunks; every chunk
//      writes, in position order, the positions whose bin is >= B;
//   3. the last chunk to finish (arrival counter) refines the threshold inside
//      bin B over the next 12 and the last 8 key bits to the exact K-th key
//      tau, then walks the chunk lists in order and emits every position with
//      key > tau plus the first K - #{key > tau} positions with key == tau.
#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

constexpr int kSelThreads = 256;
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
// Exclusive prefix of per-thread counts (0..4) built from per-element ballots:
// returns this thread's offset; *total gets the block total.
struct BlockScan {
  uint32_t wave_tot[kSelWaves];
};

template <int V>
__device__ __forceinline__ uint32_t block_prefix_flags(const bool (&flag)[V], BlockScan& sh,
                                                       uint32_t* total) {
  const int wave = threadIdx.x / kWave;
  const uint64_t lt = lanemask_lt();
  uint32_t before = 0, wave_total = 0;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const uint64_t m = __ballot(flag[j]);
    before += __popcll(m & lt);
    wave_total += __popcll(m);
  }
  __syncthreads();
  if (lane_id() == 0) sh.wave_tot[wave] = wave_total;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    if (w < wave) off += sh.wave_tot[w];
    tot += sh.wave_tot[w];
  }
  *total = tot;
  return off + before;
}

// Largest bin B (of nbins, nbins / 256 consecutive bins per thread) whose
// suffix count sum_{i >= B} h[i] reaches `need`; *above = sum_{i > B} h[i].
// Every thread returns the same values.  h may be global or shared memory.
template <int NB>
__device__ void find_threshold_bin(const uint32_t* h, uint32_t need, uint32_t* s_u32,
                                   uint32_t* bin, uint32_t* above) {
  constexpr int PER = NB / kSelThreads;
  const int tid = threadIdx.x;
  uint32_t own = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) own += h[tid * PER + i];
  // suffix sums over threads: inclusive suffix of thread tid = sum_{j >= tid} own_j
  s_u32[tid] = own;
  __syncthreads();
  for (int o = 1; o < kSelThreads; o <<= 1) {
    uint32_t v = (tid + o < kSelThreads) ? s_u32[tid + o] : 0u;
    __syncthreads();
    s_u32[tid] += v;
    __syncthreads();
  }
  const uint32_t incl = s_u32[tid];
  const uint32_t excl = incl - own;  // count strictly above this thread's bins
  __syncthreads();
  if (excl < need && need <= incl) {
    uint32_t run = excl;
    for (int i = PER - 1; i >= 0; --i) {
      const uint32_t c = h[tid * PER + i];
      if (run + c >= need) {
        s_u32[0] = (uint32_t)(tid * PER + i);
        s_u32[1] = run;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
  *bin = s_u32[0];
  *above = s_u32[1];
  __syncthreads();
}

constexpr int kSelV = 4;  // consecutive positions per thread per step

__global__ __launch_bounds__(kSelThreads) void select_kernel(TopkParams p) {
  __shared__ uint32_t s_u32[kSelThreads];
  __shared__ uint32_t s_sub[kHistBins];
  __shared__ BlockScan s_scan;
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int c = blockIdx.x;
  const int bt = blockIdx.y, b = bt / p.T, t = bt % p.T;
  const int len = clamp_len(p.seq_lens[b], p.Lmax);
  const int64_t vis = max((int64_t)0, (int64_t)len - p.T + 1 + t);
  const int K = p.K;
  int32_t* out = p.topk_idx + (int64_t)bt * K;
  const int64_t c_lo = (int64_t)c * p.chunk;
  const int64_t c_hi = min(c_lo + p.chunk, vis);

  if (vis <= K) {  // every visible position is selected
    for (int64_t s = c_lo + tid; s < c_hi; s += kSelThreads) out[s] = (int32_t)s;
    if (c == 0) {
      for (int64_t j = vis + tid; j < K; j += kSelThreads) out[j] = -1;
      if (tid == 0 && p.topk_count) p.topk_count[bt] = (int32_t)vis;
    }
    return;
  }
  if (c_lo >= c_hi) return;  // beyond this query's visible range
  const int n_chunks_q = (int)((vis + p.chunk - 1) / p.chunk);

  // 1. threshold bin from the complete histogram
  uint32_t bin, above;
  find_threshold_bin<kHistBins>(p.hist + (int64_t)bt * kHistBins, (uint32_t)K, s_u32, &bin, &above);

  // 2. ordered candidates of this chunk: positions whose key bin is >= bin
  const float* row = p.scores + (int64_t)bt * p.Lmax;
  uint32_t* cand = p.cand + (int64_t)bt * p.Lmax + c_lo;
  uint32_t n_out = 0;
  for (int64_t base = c_lo; base < c_hi; base += kSelThreads * kSelV) {
    bool f[kSelV];
    const int64_t s0 = base + (int64_t)tid * kSelV;
#pragma unroll
    for (int j = 0; j < kSelV; ++j) {
      const int64_t s = s0 + j;
      f[j] = (s < c_hi) && ((score_key(row[s]) >> kHistShift) >= bin);
    }
    uint32_t total;
    uint32_t off = n_out + block_prefix_flags<kSelV>(f, s_scan, &total);
#pragma unroll
    for (int j = 0; j < kSelV; ++j)
      if (f[j]) cand[off++] = (uint32_t)(s0 + j);
    n_out += total;
  }
  if (tid == 0) p.chunk_cnt[(int64_t)bt * p.n_chunks + c] = n_out;

  // 3. arrival: the last chunk of this query finishes the selection
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(&p.arrive[bt], 1u) == (uint32_t)(n_chunks_q - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  const uint32_t* cand_q = p.cand + (int64_t)bt * p.Lmax;
  const uint32_t* cnt_q = p.chunk_cnt + (int64_t)bt * p.n_chunks;
  const uint32_t need = (uint32_t)K - above;  // how many to take from bin `bin`

  // refine: next 12 key bits among keys in `bin`
  for (int i = tid; i < kHistBins; i += kSelThreads) s_sub[i] = 0;
  __syncthreads();
  for (int cc = 0; cc < n_chunks_q; ++cc) {
    const uint32_t n = cnt_q[cc];
    const uint32_t* lst = cand_q + (int64_t)cc * p.chunk;
    for (uint32_t j = tid; j < n; j += kSelThreads) {
      const uint32_t key = score_key(row[lst[j]]);
      if ((key >> kHistShift) == bin) atomicAdd(&s_sub[(key >> 8) & 0xFFFu], 1u);
    }
  }
  __syncthreads();
  uint32_t bin2, above2;
  find_threshold_bin<kHistBins>(s_sub, need, s_u32, &bin2, &above2);
  const uint32_t need2 = need - above2;
  const uint32_t prefix24 = (bin << 12) | bin2;

  // refine: last 8 key bits
  for (int i = tid; i < 256; i += kSelThreads) s_sub[i] = 0;
  __syncthreads();
  for (int cc = 0; cc < n_chunks_q; ++cc) {
    const uint32_t n = cnt_q[cc];
    const uint32_t* lst = cand_q + (int64_t)cc * p.chunk;
    for (uint32_t j = tid; j < n; j += kSelThreads) {
      const uint32_t key = score_key(row[lst[j]]);
      if ((key >> 8) == prefix24) atomicAdd(&s_sub[key & 0xFFu], 1u);
    }
  }
  __syncthreads();
  uint32_t bin3, above3;
  find_threshold_bin<256>(s_sub, need2, s_u32, &bin3, &above3);
  const uint32_t tau = (prefix24 << 8) | bin3;
  const uint32_t take_ties = need2 - above3;  // ties at tau to keep, lowest positions first

  // emit in position order
  uint32_t n_sel = 0, ties_seen = 0;
  for (int cc = 0; cc < n_chunks_q; ++cc) {
    const uint32_t n = cnt_q[cc];
    const uint32_t* lst = cand_q + (int64_t)cc * p.chunk;
    for (uint32_t j0 = 0; j0 < n; j0 += kSelThreads) {
      const uint32_t j = j0 + tid;
      uint32_t pos = 0, key = 0;
      if (j < n) {
        pos = lst[j];
        key = score_key(row[pos]);
      }
      bool eq[1] = {j < n && key == tau};
      uint32_t tie_total;
      const uint32_t tie_rank = ties_seen + block_prefix_flags<1>(eq, s_scan, &tie_total);
      bool sel[1] = {j < n && (key > tau || (eq[0] && tie_rank < take_ties))};
      uint32_t sel_total;
      const uint32_t o = n_sel + block_prefix_flags<1>(sel, s_scan, &sel_total);
      if (sel[0] && o < (uint32_t)K) out[o] = (int32_t)pos;
      n_sel += sel_total;
      ties_seen += tie_total;
    }
  }
  if (tid == 0 && p.topk_count) p.topk_count[bt] = K;
}

hipError_t launch_select(const TopkParams& p, hipStream_t stream) {
  dim3 grid((unsigned)p.n_chunks, (unsigned)(p.B * p.T));
  hipLaunchKernelGGL(select_kernel, grid, dim3(kSelThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dsa
