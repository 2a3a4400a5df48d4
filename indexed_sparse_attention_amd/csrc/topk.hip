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
//      writes, in position order, the (key, position) pairs whose bin is >= B
//      (typically about 2K entries per query);
//   3. the last chunk to finish (arrival counter) gathers the concatenated
//      lists into LDS, refines the threshold inside bin B over the next 12 and
//      the last 8 key bits to the exact K-th key tau, and emits every position
//      with key > tau plus the first K - #{key > tau} positions with key == tau.
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
constexpr int kFinalCap = 5120;   // candidates the finaliser keeps in LDS (LDS < 64 KB)
constexpr int kMaxChunksLds = 1024;

struct SelectShared {
  uint32_t wave[kSelWaves];
  uint32_t res[2];
  int last;
  uint32_t sub[kHistBins];
  uint32_t chunk_off[kMaxChunksLds + 1];
  uint32_t key[kFinalCap];
  uint32_t pos[kFinalCap];
};

// Candidate n of the concatenated per-chunk lists (all chunks' lists in order).
__device__ __forceinline__ uint2 cand_at(const uint2* cand_q, const uint32_t* off, int n_chunks,
                                         int64_t chunk, uint32_t n) {
  int lo = 0, hi = n_chunks - 1;  // last chunk with off[c] <= n
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= n) lo = mid; else hi = mid - 1;
  }
  return cand_q[(int64_t)lo * chunk + (n - off[lo])];
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(TopkParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t select_lds[];
  SelectShared& sh = *(SelectShared*)select_lds;

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
  find_threshold_bin<kHistBins>(p.hist + (int64_t)bt * kHistBins, (uint32_t)K, sh.wave, sh.res, &bin,
                                &above);

  // 2. ordered (key, position) candidates of this chunk: key bin >= bin.
  // Each thread takes kSelV consecutive positions per step (one 4096-position
  // step per default chunk), loaded together.
  const float* row = p.scores + (int64_t)bt * p.Lmax;
  uint2* cand_q = p.cand + (int64_t)bt * p.Lmax;
  uint2* cand = cand_q + c_lo;
  const bool vec_ok = (((uintptr_t)(row + c_lo)) & 15) == 0;
  uint32_t n_out = 0;
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
    bool f[kSelV];
    uint32_t key[kSelV];
#pragma unroll
    for (int j = 0; j < kSelV; ++j) {
      key[j] = score_key(v[j]);
      f[j] = (s0 + j < c_hi) && ((key[j] >> kHistShift) >= bin);
    }
    uint32_t total;
    uint32_t off = n_out + block_prefix_flags<kSelV>(f, sh.wave, &total);
#pragma unroll
    for (int j = 0; j < kSelV; ++j)
      if (f[j]) cand[off++] = make_uint2(key[j], (uint32_t)(s0 + j));
    n_out += total;
  }
  if (tid == 0) p.chunk_cnt[(int64_t)bt * p.n_chunks + c] = n_out;

  // 3. arrival: the last chunk of this query finishes the selection.  Writers
  // only need release ordering (their candidate stores written back past the
  // XCD's L2 before the counter moves); only the last workgroup needs acquire.
  __syncthreads();
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    sh.last = (atomicAdd(&p.arrive[bt], 1u) == (uint32_t)(n_chunks_q - 1));
  }
  __syncthreads();
  if (!sh.last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  // chunk offsets of the concatenated candidate list
  const uint32_t* cnt_q = p.chunk_cnt + (int64_t)bt * p.n_chunks;
  // (the host keeps n_chunks <= kMaxChunksLds)
  uint32_t N = 0;
  for (int c0 = 0; c0 < n_chunks_q; c0 += kSelThreads) {
    const uint32_t v = (c0 + tid < n_chunks_q) ? cnt_q[c0 + tid] : 0u;
    uint32_t tot;
    const uint32_t incl = block_incl_scan(v, sh.wave, &tot);
    if (c0 + tid < n_chunks_q) sh.chunk_off[c0 + tid] = N + incl - v;
    N += tot;
  }
  __syncthreads();
  const uint32_t need = (uint32_t)K - above;  // entries to take from bin `bin`
  const bool in_lds = N <= kFinalCap;

  if (in_lds) {
    // gather every candidate into LDS with many loads in flight
    constexpr int U = 8;
    for (uint32_t n0 = 0; n0 < N; n0 += kSelThreads * U) {
      uint2 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t n = n0 + u * kSelThreads + tid;
        v[u] = n < N ? cand_at(cand_q, sh.chunk_off, n_chunks_q, p.chunk, n) : make_uint2(0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t n = n0 + u * kSelThreads + tid;
        if (n < N) {
          sh.key[n] = v[u].x;
          sh.pos[n] = v[u].y;
        }
      }
    }
  }
  auto key_at = [&](uint32_t n) -> uint32_t {
    return in_lds ? sh.key[n] : cand_at(cand_q, sh.chunk_off, n_chunks_q, p.chunk, n).x;
  };
  auto pos_at = [&](uint32_t n) -> uint32_t {
    return in_lds ? sh.pos[n] : cand_at(cand_q, sh.chunk_off, n_chunks_q, p.chunk, n).y;
  };

  // refine: next 12 key bits among keys in `bin`
  for (int i = tid; i < kHistBins; i += kSelThreads) sh.sub[i] = 0;
  __syncthreads();
  for (uint32_t n = tid; n < N; n += kSelThreads) {
    const uint32_t key = key_at(n);
    if ((key >> kHistShift) == bin) atomicAdd(&sh.sub[(key >> 8) & 0xFFFu], 1u);
  }
  __syncthreads();
  uint32_t bin2, above2;
  find_threshold_bin<kHistBins>(sh.sub, need, sh.wave, sh.res, &bin2, &above2);
  const uint32_t need2 = need - above2;
  const uint32_t prefix24 = (bin << 12) | bin2;

  // refine: last 8 key bits
  for (int i = tid; i < 256; i += kSelThreads) sh.sub[i] = 0;
  __syncthreads();
  for (uint32_t n = tid; n < N; n += kSelThreads) {
    const uint32_t key = key_at(n);
    if ((key >> 8) == prefix24) atomicAdd(&sh.sub[key & 0xFFu], 1u);
  }
  __syncthreads();
  uint32_t bin3, above3;
  find_threshold_bin<256>(sh.sub, need2, sh.wave, sh.res, &bin3, &above3);
  const uint32_t tau = (prefix24 << 8) | bin3;
  const uint32_t take_ties = need2 - above3;  // ties at tau to keep, lowest positions first

  // emit in position order: each thread owns E consecutive candidates.  The
  // output slot of an entry = (entries above tau before it) + (ties before it
  // that are kept, at most take_ties).
  constexpr int E = 8;
  uint32_t gt_seen = 0, ties_seen = 0;
  for (uint32_t n0 = 0; n0 < N; n0 += kSelThreads * E) {
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
    uint32_t rank = ties_seen + block_incl_scan(eq, sh.wave, &eq_tot) - eq;  // tie rank of my first tie
    const uint32_t gt_before = gt_seen + block_incl_scan(gt, sh.wave, &gt_tot) - gt;
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

hipError_t launch_select(const TopkParams& p, hipStream_t stream) {
  dim3 grid((unsigned)p.n_chunks, (unsigned)(p.B * p.T));
  hipLaunchKernelGGL(select_kernel, grid, dim3(kSelThreads), sizeof(SelectShared), stream, p);
  return hipGetLastError();
}

}  // namespace dsa
