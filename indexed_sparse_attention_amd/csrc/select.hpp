// Exact Top-K threshold resolution over the chunk step's outputs, shared by
// the emit step (one workgroup per query chunk) and the sparse attention's
// fused prologue (one workgroup per query split), plus the block-wide scan
// helpers both use.  See topk.hip for the selection scheme.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;

// --------------------------------------------------------------------------
// block-wide helpers (256 threads = 4 waves)
// --------------------------------------------------------------------------
// Inclusive prefix sum over the 64 lanes of a wave with DPP adds: shifts by
// 1, 2, 4, 8 within each 16-lane row, then the last lane of row 0 is added
// to row 1 and row 2 to row 3 (row_bcast:15), and lane 31 to rows 2 and 3
// (row_bcast:31).  Lanes without a source add 0.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Inclusive prefix sums of N values per thread, in thread order, over a
// workgroup of NW waves; total[i] gets the block total of value i.
// s_wave: N * NW words of shared scratch.
template <int N, int NW>
__device__ __forceinline__ void block_scan(uint32_t (&v)[N], uint32_t* s_wave, uint32_t (&total)[N]) {
  const int wave = threadIdx.x / kWave, l = lane_id();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    v[i] = wave_incl_scan(v[i]);
    if (l == kWave - 1) s_wave[i * NW + wave] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t x = s_wave[i * NW + w];
      if (w < wave) off += x;
      tot += x;
    }
    v[i] += off;
    total[i] = tot;
  }
  __syncthreads();
}

__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* s_wave, uint32_t* total) {
  uint32_t a[1] = {v}, t[1];
  block_scan<1, kSelWaves>(a, s_wave, t);
  *total = t[0];
  return a[0];
}

// Thread tid's share of an NB-bin histogram: the PER bins just below
// NB - PER*tid, highest first.  Loading it is separate from the scan below so
// that the loads can be in flight together with a kernel's other loads.
template <int NB>
struct BinSlice {
  static constexpr int PER = NB / kSelThreads;
  uint32_t c[PER];
};

template <int NB>
__device__ __forceinline__ void load_bin_slice(const uint32_t* h, BinSlice<NB>& s) {
  const int top = NB - 1 - BinSlice<NB>::PER * (int)threadIdx.x;
#pragma unroll
  for (int i = 0; i < BinSlice<NB>::PER; ++i) s.c[i] = h[top - i];
}

// Largest bin B of the histogram whose suffix count sum_{i >= B} h[i]
// reaches `need`; *above = sum_{i > B} h[i].  An inclusive scan of the
// slices in thread order counts the entries at or above each thread's lowest
// bin.  All threads get the result.
template <int NB>
__device__ void threshold_from_slice(const BinSlice<NB>& s, uint32_t need, uint32_t* s_wave, uint32_t* s_res,
                                     uint32_t* bin, uint32_t* above) {
  constexpr int PER = BinSlice<NB>::PER;
  const int top = NB - 1 - PER * (int)threadIdx.x;
  uint32_t own = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) own += s.c[i];
  uint32_t total;
  const uint32_t incl = block_incl_scan(own, s_wave, &total);
  const uint32_t excl = incl - own;
  if (excl < need && need <= incl) {
    uint32_t run = excl;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (run + s.c[i] >= need) {
        s_res[0] = (uint32_t)(top - i);
        s_res[1] = run;
        break;
      }
      run += s.c[i];
    }
  }
  __syncthreads();
  *bin = s_res[0];
  *above = s_res[1];
  __syncthreads();
}

template <int NB>
__device__ void find_threshold_bin(const uint32_t* h, uint32_t need, uint32_t* s_wave, uint32_t* s_res,
                                   uint32_t* bin, uint32_t* above) {
  BinSlice<NB> s;
  load_bin_slice<NB>(h, s);
  threshold_from_slice<NB>(s, need, s_wave, s_res, bin, above);
}

constexpr int kEmitCap = 10240;    // threshold-bin keys the emit step keeps in LDS
static_assert(kEmitCap % 4 == 0, "keys are read four at a time");
constexpr int kMaxChunks = 1024;   // chunks per query (the host sizes chunks to respect it)

// Row stride of the bin-key lists: Lmax rounded up to 4 keys, so that a row
// starts 16-byte aligned.
__device__ __forceinline__ int64_t bin_key_stride(int64_t Lmax) { return (Lmax + 3) & ~(int64_t)3; }

// Clears the query's step-1 histogram (run once its last reader has finished).
__device__ __forceinline__ void clear_query_hist(const TopkParams& p, int bt, int nthreads) {
  uint32_t* h = p.hist + (int64_t)bt * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += nthreads) h[i] = 0;
}

// The emit step refines the threshold bin B with two more digits of 10 key
// bits each (12 + 10 + 10 = 32).
constexpr int kDigitBins = 1024;

struct EmitShared {
  uint32_t wave[2 * kSelWaves];
  uint32_t res[3];                  // [2]: most bin-B entries in one chunk
  uint32_t h2[kDigitBins];          // second digit of the bin-B keys
  uint32_t h3[kDigitBins];          // third digit of the keys matching the first two
  uint32_t boff[kMaxChunks + 1];    // bin-B entries in chunks before c' (chunk order)
  uint32_t aoff[kMaxChunks + 1];    // entries above bin B in chunks before c'
  alignas(16) uint32_t key[kEmitCap];  // the query's bin-B keys in chunk order
};

// Step 3: exact threshold, then this chunk's kept positions at their final slots.
// Every load is issued before any is used: all chunks' counts, this chunk's
// first kSelThreads * kEmitE candidates, and the first S (the largest power
// of two with n_chunks * S <= kEmitFirst) bin-B keys of every chunk, read
// speculatively four at a time inside their regions and masked afterwards;
// a typical workgroup waits for memory once (a chunk with more than S bin-B
// keys costs one more round per S).  The keys are gathered into LDS in chunk
// order (key j of chunk c' at boff[c'] + j), so "the keys of chunks before
// c" is an index range.  More than kEmitCap of them (heavy ties) are read
// from global memory chunk by chunk instead.
constexpr int kEmitG = 8;                           // speculative groups of 4 bin-B keys per thread
constexpr int kEmitFirst = kSelThreads * kEmitG * 4;  // 8192
constexpr int kEmitE = 8;                           // candidates per thread per round
constexpr int kCntPer = kMaxChunks / kSelThreads;   // chunk counts per thread (chunks 4 tid + i)


// ---------------------------------------------------------------------------
// Threshold resolution
// ---------------------------------------------------------------------------
// The loads it needs that depend on no other, issued before any is used: the
// query's threshold header, every chunk's counts, and the first S bin-B keys
// of every chunk.
struct ResolveLoads {
  uint2 hdr;
  uint32_t cn[kCntPer], ca[kCntPer];
  uint4 bk[kEmitG];
};

// log2 of S, the speculative bin-B key slots read per chunk
__device__ __forceinline__ int spec_log_s(int nch) {
  int log_s = 2;  // (>= 8 slots: n_chunks <= 1024)
  while ((nch << (log_s + 1)) <= kEmitFirst) ++log_s;
  return log_s;
}

// bin-B keys j .. j+3 of chunk cc of query bt (j % 4 == 0), clamped into the query's row
__device__ __forceinline__ uint4 bin_keys4(const TopkParams& p, int bt, int cc, uint32_t j) {
  const int64_t kstride = bin_key_stride(p.Lmax);
  const uint32_t* bkeys = p.bin_keys + (int64_t)bt * kstride;
  return *(const uint4*)(bkeys + min((int64_t)min(cc, p.n_chunks - 1) * p.chunk + j, kstride - 4));
}

__device__ __forceinline__ void issue_resolve_loads(const TopkParams& p, int bt, ResolveLoads& r) {
  const int tid = threadIdx.x, nch = p.n_chunks;
  const uint32_t* ccnt = p.chunk_cnt + (int64_t)bt * nch;
  const uint32_t* cabv = p.chunk_above + (int64_t)bt * nch;
  const int log_s = spec_log_s(nch);
  const uint32_t S = 1u << log_s;
  r.hdr = p.header[bt];
#pragma unroll
  for (int i = 0; i < kCntPer; ++i) {
    const int cc = min(kCntPer * tid + i, nch - 1);
    r.cn[i] = ccnt[cc];
    r.ca[i] = cabv[cc];
  }
  // group g = tid + 256 i holds slots 4g .. 4g+3; slot sl = key sl % S of chunk sl / S
#pragma unroll
  for (int i = 0; i < kEmitG; ++i) {
    const int sl = 4 * (tid + i * kSelThreads);
    r.bk[i] = bin_keys4(p, bt, sl >> log_s, sl & (S - 1));
  }
}

// Calls f(key) for the bin-B keys of chunks [0, c_stop) of query bt, each
// thread a share: from LDS (four keys per read; kEmitCap is a multiple of 4)
// when they were staged there, else from global memory chunk by chunk.
template <class F>
__device__ __forceinline__ void for_each_bin_key(const TopkParams& p, int bt, const EmitShared& sh, bool in_lds,
                                                 int c_stop, F&& f) {
  const int tid = threadIdx.x;
  if (in_lds) {
    const uint32_t n_end = sh.boff[c_stop];
    for (uint32_t n = 4 * tid; n < n_end; n += 4 * kSelThreads) {
      const uint4 k4 = *(const uint4*)&sh.key[n];
      f(k4.x);
      if (n + 1 < n_end) f(k4.y);
      if (n + 2 < n_end) f(k4.z);
      if (n + 3 < n_end) f(k4.w);
    }
  } else {
    const uint32_t* bkeys = p.bin_keys + (int64_t)bt * bin_key_stride(p.Lmax);
    for (int cc = 0; cc < c_stop; ++cc) {
      const uint32_t n = sh.boff[cc + 1] - sh.boff[cc];
      for (uint32_t j = tid; j < n; j += kSelThreads) f(bkeys[(int64_t)cc * p.chunk + j]);
    }
  }
}

struct Resolved {
  uint32_t tau;        // the K-th largest key
  uint32_t take_ties;  // keys equal to tau that are kept: the lowest positions
  int n_act;           // chunks that ran the chunk step
  bool in_lds;         // the bin-B keys are staged in sh.key
};

// The exact K-th key of query bt, which sees vis > K positions.  Leaves in sh
// the chunk-order offsets of the bin-B keys (boff[c]: bin-B keys of chunks
// before c) and of the entries above bin B (aoff[c]), and, when there are at
// most kEmitCap of them, the bin-B keys themselves in chunk order (key j of
// chunk c at boff[c] + j).  Two further 10-bit digits of those keys, counted
// in LDS, give tau.  All kSelThreads threads call it; it ends with a barrier.
static __device__ Resolved resolve_threshold(const TopkParams& p, int bt, int64_t vis, ResolveLoads& r,
                                      EmitShared& sh) {
  const int tid = threadIdx.x, nch = p.n_chunks;
  const int64_t chunk = p.chunk;
  const int log_s = spec_log_s(nch);
  const uint32_t S = 1u << log_s;
  const int n_act = (int)((vis + chunk - 1) / chunk);
  const uint32_t bin = r.hdr.x, need = (uint32_t)p.K - r.hdr.y;  // entries to take from bin `bin`

  // ---- chunk-order offsets of the bin-B keys and of the entries above ----
  for (int i = tid; i < kDigitBins; i += kSelThreads) {
    sh.h2[i] = 0;
    sh.h3[i] = 0;
  }
  if (tid == 0) sh.res[2] = 0;
  uint32_t nb[kCntPer], na[kCntPer];
  uint32_t sums[2] = {0u, 0u}, tot[2], nb_max = 0;
#pragma unroll
  for (int i = 0; i < kCntPer; ++i) {
    const bool act = kCntPer * tid + i < n_act;
    nb[i] = act ? r.cn[i] - r.ca[i] : 0u;
    na[i] = act ? r.ca[i] : 0u;
    sums[0] += nb[i];
    sums[1] += na[i];
    nb_max = max(nb_max, nb[i]);
  }
  const uint32_t own[2] = {sums[0], sums[1]};
  block_scan<2, kSelWaves>(sums, sh.wave, tot);  // (its barriers also cover the clearing above)
  {
    uint32_t xb = sums[0] - own[0], xa = sums[1] - own[1];
#pragma unroll
    for (int i = 0; i < kCntPer; ++i) {
      const int cc = kCntPer * tid + i;
      if (cc <= nch) {
        sh.boff[cc] = xb;
        sh.aoff[cc] = xa;
      }
      xb += nb[i];
      xa += na[i];
    }
    if (tid == 0) {  // n_chunks == kMaxChunks: the closing offsets
      sh.boff[kMaxChunks] = tot[0];
      sh.aoff[kMaxChunks] = tot[1];
    }
    if (nb_max > 0) atomicMax(&sh.res[2], nb_max);
  }
  __syncthreads();
  const uint32_t M = tot[0];
  const uint32_t max_per_chunk = sh.res[2];
  const bool in_lds = M <= (uint32_t)kEmitCap;

  // ---- bin-B keys into LDS (chunk order) with their second digit counted ----
  if (in_lds) {
    auto stage = [&](const uint4 (&k)[kEmitG], uint32_t j0) {
      uint32_t o[kEmitG], n[kEmitG];  // all offset reads first (independent LDS loads)
#pragma unroll
      for (int i = 0; i < kEmitG; ++i) {
        const int cc = min((4 * (tid + i * kSelThreads)) >> log_s, nch);
        o[i] = sh.boff[cc];
        n[i] = sh.boff[min(cc + 1, nch)] - o[i];
      }
#pragma unroll
      for (int i = 0; i < kEmitG; ++i) {
        const int sl = 4 * (tid + i * kSelThreads);
        const bool act = (sl >> log_s) < n_act;
        const uint32_t j = j0 + (sl & (S - 1));
        const uint32_t kv[4] = {k[i].x, k[i].y, k[i].z, k[i].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (act && j + q < n[i]) {
            sh.key[o[i] + j + q] = kv[q];
            atomicAdd(&sh.h2[(kv[q] >> 10) & (kDigitBins - 1)], 1u);
          }
        }
      }
    };
    stage(r.bk, 0);
    for (uint32_t j0 = S; j0 < max_per_chunk; j0 += S) {  // chunks with more than S bin-B keys
#pragma unroll
      for (int i = 0; i < kEmitG; ++i) {
        const int sl = 4 * (tid + i * kSelThreads);
        r.bk[i] = bin_keys4(p, bt, sl >> log_s, j0 + (sl & (S - 1)));
      }
      stage(r.bk, j0);
    }
  } else {
    const uint32_t* bkeys = p.bin_keys + (int64_t)bt * bin_key_stride(p.Lmax);
    for (int cc = 0; cc < n_act; ++cc) {
      const uint32_t n = sh.boff[cc + 1] - sh.boff[cc];
      for (uint32_t j = tid; j < n; j += kSelThreads)
        atomicAdd(&sh.h2[(bkeys[(int64_t)cc * chunk + j] >> 10) & (kDigitBins - 1)], 1u);
    }
  }
  __syncthreads();

  // second digit -> 22-bit prefix of the K-th key
  uint32_t bin2, above2;
  find_threshold_bin<kDigitBins>(sh.h2, need, sh.wave, sh.res, &bin2, &above2);
  const uint32_t need2 = need - above2;
  const uint32_t prefix22 = (bin << 10) | bin2;
  // third digit -> exact K-th key tau
  for_each_bin_key(p, bt, sh, in_lds, n_act, [&](uint32_t k) {
    if ((k >> 10) == prefix22) atomicAdd(&sh.h3[k & (kDigitBins - 1)], 1u);
  });
  __syncthreads();
  uint32_t bin3, above3;
  find_threshold_bin<kDigitBins>(sh.h3, need2, sh.wave, sh.res, &bin3, &above3);
  Resolved rs;
  rs.tau = (prefix22 << 10) | bin3;
  rs.take_ties = need2 - above3;
  rs.n_act = n_act;
  rs.in_lds = in_lds;
  return rs;
}

}  // namespace dsa
