// Sparse MLA attention over the Top-K selected latent rows.
//
// For query (b, t) and head h, with c_j the latent row kv[b, idx_j, :] (times
// its scale for an E4M3 cache):
//     z_j = softmax_scale * q[b,t,h,:] . c_j            (all qk_dim columns)
//     out[b,t,h,:] = sum_j softmax(z)_j * c_j[:v_dim]   (value = leading columns)
// Only the selected rows are read ("Optimization and Deployment Practices for
// Next-Generation Sparse Attention LLMs" §2: the sparse attention reads the KV
// entries the indexer selected; "Engineering Practices for Optimizing
// Ultra-Large Sparse Attention Model Inference" §3.1: load the selected blocks,
// then attend with the matrix units).  In MLA one latent row serves every
// head, so a workgroup stages each selected row into LDS once and all of its
// heads read it from there.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

// ---------------------------------------------------------------------------
// Portable SIMT kernel: one workgroup per (head, query); any dims <= limits.
// Online softmax over chunks of the index list.
// ---------------------------------------------------------------------------
constexpr int kGenThreads = 256;
constexpr int kGenChunk = 512;      // index entries per chunk
constexpr int kGenMaxDqk = 2048;
constexpr int kGenMaxDvPerThread = 4;  // Dv <= 1024

__device__ __forceinline__ float mla_load(const void* p, int dtype, int64_t i) {
  if (dtype == kF32) return ((const float*)p)[i];
  if (dtype == kBF16) return bf16_bits_to_f32(((const uint16_t*)p)[i]);
  return e4m3_to_f32(((const uint8_t*)p)[i]);
}

__device__ __forceinline__ void store_out(void* out, int dtype, int64_t i, float v) {
  if (dtype == kF32) ((float*)out)[i] = v;
  else ((uint16_t*)out)[i] = (uint16_t)f32_to_bf16_bits(v);
}

__global__ __launch_bounds__(kGenThreads) void mla_generic_kernel(MlaParams p) {
  __shared__ float s_q[kGenMaxDqk];
  __shared__ float s_z[kGenChunk];
  __shared__ int64_t s_row[kGenChunk];
  __shared__ float s_red[kGenThreads / kWave];

  const int h = blockIdx.x, bt = blockIdx.y, b = bt / p.T;
  const int tid = threadIdx.x, wave = tid / kWave;
  const int len = clamp_len(p.seq_lens[b], p.Lmax);
  const int64_t qoff = ((int64_t)bt * p.H + h) * p.Dqk;
  for (int i = tid; i < p.Dqk; i += kGenThreads) s_q[i] = mla_load(p.q, p.q_dtype, qoff + i);

  float o[kGenMaxDvPerThread];
#pragma unroll
  for (int k = 0; k < kGenMaxDvPerThread; ++k) o[k] = 0.0f;
  float m = -INFINITY, lsum = 0.0f;
  const int32_t* sel = p.topk_idx + (int64_t)bt * p.K;

  for (int j0 = 0; j0 < p.K; j0 += kGenChunk) {
    const int n = min(kGenChunk, p.K - j0);
    __syncthreads();
    // logits of this chunk (natural-log units)
    for (int j = tid; j < n; j += kGenThreads) {
      const int32_t r = sel[j0 + j];
      float z = -INFINITY;
      int64_t row = -1;
      if (r >= 0 && r < len) {
        row = (int64_t)b * p.Lmax + r;
        const float sc = p.kv_scale ? p.kv_scale[row] : 1.0f;
        float d = 0.0f;
        for (int i = 0; i < p.Dqk; ++i) d = fmaf(s_q[i], mla_load(p.kv, p.kv_dtype, row * p.Dqk + i) * sc, d);
        z = d * p.scale;
      }
      s_z[j] = z;
      s_row[j] = row;
    }
    __syncthreads();
    // chunk maximum
    float cm = -INFINITY;
    for (int j = tid; j < n; j += kGenThreads) cm = fmaxf(cm, s_z[j]);
    cm = wave_max(cm);
    if (lane_id() == 0) s_red[wave] = cm;
    __syncthreads();
    cm = s_red[0];
    for (int w = 1; w < kGenThreads / kWave; ++w) cm = fmaxf(cm, s_red[w]);
    const float m_new = fmaxf(m, cm);
    if (m_new == -INFINITY) continue;  // nothing valid yet
    const float alpha = (m == -INFINITY) ? 0.0f : expf(m - m_new);
    lsum *= alpha;
#pragma unroll
    for (int k = 0; k < kGenMaxDvPerThread; ++k) o[k] *= alpha;
    for (int j = 0; j < n; ++j) {
      if (s_row[j] < 0) continue;
      const float pj = expf(s_z[j] - m_new);
      lsum += pj;
      const float sc = p.kv_scale ? p.kv_scale[s_row[j]] : 1.0f;
#pragma unroll
      for (int k = 0; k < kGenMaxDvPerThread; ++k) {
        const int d = tid + k * kGenThreads;
        if (d < p.Dv) o[k] = fmaf(pj, mla_load(p.kv, p.kv_dtype, s_row[j] * p.Dqk + d) * sc, o[k]);
      }
    }
    m = m_new;
  }
  const int64_t ooff = ((int64_t)bt * p.H + h) * p.Dv;
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
#pragma unroll
  for (int k = 0; k < kGenMaxDvPerThread; ++k) {
    const int d = tid + k * kGenThreads;
    if (d < p.Dv) store_out(p.out, p.out_dtype, ooff + d, o[k] * inv);
  }
  if (p.lse && tid == 0) p.lse[(int64_t)bt * p.H + h] = lsum > 0.0f ? m + logf(lsum) : -INFINITY;
}

// ---------------------------------------------------------------------------
// Matrix-core kernel: qk_dim 576, v_dim 512, 64 heads per workgroup (4 waves x
// 16 heads), row tiles of 32 selected rows staged in LDS.
//
// QK^T is computed transposed, S^T[row, head], with the LDS row tile as MFMA
// operand A and the wave's 16 query heads (registers) as operand B, so in the
// 16x16 accumulator lane l holds head l%16 and rows 4*(l/16)+e of each
// 16-row half.  Those 8 probabilities are exactly the A operand the PV product
// needs for head l%16 (the 32 k-slots of the PV step are a fixed permutation
// of the tile's rows; the V operand is read from LDS in the same order), so P
// never leaves registers.  Online softmax (running max/sum per head) in base 2.
// Splits of the index list run in separate workgroups and are merged by
// mla_combine_kernel with their (max, sum) pairs.
// ---------------------------------------------------------------------------
constexpr int kDqk = 576, kDv = 512;
constexpr int kMlaWaves = 4, kMlaThreads = kMlaWaves * kWave;
constexpr int kHeadsPerWave = 16, kHeadsPerWG = kMlaWaves * kHeadsPerWave;
constexpr int kTile = 32;
constexpr int kRowStride = kDqk + 8;  // bf16 elements per LDS row (1168 bytes)
constexpr int kKSteps = kDqk / 32;    // 18
constexpr int kNTiles = kDv / 16;     // 32

int mla_row_tile() { return kTile; }

// Global chunks (16 bytes) per tile and per thread for staging.
template <bool FP8>
struct Stage {
  static constexpr int kChunksPerRow = FP8 ? kDqk / 16 : kDqk / 8;  // 36 or 72
  static constexpr int kChunks = kTile * kChunksPerRow;
  static constexpr int kPerThread = (kChunks + kMlaThreads - 1) / kMlaThreads;
  i32x4 v[kPerThread];
  float sc[kPerThread];
};

template <bool FP8>
__device__ __forceinline__ void stage_load(Stage<FP8>& st, const MlaParams& p, const int32_t* sel,
                                           int j0, int n_rows, int b, int len) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < Stage<FP8>::kPerThread; ++k) {
    const int id = tid + k * kMlaThreads;
    const int r = id / Stage<FP8>::kChunksPerRow, c = id % Stage<FP8>::kChunksPerRow;
    int32_t pos = 0;
    if (id < Stage<FP8>::kChunks && r < n_rows) {
      const int32_t v = sel[j0 + r];
      pos = (v >= 0 && v < len) ? v : 0;
    }
    const int64_t row = (int64_t)b * p.Lmax + pos;
    if (id < Stage<FP8>::kChunks) {
      const i32x4* src = (const i32x4*)((const uint8_t*)p.kv + row * (FP8 ? kDqk : 2 * kDqk)) + c;
      st.v[k] = *src;
      if constexpr (FP8) st.sc[k] = p.kv_scale[row];
    }
  }
}

template <bool FP8>
__device__ __forceinline__ void stage_store(const Stage<FP8>& st, uint16_t* lds) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < Stage<FP8>::kPerThread; ++k) {
    const int id = tid + k * kMlaThreads;
    if (id >= Stage<FP8>::kChunks) break;
    const int r = id / Stage<FP8>::kChunksPerRow, c = id % Stage<FP8>::kChunksPerRow;
    if constexpr (!FP8) {
      *(i32x4*)(lds + r * kRowStride + c * 8) = st.v[k];
    } else {
      // 16 e4m3 codes -> 16 bf16 (exact: code * 2^e fits bf16)
      uint32_t w[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t word = (uint32_t)st.v[k][q];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const float a = e4m3_to_f32((word >> (16 * h2)) & 0xFFu) * st.sc[k];
          const float bb = e4m3_to_f32((word >> (16 * h2 + 8)) & 0xFFu) * st.sc[k];
          w[2 * q + h2] = (__float_as_uint(a) >> 16) | (__float_as_uint(bb) & 0xFFFF0000u);
        }
      }
      i32x4* dst = (i32x4*)(lds + r * kRowStride + c * 16);
      dst[0] = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
      dst[1] = i32x4{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
    }
  }
}

template <bool FP8>
__global__ __launch_bounds__(kMlaThreads) void mla_mfma_kernel(MlaParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t s_rows[kTile * kRowStride];

  const int split = blockIdx.x, bt = blockIdx.y, hg = blockIdx.z;
  const int b = bt / p.T;
  const int tid = threadIdx.x, wave = tid / kWave, l = lane_id();
  const int lg = l >> 4, lc = l & 15;
  const int len = clamp_len(p.seq_lens[b], p.Lmax);
  const int h0 = hg * kHeadsPerWG + wave * kHeadsPerWave;  // this wave's first head
  const int32_t* sel = p.topk_idx + (int64_t)bt * p.K;
  const int j_begin = split * p.rows_per_split;
  const int j_end = min(p.K, j_begin + p.rows_per_split);

  // query heads h0 + lc, dims 32 ks + 8 lg .. +8  (operand B of QK^T)
  bf16x8 qreg[kKSteps];
  {
    const bf16x8* qrow = (const bf16x8*)((const uint16_t*)p.q + ((int64_t)bt * p.H + h0 + lc) * kDqk);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) qreg[ks] = qrow[ks * 4 + lg];
  }
  const float zscale = p.scale * 1.4426950408889634f;  // logits in base-2 units

  f32x4 o[kNTiles];
#pragma unroll
  for (int n = 0; n < kNTiles; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;  // for head h0 + lc

  Stage<FP8> stage;
  if (j_begin < j_end) stage_load<FP8>(stage, p, sel, j_begin, min(kTile, j_end - j_begin), b, len);

  for (int j0 = j_begin; j0 < j_end; j0 += kTile) {
    const int n_rows = min(kTile, j_end - j0);
    __syncthreads();
    stage_store<FP8>(stage, s_rows);
    __syncthreads();
    if (j0 + kTile < j_end) stage_load<FP8>(stage, p, sel, j0 + kTile, min(kTile, j_end - j0 - kTile), b, len);

    // ---- S^T[32 rows x 16 heads] ----
    f32x4 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* arow = s_rows + (mt * 16 + lc) * kRowStride + 8 * lg;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        const bf16x8 a = *(const bf16x8*)(arow + ks * 32);
        s[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[ks], s[mt], 0, 0, 0);
      }
    }
    // ---- online softmax for head h0 + lc over rows 4 lg + e (+16) ----
    float z[2][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = mt * 16 + 4 * lg + e;
        bool valid = r < n_rows;
        if (valid) {
          const int32_t v = sel[j0 + r];
          valid = v >= 0 && v < len;
        }
        z[mt][e] = valid ? s[mt][e] * zscale : -INFINITY;
        tmax = fmaxf(tmax, z[mt][e]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    const float m_new = fmaxf(m_run, tmax);
    float alpha = 1.0f, psum = 0.0f;
    float pr[2][4];
    if (m_new == -INFINITY) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) pr[mt][e] = 0.0f;
    } else {
      alpha = exp2f(m_run - m_new);  // m_run = -inf gives 0
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pr[mt][e] = exp2f(z[mt][e] - m_new);
          psum += pr[mt][e];
        }
    }
    psum += __shfl_xor(psum, 16, kWave);
    psum += __shfl_xor(psum, 32, kWave);
    l_run = l_run * alpha + psum;
    m_run = m_new;

    // rescale O rows (heads h0 + 4 lg + e) by their head's alpha
    float al[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) al[e] = __shfl(alpha, 4 * lg + e, kWave);
#pragma unroll
    for (int n = 0; n < kNTiles; ++n)
#pragma unroll
      for (int e = 0; e < 4; ++e) o[n][e] *= al[e];

    // P operand (A of PV): head lc, k-slot 8 lg + j <-> row (j < 4 ? 4 lg + j : 16 + 4 lg + j - 4)
    bf16x8 pa;
    {
      uint16_t pb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[j] = (uint16_t)f32_to_bf16_bits(pr[j >> 2][j & 3]);
      pa = __builtin_bit_cast(bf16x8, pb);
    }
    // ---- O[16 heads x 512] += P V ----
    const uint16_t* v0 = s_rows + (4 * lg) * kRowStride + lc;
    const uint16_t* v1 = s_rows + (16 + 4 * lg) * kRowStride + lc;
#pragma unroll
    for (int n = 0; n < kNTiles; ++n) {
      uint16_t vb[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vb[j] = v0[j * kRowStride + n * 16];
        vb[4 + j] = v1[j * kRowStride + n * 16];
      }
      o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8, vb), o[n], 0, 0, 0);
    }
  }

  // ---- write-out: O rows are heads h0 + 4 lg + e, columns 16 n + lc ----
  float lh[4], mh[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lh[e] = __shfl(l_run, 4 * lg + e, kWave);
    mh[e] = __shfl(m_run, 4 * lg + e, kWave);
  }
  if (p.splits == 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int h = h0 + 4 * lg + e;
      const float inv = lh[e] > 0.0f ? 1.0f / lh[e] : 0.0f;
      const int64_t ooff = ((int64_t)bt * p.H + h) * kDv;
#pragma unroll
      for (int n = 0; n < kNTiles; ++n) store_out(p.out, p.out_dtype, ooff + n * 16 + lc, o[n][e] * inv);
      if (p.lse && lc == 0)
        p.lse[(int64_t)bt * p.H + h] = lh[e] > 0.0f ? (mh[e] + log2f(lh[e])) * 0.6931471805599453f : -INFINITY;
    }
  } else {
    const int64_t BT = (int64_t)p.B * p.T;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int h = h0 + 4 * lg + e;
      const int64_t slot = ((int64_t)split * BT + bt) * p.H + h;
      float* po = p.part_o + slot * kDv;
#pragma unroll
      for (int n = 0; n < kNTiles; ++n) po[n * 16 + lc] = o[n][e];
      if (lc == 0) {
        p.part_ml[slot * 2] = mh[e];
        p.part_ml[slot * 2 + 1] = lh[e];
      }
    }
  }
}

// Merge the per-split partial (O, max, sum) of one (query, head).
__global__ __launch_bounds__(128) void mla_combine_kernel(MlaParams p) {
  const int h = blockIdx.x, bt = blockIdx.y;
  const int64_t BT = (int64_t)p.B * p.T;
  const float* ml = p.part_ml + ((int64_t)bt * p.H + h) * 2;
  const int64_t ml_stride = BT * p.H * 2;
  float M = -INFINITY;
  for (int s = 0; s < p.splits; ++s)
    if (ml[s * ml_stride + 1] > 0.0f) M = fmaxf(M, ml[s * ml_stride]);
  float L = 0.0f;
  for (int s = 0; s < p.splits; ++s) {
    const float ls = ml[s * ml_stride + 1];
    if (ls > 0.0f) L += ls * exp2f(ml[s * ml_stride] - M);
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const int64_t ooff = ((int64_t)bt * p.H + h) * p.Dv;
  const float* po = p.part_o + ((int64_t)bt * p.H + h) * p.Dv;
  const int64_t po_stride = BT * p.H * p.Dv;
  for (int d = threadIdx.x; d < p.Dv; d += blockDim.x) {
    float acc = 0.0f;
    for (int s = 0; s < p.splits; ++s) {
      const float ls = ml[s * ml_stride + 1];
      if (ls > 0.0f) acc = fmaf(po[s * po_stride + d], exp2f(ml[s * ml_stride] - M), acc);
    }
    store_out(p.out, p.out_dtype, ooff + d, acc * inv);
  }
  if (p.lse && threadIdx.x == 0)
    p.lse[(int64_t)bt * p.H + h] = L > 0.0f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
}

bool mla_mfma_supported(const MlaParams& p) {
  return p.Dqk == kDqk && p.Dv == kDv && p.H % kHeadsPerWG == 0 && p.q_dtype == kBF16 &&
         (p.kv_dtype == kBF16 || p.kv_dtype == kE4M3);
}

hipError_t launch_mla(const MlaParams& p, bool allow_mfma, hipStream_t stream) {
  if (allow_mfma && mla_mfma_supported(p)) {
    dim3 grid((unsigned)p.splits, (unsigned)(p.B * p.T), (unsigned)(p.H / kHeadsPerWG));
    if (p.kv_dtype == kBF16)
      hipLaunchKernelGGL(mla_mfma_kernel<false>, grid, dim3(kMlaThreads), 0, stream, p);
    else
      hipLaunchKernelGGL(mla_mfma_kernel<true>, grid, dim3(kMlaThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)p.H, (unsigned)(p.B * p.T)), dim3(128), 0,
                       stream, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(mla_generic_kernel, dim3((unsigned)p.H, (unsigned)(p.B * p.T)), dim3(kGenThreads),
                     0, stream, p);
  return hipGetLastError();
}

}  // namespace dsa
