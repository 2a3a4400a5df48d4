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
// Matrix-core kernel: qk_dim 576, v_dim 512, 64 heads per workgroup, row tiles
// of 32 selected rows staged in LDS once and read by every wave.
//
// Eight waves: wave w serves heads 16*(w/2) .. +16 and half h = w%2 of the
// work: dims [288h, 288h+288) of the QK^T contraction and value columns
// [256h, 256h+256) of PV.  The two halves of a head group exchange their
// partial logits through LDS, so each wave keeps only 36 query registers and
// 64 output accumulators.
//
// QK^T is computed transposed, S^T[row, head], with the LDS row tile as MFMA
// operand A and 16 query heads (registers) as operand B; in the 16x16
// accumulator lane l holds head l%16 and rows 4*(l/16)+e of each 16-row half.
// Those 8 probabilities are exactly the A operand the PV product needs for
// head l%16 (the PV k-slots are a fixed permutation of the tile's rows; the V
// operand is read from LDS in the same order), so P never leaves registers.
// The V operand needs 8 rows at one column per lane; gfx950's LDS transpose
// read (ds_read_b64_tr_b16) delivers that from the row-major tile: within each
// 16-lane group, output lane j receives element j%4 of the 4-element segments
// addressed by lanes j/4 + 4k, k < 4.  MFMA lane i of 16-row block mt reads
// LDS row perm(mt, i) = 16 mt + 2 (i%4) + (i/4)%2 + 8 (i/8), which keeps both
// the QK^T operand reads and the transpose reads free of bank conflicts.
// Online softmax (running max/sum per head) in base 2.  Row splits of the
// index list run in separate workgroups and are merged by mla_combine_kernel
// from their (O, max, sum) partials.
// ---------------------------------------------------------------------------
constexpr int kDqk = 576, kDv = 512;
constexpr int kMlaWaves = 8, kMlaThreads = kMlaWaves * kWave;
constexpr int kHeadsPerWave = 16, kHeadsPerWG = 64;
constexpr int kTile = 32;
constexpr int kRowStride = kDqk + 8;  // bf16 elements per LDS row (1168 bytes)
constexpr int kKStepsHalf = kDqk / 2 / 32;  // 9 k-steps of 32 dims per half
constexpr int kNTilesHalf = kDv / 2 / 16;   // 16 value tiles of 16 columns per half
constexpr int kIdxCap = 2048;               // index entries staged in LDS at a time

int mla_row_tile() { return kTile; }

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

// LDS row holding row i (0..15) of 16-row block mt of the MFMA row order.
__device__ __forceinline__ int tile_row(int mt, int i) {
  return 16 * mt + 2 * (i & 3) + ((i >> 2) & 1) + 8 * (i >> 3);
}

__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
}

// Global 16-byte chunks per tile and per thread for staging.
template <bool FP8>
struct Stage {
  static constexpr int kChunksPerRow = FP8 ? kDqk / 16 : kDqk / 8;  // 36 or 72
  static constexpr int kChunks = kTile * kChunksPerRow;
  static constexpr int kPerThread = (kChunks + kMlaThreads - 1) / kMlaThreads;
  i32x4 v[kPerThread];
  float sc[kPerThread];
};

// s_pos: resolved row positions of the current tile (-1: not a row).
template <bool FP8>
__device__ __forceinline__ void stage_load(Stage<FP8>& st, const MlaParams& p, const int32_t* s_pos,
                                           int64_t seq_row0) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < Stage<FP8>::kPerThread; ++k) {
    const int id = tid + k * kMlaThreads;
    if (id < Stage<FP8>::kChunks) {
      const int r = id / Stage<FP8>::kChunksPerRow, c = id % Stage<FP8>::kChunksPerRow;
      const int32_t pos = max(s_pos[r], 0);
      const int64_t row = seq_row0 + pos;
      st.v[k] = *((const i32x4*)((const uint8_t*)p.kv + row * (FP8 ? kDqk : 2 * kDqk)) + c);
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
  __shared__ float s_xch[kMlaWaves][8][kWave];  // partial logits exchanged between halves
  __shared__ int32_t s_idx[kIdxCap];            // resolved positions of the split's rows

  const int split = blockIdx.x, bt = blockIdx.y, hg = blockIdx.z;
  const int b = bt / p.T;
  const int tid = threadIdx.x, wave = tid / kWave, l = lane_id();
  const int lg = l >> 4, lc = l & 15;
  const int half = wave & 1;
  const int len = clamp_len(p.seq_lens[b], p.Lmax);
  const int h0 = hg * kHeadsPerWG + (wave >> 1) * kHeadsPerWave;  // this wave's first head
  const int64_t seq_row0 = (int64_t)b * p.Lmax;
  const int32_t* sel = p.topk_idx + (int64_t)bt * p.K;
  const int j_begin = split * p.rows_per_split;
  const int j_end = min(p.K, j_begin + p.rows_per_split);

  // query heads h0 + lc, dims 288 half + 32 ks + 8 lg .. +8  (operand B of QK^T)
  bf16x8 qreg[kKStepsHalf];
  {
    const bf16x8* qrow =
        (const bf16x8*)((const uint16_t*)p.q + ((int64_t)bt * p.H + h0 + lc) * kDqk + 288 * half);
#pragma unroll
    for (int ks = 0; ks < kKStepsHalf; ++ks) qreg[ks] = qrow[ks * 4 + lg];
  }
  const float zscale = p.scale * 1.4426950408889634f;  // logits in base-2 units

  f32x4 o[kNTilesHalf];
#pragma unroll
  for (int n = 0; n < kNTilesHalf; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;  // for head h0 + lc

  Stage<FP8> stage;
  for (int jc = j_begin; jc < j_end; jc += kIdxCap) {
    const int jc_end = min(j_end, jc + kIdxCap);
    __syncthreads();  // previous users of s_idx are done
    for (int i = tid; i < jc_end - jc; i += kMlaThreads) {
      const int32_t v = sel[jc + i];
      s_idx[i] = (v >= 0 && v < len) ? v : -1;
    }
    // pad the last tile
    for (int i = jc_end - jc + tid; i < ((jc_end - jc + kTile - 1) / kTile) * kTile; i += kMlaThreads)
      s_idx[i] = -1;
    __syncthreads();
    stage_load<FP8>(stage, p, s_idx, seq_row0);

    for (int j0 = 0; j0 < jc_end - jc; j0 += kTile) {
      __syncthreads();
      stage_store<FP8>(stage, s_rows);
      __syncthreads();
      if (j0 + kTile < jc_end - jc) stage_load<FP8>(stage, p, s_idx + j0 + kTile, seq_row0);

      // ---- partial S^T[32 rows x 16 heads] over this wave's 288 dims ----
      f32x4 s[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint16_t* arow = s_rows + tile_row(mt, lc) * kRowStride + 288 * half + 8 * lg;
#pragma unroll
        for (int ks = 0; ks < kKStepsHalf; ++ks) {
          const bf16x8 a = *(const bf16x8*)(arow + ks * 32);
          s[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[ks], s[mt], 0, 0, 0);
        }
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) s_xch[wave][mt * 4 + e][l] = s[mt][e];
      __syncthreads();
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[mt][e] += s_xch[wave ^ 1][mt * 4 + e][l];

      // ---- online softmax for head h0 + lc over rows 4 lg + e (+16) ----
      float z[2][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool valid = s_idx[j0 + tile_row(mt, 4 * lg + e)] >= 0;
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
      for (int n = 0; n < kNTilesHalf; ++n)
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
      // ---- O[16 heads x 256 value columns] += P V ----
      // k-slot 8 lg + k (k < 4) is LDS row tile_row(0, 4 lg + k), slot 8 lg + 4 + k
      // is tile_row(1, 4 lg + k): lane lc addresses row k = lc/4 of its group and
      // columns 4 (lc%4) .. +4 of the 16-column tile.
      const uint16_t* va = s_rows + tile_row(0, 4 * lg + (lc >> 2)) * kRowStride + 256 * half + 4 * (lc & 3);
      const uint16_t* vb = s_rows + tile_row(1, 4 * lg + (lc >> 2)) * kRowStride + 256 * half + 4 * (lc & 3);
#pragma unroll
      for (int n = 0; n < kNTilesHalf; ++n) {
        const i16x4 lo = lds_read_tr16(va + n * 16);
        const i16x4 hi = lds_read_tr16(vb + n * 16);
        const bf16x8 vop = __builtin_bit_cast(bf16x8, (i32x4){__builtin_bit_cast(int, (short2){lo[0], lo[1]}),
                                                               __builtin_bit_cast(int, (short2){lo[2], lo[3]}),
                                                               __builtin_bit_cast(int, (short2){hi[0], hi[1]}),
                                                               __builtin_bit_cast(int, (short2){hi[2], hi[3]})});
        o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vop, o[n], 0, 0, 0);
      }
    }
  }

  // ---- write-out: O rows are heads h0 + 4 lg + e, columns 256 half + 16 n + lc ----
  float lh[4], mh[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lh[e] = __shfl(l_run, 4 * lg + e, kWave);
    mh[e] = __shfl(m_run, 4 * lg + e, kWave);
  }
  const int col0 = 256 * half + lc;
  if (p.splits == 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int h = h0 + 4 * lg + e;
      const float inv = lh[e] > 0.0f ? 1.0f / lh[e] : 0.0f;
      const int64_t ooff = ((int64_t)bt * p.H + h) * kDv + col0;
#pragma unroll
      for (int n = 0; n < kNTilesHalf; ++n) store_out(p.out, p.out_dtype, ooff + n * 16, o[n][e] * inv);
      if (p.lse && lc == 0 && half == 0)
        p.lse[(int64_t)bt * p.H + h] = lh[e] > 0.0f ? (mh[e] + log2f(lh[e])) * 0.6931471805599453f : -INFINITY;
    }
  } else {
    const int64_t BT = (int64_t)p.B * p.T;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int h = h0 + 4 * lg + e;
      const int64_t slot = ((int64_t)split * BT + bt) * p.H + h;
      float* po = p.part_o + slot * kDv + col0;
#pragma unroll
      for (int n = 0; n < kNTilesHalf; ++n) po[n * 16] = o[n][e];
      if (lc == 0 && half == 0) {
        p.part_ml[slot * 2] = mh[e];
        p.part_ml[slot * 2 + 1] = lh[e];
      }
    }
  }
}

// Merge the per-split partials (O, max, sum) of one (query, head): 128
// threads, 4 consecutive value columns each.
__global__ __launch_bounds__(128) void mla_combine_kernel(MlaParams p) {
  __shared__ float s_w[64];
  __shared__ float s_stat[2];
  const int h = blockIdx.x, bt = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t BT = (int64_t)p.B * p.T;
  const int64_t slot0 = (int64_t)bt * p.H + h;
  const int64_t slot_stride = BT * p.H;
  if (tid < kWave) {
    float ms = -INFINITY, ls = 0.0f;
    if (tid < p.splits) {
      ms = p.part_ml[(slot0 + tid * slot_stride) * 2];
      ls = p.part_ml[(slot0 + tid * slot_stride) * 2 + 1];
    }
    const float M = wave_max(ls > 0.0f ? ms : -INFINITY);
    const float wgt = (ls > 0.0f) ? exp2f(ms - M) : 0.0f;
    const float L = wave_sum(ls * wgt);
    if (tid < 64) s_w[tid] = wgt;
    if (tid == 0) {
      s_stat[0] = M;
      s_stat[1] = L;
    }
  }
  __syncthreads();
  const float M = s_stat[0], L = s_stat[1];
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const int d = tid * 4;
  if (d < p.Dv) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    const float* po = p.part_o + slot0 * p.Dv + d;
    const int64_t stride = slot_stride * p.Dv;
#pragma unroll 4
    for (int s = 0; s < p.splits; ++s) {
      const float wgt = s_w[s];
      const f32x4 v = *(const f32x4*)(po + s * stride);
      acc[0] = fmaf(v[0], wgt, acc[0]);
      acc[1] = fmaf(v[1], wgt, acc[1]);
      acc[2] = fmaf(v[2], wgt, acc[2]);
      acc[3] = fmaf(v[3], wgt, acc[3]);
    }
    const int64_t ooff = slot0 * p.Dv + d;
#pragma unroll
    for (int k = 0; k < 4; ++k) store_out(p.out, p.out_dtype, ooff + k, acc[k] * inv);
  }
  if (p.lse && tid == 0)
    p.lse[slot0] = L > 0.0f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
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
                       stream, p);  // needs Dv <= 512 and splits <= 64
    return hipGetLastError();
  }
  hipLaunchKernelGGL(mla_generic_kernel, dim3((unsigned)p.H, (unsigned)(p.B * p.T)), dim3(kGenThreads),
                     0, stream, p);
  return hipGetLastError();
}

}  // namespace dsa
