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

// Scale of column i of cache row `row` (1 for f32/bf16 caches).
__device__ __forceinline__ float kv_col_scale(const MlaParams& p, int64_t row, int i) {
  if (p.kv_dtype == kE4M3) return p.kv_scale[row];
  if (p.kv_dtype == kE4M3T128) return p.kv_scale[row * ((p.Dqk + 127) / 128) + i / 128];
  return 1.0f;
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
  const int len = filled_rows(p.seq_lens[b], p.Lmax, p.len_sub);
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
        float d = 0.0f;
        for (int i = 0; i < p.Dqk; ++i)
          d = fmaf(s_q[i], mla_load(p.kv, p.kv_dtype, row * p.Dqk + i) * kv_col_scale(p, row, i), d);
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
#pragma unroll
      for (int k = 0; k < kGenMaxDvPerThread; ++k) {
        const int d = tid + k * kGenThreads;
        if (d < p.Dv)
          o[k] = fmaf(pj, mla_load(p.kv, p.kv_dtype, s_row[j] * p.Dqk + d) * kv_col_scale(p, s_row[j], d), o[k]);
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
// of 64 selected rows staged in LDS once and read by every wave.
//
// Four waves, one per SIMD (so a wave may hold up to 512 registers).  For
// QK^T and the softmax, wave w owns heads 16w .. 16w+15 over all 576 dims
// (its queries stay in registers).  For PV it owns value columns 128w ..
// 128w+127 of all 64 heads: each wave then reads only its quarter of the
// tile's value columns, and the probabilities of all heads (8 KB of bf16 per
// tile) plus each head's rescale factor pass through LDS between the two
// halves, behind one extra barrier.  Tiles of 64 rows amortise each tile's
// fixed costs (barriers, copy issue, softmax reductions) over more rows and
// give 8 independent accumulation chains for QK^T.
//
// Row tiles alternate between two LDS buffers: while tile t is computed, tile
// t+1 is in flight.  A bf16 cache is copied global -> LDS directly
// (global_load_lds_dwordx4, no registers); an e4m3 cache is copied the
// same way as raw codes, each wave then decodes its own rows to bf16 (x the
// row scale) in place.  A tile
// is 64 rows x 72 chunks of 16 bytes, stored in 1 KB segments of 8 rows x 8
// chunks with the chunk slot XOR-swizzled by row, so that one DMA
// instruction fills one segment with eight 128-byte row pieces and both
// operand reads below are free of bank conflicts.
//
// QK^T is computed transposed, S^T[row, head], with the LDS row tile as MFMA
// operand A and 16 query heads (registers) as operand B; in the 16x16
// accumulator lane l holds head l%16 and rows 4*(l/16)+e of each 16-row
// block.  Those probabilities, in bf16, are exactly the B operand the PV
// product needs for head l%16 (the PV k-slots are a fixed permutation of the
// tile's rows; the V operand is read from LDS in the same order), so each
// lane stores them as two 16-byte chunks and every wave reads the four head
// blocks back.  The V operand needs 8 rows at one column per lane; gfx950's
// LDS transpose read (ds_read_b64_tr_b16) delivers that: within each 16-lane
// group, output lane j receives element j%4 of the 4-element segments
// addressed by lanes j/4 + 4k, k < 4.  MFMA lane i of 16-row block mt uses
// tile row perm(mt, i) = 16 mt + 2 (i%4) + (i/4)%2 + 8 (i/8).  Online softmax
// in base 2 with a lazily moved reference max.  Row splits of the index list
// run in separate workgroups and are merged by mla_combine_kernel from their
// (O, max, sum) partials.
// ---------------------------------------------------------------------------
constexpr int kDqk = 576, kDv = 512;
constexpr int kMlaWaves = 4, kMlaThreads = kMlaWaves * kWave;
constexpr int kHeadsPerWave = 16, kHeadsPerWG = kMlaWaves * kHeadsPerWave;
constexpr int kTile = 64;
constexpr int kBlocks = kTile / 16;                      // 16-row MFMA blocks per tile
constexpr int kChunksPerRow = kDqk / 8;                  // 72 bf16 chunks of 16 bytes
constexpr int kTileBytes = kTile * kChunksPerRow * 16;   // 72 KB
// row stride of the output block staged in LDS at write-out: 32 B of padding
// per 1 KB row spreads the sixteen rows one store instruction touches over
// the banks
constexpr int kStageRow = 2 * kDv + 32;
constexpr int kKSteps = kDqk / 32;                       // 18 k-steps of 32 dims
constexpr int kIdxCap = 1536;                            // most index entries of one split
constexpr int kIdxPad = 3 * kTile;                       // the last tile's padding + 2 tiles read ahead
constexpr float kSlack = 8.0f;                           // log2 headroom before the running max moves
static_assert(kMlaWaves * 16 == kTile, "two 8-row groups of the tile per wave");

int mla_row_tile() { return kTile; }
int mla_max_rows_per_split() { return kIdxCap; }

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

// Tile row used by row i (0..15) of 16-row block mt of the MFMA row order.
__device__ __forceinline__ int tile_row(int mt, int i) {
  return 16 * mt + 2 * (i & 3) + ((i >> 2) & 1) + 8 * (i >> 3);
}

// Byte offset of 16-byte chunk c (0..71) of tile row r (0..63): chunk c of
// a segment sits in slot (c ^ r ^ r/4) % 8 of the row's 128 bytes.  Of the
// XOR swizzles tried on the LDS bank-conflict counter, this one leaves both
// the score operand reads (16 rows x 4 chunks per instruction) and the
// transposed value reads conflict-free; with (c ^ r ^ r/8) % 8 the score
// reads took two passes each.
__device__ __forceinline__ int chunk_off(int r, int c) {
  return ((r >> 3) * 9 + (c >> 3)) * 1024 + 16 * (8 * (r & 7) + ((c ^ r ^ (r >> 2)) & 7));
}

// Reductions over the lanes l, l^16, l^32, l^48 (the four 16-lane groups
// holding one head's rows) with the gfx950 lane-swap instructions: VALU
// work, no LDS round trip.  permlane{16,32}_swap(x, x) returns, per lane,
// x(l) and x(l ^ 16) (or x(l ^ 32)) in some order.
__device__ __forceinline__ float group4_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float group4_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Operand reads of a tile go through inline asm: the compiler's own wait
// insertion treats LDS reads as aliasing every pending global->LDS copy and
// would drain them all before each read.  The tile being read is known to be
// complete (its copies were waited for before the barrier that opened it),
// so only the LDS counter matters.  Reads go in groups; each block issues a
// later group and then waits until only the groups issued after the one it
// completes are outstanding.  A completed group's registers are in/out
// operands of that block, so nothing reads them before the wait, and no
// register of an in-flight read is reused.
struct QkGroup {
  bf16x8 r[4];  // [2 j + k-step parity], 16-row block 2h + j
};

// QK^T operand A: group (g, h) = k-steps 2g, 2g+1 of 16-row blocks 2h, 2h+1,
// at addr[j][parity] + g KB.
template <int G>
__device__ __forceinline__ void qk_issue(QkGroup& nxt, const uint32_t (&addr)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:%8\n"
      "ds_read_b128 %1, %5 offset:%8\n"
      "ds_read_b128 %2, %6 offset:%8\n"
      "ds_read_b128 %3, %7 offset:%8"
      : "=&v"(nxt.r[0]), "=&v"(nxt.r[1]), "=&v"(nxt.r[2]), "=&v"(nxt.r[3])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "i"(G * 1024)
      : "memory");
}

// Issues group `nxt` (4 reads at addr + G KB), then waits until the reads
// still outstanding are the last N (`done`, issued before, is complete).
template <int G, int N>
__device__ __forceinline__ void qk_issue_wait(QkGroup& nxt, QkGroup& done, const uint32_t (&addr)[4]) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:%12\n"
      "ds_read_b128 %1, %9 offset:%12\n"
      "ds_read_b128 %2, %10 offset:%12\n"
      "ds_read_b128 %3, %11 offset:%12\n"
      "s_waitcnt lgkmcnt(%13)"
      : "=&v"(nxt.r[0]), "=&v"(nxt.r[1]), "=&v"(nxt.r[2]), "=&v"(nxt.r[3]), "+v"(done.r[0]), "+v"(done.r[1]),
        "+v"(done.r[2]), "+v"(done.r[3])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "i"(G * 1024), "i"(N)
      : "memory");
}

template <int N>
__device__ __forceinline__ void qk_wait(QkGroup& done) {
  asm volatile("s_waitcnt lgkmcnt(%4)"
               : "+v"(done.r[0]), "+v"(done.r[1]), "+v"(done.r[2]), "+v"(done.r[3])
               : "i"(N)
               : "memory");
}

struct TrGroup {
  i16x4 r[8];  // [2 k + h]: value tile 4 g + k, row half h
};

// PV operand (V^T): addr[2 k + h] = value tile k (mod 4), row half h of the
// k-step's first 4-tile group; group G sits G KB further.
template <int G>
__device__ __forceinline__ void tr_issue_wait(TrGroup& nxt, TrGroup& prev, const uint32_t (&addr)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:%24\n"
      "ds_read_b64_tr_b16 %1, %17 offset:%24\n"
      "ds_read_b64_tr_b16 %2, %18 offset:%24\n"
      "ds_read_b64_tr_b16 %3, %19 offset:%24\n"
      "ds_read_b64_tr_b16 %4, %20 offset:%24\n"
      "ds_read_b64_tr_b16 %5, %21 offset:%24\n"
      "ds_read_b64_tr_b16 %6, %22 offset:%24\n"
      "ds_read_b64_tr_b16 %7, %23 offset:%24\n"
      "s_waitcnt lgkmcnt(8)"
      : "=&v"(nxt.r[0]), "=&v"(nxt.r[1]), "=&v"(nxt.r[2]), "=&v"(nxt.r[3]), "=&v"(nxt.r[4]), "=&v"(nxt.r[5]),
        "=&v"(nxt.r[6]), "=&v"(nxt.r[7]), "+v"(prev.r[0]), "+v"(prev.r[1]), "+v"(prev.r[2]), "+v"(prev.r[3]),
        "+v"(prev.r[4]), "+v"(prev.r[5]), "+v"(prev.r[6]), "+v"(prev.r[7])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6]),
        "v"(addr[7]), "i"(G * 1024)
      : "memory");
}

__device__ __forceinline__ void tr_wait_last(TrGroup& prev) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(prev.r[0]), "+v"(prev.r[1]), "+v"(prev.r[2]), "+v"(prev.r[3]), "+v"(prev.r[4]),
                 "+v"(prev.r[5]), "+v"(prev.r[6]), "+v"(prev.r[7])
               :
               : "memory");
}

struct MlaShared {
  uint8_t rows[2][kTileBytes];  // tile buffers (read only through inline asm)
  uint8_t pt[kHeadsPerWG * kTile * 2];  // P of the current tile, bf16 [head][PV k-slot], 16-byte chunks swizzled
  float hv[kHeadsPerWG];        // per head: rescale factor of the current tile, at the end 1 / sum
  int32_t idx[kIdxCap + kIdxPad];
  uint64_t vmask[(kIdxCap + kIdxPad) / kTile];  // bit r of word t: row r of tile t is a valid entry
};
static_assert(sizeof(MlaShared) <= 160 * 1024, "LDS");
static_assert(kHeadsPerWG * kStageRow <= kTileBytes, "write-out block fits in a tile buffer");

// P in LDS: row = head of the workgroup (128 bytes = 64 k-slots), chunk c of
// 8 k-slots stored at slot c ^ (head % 8) so that 16 lanes reading 16 heads'
// same chunk hit distinct banks.
__device__ __forceinline__ uint32_t pt_off(int head, int c) { return head * 128 + ((c ^ (head & 7)) << 4); }

// LDS accesses that sit between the tile copies go through inline asm as
// well: the compiler would make an ordinary LDS access wait for every copy
// in flight.  The caller waits (lgkmcnt) before using or publishing them.
__device__ __forceinline__ void lds_store16(uint32_t addr, bf16x8 v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_store4(uint32_t addr, float v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}

// Opens a tile of the copy pipeline: this wave's copies of the tile have
// landed and its earlier LDS accesses are done, then the workgroup barrier.
// The barrier is issued bare: __syncthreads() would also drain any copy
// still in flight, since its release fence covers the copies' pending LDS
// writes.  All waves share one LDS, so once every wave has passed its own
// waits, the tile is complete for all of them.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wave w copies rows 16w .. 16w+15 of a tile (two 8-row groups) with
// eighteen 1 KB DMA instructions; pos[g] is the position of this lane's row
// 16w + 8g + l/8 (< 0: row 0).  Lane l of copy i of a group fills slot l of
// segment i, i.e. bf16 chunk 8i + cx of its row.  A bf16 cache copies that
// chunk.  An e4m3 cache copies the 16 codes that decode to bf16 chunks
// 2m, 2m+1 (raw chunk m) into the slot of chunk 2m, and the same codes again
// into the slot of chunk 2m+1, where the decode's second half lands; so each
// raw chunk sits where its own decoded first half goes, and fp8_decode can
// expand a wave's rows in place with no exchange between lanes.
template <bool FP8>
__device__ __forceinline__ void tile_dma(uint8_t* dst, const MlaParams& p, const int32_t (&pos)[2], int64_t seq_row0,
                                         int wave, int l) {
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int rg = 2 * wave + g;  // 8-row group
    const int64_t row = seq_row0 + max(pos[g], 0);
    // the chunk whose slot is l % 8 in row 8 rg + l / 8 (the inverse of chunk_off's swizzle)
    const int cx = ((l & 7) ^ (l >> 3) ^ (2 * rg + (l >> 5))) & 7;
    const uint8_t* src = FP8 ? (const uint8_t*)p.kv + row * kDqk + (cx >> 1) * 16
                             : (const uint8_t*)p.kv + row * (2 * kDqk) + cx * 16;
    uint8_t* seg = dst + rg * 9 * 1024;
#pragma unroll
    for (int i = 0; i < 9; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(src + (FP8 ? 64 : 128) * i),
                                       (__attribute__((address_space(3))) void*)(seg + 1024 * i), 16, 0, 0);
  }
}

// The same copy, issued one instruction at a time (k = 0 .. 17) between the
// compute steps of the previous tile: a wave that issued all eighteen at once
// would stall on the memory pipeline's back-pressure with its MFMA idle.
// Without a next tile (!live) every lane reads the same 16 bytes (one
// request per instruction, written to a buffer nobody reads): the issue stays
// unconditional, and so the code stays one basic block.
template <bool FP8>
struct TileCopy {
  const uint8_t* src[2];
  uint8_t* seg[2];
  __device__ __forceinline__ TileCopy(uint8_t* dst, const MlaParams& p, const int32_t (&pos)[2], int64_t seq_row0,
                                      int wave, int l, bool live) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int rg = 2 * wave + g;
      const int64_t row = seq_row0 + (live ? max(pos[g], 0) : 0);
      const int cx = live ? ((l & 7) ^ (l >> 3) ^ (2 * rg + (l >> 5))) & 7 : 0;
      src[g] = FP8 ? (const uint8_t*)p.kv + row * kDqk + (cx >> 1) * 16
                   : (const uint8_t*)p.kv + row * (2 * kDqk) + cx * 16;
      seg[g] = dst + rg * 9 * 1024;
    }
  }
  __device__ __forceinline__ void issue(int k) const {
    const int g = k / 9, i = k % 9;
    __builtin_amdgcn_global_load_lds((const void*)(src[g] + (FP8 ? 64 : 128) * i),
                                     (__attribute__((address_space(3))) void*)(seg[g] + 1024 * i), 16, 0, 0);
  }
};

// e4m3 cache: expands, in place, the rows this wave copied: lane l takes row
// 16w + l/4 (whose scales it holds: one per row, or one per 128-column tile)
// and raw chunks m = l%4 + 4k, k < 9, i.e. columns 16 m .. +16, which lie in
// tile m / 8 = k / 2 for every lane.  The wave's copies must have landed
// (vmcnt(0)).  Code x power-of-two scale is exact in bf16.
template <int NSC>
__device__ __forceinline__ void fp8_decode(uint8_t* buf, const float (&sc)[NSC], int wave, int l) {
  constexpr int kSteps = kDqk / 64;                    // k = 0 .. 8
  constexpr int kPerScale = NSC == 1 ? kSteps : 2;     // k-steps under one scale (a tile: 2)
  const int r = 16 * wave + (l >> 2);
  // one pass per scale, so each scale is a fixed register (selecting it by k
  // would become an indexed scratch load); the steps are unrolled so their
  // LDS reads overlap (about 1 us less per tile pair at the 128K decode shape)
#pragma unroll
  for (int i = 0; i < NSC; ++i) {
    const float scale = sc[i];
    const uint32_t sb = __float_as_uint(scale);
    const bool pow2 = (sb & 0x807FFFFFu) == 0 && (sb >> 23) != 0;  // a positive normal power of two
    const float hw_scale = pow2 ? scale : 1.0f;
#pragma unroll
    for (int k = i * kPerScale; k < min((i + 1) * kPerScale, kSteps); ++k) {
      const int m = (l & 3) + 4 * k;
      uint8_t* d0 = buf + chunk_off(r, 2 * m);
      const i32x4 v = *(const i32x4*)d0;
      // codes 4q .. 4q+3 -> bf16 pairs with the hardware's scaled OCP e4m3
      // conversion, exact for a power-of-two scale (checked against the
      // format's definition for all 256 codes and the scales 2^-2 .. 2^2).
      // The instruction takes only the scale's exponent, so a scale that is
      // not a power of two is converted unscaled and multiplied in fp32.
      uint32_t w[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w[2 * q] =
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)v[q], hw_scale, false));
        w[2 * q + 1] =
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)v[q], hw_scale, true));
      }
      if (!pow2) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          w[j] = pack_bf16x2(__uint_as_float(w[j] << 16) * scale, __uint_as_float(w[j] & 0xFFFF0000u) * scale);
      }
      *(i32x4*)d0 = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
      *(i32x4*)(buf + chunk_off(r, 2 * m + 1)) = i32x4{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
    }
  }
}

// NSC: scales per cache row (e4m3: 1 per row, or one per 128-column tile)
template <bool FP8, int NSC = 1>
__global__ __launch_bounds__(kMlaThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_mfma_kernel(MlaParams p) {
  const WgTrace wg_trace_(p.wg_trace);
  extern __shared__ __attribute__((aligned(16))) uint8_t mla_smem[];
  MlaShared& sh = *reinterpret_cast<MlaShared*>(mla_smem);
  int32_t* s_idx = sh.idx;
  // An accumulation-register operand makes the compiler select the MFMA
  // forms that accumulate in AGPRs, so the 128 output accumulators live there
  // and the arithmetic registers stay free for operands and addresses.
  asm volatile("" ::"a"(0.0f));

  const int split = blockIdx.x, bt = blockIdx.y, hg = blockIdx.z;
  const int b = bt / p.T;
  const int tid = threadIdx.x, wave = tid / kWave, l = lane_id();
  const int lg = l >> 4, lc = l & 15;
  const int len = filled_rows(p.seq_lens[b], p.Lmax, p.len_sub);
  const int h0 = hg * kHeadsPerWG + wave * kHeadsPerWave;  // this wave's first head
  // row index of position 0 of this sequence (paged cache: rows are
  // translated to physical rows when the index list is loaded)
  const bool paged = p.block_table != nullptr;
  const int64_t seq_row0 = paged ? 0 : (int64_t)b * p.Lmax;
  const int32_t* sel = p.topk_idx + (int64_t)bt * p.K;
  // The split's entries j_split .. +split_rows go through LDS in chunks of
  // at most kIdxCap (whole tiles), one after another, with the softmax
  // state carried across: a split needs no more rows than the host's
  // parallelism asks for, whatever the LDS holds.
  const int j_split = split * p.rows_per_split;
  const int split_rows = max(0, min(p.K, j_split + p.rows_per_split) - j_split);
  const int n_chunks = max(1, (split_rows + kIdxCap - 1) / kIdxCap);
  const int chunk_rows = (((split_rows + n_chunks - 1) / n_chunks) + kTile - 1) / kTile * kTile;  // <= kIdxCap
  int j_begin = j_split, n_rows = 0;  // the current chunk's entries
  const int my_row = 16 * wave + (l >> 3);  // this lane's row of 8-row group 0 (group 1: +8)
  // index entry j of the split -> position (-1: none); the load is
  // unconditional and clamped into the list, so that several of them can be
  // in flight at once
  auto resolve = [&](int j) -> int32_t {
    const int32_t v = sel[min(j_begin + j, p.K - 1)];
    return (j < n_rows && v >= 0 && v < len) ? v : -1;
  };

  float kscale[NSC] = {};  // e4m3: scales of row 16 wave + l/4 of the tile being copied
  auto load_kscale = [&](int64_t row) {
#pragma unroll
    for (int i = 0; i < NSC; ++i) kscale[i] = p.kv_scale[row * NSC + i];
  };
  // Prologue of a chunk: every load of its index list is issued at once;
  // once they land the list is stored to LDS and the first tile's copy
  // starts (its rows come straight from registers).  The LDS stores go
  // first: stored after the copy was issued, they would wait for it to land.
  // Returns the chunk's tile count.
  constexpr int kPer = kIdxCap / kMlaThreads;
  auto load_chunk = [&](int c) -> int {
    j_begin = j_split + c * chunk_rows;
    n_rows = max(0, min(chunk_rows, j_split + split_rows - j_begin));
    int32_t iv[kPer];  // entries tid + 256 k
#pragma unroll
    for (int k = 0; k < kPer; ++k) iv[k] = resolve(tid + k * kMlaThreads);
    if (paged) {
      // position -> physical row: page table[b][pos / page] (clamped into the
      // cache), row pos % page within it; every entry's load is issued first
      const int64_t prow = (int64_t)1 << p.page_shift;
      const int32_t* btab = p.block_table + (int64_t)b * p.max_pages;
      int32_t pe[kPer];
#pragma unroll
      for (int k = 0; k < kPer; ++k)
        pe[k] = btab[min((int64_t)(max(iv[k], 0) >> p.page_shift), (int64_t)p.max_pages - 1)];
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int64_t pp = min(max((int64_t)pe[k], (int64_t)0), p.num_pages - 1);
        iv[k] = iv[k] >= 0 ? (int32_t)(pp * prow + (iv[k] & (prow - 1))) : -1;
      }
    }
    // the list in LDS, padded with -1 through the last tile plus the 2 tiles
    // whose positions are read ahead
    const int n_tiles = (n_rows + kTile - 1) / kTile;
    const int n_pad = (n_tiles + 2) * kTile;
#pragma unroll
    for (int k = 0; k < kPer; ++k) s_idx[tid + k * kMlaThreads] = iv[k];  // -1 past the list
    for (int i = kIdxCap + tid; i < n_pad; i += kMlaThreads) s_idx[i] = -1;
    if (paged) {  // the first tile's rows come back from LDS
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      const int32_t pos0[2] = {s_idx[my_row], s_idx[my_row + 8]};
      tile_dma<FP8>(sh.rows[0], p, pos0, seq_row0, wave, l);
      if constexpr (FP8) load_kscale(max(s_idx[16 * wave + (l >> 2)], 0));
    } else {
      const int32_t pos0[2] = {resolve(my_row), resolve(my_row + 8)};
      tile_dma<FP8>(sh.rows[0], p, pos0, seq_row0, wave, l);
      if constexpr (FP8) load_kscale(seq_row0 + max(resolve(16 * wave + (l >> 2)), 0));
    }
    return n_tiles;
  };
  // the list is complete in LDS (a bare barrier lets the first tile's copy
  // stay in flight: __syncthreads() would wait for it); then each tile's
  // mask of valid rows
  auto chunk_masks = [&](int n_tiles) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    for (int t = wave; t < n_tiles + 2; t += kMlaWaves) {
      const uint64_t bal = __ballot(s_idx[t * kTile + l] >= 0);
      if (l == 0) sh.vmask[t] = bal;
    }
  };
  int n_tiles = load_chunk(0);

  // query heads h0 + lc, dims 32 ks + 8 lg .. +8  (operand B of QK^T)
  bf16x8 qreg[kKSteps];
  {
    const bf16x8* qrow = (const bf16x8*)((const uint16_t*)p.q + ((int64_t)bt * p.H + h0 + lc) * kDqk);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) qreg[ks] = qrow[ks * 4 + lg];
  }

  const float zscale = p.scale * 1.4426950408889634f;  // logits in base-2 units

  // LDS byte offsets of this lane's operand reads within a tile
  uint32_t a_off[kBlocks][2];  // QK^T operand A: [16-row block][k-step parity], plus 1 KB per 2 k-steps
#pragma unroll
  for (int mt = 0; mt < kBlocks; ++mt)
#pragma unroll
    for (int par = 0; par < 2; ++par) a_off[mt][par] = chunk_off(tile_row(mt, lc), 4 * par + lg);
  uint32_t v_off[2][2];  // PV operand, value tile 0: [k-step][row half]
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      v_off[kk][hh] = chunk_off(tile_row(2 * kk + hh, 4 * lg + (lc >> 2)), (lc & 3) >> 1) + 8 * (lc & 1);

  // O^T accumulators of the PV product: this wave owns value columns
  // 128 wave .. +128 of all 64 heads; o[hb][db] = columns 128 wave + 16 db +
  // 4 lg .. +4 of head 16 hb + lc.
  f32x4 o[4][8];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int db = 0; db < 8; ++db) o[hb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;  // softmax state of head h0 + lc (this wave's QK heads)
  const uint32_t pt_base = (uint32_t)(uintptr_t)sh.pt, hv_base = (uint32_t)(uintptr_t)sh.hv;

  // dma(k), k = 0 .. 17, is called once after each QK^T step: it issues the
  // next tile's copy instruction k.
  auto compute = [&](const uint8_t* rows, int j0, auto&& dma) {
    const uint64_t vm = sh.vmask[j0 / kTile];  // read early: its latency hides behind QK^T
    const uint32_t base = (uint32_t)(uintptr_t)rows;
    // ---- S^T[64 rows x 16 heads] over all 576 dims: 8 accumulation chains ----
    f32x4 s[kBlocks][2];
#pragma unroll
    for (int mt = 0; mt < kBlocks; ++mt) {
      s[mt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      s[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    uint32_t qaddr[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int par = 0; par < 2; ++par) qaddr[h][2 * j + par] = base + a_off[2 * h + j][par];
    QkGroup qg[2];
    auto qk_group = [&](const QkGroup& cur, int g, int h) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int par = 0; par < 2; ++par)
          s[2 * h + j][par] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.r[2 * j + par], qreg[2 * g + par],
                                                                      s[2 * h + j][par], 0, 0, 0);
    };
    static_assert(kKSteps == 18, "nine pairs of k-steps");
    // 18 groups n = (g, h) = (n/2, n%2) in the order (0,0) (0,1) (1,0) ... (8,1),
    // the next one in flight while one is multiplied
    qk_issue<0>(qg[0], qaddr[0]);
    qk_issue_wait<0, 4>(qg[1], qg[0], qaddr[1]);
    qk_group(qg[0], 0, 0);
    dma(0);
    qk_issue_wait<1, 4>(qg[0], qg[1], qaddr[0]);
    qk_group(qg[1], 0, 1);
    dma(1);
    qk_issue_wait<1, 4>(qg[1], qg[0], qaddr[1]);
    qk_group(qg[0], 1, 0);
    dma(2);
    qk_issue_wait<2, 4>(qg[0], qg[1], qaddr[0]);
    qk_group(qg[1], 1, 1);
    dma(3);
    qk_issue_wait<2, 4>(qg[1], qg[0], qaddr[1]);
    qk_group(qg[0], 2, 0);
    dma(4);
    qk_issue_wait<3, 4>(qg[0], qg[1], qaddr[0]);
    qk_group(qg[1], 2, 1);
    dma(5);
    qk_issue_wait<3, 4>(qg[1], qg[0], qaddr[1]);
    qk_group(qg[0], 3, 0);
    dma(6);
    qk_issue_wait<4, 4>(qg[0], qg[1], qaddr[0]);
    qk_group(qg[1], 3, 1);
    dma(7);
    qk_issue_wait<4, 4>(qg[1], qg[0], qaddr[1]);
    qk_group(qg[0], 4, 0);
    dma(8);
    qk_issue_wait<5, 4>(qg[0], qg[1], qaddr[0]);
    qk_group(qg[1], 4, 1);
    dma(9);
    qk_issue_wait<5, 4>(qg[1], qg[0], qaddr[1]);
    qk_group(qg[0], 5, 0);
    dma(10);
    qk_issue_wait<6, 4>(qg[0], qg[1], qaddr[0]);
    qk_group(qg[1], 5, 1);
    dma(11);
    qk_issue_wait<6, 4>(qg[1], qg[0], qaddr[1]);
    qk_group(qg[0], 6, 0);
    dma(12);
    qk_issue_wait<7, 4>(qg[0], qg[1], qaddr[0]);
    qk_group(qg[1], 6, 1);
    dma(13);
    qk_issue_wait<7, 4>(qg[1], qg[0], qaddr[1]);
    qk_group(qg[0], 7, 0);
    dma(14);
    qk_issue_wait<8, 4>(qg[0], qg[1], qaddr[0]);
    qk_group(qg[1], 7, 1);
    dma(15);
    qk_issue_wait<8, 4>(qg[1], qg[0], qaddr[1]);
    qk_group(qg[0], 8, 0);
    dma(16);
    qk_wait<0>(qg[1]);
    qk_group(qg[1], 8, 1);
    dma(17);

    // ---- online softmax for head h0 + lc over rows 4 lg + e of each block ----
    // this lane's rows are tile_row(mt, 4 lg + e) = 16 mt + 2 e + (lg & 1) + 8 (lg >> 1)
    const uint64_t vml = vm >> ((lg & 1) + 8 * (lg >> 1));
    float z[kBlocks][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < kBlocks; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool valid = (vml >> (16 * mt + 2 * e)) & 1u;
        z[mt][e] = valid ? (s[mt][0][e] + s[mt][1][e]) * zscale : -INFINITY;
        tmax = fmaxf(tmax, z[mt][e]);
      }
    tmax = group4_max(tmax);
    // Lazy rescaling: the reference max m_run only moves when the tile's
    // max exceeds it by more than kSlack (probabilities then stay <= 2^kSlack,
    // exact enough in bf16 and fp32), or when it is still -inf (O and l are
    // zero then, so nothing needs rescaling).  Moving it costs a pass over the
    // 128 accumulators; with a stable max that pass is skipped for the wave.
    const bool move = tmax > m_run + kSlack;
    const float m_new = move ? tmax : m_run;
    // v_exp_f32 directly: exp2(-inf) = 0, and results below 2^-126 (which
    // cannot matter next to the reference max) may flush to 0
    const float alpha = move ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;  // m_run = -inf gives 0
    const float m_ref = m_new > -INFINITY ? m_new : 0.0f;  // no row valid yet: every z is -inf
    float psum = 0.0f;
    float pr[kBlocks][4];
#pragma unroll
    for (int mt = 0; mt < kBlocks; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pr[mt][e] = __builtin_amdgcn_exp2f(z[mt][e] - m_ref);  // m_ref >= z when z is finite
        psum += pr[mt][e];
      }
    psum = group4_sum(psum);
    l_run = l_run * alpha + psum;
    m_run = m_new;

    // ---- hand P and the rescale factors to every wave ----
    // P^T operand of k-step kk for head lc: k-slot 8 lg + j <-> row
    // (j < 4 ? block 2kk row 4 lg + j : block 2kk+1 row 4 lg + j - 4), i.e.
    // chunk 4 kk + lg of the head's P row.
    {
      const int hl = wave * kHeadsPerWave + lc;  // this lane's head within the workgroup
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        uint32_t pw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pw[j] = pack_bf16x2(pr[2 * kk + (j >> 1)][2 * (j & 1)], pr[2 * kk + (j >> 1)][2 * (j & 1) + 1]);
        lds_store16(pt_base + pt_off(hl, 4 * kk + lg), __builtin_bit_cast(bf16x8, pw));
      }
      if (lg == 0) lds_store4(hv_base + 4 * hl, alpha);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // P and factors complete (copies may be in flight)

    // ---- O^T[128 value columns x 64 heads] += V^T P^T ----
    // Rescale factors of this lane's 4 heads 16 hb + lc.  Only heads whose
    // reference max moved past a nonzero O need work (a factor of 0 meets an
    // O that is still 0), which is rare after the first tiles.
    float al[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
      asm volatile("ds_read_b32 %0, %1" : "=&v"(al[hb]) : "v"(hv_base + 4 * (16 * hb + lc)) : "memory");
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(al[0]), "+v"(al[1]), "+v"(al[2]), "+v"(al[3])::"memory");
    if (__any((al[0] != 1.0f && al[0] != 0.0f) || (al[1] != 1.0f && al[1] != 0.0f) ||
              (al[2] != 1.0f && al[2] != 0.0f) || (al[3] != 1.0f && al[3] != 0.0f))) {
      // Each scaled accumulator goes back through an MFMA with zero operands
      // (0 x 0 + C = C), so it leaves this block, like the PV product, as an
      // MFMA result and stays in the accumulation registers on both paths.
      // The empty asm pins each accumulator's input to those registers
      // inside this block: the copies to ordinary registers that the
      // multiply needs are then made here, on the rare path, and not in the
      // score phase of every tile.
      const bf16x8 zero = {};
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          f32x4 acc = o[hb][db];
          asm volatile("" : "+a"(acc));
          o[hb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(zero, zero, acc * al[hb], 0, 0, 0);
        }
    }
    // V^T operand (A) of k-step kk: k-slot 8 lg + k (k < 4) is tile row
    // tile_row(2kk, 4 lg + k), slot 8 lg + 4 + k is tile_row(2kk+1, 4 lg + k):
    // lane lc addresses row k = lc/4 of its group and columns 4 (lc%4) .. +4
    // of the 16-column tile.  This wave's value tiles 8 wave + db sit 2 wave
    // KB (plus 1 KB per 4 tiles) past those of tiles 0 .. 3; within a KB the
    // tiles' offsets differ in bits 5-6 only (the swizzle is an XOR), so
    // tile n4's offset is that of tile 0 XOR 32 n4.
    const uint32_t vbase = base + 2048 * wave;
    TrGroup grp[2];
    bf16x8 pbt[4];  // P^T operands of the current k-step, head blocks 0..3
    auto pv_group = [&](const TrGroup& cur, int g) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const i16x4 lo = cur.r[2 * k], hi = cur.r[2 * k + 1];
        const bf16x8 vop = __builtin_bit_cast(bf16x8, (i32x4){__builtin_bit_cast(int, (short2){lo[0], lo[1]}),
                                                               __builtin_bit_cast(int, (short2){lo[2], lo[3]}),
                                                               __builtin_bit_cast(int, (short2){hi[0], hi[1]}),
                                                               __builtin_bit_cast(int, (short2){hi[2], hi[3]})});
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          o[hb][4 * g + k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pbt[hb], o[hb][4 * g + k], 0, 0, 0);
      }
    };
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint32_t taddr[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        taddr[2 * k] = vbase + (v_off[kk][0] ^ (32 * k));
        taddr[2 * k + 1] = vbase + (v_off[kk][1] ^ (32 * k));
      }
      // P^T of head block hb, k-step kk: head 16 hb + lc, chunk 4 kk + lg
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
        asm volatile("ds_read_b128 %0, %1" : "=&v"(pbt[hb]) : "v"(pt_base + pt_off(16 * hb + lc, 4 * kk + lg)) : "memory");
      tr_issue_wait<0>(grp[0], grp[1], taddr);  // (waits for the P^T reads; grp[1] is not live here)
      tr_issue_wait<1>(grp[1], grp[0], taddr);
      pv_group(grp[0], 0);
      tr_wait_last(grp[1]);
      pv_group(grp[1], 1);
    }
  };

  int cur = 0;
  for (int c = 0; c < n_chunks; ++c) {
  if (c > 0) {
    // the last chunk's copies have landed and every wave is done with its
    // list and tiles before the next list and first tile overwrite them
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    n_tiles = load_chunk(c);
    cur = 0;
  }
  chunk_masks(n_tiles);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // vmask complete (copies may be in flight)
  // Tiles after the chunk's last valid entry are skipped: a query that sees
  // fewer than K positions has an index list ending in -1s (the first
  // tokens of a fresh prompt), and its split would otherwise run them all.
  int n_live = 0;
  for (int t = 0; t < n_tiles; ++t)
    if (sh.vmask[t] != 0) n_live = t + 1;
  n_live = __builtin_amdgcn_readfirstlane(n_live);
  // One compact loop over the tiles (the body stays in the instruction
  // cache).  Tile t sits in buffer t % 2.  The rows this lane copies for
  // tile t are entries 64 t + 16 wave + l/8 (+8); they are read one tile
  // ahead, so the copy is issued without an LDS round trip.
  int32_t pos[2] = {s_idx[kTile + my_row], s_idx[kTile + my_row + 8]};
  if constexpr (!FP8) {
    // Step t: wait for this wave's copy of tile t, barrier (tile t complete;
    // every wave is done with tile t-1, whose buffer is reused), compute tile
    // t while issuing the copy of tile t+1 step by step (a token copy after
    // the last tile).
    for (int t = 0; t < n_live; ++t) {
      tile_barrier();
      const TileCopy<false> next(sh.rows[cur ^ 1], p, pos, seq_row0, wave, l, t + 1 < n_live);
      pos[0] = s_idx[(t + 2) * kTile + my_row];
      pos[1] = s_idx[(t + 2) * kTile + my_row + 8];
      compute(sh.rows[cur], t * kTile, [&](int k) { next.issue(k); });
      cur ^= 1;
    }
    // the token copy after the last tile is still in flight into rows[cur]:
    // the write-out stages its block in the other buffer and waits for the
    // copy only at the very end
  } else {
    // Step t: barrier (every wave has decoded its rows of tile t and is done
    // with tile t-1), start copying tile t+1, compute tile t, then wait for
    // this wave's copy and decode its rows of tile t+1.
    const int srow = 16 * wave + (l >> 2);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    fp8_decode(sh.rows[0], kscale, wave, l);
    for (int t = 0; t < n_live; ++t) {
      __syncthreads();
      tile_dma<true>(sh.rows[cur ^ 1], p, pos, seq_row0, wave, l);
      load_kscale(seq_row0 + max(s_idx[(t + 1) * kTile + srow], 0));
      pos[0] = s_idx[(t + 2) * kTile + my_row];
      pos[1] = s_idx[(t + 2) * kTile + my_row + 8];
      compute(sh.rows[cur], t * kTile, [](int) {});
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      fp8_decode(sh.rows[cur ^ 1], kscale, wave, l);
      cur ^= 1;
    }
  }
  }  // chunks

  // ---- write-out ----
  // The owner wave of each head publishes 1 / sum (after every wave's last
  // read of the rescale factors) and writes the head's statistics; lane l
  // then holds columns 128 wave + 16 db + 4 lg .. +4 of heads 16 hb + lc.
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (lg == 0) sh.hv[wave * kHeadsPerWave + lc] = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  {
    const int h = h0 + lc;
    if (p.splits == 1) {
      if (p.lse && lg == 0)
        store_through(&p.lse[(int64_t)bt * p.H + h],
                      l_run > 0.0f ? (m_run + log2f(l_run)) * 0.6931471805599453f : -INFINITY);
    } else if (lg == 0) {
      const int64_t slot = ((int64_t)split * p.B * p.T + bt) * p.H + h;
      store_through(&p.part_ml[slot * 2], m_run);
      store_through(&p.part_ml[slot * 2 + 1], l_run);
    }
  }
  if (p.splits == 1 && p.out_dtype == kF32) {
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const int h = hg * kHeadsPerWG + 16 * hb + lc;
      const float inv = sh.hv[16 * hb + lc];
      const int64_t ooff = ((int64_t)bt * p.H + h) * kDv + 128 * wave + 4 * lg;
#pragma unroll
      for (int db = 0; db < 8; ++db)
        store_through((float*)p.out + ooff + 16 * db,
                      __builtin_bit_cast(i32x4, f32x4{o[hb][db][0] * inv, o[hb][db][1] * inv,
                                                      o[hb][db][2] * inv, o[hb][db][3] * inv}));
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no copy into LDS outlives the workgroup
    return;
  }
  // bf16 rows: the workgroup's 64 heads are 64 consecutive rows of Dv values
  // in the output and in the split's partial alike, so the block is staged in
  // LDS (in the last tile's buffer, free after the barrier above) and written
  // back as whole rows, one 1 KB row per wave instruction.  Written straight from the accumulator
  // layout, every store instruction would cover sixteen 32-byte pieces of
  // sixteen rows.  (All results are stored through the L2 to memory: the
  // partials are the merge's input, tens of MB at long contexts, which as
  // dirty L2 lines would be written back only after the last workgroup.)
  uint8_t* stage = sh.rows[cur ^ 1];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const int hl = 16 * hb + lc;
    const float inv = sh.hv[hl];
#pragma unroll
    for (int db = 0; db < 8; ++db)
      *(i32x2*)(stage + hl * kStageRow + 2 * (128 * wave + 16 * db + 4 * lg)) =
          i32x2{(int)pack_bf16x2(o[hb][db][0] * inv, o[hb][db][1] * inv),
                (int)pack_bf16x2(o[hb][db][2] * inv, o[hb][db][3] * inv)};
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  uint16_t* dst = p.splits == 1
                      ? (uint16_t*)p.out + ((int64_t)bt * p.H + hg * kHeadsPerWG) * kDv
                      : p.part_o + (((int64_t)split * p.B * p.T + bt) * p.H + hg * kHeadsPerWG) * kDv;
#pragma unroll
  for (int r = 0; r < kHeadsPerWG / kMlaWaves; ++r) {
    const int hl = kMlaWaves * r + wave;
    store_through(dst + (int64_t)hl * kDv + 8 * l, *(const i32x4*)(stage + hl * kStageRow + 16 * l));
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no copy into LDS outlives the workgroup
}

// Merge the per-split partials of one (query, head): split s holds its
// output normalised by its own sum l_s and its running max m_s (base 2), so
//   out = sum_s w_s O_s / sum_s w_s,   w_s = l_s 2^(m_s - M),  M = max_s m_s.
// 64 threads, 8 consecutive value columns (16 bytes of bf16 partials) each;
// the partials of up to 16 splits are loaded before any is used, so their
// latencies overlap.
constexpr int kCombineBatch = 16;

__global__ __launch_bounds__(64) void mla_combine_kernel(MlaParams p) {
  const WgTrace wg_trace_(p.wg_trace);
  const int h = blockIdx.x, bt = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t BT = (int64_t)p.B * p.T;
  const int64_t slot0 = (int64_t)bt * p.H + h;
  const int64_t slot_stride = BT * p.H;
  const int d = min(tid * 8, p.Dv - 8);  // this lane's 8 value columns (lanes past Dv repeat the last 8)
  const uint16_t* po = p.part_o + slot0 * p.Dv + d;
  const int64_t stride = slot_stride * p.Dv;
  // The first batch of partials is loaded together with the statistics (the
  // addresses do not depend on them), so the workgroup waits for memory once.
  i32x4 v[kCombineBatch];
#pragma unroll
  for (int j = 0; j < kCombineBatch; ++j)  // splits past the end reread split 0 (weight 0)
    v[j] = *(const i32x4*)(po + (j < p.splits ? j : 0) * stride);
  const int sl = min(tid, p.splits - 1);
  const float ms_raw = p.part_ml[(slot0 + sl * slot_stride) * 2];
  const float ls_raw = p.part_ml[(slot0 + sl * slot_stride) * 2 + 1];
  const float ms = tid < p.splits ? ms_raw : -INFINITY, ls = tid < p.splits ? ls_raw : 0.0f;
  const float M = wave_max(ls > 0.0f ? ms : -INFINITY);
  const float wgt = (ls > 0.0f) ? ls * exp2f(ms - M) : 0.0f;
  const float L = wave_sum(wgt);
  const float wn = L > 0.0f ? wgt / L : 0.0f;  // lane s: normalised weight of split s
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
  for (int s0 = 0; s0 < p.splits; s0 += kCombineBatch) {
    if (s0 > 0) {
#pragma unroll
      for (int j = 0; j < kCombineBatch; ++j)
        v[j] = *(const i32x4*)(po + (s0 + j < p.splits ? s0 + j : s0) * stride);
    }
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) {
      const float w = s0 + j < p.splits ? __shfl(wn, s0 + j, kWave) : 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[2 * k] = fmaf(bf16_bits_to_f32((uint32_t)v[j][k] & 0xFFFFu), w, acc[2 * k]);
        acc[2 * k + 1] = fmaf(bf16_bits_to_f32((uint32_t)v[j][k] >> 16), w, acc[2 * k + 1]);
      }
    }
  }
  if (tid * 8 < p.Dv) {
    const int64_t ooff = slot0 * p.Dv + d;
    if (p.out_dtype == kF32) {
      *(f32x4*)((float*)p.out + ooff) = f32x4{acc[0], acc[1], acc[2], acc[3]};
      *(f32x4*)((float*)p.out + ooff + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    } else {
      i32x4 ob;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        ob[k] = (int)pack_bf16x2(acc[2 * k], acc[2 * k + 1]);
      *(i32x4*)((uint16_t*)p.out + ooff) = ob;
    }
  }
  if (p.lse && tid == 0) p.lse[slot0] = L > 0.0f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
}

bool mla_mfma_supported(const MlaParams& p) {
  return p.Dqk == kDqk && p.Dv == kDv && p.H % kHeadsPerWG == 0 && p.q_dtype == kBF16 &&
         (p.kv_dtype == kBF16 || p.kv_dtype == kE4M3 || p.kv_dtype == kE4M3T128);
}

hipError_t launch_mla(const MlaParams& p_in, bool allow_mfma, hipStream_t stream) {
  MlaParams p = p_in;
  p.wg_trace = nullptr;
  if (allow_mfma && mla_mfma_supported(p)) {
    dim3 grid((unsigned)p.splits, (unsigned)(p.B * p.T), (unsigned)(p.H / kHeadsPerWG));
    p.wg_trace = trace_region(kTraceMla, (int64_t)grid.x * grid.y * grid.z);
    const size_t lds = sizeof(MlaShared);
    hipError_t e;
    if (p.kv_dtype == kBF16) {
      e = set_max_dynamic_lds((const void*)mla_mfma_kernel<false>, (int)lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(mla_mfma_kernel<false>, grid, dim3(kMlaThreads), lds, stream, p);
    } else if (p.kv_dtype == kE4M3) {
      e = set_max_dynamic_lds((const void*)mla_mfma_kernel<true>, (int)lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(mla_mfma_kernel<true>, grid, dim3(kMlaThreads), lds, stream, p);
    } else {  // one scale per 128-column tile: ceil(576 / 128) per row
      constexpr int kTiles = (kDqk + 127) / 128;
      e = set_max_dynamic_lds((const void*)mla_mfma_kernel<true, kTiles>, (int)lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((mla_mfma_kernel<true, kTiles>), grid, dim3(kMlaThreads), lds, stream, p);
    }
    e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    p.wg_trace = trace_region(kTraceMlaCombine, (int64_t)p.H * p.B * p.T);
    hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)p.H, (unsigned)(p.B * p.T)), dim3(kWave), 0,
                       stream, p);  // needs Dv <= 512 and splits <= 64
    return hipGetLastError();
  }
  p.wg_trace = nullptr;
  hipLaunchKernelGGL(mla_generic_kernel, dim3((unsigned)p.H, (unsigned)(p.B * p.T)), dim3(kGenThreads),
                     0, stream, p);
  return hipGetLastError();
}

}  // namespace dsa
