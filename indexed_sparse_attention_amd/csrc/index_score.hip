// Indexer scores: S[b,t,s] = sum_h w[b,t,h] * max(0, (q_idx[b,t,h,:] . k_idx[b,s,:]) * k_scale[b,s])
// for every visible position s < vis(b,t) = len_b - T + 1 + t.
//
// The pages ("Optimizing Next-Gen LLM Inference" §3.1, "Inference Acceleration
// for New Large Model Architectures" §3.1) fuse relevance scoring and the
// head-weighted aggregation into one pass over the key cache; here that pass
// is a matrix-core contraction over (index heads x key rows) with the ReLU,
// the weights and the head sum applied to the accumulators in registers.  The
// same pass builds the per-query histogram of the top 12 bits of each score's
// order-preserving key, which the Top-K threshold search consumes.
#include <hip/hip_ext.h>
#include <stdlib.h>

#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

// ---------------------------------------------------------------------------
// Portable SIMT kernel: one thread per (query, position).  Any dims/dtypes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float load_elem(const void* p, int dtype, int64_t i) {
  if (dtype == kF32) return ((const float*)p)[i];
  if (dtype == kBF16) return bf16_bits_to_f32(((const uint16_t*)p)[i]);
  return e4m3_to_f32(((const uint8_t*)p)[i]);
}

__global__ __launch_bounds__(256) void score_generic_kernel(ScoreParams p) {
  const int bt = blockIdx.y;
  const int b = bt / p.T, t = bt % p.T;
  const int len = filled_rows(p.seq_lens[b], p.Lmax, p.len_sub);
  const int64_t vis = (int64_t)len - p.T + 1 + t;
  const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= vis) return;
  const bool fp8 = (p.k_dtype == kE4M3);
  const int64_t krow = ((int64_t)b * p.Lmax + s) * p.Di;
  float S = 0.0f;
  if (p.k_dtype == kMXE4M3) {
    // MXFP8: the query is quantised group by group (32 dims, the last group
    // may be shorter) with a shared power-of-two scale 2^E, E = floor(log2
    // amax) - 8 (the largest magnitude lands in E4M3's top binade; OCP MX
    // v1.0 conversion), and each group's products carry both groups' scales.
    const int G = (p.Di + 31) / 32;
    const uint8_t* ks = (const uint8_t*)p.k_scale + ((int64_t)b * p.Lmax + s) * G;
    for (int h = 0; h < p.Hi; ++h) {
      const int64_t qrow = ((int64_t)bt * p.Hi + h) * p.Di;
      float d = 0.0f;
      for (int g = 0; g < G; ++g) {
        const int i0 = 32 * g, n = min(32, p.Di - i0);
        float amax = 0.0f;
        for (int i = 0; i < n; ++i) amax = fmaxf(amax, fabsf(load_elem(p.q_idx, p.q_dtype, qrow + i0 + i)));
        const int ef = (int)(__float_as_uint(amax) >> 23);  // biased exponent (amax >= 0)
        const int E = ef == 0 ? -127 : max(ef - 127 - 8, -127);
        const float inv = __uint_as_float((uint32_t)(127 - E) << 23);  // 2^-E
        float gd = 0.0f;
        for (int i = 0; i < n; ++i)
          gd = fmaf(e4m3_quantize(load_elem(p.q_idx, p.q_dtype, qrow + i0 + i) * inv),
                    load_elem(p.k_idx, kE4M3, krow + i0 + i), gd);
        d += ldexpf(gd, E + (int)ks[g] - 127);
      }
      S = fmaf(p.head_w[(int64_t)bt * p.Hi + h], fmaxf(d, 0.0f), S);
    }
    p.scores[(int64_t)bt * p.Lmax + s] = S;
    if (p.hist) atomicAdd(&p.hist[(int64_t)bt * kHistBins + (score_key(S) >> kHistShift)], 1u);
    return;
  }
  const float scale = p.k_scale ? ((const float*)p.k_scale)[(int64_t)b * p.Lmax + s] : 1.0f;
  for (int h = 0; h < p.Hi; ++h) {
    const int64_t qrow = ((int64_t)bt * p.Hi + h) * p.Di;
    float d = 0.0f;
    for (int i = 0; i < p.Di; ++i) {
      float qv = load_elem(p.q_idx, p.q_dtype, qrow + i);
      if (fp8) qv = e4m3_quantize(qv);
      d = fmaf(qv, load_elem(p.k_idx, p.k_dtype, krow + i), d);
    }
    d *= scale;
    S = fmaf(p.head_w[(int64_t)bt * p.Hi + h], fmaxf(d, 0.0f), S);
  }
  p.scores[(int64_t)bt * p.Lmax + s] = S;
  if (p.hist) atomicAdd(&p.hist[(int64_t)bt * kHistBins + (score_key(S) >> kHistShift)], 1u);
}

// ---------------------------------------------------------------------------
// Matrix-core kernel for 64 index heads x 128 dims.
//
// Work: for each sequence b and group g of TQ consecutive query tokens, the
// positions [0, vis_end) with vis_end = vis of the group's last token, cut
// into units of 64 positions (a "segment").  Each segment gets a contiguous
// run of workgroups in proportion to its units (at least one), and the waves
// of that run take its 16-position sub-tiles round-robin, so all of them
// sweep the segment's key rows together through one contiguous window:
// neighbouring waves read neighbouring 4 KB tiles, which keeps HBM pages and
// channels evenly busy.  A wave's unit is 4 of its sub-tiles.
//
// Per wave and sub-tile of 16 positions, the MFMA computes D[16 heads x 16
// positions] for each of the 4 head tiles: operand A is the index query (kept
// in registers for the whole segment), operand B the key rows loaded straight
// from HBM, 16 bytes per lane.  In the 16x16 accumulator layout lane l holds
// position l%16 and heads 4*(l/16) + e, e < 4, so ReLU, weight and a partial
// head sum happen in-lane; after 4 sub-tiles a 3-shuffle reduce-scatter across
// the 4 lane groups leaves lane l with the full score of column l%16 of the
// unit's sub-tile l/16.
//
// Operand k-ordering: bf16 operands A and B share one (lane group, element)
// -> k assignment, so any fixed permutation of the 128 dims gives the same
// dot product; lane group j of k-step ks carries dims 32 ks + 8 j .. +8.  The
// e4m3 product (one k-step of 128) applies its scales per 32 consecutive k,
// so there the operands follow the hardware's own order: lane group j holds k
// 16 j .. +16 in its first 16 bytes and 64 + 16 j .. +16 in the next 16, and
// lane l's scale operand applies to row (A) / column (B) l%16 of the group of
// k = 32 (l/16) .. +32 (both checked on the device against an exact sum).
//
// Key formats: bf16; e4m3 with one scale per row (applied to the score,
// the operands' scales are 1); MXFP8, e4m3 with an E8M0 scale per 32 dims,
// whose index query is quantised the same way while it is staged, both
// scales going into the scaled e4m3 MFMA.
// ---------------------------------------------------------------------------
constexpr int kHi = 64, kDi = 128;
constexpr int kSharedTokens = 8;    // tokens per segment of the shared-key variant
constexpr int kSharedThreads = 512;  // its workgroup: 8 waves, two per SIMD, one token each
// Its LDS key ring (16-row sub-tiles of 4 KB): what the 8 tokens' packed
// histograms (64 KB) and the static arrays leave of 160 KB.
__host__ __device__ constexpr int ks_ring_slots(int threads) { return threads == 512 ? 20 : 0; }
// Units a shared-key workgroup takes before flushing its 16-bit counters
// (1008 x 64 positions per token stay below 2^16); a multiple of its store batch.
constexpr int kPassUnits = 1008;
constexpr int kKeyBF16 = 0, kKeyE4M3 = 1, kKeyMX = 2;
constexpr int kGroups = kDi / 32;  // MX groups per row

template <int KF>
struct KeyTile {  // e4m3: one k-step of 128 dims, 32 bytes
  i32x8 v;
};
template <>
struct KeyTile<kKeyBF16> {  // bf16: 4 k-steps of 32 dims, 16 bytes each
  bf16x8 v[4];
};
template <>
struct KeyTile<kKeyMX> {  // MXFP8: the codes and this lane's group scale (E8M0)
  i32x8 v;
  int sc;
};

// Key rows are read through a buffer resource over the sequence's filled rows
// (num_records = len x row bytes): a read at or past that bound returns zeros
// without touching memory.  The ring reads ahead past a wave's last sub-tile
// and its last sub-tile may run past the sequence's end; those reads cost
// nothing this way, with no branch around the loads (a branch would make the
// compiler wait for the whole ring at every use).
constexpr uint32_t kNoRow = 0x80000000u;  // offset of a read that must not happen
constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format

// scales: (MXFP8) a buffer resource over the rows' E8M0 bytes, kGroups per
// row, in the same row order as `rows` (a row past the bound reads scale 0).
template <int KF>
__device__ __forceinline__ void load_key_tile(KeyTile<KF>& kt, __amdgpu_buffer_rsrc_t rows,
                                              __amdgpu_buffer_rsrc_t scales, uint32_t row_off, int lg) {
  if constexpr (KF == kKeyBF16) {  // 128 bf16 = 16 x 16 B
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      kt.v[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rows, row_off + 16 * (ks * 4 + lg), 0, 0));
  } else {  // 128 bytes = 8 x 16 B: dims 16 lg .. +16 and 64 + 16 lg .. +16
    const i32x4 a = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rows, row_off + 16 * lg, 0, 0));
    const i32x4 c = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rows, row_off + 64 + 16 * lg, 0, 0));
    kt.v = i32x8{a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
    if constexpr (KF == kKeyMX)  // scale of group lg of this row
      kt.sc = __builtin_amdgcn_raw_buffer_load_b8(scales, row_off / kDi * kGroups + lg, 0, 0);
  }
}

template <int TQ, int KF>
struct QRegs {
  i32x8 a[TQ][4];  // [token][head tile], 32 e4m3 codes
};
template <int TQ>
struct QRegs<TQ, kKeyBF16> {
  bf16x8 a[TQ][4][4];  // [token][head tile][k-step]
};
template <int TQ>
struct QRegs<TQ, kKeyMX> {
  i32x8 a[TQ][4];  // [token][head tile], 32 e4m3 codes
  int sc[TQ][4];   // [token][head tile]: E8M0 scale of this lane's head row and group
};

// ReLU on the bit pattern: a float with its sign bit set is a negative
// integer, so max(bits, 0) is x for x > 0 and +0 otherwise (-0 included), in
// one integer max.  fmaxf(x, 0) costs two float maxes on a matrix-core result
// (the first quiets a possible signalling NaN), and the epilogue's VALU time
// rivals the MFMA time in the two-token kernel.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

template <int TQ, int NSLOT, int KF, int MINB, int NT, bool PAGED>
__global__ __launch_bounds__(NT, MINB) void score_mfma_kernel(ScoreParams p) {
  const WgTrace wg_trace_(p.wg_trace);
  constexpr bool FP8 = KF != kKeyBF16, MX = KF == kKeyMX;
  constexpr int kScoreThreads = NT, kScoreWaves = NT / kWave;
  // Eight tokens per segment (bf16 keys, contiguous cache, many query
  // tokens): the workgroup's four waves take two tokens each and share every
  // key sub-tile through an LDS ring (see the segment body).
  constexpr bool KS = TQ == kSharedTokens;
  static_assert(!KS || (KF == kKeyBF16 && !PAGED && MINB == 1 && NT == 512), "shared-key variant: bf16, contiguous, 8 waves");
  constexpr int TW = KS ? TQ / kScoreWaves : 1;  // (shared-key variant) tokens per wave
  constexpr int kRing = KS ? ks_ring_slots(NT) : 1;
  // LDS histogram words per token: the shared-key variant packs two 16-bit
  // counters per word (bins 2i, 2i + 1), which leaves room for its key ring;
  // it flushes them at least every kPassUnits units, before one can overflow
  constexpr int kHistWords = KS ? kHistBins / 2 : kHistBins;
  // LDS: [TQ] index queries in operand order (bf16: 64 x 128 x 2 B; e4m3: 64 x 128 B),
  // then [TQ][kHistBins] histogram counters when p.hist.  Shared-key variant:
  // [TQ][kHistBins / 2] packed histogram counters, then the key ring.
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  __shared__ uint8_t s_qsc[MX ? TQ * kHi * kGroups : 4];  // (MXFP8) query group scales [TQ][head][group]
  constexpr int kQBytes = FP8 ? kHi * kDi : kHi * kDi * 2;
  uint8_t* lds_q = (uint8_t*)lds;
  uint32_t* lds_hist = lds + (KS ? 0 : TQ * kQBytes / 4);
  __shared__ int64_t s_total;
  __shared__ int64_t s_wsum[kScoreWaves];
  __shared__ int64_t s_excl[kScoreThreads];
  __shared__ int s_len[kScoreThreads];  // clamped length of each segment's sequence in the current chunk
  __shared__ int s_list[kScoreThreads];  // the segments of the current chunk this workgroup serves, in order
  __shared__ int s_wcnt[kScoreWaves];
  __shared__ int64_t s_hist_row;  // global histogram row of the current segment's first token

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int l = lane_id();
  const int lg = l >> 4;   // lane group 0..3
  const int lc = l & 15;   // column within a 16-wide tile
  const int n_groups = (p.T + TQ - 1) / TQ;
  const int n_seg = p.B * n_groups;

  // A segment's weight in the work split: its units of 64 positions plus
  // kSegCost for what every segment costs besides its units (its queries and
  // weights staged, the key ring filled, its histogram flushed), about 16
  // units' time.  (Without it a fresh 8192-token prompt gave its first
  // workgroup the first 256 token pairs, a unit or two each, and that
  // workgroup finished at 3.1 ms where the median one did at 0.9 ms.)  The
  // weight puts kSegCost virtual units in front of the segment's real ones.
  constexpr int64_t kSegCost = 16;
  auto seg_units_len = [&](int seg, int len) -> int64_t {
    const int g = seg % n_groups;
    const int t_last = min(g * TQ + TQ - 1, p.T - 1);
    const int64_t vis_end = (int64_t)len - p.T + 1 + t_last;
    return vis_end > 0 ? (vis_end + 63) / 64 + kSegCost : 0;
  };
  auto seg_units = [&](int seg) -> int64_t {
    return seg_units_len(seg, filled_rows(p.seq_lens[seg / n_groups], p.Lmax, p.len_sub));
  };

  // Pass 1: total units.  Segment tid's length and units are kept for the
  // first chunk of pass 2, which then starts without another memory round trip.
  const int len0 = tid < n_seg ? filled_rows(p.seq_lens[tid / n_groups], p.Lmax, p.len_sub) : 0;
  const int64_t units0 = tid < n_seg ? seg_units_len(tid, len0) : 0;
  int64_t acc = units0;
  for (int s = tid + kScoreThreads; s < n_seg; s += kScoreThreads) acc += seg_units(s);
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kWave);
  if (l == 0) s_wsum[wave] = acc;
  __syncthreads();
  if (tid == 0) {
    int64_t tot = 0;
    for (int w = 0; w < kScoreWaves; ++w) tot += s_wsum[w];
    s_total = tot;
  }
  __syncthreads();
  const int64_t U = s_total;
  if (U == 0) return;
  const int64_t G = gridDim.x;
  const int64_t wg = blockIdx.x;
  // Two ways to share a segment's units among workgroups, chosen per
  // segment from its size alone (so every workgroup takes the same choice):
  //  - a segment of at least 8 workgroups' shares U / G (a long sequence
  //    with few query tokens: decode) goes to the workgroups
  //    [wg_first, wg_end) its units start and end in, its 16-position
  //    sub-tiles round-robin over all their waves, so at any moment they
  //    read one window of consecutive rows (7 us faster than the exact split
  //    at 8 sequences x 128K keys);
  //  - a smaller one is split exactly: workgroup wg takes the units in
  //    [u_lo, u_hi), its own U / G share of all segments' units in order.
  //    (The round-robin ranges round to whole workgroups: with segments near
  //    one share, some workgroup got two whole segments and the launch took
  //    twice as long, 4096 prefill tokens over 64K keys split in 512-token
  //    launches 1.50 ms per launch against 0.79 ms exact.)
  auto wg_first = [&](int64_t start) -> int64_t { return start * G / U; };
  auto wg_end = [&](int64_t start, int64_t n) -> int64_t {
    return max(wg_first(start) + 1, (start + n) * G / U);
  };
  auto round_robin = [&](int64_t n) -> bool {
    return !KS && (p.split_mode == 1 || (p.split_mode == 0 && n * G >= 8 * U));
  };
  const int64_t u_lo = wg * U / G, u_hi = (wg + 1) * U / G;

  if (p.hist)
    for (int i = tid; i < TQ * kHistWords; i += kScoreThreads) lds_hist[i] = 0;

  // Pass 2: walk the segments in chunks of kScoreThreads, with an exclusive
  // scan of their unit counts, and process the segments this workgroup serves.
  int64_t chunk_base = 0;
  // (a chunk starting at or past u_hi can still hold a round-robin segment
  // that wg serves while wg_first(its start) <= wg, never past that)
  for (int c0 = 0; c0 < n_seg && wg_first(chunk_base) <= wg; c0 += kScoreThreads) {
    const int n_here = min(kScoreThreads, n_seg - c0);
    const int64_t mine = tid < n_here ? (c0 == 0 ? units0 : seg_units(c0 + tid)) : 0;
    if (tid < n_here) s_len[tid] = c0 == 0 ? len0 : filled_rows(p.seq_lens[(c0 + tid) / n_groups], p.Lmax, p.len_sub);
    int64_t v = mine;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int64_t y = __shfl_up(v, o, kWave);
      if (l >= o) v += y;
    }
    if (l == kWave - 1) s_wsum[wave] = v;
    __syncthreads();
    int64_t off = 0, chunk_total = 0;
#pragma unroll
    for (int w = 0; w < kScoreWaves; ++w) {
      if (w < wave) off += s_wsum[w];
      chunk_total += s_wsum[w];
    }
    s_excl[tid] = off + v - mine;
    // The segments this workgroup serves (those whose workgroup range holds
    // wg): every thread tests its own segment, and the hits are listed in
    // order.  (Testing them one after another, with a 64-bit division each,
    // held the workgroups of the last segments back for microseconds before
    // their first key load.)
    // wg_first(st) <= wg < wg_end(st, n), without the divisions:
    //   floor(st G / U) <= wg        <=>  st G < (wg + 1) U
    //   wg < floor(st G / U) + 1     <=>  wg U <= st G
    //   wg < floor((st + n) G / U)   <=>  (wg + 1) U <= (st + n) G
    bool serves = false;
    if (tid < n_here && mine > 0) {
      const int64_t st = chunk_base + off + v - mine;
      if (round_robin(mine))
        serves = st * G < (wg + 1) * U && (wg * U <= st * G || (wg + 1) * U <= (st + mine) * G);
      else
        serves = st < u_hi && st + mine > u_lo;
    }
    const uint64_t hits = __ballot(serves);
    if (l == 0) s_wcnt[wave] = __popcll(hits);
    __syncthreads();
    int n_list = 0, list_base = 0;
#pragma unroll
    for (int w = 0; w < kScoreWaves; ++w) {
      if (w < wave) list_base += s_wcnt[w];
      n_list += s_wcnt[w];
    }
    if (serves) s_list[list_base + __popcll(hits & ((1ull << l) - 1))] = tid;
    __syncthreads();

    for (int k = 0; k < n_list; ++k) {
      const int i = __builtin_amdgcn_readfirstlane(s_list[k]);  // (uniform: it selects the key buffer)
      const int64_t seg_start = chunk_base + s_excl[i];
      const int seg = c0 + i;
      const int64_t seg_w = (i + 1 < n_here ? s_excl[i + 1] : chunk_total) - s_excl[i];  // weight
      const int64_t seg_n = seg_w - kSegCost;  // real units (>= 1: the segment is served)
      // The segment's work is its seg_n units of 64 consecutive positions
      // (4 sub-tiles of 16).  This wave takes units id_0 + k stride (k = 0,
      // 1, ...) below u_end: round-robin over the `stride` waves of all the
      // segment's workgroups, or of this one's share under the exact split.
      // Round-robin keeps the waves reading one window of consecutive rows.
      const bool rr = round_robin(seg_w);
      int id_0, stride, u_end;
      if (rr) {
        const int64_t g0 = wg_first(seg_start), g1 = wg_end(seg_start, seg_w);
        stride = (int)((g1 - g0) * kScoreWaves);
        id_0 = (int)((wg - g0) * kScoreWaves + wave);
        u_end = (int)seg_n;
      } else {
        // this workgroup's share of the weight, less the virtual units
        const int64_t ua = max(max(seg_start, u_lo) - seg_start - kSegCost, (int64_t)0);
        const int64_t ub = max(min(seg_start + seg_w, u_hi) - seg_start - kSegCost, (int64_t)0);
        if (ub <= ua) continue;  // (uniform) only virtual units: nothing to do
        stride = kScoreWaves;
        id_0 = (int)ua + wave;
        u_end = (int)ub;
      }

      // ---------------- one segment: sequence b, tokens t0 .. t0+TQ-1 ----------------
      const int b = seg / n_groups;
      const int t0 = (seg % n_groups) * TQ;
      // (read back from LDS, so the compiler cannot tell it is uniform; the
      // key buffer resource built from it must sit in scalar registers)
      const int len = __builtin_amdgcn_readfirstlane(s_len[i]);
      const int vis_last = len - p.T + 1 + min(t0 + TQ - 1, p.T - 1);  // >= 1 here

      // (A counter handing units out to whichever wave is ready was tried
      // for round-robin segments: device-scope atomics on one address
      // serialise in memory across the XCDs, about 90 ns each, and 128K-key
      // decode went from 41 to 200 us.)
      constexpr int D = NSLOT / 4;  // units in the ring ahead of the current one
      // (wave-uniform: kept in scalar registers)
      id_0 = __builtin_amdgcn_readfirstlane(id_0);
      stride = __builtin_amdgcn_readfirstlane(stride);
      u_end = __builtin_amdgcn_readfirstlane(u_end);
      const int n_units = id_0 < u_end ? (u_end - id_0 + stride - 1) / stride : 0;  // this wave's
      auto unit_id = [&](int k) -> int { return id_0 + k * stride; };  // (< 2^25: positions fit int64 x 64)
      constexpr int kRowBytes = FP8 ? kDi : kDi * 2;
      const __amdgpu_buffer_rsrc_t krows = __builtin_amdgcn_make_buffer_rsrc(
          (void*)((const uint8_t*)p.k_idx + (int64_t)b * p.Lmax * kRowBytes), (short)0, len * kRowBytes, kBufferFlags);
      const __amdgpu_buffer_rsrc_t kscales =
          MX ? __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)p.k_scale + (int64_t)b * p.Lmax * kGroups),
                                                 (short)0, len * kGroups, kBufferFlags)
             : krows;
      const int last_row = len - 1;
      // the segment's histogram counters into the global histograms (after a
      // barrier); leaves them zero
      // (the histogram row is read back from LDS, after a barrier: a flush
      // inside the key loop must not keep eight row addresses in registers)
      if (tid == 0) s_hist_row = (int64_t)b * p.T + t0;
      auto flush_hist = [&]() {
        if (!p.hist) return;
        const int64_t row0 = s_hist_row;
        for (int tq = 0; tq < TQ; ++tq) {
          if (t0 + tq >= p.T) break;
          uint32_t* gh = p.hist + (row0 + tq) * kHistBins;
          for (int i = tid; i < kHistWords; i += kScoreThreads) {
            const uint32_t c = lds_hist[tq * kHistWords + i];
            if (c) {
              if constexpr (KS) {  // bins 2i (low half) and 2i + 1
                if (c & 0xFFFFu) atomicAdd(&gh[2 * i], c & 0xFFFFu);
                if (c >> 16) atomicAdd(&gh[2 * i + 1], c >> 16);
              } else {
                atomicAdd(&gh[i], c);
              }
              lds_hist[tq * kHistWords + i] = 0;
            }
          }
        }
      };

      if constexpr (KS) {
        // ---- keys shared through LDS ----
        // All eight waves walk the workgroup's units [u_a, u_end) of the
        // segment together.  Each unit's keys (64 rows, 16 KB) are copied into
        // a ring of kRingU unit slots in LDS once, by DMA (no registers), and
        // every wave multiplies them with its own token's queries, so one key
        // read feeds 8 tokens where the register ring feeds 2.  Per pair of
        // units k, k + 1: each wave waits for its own copies of them, then a
        // barrier (both are complete; every wave is done with the previous
        // pair), then the copies of units k + kRingU - 2 and k + kRingU - 1 go
        // into the previous pair's slots.  (Barriers per 16-row sub-tile made
        // the 512-token prefill tile's scores 517 us, per two sub-tiles 486,
        // per unit 482 and, with the later changes, per unit 418, per pair 404.)
        constexpr int kRingU = kRing / 4;  // the ring in units (4 sub-tiles, 16 KB)
        const int u_a = __builtin_amdgcn_readfirstlane(id_0 - wave);
        const int n_wg_units = u_end - u_a;  // >= 1
        const int n_sub = 4 * n_wg_units;
        uint8_t* ring = (uint8_t*)(lds_hist + TQ * kHistWords);
        const int tw = t0 + TW * wave;  // this wave's tokens tw .. tw + TW - 1
        // Lane l copies row 4 (wave % 4) + l/16 of a sub-tile, chunk (l%16) ^
        // row into chunk slot l%16 (rows 256 B apart; the XOR spreads the 16
        // rows a 16-lane read of one chunk touches over distinct banks).
        const int drow = 4 * (wave & 3) + (l >> 4);
        const uint8_t* kbase =
            (const uint8_t*)p.k_idx + (int64_t)b * p.Lmax * (kDi * 2) + (((l & 15) ^ drow) << 4);
        // The copy is written as asm, so the compiler does not see an LDS
        // write in flight: seeing one, it would make every LDS access in the
        // loop wait for all copies (the ring and the histograms share one
        // array).  The ring's own waits and barriers order the copies with the
        // reads.  (M0, which the instruction takes its LDS address from, is
        // restored in the block.)
        const uint32_t ring_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)ring;
        // Unit k's copies into unit slot us (sub-tile slots 4 us .. 4 us + 3):
        // wave w copies rows 4 (w % 4) + l/16 of its sub-tiles w/4 and w/4 + 2,
        // so every wave issues two of the unit's sixteen 1 KB copies.  (k past
        // the range re-copies the last unit: nobody reads it.)
        const int dsub = wave >> 2;
        auto dma_unit = [&](int k, int us) {
          const int64_t r0 = 64 * (int64_t)(u_a + min(k, n_wg_units - 1)) + drow;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int h = dsub + 2 * j;
            const int64_t row = min(r0 + 16 * h, (int64_t)last_row);
            uint32_t m0_saved;
            asm volatile(
                "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
                : "=&s"(m0_saved)
                : "s"(__builtin_amdgcn_readfirstlane(ring_base + (uint32_t)((us * 4 + h) * 4096 + (wave & 3) * 1024))),
                  "v"(kbase + row * (kDi * 2))
                : "memory");
          }
        };
        // operand A: this wave's TW tokens' queries, straight from memory
        // (head 16 ht + lc, dims 32 ks + 8 lg .. +8), and their head weights
        bf16x8 qa[TW][4][4];
        float w2[TW][4][4];
#pragma unroll
        for (int tq = 0; tq < TW; ++tq) {
          const int t = min(tw + tq, p.T - 1);
          const bf16x8* qrow = (const bf16x8*)((const uint16_t*)p.q_idx + ((int64_t)b * p.T + t) * kHi * kDi);
          const float* wrow = p.head_w + ((int64_t)b * p.T + t) * kHi;
#pragma unroll
          for (int ht = 0; ht < 4; ++ht) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) qa[tq][ht][ks] = qrow[(ht * 16 + lc) * (kDi / 8) + ks * 4 + lg];
#pragma unroll
            for (int e = 0; e < 4; ++e) w2[tq][ht][e] = wrow[ht * 16 + 4 * lg + e];
          }
        }
        // (pinned in accumulation registers, which the MFMA reads directly;
        // the ring's first copies go out after them, since the compiler's
        // wait for the queries would otherwise wait for the copies too)
#pragma unroll
        for (int tq = 0; tq < TW; ++tq)
#pragma unroll
          for (int ht = 0; ht < 4; ++ht)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) asm volatile("" : "+a"(qa[tq][ht][ks]));
#pragma unroll
        for (int k = 0; k < kRingU - 2; ++k) dma_unit(k, k);
        // this lane's operand-B read of chunk 4 ks + lg of row lc, within a slot
        uint32_t boff[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) boff[ks] = (uint32_t)(lc * 256 + (((4 * ks + lg) ^ lc) << 4));

        const bool upper = l >= 32, odd = (lg & 1) != 0;
        int uslot = 0;  // unit slot of the current unit (its index % kRingU)
        constexpr int RBK = 16;  // units per store batch
        static_assert(kRingU == 5 && RBK % 2 == 0, "a pair of units in use, one landed, two being copied");
        static_assert(kPassUnits % RBK == 0, "flushes fall between store batches");
        for (int u0 = 0; u0 < n_wg_units; u0 += RBK) {
          if (u0 > 0 && u0 % kPassUnits == 0) {  // (uniform; rare) flush the packed counters before they can overflow
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __syncthreads();
            flush_hist();
            __syncthreads();
          }
          float sbuf[TW][RBK];
#pragma unroll
          for (int ub = 0; ub < RBK; ++ub) {
            if (u0 + ub < n_wg_units) {  // (uniform over the workgroup)
              float part[TW][4];
              {
                // unit k = u0 + ub; at an even k, this wave's copies of units
                // k and k + 1 have landed (those of k + 2 may be in flight:
                // copies complete in order), barrier, then units k + 3 and
                // k + 4 go into the slots of k - 2 and k - 1
                if (ub % 2 == 0) {  // (u0 is even: units pair up as k, k + 1)
                  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * (kRingU - 4)) : "memory");
                  dma_unit(u0 + ub + kRingU - 2, uslot + kRingU - 2 >= kRingU ? uslot - 2 : uslot + kRingU - 2);
                  dma_unit(u0 + ub + kRingU - 1, uslot + kRingU - 1 >= kRingU ? uslot - 1 : uslot + kRingU - 1);
                }
                // operand B of the unit's four sub-tiles (plain LDS loads: the
                // compiler issues them together and waits for each just
                // before its first MFMA)
                bf16x8 kb[4][4];
#pragma unroll
                for (int h = 0; h < 4; ++h)
#pragma unroll
                  for (int ks = 0; ks < 4; ++ks) kb[h][ks] = *(const bf16x8*)(ring + (uslot * 4 + h) * 4096 + boff[ks]);
                uslot = uslot + 1 == kRingU ? 0 : uslot + 1;
                // Software-pipelined: sub-tile h's MFMAs are issued next to
                // the ReLU-weighted sums of sub-tile h - 1, which do not
                // depend on them, so the matrix core and the VALU overlap.
                f32x4 accp[TW][4];
                auto head_sums = [&](const f32x4 (&a)[TW][4], int st) {
#pragma unroll
                  for (int tq = 0; tq < TW; ++tq) {
                    float sacc = 0.0f;
#pragma unroll
                    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
                      for (int e = 0; e < 4; ++e) sacc = fmaf(w2[tq][ht][e], relu_bits(a[tq][ht][e]), sacc);
                    part[tq][st] = sacc;
                  }
                };
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                  f32x4 acc[TW][4];
#pragma unroll
                  for (int tq = 0; tq < TW; ++tq)
#pragma unroll
                    for (int ht = 0; ht < 4; ++ht) {
                      f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                      for (int ks = 0; ks < 4; ++ks)
                        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[tq][ht][ks], kb[h][ks], a, 0, 0, 0);
                      acc[tq][ht] = a;
                    }
                  if (h > 0) {
                    head_sums(accp, h - 1);
                    // (the schedule: each MFMA followed by two VALU instructions)
#pragma unroll
                    for (int i = 0; i < 16 * TW; ++i) {
                      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two VALU
                    }
                  }
#pragma unroll
                  for (int tq = 0; tq < TW; ++tq)
#pragma unroll
                    for (int ht = 0; ht < 4; ++ht) accp[tq][ht] = acc[tq][ht];
                }
                head_sums(accp, 3);
              }
              // reduce-scatter over the 4 lane groups: lane l gets column lc of sub-tile lg
              const int64_t pos = 64 * (int64_t)(u_a + u0 + ub) + 16 * lg + lc;
#pragma unroll
              for (int tq = 0; tq < TW; ++tq) {
                const float r0 = (upper ? part[tq][2] : part[tq][0]) +
                                 __shfl_xor(upper ? part[tq][0] : part[tq][2], 32, kWave);
                const float r1 = (upper ? part[tq][3] : part[tq][1]) +
                                 __shfl_xor(upper ? part[tq][1] : part[tq][3], 32, kWave);
                const float sc = (odd ? r1 : r0) + __shfl_xor(odd ? r0 : r1, 16, kWave);
                sbuf[tq][ub] = sc;
                if (p.hist && tw + tq < p.T && pos < (int64_t)len - p.T + 1 + tw + tq) {
                  const uint32_t bin = score_key(sc) >> kHistShift;
                  atomicAdd(&lds_hist[(TW * wave + tq) * kHistWords + (bin >> 1)], 1u << (16 * (bin & 1)));
                }
              }
            }
          }
          // store the batch, then let the stores complete: on this target
          // loads and stores share one completion counter, and the ring's
          // partial waits assume that only its copies are outstanding
#pragma unroll
          for (int ub = 0; ub < RBK; ++ub) {
            const int64_t pos = 64 * (int64_t)(u_a + u0 + ub) + 16 * lg + lc;
            if (u0 + ub < n_wg_units && pos < vis_last) {
#pragma unroll
              for (int tq = 0; tq < TW; ++tq)
                if (tw + tq < p.T) p.scores[((int64_t)b * p.T + tw + tq) * p.Lmax + pos] = sbuf[tq][ub];
            }
          }
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        // (the copies past the range have landed; the histogram adds are done)
        asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)" ::: "memory");
      } else {

      // Paged caches: a 16-row sub-tile never straddles a page (pages hold a
      // multiple of 64 rows), so each sub-tile's rows are read through a
      // buffer resource over its page.  The block-table entries of the
      // sub-tiles NSLOT ahead of the ring are loaded one ring's length before
      // they are needed (their wait then costs nothing: the ring's own waits
      // already cover them).
      const int64_t page_rows = PAGED ? ((int64_t)1 << p.page_shift) : 1;
      // (read as constant memory: with a uniform index these are scalar loads,
      // so the entries sit in scalar registers)
      typedef const __attribute__((address_space(4))) int32_t* const_i32p;
      const const_i32p btab = PAGED ? (const_i32p)(p.block_table + (int64_t)b * p.max_pages) : nullptr;
      // block-table entry of sub-tile st of the wave's unit k (clamped into the wave's units)
      auto page_entry = [&](int k, int st) -> int32_t {
        const int64_t pos = 64 * unit_id(min(k, max(n_units - 1, 0))) + 16 * st;
        return btab[__builtin_amdgcn_readfirstlane((int)min(pos >> p.page_shift, (int64_t)p.max_pages - 1))];
      };
      auto phys_page = [&](int32_t entry) -> int64_t { return min(max((int64_t)entry, (int64_t)0), p.num_pages - 1); };
      auto key_rsrc = [&](int32_t entry) -> __amdgpu_buffer_rsrc_t {
        if constexpr (!PAGED) {
          return krows;
        } else {
          const int64_t pp = phys_page(__builtin_amdgcn_readfirstlane(entry));
          return __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)p.k_idx + pp * page_rows * kRowBytes),
                                                   (short)0, (int)(page_rows * kRowBytes), kBufferFlags);
        }
      };
      auto scale_rsrc = [&](int32_t entry) -> __amdgpu_buffer_rsrc_t {  // (MXFP8) the scales of key_rsrc's rows
        if constexpr (!PAGED || !MX) {
          return kscales;
        } else {
          const int64_t pp = phys_page(__builtin_amdgcn_readfirstlane(entry));
          return __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)p.k_scale + pp * page_rows * kGroups),
                                                   (short)0, (int)(page_rows * kGroups), kBufferFlags);
        }
      };
      // offset of the key row this lane loads for sub-tile st of the wave's unit k
      auto st_off = [&](int k, int st) -> uint32_t {
        const int64_t pos = 64 * unit_id(k) + 16 * st + lc;
        const int64_t r = PAGED ? (pos & (page_rows - 1)) : pos;
        return (k < n_units && pos < len) ? (uint32_t)(r * kRowBytes) : kNoRow;
      };
      int32_t pg_cur[NSLOT], pg_next[NSLOT];  // (paged) entries of the slots' sub-tiles and of those NSLOT ahead

      // Key tiles stream through a ring of NSLOT sub-tile register slots,
      // filled first, before the queries are staged: the key stream starts
      // as soon as the segment is known and its latency hides the staging.  The
      // scores of RB units are kept in registers and stored together after
      // each batch: on this target loads and stores share one completion
      // counter, so any store inside the streaming loop would make every
      // iteration wait for all loads in flight.
      constexpr int RB = 8;
      static_assert((4 * RB) % NSLOT == 0 && NSLOT % 4 == 0, "ring must tile the batch");
      KeyTile<KF> slot[NSLOT];
      auto fill_ring = [&]() {
        if constexpr (PAGED) {
#pragma unroll
          for (int j = 0; j < NSLOT; ++j) pg_cur[j] = page_entry(j >> 2, j & 3);
#pragma unroll
          for (int j = 0; j < NSLOT; ++j) pg_next[j] = page_entry(D + (j >> 2), j & 3);
        }
#pragma unroll
        for (int j = 0; j < NSLOT; ++j)
          load_key_tile<KF>(slot[j], key_rsrc(pg_cur[j]), scale_rsrc(pg_cur[j]), st_off(j >> 2, j & 3), lg);
      };

      // head weights (used from the first unit on), then the index queries
      // -> LDS (e4m3: quantised) -> registers.  bf16: the query loads go out
      // first and the ring right behind them, so waiting for the queries does
      // not wait for the ring, and the LDS hand-over uses a bare barrier
      // (__syncthreads() would drain the ring): the first unit starts while
      // the ring is still arriving and its refills keep the stream going.
      // e4m3 (converted queries): the ring goes first.
      if constexpr (FP8) fill_ring();
      float w[TQ][4][4];
#pragma unroll
      for (int tq = 0; tq < TQ; ++tq) {
        const float* wrow = p.head_w + ((int64_t)b * p.T + min(t0 + tq, p.T - 1)) * kHi;
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
#pragma unroll
          for (int e = 0; e < 4; ++e) w[tq][ht][e] = wrow[ht * 16 + 4 * lg + e];
      }
      for (int tq = 0; tq < TQ; ++tq) {
        const int t = min(t0 + tq, p.T - 1);
        const int64_t qoff = ((int64_t)b * p.T + t) * kHi * kDi;
        if constexpr (!FP8) {
          constexpr int kVecs = kHi * kDi / 8 / kScoreThreads;  // 4 per thread, all loads issued first
          const i32x4* src = (const i32x4*)((const uint16_t*)p.q_idx + qoff);
          i32x4 x[kVecs];
#pragma unroll
          for (int k = 0; k < kVecs; ++k) x[k] = src[tid + k * kScoreThreads];
          if (tq == TQ - 1) {
            __builtin_amdgcn_sched_barrier(0);  // keep the query loads ahead of the ring
            fill_ring();
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int k = 0; k < kVecs; ++k) ((i32x4*)(lds_q + tq * kQBytes))[tid + k * kScoreThreads] = x[k];
        } else {
          // 4 consecutive values per word; all loads issued before converting
          constexpr int kWords = kHi * kDi / 4 / kScoreThreads;  // 8 per thread
          f32x4 x[kWords];
          if (p.q_dtype == kF32) {
            const f32x4* src = (const f32x4*)((const float*)p.q_idx + qoff);
#pragma unroll
            for (int k = 0; k < kWords; ++k) x[k] = src[tid + k * kScoreThreads];
          } else {
            const i32x2* src = (const i32x2*)((const uint16_t*)p.q_idx + qoff);
#pragma unroll
            for (int k = 0; k < kWords; ++k) {
              const i32x2 v = src[tid + k * kScoreThreads];
              x[k] = f32x4{bf16_bits_to_f32((uint32_t)v[0] & 0xFFFFu), bf16_bits_to_f32((uint32_t)v[0] >> 16),
                           bf16_bits_to_f32((uint32_t)v[1] & 0xFFFFu), bf16_bits_to_f32((uint32_t)v[1] >> 16)};
            }
          }
          // MXFP8: word tid + 256 k is word tid%8 of group (tid + 256 k)/8, so the
          // 8 words of a group sit in 8 neighbouring lanes: their largest
          // magnitude sets the group's shared exponent E = floor(log2 amax) - 8
          // (within E8M0's range) and the codes are of x / 2^E (OCP MX v1.0)
          float inv[kWords];
#pragma unroll
          for (int k = 0; k < kWords; ++k) {
            inv[k] = 1.0f;
            if constexpr (MX) {
              float m = fmaxf(fmaxf(fabsf(x[k][0]), fabsf(x[k][1])), fmaxf(fabsf(x[k][2]), fabsf(x[k][3])));
              m = fmaxf(m, __shfl_xor(m, 1, kWave));
              m = fmaxf(m, __shfl_xor(m, 2, kWave));
              m = fmaxf(m, __shfl_xor(m, 4, kWave));
              const int ef = (int)(__float_as_uint(m) >> 23);  // biased exponent (m >= 0)
              const int E = ef == 0 ? -127 : max(ef - 127 - 8, -127);
              inv[k] = __uint_as_float((uint32_t)(127 - E) << 23);  // 2^-E
              if ((tid & 7) == 0) s_qsc[tq * kHi * kGroups + (tid + k * kScoreThreads) / 8] = (uint8_t)(E + 127);
            }
          }
#pragma unroll
          for (int k = 0; k < kWords; ++k) {
            uint32_t word = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) word |= e4m3_code_exact(e4m3_quantize(x[k][e] * inv[k])) << (8 * e);
            ((uint32_t*)(lds_q + tq * kQBytes))[tid + k * kScoreThreads] = word;
          }
        }
      }
      if constexpr (FP8)
        __syncthreads();
      else
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      QRegs<TQ, KF> q;
#pragma unroll
      for (int tq = 0; tq < TQ; ++tq) {
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) {
          const uint8_t* qrow = lds_q + tq * kQBytes + (ht * 16 + lc) * (kQBytes / kHi);
          if constexpr (!FP8) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) q.a[tq][ht][ks] = ((const bf16x8*)qrow)[ks * 4 + lg];
          } else {  // dims 16 lg .. +16 and 64 + 16 lg .. +16
            const i32x4* r = (const i32x4*)qrow;
            const i32x4 x0 = r[lg], x1 = r[4 + lg];
            q.a[tq][ht] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
            if constexpr (MX) q.sc[tq][ht] = s_qsc[(tq * kHi + ht * 16 + lc) * kGroups + lg];
          }
        }
      }
      // One workgroup per CU gives a wave 256 arithmetic registers and 256
      // accumulation registers.  The queries (64 registers a token) are pinned
      // in the accumulation registers, which the matrix core reads its A
      // operand from directly: left to itself the compiler ran out of
      // arithmetic registers, parked them there anyway and copied each back
      // before every MFMA (1434 copies per batch of two-token prefill), and
      // kept every MFMA result in one accumulator tile, serialising them.
      if constexpr (MINB == 1 && NT == 256) {
#pragma unroll
        for (int tq = 0; tq < TQ; ++tq)
#pragma unroll
          for (int ht = 0; ht < 4; ++ht) {
            if constexpr (!FP8) {
#pragma unroll
              for (int ks = 0; ks < 4; ++ks) asm volatile("" : "+a"(q.a[tq][ht][ks]));
            } else {
              asm volatile("" : "+a"(q.a[tq][ht]));
            }
          }
      }

      const bool upper = l >= 32, odd = (lg & 1) != 0;
      for (int u0 = 0; u0 < n_units; u0 += RB) {
        float sbuf[TQ][RB];
#pragma unroll
        for (int ub = 0; ub < RB; ++ub) {
          const bool live = u0 + ub < n_units;
          // this unit's position for lane l, and (e4m3 keys) its row scale, loaded
          // before the ring refills so waiting for it does not drain them
          // after the reduce-scatter lane l holds position lc of its sub-tile lg
          const int64_t pos = 64 * unit_id(u0 + ub) + 16 * lg + lc;
          float kscale = 1.0f;
          const float* k_scale = (const float*)p.k_scale;
          if constexpr (KF == kKeyE4M3 && !PAGED) {
            kscale = k_scale[(int64_t)b * p.Lmax + (pos < len ? pos : last_row)];
          } else if constexpr (KF == kKeyE4M3) {
            // this lane's sub-tile lg of the unit sits in slot (4 ub + lg) % NSLOT (u0 is a multiple of NSLOT)
            const int s0 = (4 * ub) % NSLOT;
            const int32_t e = lg == 0 ? pg_cur[s0] : lg == 1 ? pg_cur[s0 + 1] : lg == 2 ? pg_cur[s0 + 2] : pg_cur[s0 + 3];
            kscale = k_scale[phys_page(e) * page_rows + (pos < len ? (pos & (page_rows - 1)) : 0)];
          }
          float part[TQ][4];
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const int j = (ub * 4 + st) % NSLOT;
            if (live) {
              // every head tile's MFMA chain first, each into its own
              // accumulator (the chains overlap in the matrix core), then
              // the ReLU-weighted head sums
              f32x4 acc[TQ][4];
#pragma unroll
              for (int tq = 0; tq < TQ; ++tq) {
#pragma unroll
                for (int ht = 0; ht < 4; ++ht) {
                  f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
                  if constexpr (!FP8) {
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                      a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q.a[tq][ht][ks], slot[j].v[ks], a, 0, 0, 0);
                  } else if constexpr (!MX) {  // unit operand scales (E8M0 127 = 1)
                    a = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(q.a[tq][ht], slot[j].v, a, 0, 0, 0,
                                                                         127, 0, 127);
                  } else {
                    a = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(q.a[tq][ht], slot[j].v, a, 0, 0, 0,
                                                                         q.sc[tq][ht], 0, slot[j].sc);
                  }
                  acc[tq][ht] = a;
                }
              }
#pragma unroll
              for (int tq = 0; tq < TQ; ++tq) {
                float sacc = 0.0f;
#pragma unroll
                for (int ht = 0; ht < 4; ++ht)
#pragma unroll
                  for (int e = 0; e < 4; ++e) sacc = fmaf(w[tq][ht][e], relu_bits(acc[tq][ht][e]), sacc);
                part[tq][st] = sacc;
              }
            }
            // refill this slot with the same sub-tile of unit k + D (nothing
            // is read past the wave's units or the sequence's end)
            if constexpr (PAGED) pg_cur[j] = pg_next[j];
            load_key_tile<KF>(slot[j], key_rsrc(pg_cur[j]), scale_rsrc(pg_cur[j]), st_off(u0 + ub + D, st), lg);
            if constexpr (PAGED) pg_next[j] = page_entry(u0 + ub + 2 * D, st);
          }
          if (live) {
            // reduce-scatter over the 4 lane groups: lane l gets column lc of sub-tile lg
#pragma unroll
            for (int tq = 0; tq < TQ; ++tq) {
              const float r0 = (upper ? part[tq][2] : part[tq][0]) +
                               __shfl_xor(upper ? part[tq][0] : part[tq][2], 32, kWave);
              const float r1 = (upper ? part[tq][3] : part[tq][1]) +
                               __shfl_xor(upper ? part[tq][1] : part[tq][3], 32, kWave);
              float sc = (odd ? r1 : r0) + __shfl_xor(odd ? r0 : r1, 16, kWave);
              if constexpr (KF == kKeyE4M3) sc *= kscale;
              sbuf[tq][ub] = sc;
              if (p.hist && t0 + tq < p.T && pos < (int64_t)len - p.T + 1 + t0 + tq)
                atomicAdd(&lds_hist[tq * kHistBins + (score_key(sc) >> kHistShift)], 1u);
            }
          }
        }
        // store the batch
#pragma unroll
        for (int ub = 0; ub < RB; ++ub) {
          const int64_t pos = 64 * unit_id(u0 + ub) + 16 * lg + lc;
          if (u0 + ub < n_units && pos < vis_last) {
#pragma unroll
            for (int tq = 0; tq < TQ; ++tq)
              if (t0 + tq < p.T) p.scores[((int64_t)b * p.T + t0 + tq) * p.Lmax + pos] = sbuf[tq][ub];
          }
        }
      }
      }  // register ring
      __syncthreads();  // all waves done with lds_q or the key ring (and their histogram updates)
      if (p.hist) {
        flush_hist();
        __syncthreads();
      }
    }
    chunk_base += chunk_total;
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
bool score_mfma_supported(const ScoreParams& p) {
  if (p.Hi != kHi || p.Di != kDi) return false;
  // key rows are addressed by 32-bit byte offsets within a sequence
  const int64_t row_bytes = p.k_dtype == kBF16 ? 2 * kDi : kDi;
  if (!p.block_table && (int64_t)p.Lmax * row_bytes >= (int64_t)kNoRow) return false;  // (paged: one page at a time)
  if (p.k_dtype == kBF16) return p.q_dtype == kBF16;
  return p.k_dtype == kE4M3 || p.k_dtype == kMXE4M3;
}

template <int TQ, int NSLOT, int KF, int MINB, int NT, bool PAGED>
static void launch_mfma_k(const ScoreParams& p_in, int grid, hipStream_t stream, hipEvent_t ev_start,
                          hipEvent_t ev_stop) {
  constexpr int kQBytes = KF != kKeyBF16 ? kHi * kDi : kHi * kDi * 2;
  size_t lds = TQ * kQBytes + (p_in.hist ? TQ * kHistBins * sizeof(uint32_t) : 0);
  if constexpr (TQ == kSharedTokens) {  // histograms, then the key ring
    lds = TQ * kHistBins * sizeof(uint16_t) + ks_ring_slots(NT) * 4096;
  }
  ScoreParams p = p_in;
  p.wg_trace = trace_region(kTraceScore, grid);
  if (ev_start || ev_stop)  // events taken by the dispatch itself at the kernel's start and end
    hipExtLaunchKernelGGL((score_mfma_kernel<TQ, NSLOT, KF, MINB, NT, PAGED>), dim3(grid), dim3(NT), lds, stream,
                          ev_start, ev_stop, 0, p);
  else
    hipLaunchKernelGGL((score_mfma_kernel<TQ, NSLOT, KF, MINB, NT, PAGED>), dim3(grid), dim3(NT), lds, stream, p);
}

template <int TQ, int NSLOT, int KF, int MINB = 2, int NT = 256>
static void launch_mfma(const ScoreParams& p, int grid, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (p.block_table)
    launch_mfma_k<TQ, NSLOT, KF, MINB, NT, true>(p, grid, stream, ev_start, ev_stop);
  else
    launch_mfma_k<TQ, NSLOT, KF, MINB, NT, false>(p, grid, stream, ev_start, ev_stop);
}

static int env_int(const char* name, int dflt) {
  const char* e = getenv(name);
  return (e && *e) ? atoi(e) : dflt;
}

// Launch shape: DSA_SCORE_VARIANT selects the bf16 key-prefetch depth,
// tokens per segment and occupancy (0, the default: one token, rings of 4
// sub-tiles, two workgroups per CU, so two waves per SIMD interleave their
// loads and MFMAs, or for short rows rings of 8 at one workgroup per CU;
// two tokens and one workgroup per CU when there are several query tokens.
// 1: rings of 8 sub-tiles at one per CU; 2: 8 waves; 3 / 4: two / four
// tokens; 5: rings of 4 at two per CU whatever the rows), and
// DSA_SCORE_WGS_PER_CU overrides the workgroups per CU and DSA_SCORE_WGS
// the total.  (Measured at the 128K decode shape: variant 0 at 2/CU streams
// the keys about 5 % faster than variant 1 at 1/CU.)
// The matrix-core kernel and grid launch_score takes for p (shared with the
// diagnostics that name the launch).
enum ScoreKernel {
  kSkBf16R8, kSkBf16W8, kSkBf16T2, kSkBf16T4, kSkBf16R4, kSkE4m3T1, kSkE4m3T2, kSkMxT1, kSkMxT2, kSkBf16S8
};
struct ScoreLaunch {
  ScoreKernel kernel;
  int grid;
};

static ScoreLaunch score_launch_plan(const ScoreParams& p, int num_cus) {
  const int variant = env_int("DSA_SCORE_VARIANT", 0);
  // two workgroups per CU (bf16 variants 1 and 2: one, with 8-deep rings or 8 waves)
  const int per_cu = (p.k_dtype != kBF16 || variant == 0) ? 2 : 1;
  int grid = max(1, env_int("DSA_SCORE_WGS_PER_CU", per_cu)) * num_cus;
  if (env_int("DSA_SCORE_WGS", 0) > 0) grid = env_int("DSA_SCORE_WGS", 0);
  if (p.k_dtype == kBF16) {
    switch (variant) {
      case 1: return {kSkBf16R8, grid};
      case 2: return {kSkBf16W8, grid};
      case 3: return {kSkBf16T2, grid};
      case 4: return {kSkBf16T4, grid};
      case 5: return {kSkBf16R4, 2 * num_cus};
      default:
        // eight or more query tokens (contiguous cache): eight per segment,
        // each key sub-tile shared by the workgroup's four waves through LDS
        if (p.T >= kSharedTokens && !p.block_table)
          return {kSkBf16S8, env_int("DSA_SCORE_WGS", 0) > 0 ? grid : num_cus};
        // several query tokens: two per segment, so each key tile feeds twice
        // the MFMAs (12 % faster at 4096 tokens over 64K keys; four tokens
        // need one workgroup per CU and were slower)
        if (p.T >= 2) return {kSkBf16T2, num_cus};
        // one token per sequence: two workgroups per CU, unless each would
        // stream fewer than 16 units (the rows are short and the start-up
        // dominates): then one per CU with 8-deep rings (32 sequences of 8K:
        // 22.4 against 25.3 us; 8 of 128K: 47.1 against 49.7 us the other
        // way round)
        if ((int64_t)p.B * (p.Lmax / 64 + 16) < (int64_t)16 * grid) return {kSkBf16R8, num_cus};
        return {kSkBf16R4, grid};
    }
  }
  if (p.k_dtype == kE4M3) return {p.T == 1 ? kSkE4m3T1 : kSkE4m3T2, grid};
  // (two tokens with their group scales need more than half the registers:
  // one workgroup per CU)
  return p.T == 1 ? ScoreLaunch{kSkMxT1, grid} : ScoreLaunch{kSkMxT2, num_cus};
}

int score_launch_desc(const ScoreParams& p, int num_cus, char* buf, size_t len) {
  if (!score_mfma_supported(p)) return snprintf(buf, len, "generic");
  // keys, query tokens per segment, key ring depth (16-row sub-tiles), waves per workgroup
  static const char* const names[] = {
      "bf16 keys, 1 token, ring 8, 4 waves",  "bf16 keys, 1 token, ring 4, 8 waves",
      "bf16 keys, 2 tokens, ring 4, 4 waves", "bf16 keys, 4 tokens, ring 4, 4 waves",
      "bf16 keys, 1 token, ring 4, 4 waves",  "e4m3 keys, 1 token, ring 8, 4 waves",
      "e4m3 keys, 2 tokens, ring 4, 4 waves", "mxfp8 keys, 1 token, ring 8, 4 waves",
      "mxfp8 keys, 2 tokens, ring 4, 4 waves", "bf16 keys, 8 tokens, shared LDS ring 20, 8 waves"};
  const ScoreLaunch l = score_launch_plan(p, num_cus);
  return snprintf(buf, len, "mfma(%s; %d workgroups)", names[l.kernel], l.grid);
}

hipError_t launch_score(const ScoreParams& p_in, bool allow_mfma, int num_cus, hipStream_t stream,
                        hipEvent_t ev_start, hipEvent_t ev_stop) {
  ScoreParams p = p_in;
  p.split_mode = env_int("DSA_SCORE_SPLIT", 0);  // (tests run both splits on small problems)
  p.wg_trace = nullptr;
  if (allow_mfma && score_mfma_supported(p)) {
    const ScoreLaunch l = score_launch_plan(p, num_cus);
    switch (l.kernel) {
      case kSkBf16R8: launch_mfma<1, 8, kKeyBF16, 1>(p, l.grid, stream, ev_start, ev_stop); break;
      case kSkBf16W8: launch_mfma<1, 4, kKeyBF16, 1, 512>(p, l.grid, stream, ev_start, ev_stop); break;
      case kSkBf16T2: launch_mfma<2, 4, kKeyBF16, 1>(p, l.grid, stream, ev_start, ev_stop); break;
      case kSkBf16T4: launch_mfma<4, 4, kKeyBF16, 1>(p, l.grid, stream, ev_start, ev_stop); break;
      case kSkBf16R4: launch_mfma<1, 4, kKeyBF16, 2>(p, l.grid, stream, ev_start, ev_stop); break;
      case kSkE4m3T1: launch_mfma<1, 8, kKeyE4M3>(p, l.grid, stream, ev_start, ev_stop); break;
      case kSkE4m3T2: launch_mfma<2, 4, kKeyE4M3>(p, l.grid, stream, ev_start, ev_stop); break;
      case kSkMxT1: launch_mfma<1, 8, kKeyMX>(p, l.grid, stream, ev_start, ev_stop); break;
      case kSkMxT2: launch_mfma<2, 4, kKeyMX, 1>(p, l.grid, stream, ev_start, ev_stop); break;
      case kSkBf16S8: {
        constexpr size_t lds = kSharedTokens * kHistBins * sizeof(uint16_t) + ks_ring_slots(kSharedThreads) * 4096;
        const hipError_t e = set_max_dynamic_lds(
            (const void*)score_mfma_kernel<kSharedTokens, 4, kKeyBF16, 1, kSharedThreads, false>, (int)lds);
        if (e != hipSuccess) return e;
        launch_mfma_k<kSharedTokens, 4, kKeyBF16, 1, kSharedThreads, false>(p, l.grid, stream, ev_start, ev_stop);
        break;
      }
    }
  } else {
    dim3 grid((unsigned)((p.Lmax + 255) / 256), (unsigned)(p.B * p.T));
    hipLaunchKernelGGL(score_generic_kernel, grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace dsa
