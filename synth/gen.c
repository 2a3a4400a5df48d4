/*
 * Seeded synthetic input generator for the indexed-sparse-attention (DSA)
 * workloads.  Test and benchmark infrastructure: it holds none of the
 * method's arithmetic (no score, selection or attention step), only the
 * recipes that fill input tensors with reproducible pseudo-random values.
 *
 * Every value is a pure function of (seed, tensor_id, flat_index): the
 * i-th output of a SplitMix64 stream whose state starts at
 * h = mix(seed * 0x100000001B3 + tensor_id).  SplitMix64 (Steele, Lea and
 * Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014)
 * advances its state by the odd constant 0x9E3779B97F4A7C15 and returns a
 * mixed copy of it, so output i is mix(h + (i + 1) * 0x9E3779B97F4A7C15)
 * and any element can be produced independently of the others.
 *
 * Output encodings (the bytes both the GPU path and the oracle read):
 *   f32   IEEE binary32
 *   bf16  upper half of binary32 after round-to-nearest-even
 *   e4m3  OCP FP8 E4M3 ("fn": bias 7, no infinities, max 448), produced by
 *         searching the 127 non-negative finite codes for the nearest value
 *         (ties to the even code), saturating at +-448.
 *
 * Built as a shared library and driven from synth/__init__.py via ctypes.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_base(uint64_t seed, uint64_t tensor_id) {
  return mix64(seed * 0x100000001B3ULL + tensor_id);
}

/* i-th SplitMix64 output of the stream whose state starts at h. */
static inline uint64_t draw(uint64_t h, uint64_t i) { return mix64(h + (i + 1) * GOLDEN); }

/* Integer uniform on [lo, hi] by multiply-shift of the upper 32 bits. */
static inline int64_t draw_int(uint64_t h, uint64_t i, int64_t lo, int64_t hi) {
  uint64_t span = (uint64_t)(hi - lo + 1);
  return lo + (int64_t)(((draw(h, i) >> 32) * span) >> 32);
}

/* Uniform in (0, 1): 53 random bits, offset by half an ulp so 0 never occurs. */
static inline double draw_open01(uint64_t h, uint64_t i) {
  return ((double)(draw(h, i) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

/* Standard normal by the Box-Muller transform from draws 2i and 2i+1. */
static inline double draw_normal(uint64_t h, uint64_t i) {
  double u1 = draw_open01(h, 2 * i), u2 = draw_open01(h, 2 * i + 1);
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* Value of a non-negative finite e4m3 code (0..126). */
static double e4m3_code_value(int c) {
  int e = (c >> 3) & 15, m = c & 7;
  if (e == 0) return ldexp((double)m, -9);
  return ldexp(8.0 + m, e - 10);
}

static double g_e4m3_pos[127];
static int g_e4m3_ready = 0;

static void e4m3_table(void) {
  if (g_e4m3_ready) return;
  for (int c = 0; c < 127; ++c) g_e4m3_pos[c] = e4m3_code_value(c);
  g_e4m3_ready = 1;
}

static uint8_t e4m3_encode_rne_sat(double x) {
  uint8_t sign = (x < 0) ? 0x80 : 0x00;
  double a = fabs(x);
  if (!(a < 448.0)) return sign | 0x7E; /* saturate (NaN inputs never occur here) */
  int lo = 0, hi = 126;                  /* largest code with value <= a */
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if (g_e4m3_pos[mid] <= a) lo = mid; else hi = mid - 1;
  }
  int c = lo;
  if (c < 126) {
    double dl = a - g_e4m3_pos[c], dh = g_e4m3_pos[c + 1] - a;
    if (dh < dl || (dh == dl && (c & 1))) c = c + 1;
  }
  return sign | (uint8_t)c;
}

/* ---------------------------------------------------------------------- */
/* Exported fillers.  dtype: 0 = f32, 1 = bf16, 2 = e4m3 (and 3, 4: e4m3 */
/* codes of the scaled formats, whose scales are filled separately).      */
/* ---------------------------------------------------------------------- */

static void store(void* out, int dtype, int64_t i, double v) {
  if (dtype == 0) ((float*)out)[i] = (float)v;
  else if (dtype == 1) ((uint16_t*)out)[i] = f32_to_bf16_rne((float)v);
  else ((uint8_t*)out)[i] = e4m3_encode_rne_sat(v);
}

/* Integers uniform on [lo, hi], stored exactly in the given dtype. */
void synth_fill_int(void* out, int dtype, int64_t n, uint64_t seed, uint64_t tensor_id,
                    int64_t lo, int64_t hi) {
  uint64_t h = stream_base(seed, tensor_id);
  if (dtype == 2) e4m3_table();
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) store(out, dtype, i, (double)draw_int(h, (uint64_t)i, lo, hi));
}

/* Standard normal samples, rounded into the dtype (f32 or bf16). */
void synth_fill_normal(void* out, int dtype, int64_t n, uint64_t seed, uint64_t tensor_id) {
  uint64_t h = stream_base(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) store(out, dtype, i, draw_normal(h, (uint64_t)i));
}

/* int32 uniform on [lo, hi]. */
void synth_fill_i32(int32_t* out, int64_t n, uint64_t seed, uint64_t tensor_id, int64_t lo,
                    int64_t hi) {
  uint64_t h = stream_base(seed, tensor_id);
  for (int64_t i = 0; i < n; ++i) out[i] = (int32_t)draw_int(h, (uint64_t)i, lo, hi);
}

/*
 * Per-row power-of-two scales 2^e, e uniform on [elo, ehi], one per row.
 * scale_out: n_rows floats.
 */
void synth_fill_pow2_scale(float* scale_out, int64_t n_rows, uint64_t seed, uint64_t tensor_id,
                           int elo, int ehi) {
  uint64_t h = stream_base(seed, tensor_id);
  for (int64_t r = 0; r < n_rows; ++r)
    scale_out[r] = (float)ldexp(1.0, (int)draw_int(h, (uint64_t)r, elo, ehi));
}

/*
 * e4m3 codes of x / scale[row] with x ~ N(0,1): the stored code times the
 * row's scale approximates the normal sample.  codes: n_rows * row_len bytes.
 */
void synth_fill_normal_e4m3_scaled(uint8_t* codes, const float* scale, int64_t n_rows,
                                   int64_t row_len, uint64_t seed, uint64_t tensor_id) {
  uint64_t h = stream_base(seed, tensor_id);
  e4m3_table();
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    double inv = 1.0 / (double)scale[r];
    for (int64_t j = 0; j < row_len; ++j) {
      int64_t i = r * row_len + j;
      codes[i] = e4m3_encode_rne_sat(draw_normal(h, (uint64_t)i) * inv);
    }
  }
}

/*
 * As above with one scale per tile of `tile` consecutive values of a row:
 * value j of row r is divided by scale[r * ceil(row_len / tile) + j / tile].
 */
void synth_fill_normal_e4m3_tiled(uint8_t* codes, const float* scale, int64_t n_rows,
                                  int64_t row_len, int64_t tile, uint64_t seed, uint64_t tensor_id) {
  uint64_t h = stream_base(seed, tensor_id);
  const int64_t nt = (row_len + tile - 1) / tile;
  e4m3_table();
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    for (int64_t j = 0; j < row_len; ++j) {
      int64_t i = r * row_len + j;
      codes[i] = e4m3_encode_rne_sat(draw_normal(h, (uint64_t)i) / (double)scale[r * nt + j / tile]);
    }
  }
}

/* Raw 64-bit draws, exposed so tests can check the stream definition. */
void synth_raw(uint64_t* out, int64_t n, uint64_t seed, uint64_t tensor_id) {
  uint64_t h = stream_base(seed, tensor_id);
  for (int64_t i = 0; i < n; ++i) out[i] = draw(h, (uint64_t)i);
}

/* Outputs 0..n-1 of a SplitMix64 generator whose state starts at `state`
 * (exposed so tests can check the stream against published values). */
void synth_splitmix64_from_state(uint64_t state, int64_t n, uint64_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = draw(state, (uint64_t)i);
}
