/*
 * CPU oracle for indexed sparse attention (DSA).  TEST INFRASTRUCTURE ONLY:
 * only tests, the smoke check and the benchmark's CPU-baseline leg may call
 * it.  It shares no code, header, table or helper with the GPU library.
 *
 * Plain and slow on purpose: fp64 direct loops, a full sort for Top-K and a
 * two-pass softmax, each step written as the definition it follows.  Work is
 * split over OpenMP threads by query (b, t) and head; the arithmetic of each
 * output is a single serial loop.
 *
 * What is computed (DSA as the pages describe it; the readings taken where
 * they are silent are listed with each function):
 *
 *   1. indexer scores   "Optimizing Next-Gen LLM Inference" §3.1 and
 *      "Inference Acceleration for New Large Model Architectures" §3.1:
 *      per-head query/key relevance, then a head-weighted aggregation.
 *      Reading: S[s] = sum_h w_h * max(0, sum_i qi[h,i] * k[s,i]).
 *   2. Top-K            same sections: keep the K most relevant historical
 *      positions.  Reading: ties go to the lower position; if fewer than K
 *      positions are visible, all of them are kept.
 *   3. sparse attention "Optimization and Deployment Practices for
 *      Next-Generation Sparse Attention LLMs" §1 and "Long-Context LLM
 *      Inference Optimization" (architecture section): attention of the MLA
 *      query over only the selected latent-cache rows.  Reading: logits
 *      z_j = scale * q . c[idx_j] over all qk_dim columns, values are the
 *      first v_dim columns of the same rows.
 *
 * Visibility: the T query tokens of a sequence are its last T filled rows;
 * token t sees positions 0 .. len - T + t (causal).
 *
 * Input encodings (decoded here with our own bit-field decoders):
 *   dtype 0 = IEEE f32, 1 = bf16, 2 = OCP FP8 E4M3 (bias 7, no inf, max 448),
 *   3 = MXFP8: E4M3 elements with one E8M0 scale byte per 32 consecutive
 *       elements of a row (index keys),
 *   4 = E4M3 elements with one fp32 scale per 128 consecutive elements of a
 *       row (latent rows).
 * dtype 2 carries one scale per row ("Inference Acceleration ..." §4.1/§4.2
 * describe group scales; one scale per row is the case where every group of a
 * row shares its scale); with such index keys the index query is quantised to
 * E4M3 (round to nearest even, saturating at +-448) before the dot product, as
 * that page's §4.1 quantises both index Q and K.  dtype 3 and 4 are the
 * pages' own granularities: groups of 32 for index Q and K (§4.1 there, and
 * "Layered Quantization" on the page "Long-Context LLM Inference
 * Optimization", which names MXFP8), tiles of 128 per token for the main
 * cache (§4.2 there).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t batch, q_len;
  int64_t max_seq_len;
  int32_t idx_heads, idx_dim;
  int32_t heads, qk_dim, v_dim;
  int32_t top_k;
  double softmax_scale;
  int32_t q_idx_dtype, idx_key_dtype, q_dtype, kv_dtype;
} oracle_dims;

/* ---------------- decoders (the formats' definitions) ---------------- */

/* OpenMP threads the oracle's parallel loops use. */
int oracle_num_threads(void) { return omp_get_max_threads(); }

double oracle_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16; /* bf16 is the upper half of binary32 */
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* E4M3: s eeee mmm; e == 0 subnormal m * 2^-9; e in 1..15: (1 + m/8) 2^(e-7);
 * s 1111 111 is NaN; there are no infinities. */
double oracle_e4m3_value(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 0xF, m = c & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* Nearest E4M3 value to x, ties to even mantissa, |x| >= 448 saturates. */
double oracle_e4m3_quantize(double x) {
  double a = fabs(x), best = 0.0;
  int best_code = 0;
  if (a >= 448.0) return x < 0 ? -448.0 : 448.0;
  for (int code = 0; code <= 0x7E; ++code) { /* all non-negative finite values */
    double v = oracle_e4m3_value((uint8_t)code);
    double d = fabs(v - a), db = fabs(best - a);
    if (d < db || (d == db && (code & 1) == 0 && (best_code & 1) == 1)) {
      best = v;
      best_code = code;
    }
  }
  return x < 0 ? -best : best;
}

/* E8M0 (the MX scale format): an unsigned biased exponent, value 2^(e-127);
 * 0xFF is NaN. */
double oracle_e8m0_value(uint8_t e) { return e == 0xFF ? NAN : ldexp(1.0, (int)e - 127); }

/*
 * MX quantisation of one group of n <= 32 values to E4M3 elements and a
 * shared E8M0 scale, following the conversion the OCP Microscaling (MX)
 * Formats Specification v1.0 gives: the shared exponent is floor(log2 of the
 * group's largest magnitude) minus the exponent of the element format's
 * largest power of two (8 for E4M3, whose largest normal is 1.75 * 2^8), kept
 * within E8M0's range; each element is the nearest E4M3 value of v / 2^shared,
 * saturating.  An all-zero group gets the smallest scale and zero elements.
 * Outputs the scale byte and the element values (E4M3 values, not codes).
 * Values must be finite.
 */
void oracle_mx_quantize(const double* v, int n, uint8_t* scale, double* elem) {
  double amax = 0.0;
  for (int i = 0; i < n; ++i)
    if (fabs(v[i]) > amax) amax = fabs(v[i]);
  int shared = -127;
  if (amax > 0.0) {
    int ex;
    frexp(amax, &ex); /* amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1 */
    shared = (ex - 1) - 8;
    if (shared < -127) shared = -127;
    if (shared > 127) shared = 127;
  }
  *scale = (uint8_t)(shared + 127);
  for (int i = 0; i < n; ++i) elem[i] = oracle_e4m3_quantize(ldexp(v[i], -shared));
}

/* Element value of a stored input (dtypes 3 and 4 store E4M3 codes). */
static double load(const void* p, int dtype, int64_t i) {
  switch (dtype) {
    case 0: return (double)((const float*)p)[i];
    case 1: return oracle_bf16_value(((const uint16_t*)p)[i]);
    default: return oracle_e4m3_value(((const uint8_t*)p)[i]);
  }
}

/* Decoded value of column i of row r of a latent cache with Dqk columns:
 * the element times its scale (per row for dtype 2, per 128-column tile for
 * dtype 4, none otherwise). */
static double kv_value(const void* kv, int dtype, const float* kv_scale, int64_t r, int Dqk, int i) {
  double v = load(kv, dtype, r * Dqk + i);
  if (dtype == 2) return v * (double)kv_scale[r];
  if (dtype == 4) return v * (double)kv_scale[r * ((Dqk + 127) / 128) + i / 128];
  return v;
}

static int64_t visible(const oracle_dims* d, const int32_t* seq_lens, int b, int t) {
  int64_t len = seq_lens[b];
  if (len > d->max_seq_len) len = d->max_seq_len;
  return len - d->q_len + 1 + t;
}

/* ---------------- 1. indexer scores ---------------- */
/*
 * scores: [B, T, Lmax] fp64; entries s >= vis are set to NaN (not visible).
 * k_scale: NULL for f32/bf16 keys; fp32 [B, Lmax] (one scale per key row) for
 * dtype 2; E8M0 bytes [B, Lmax, ceil(Di/32)] for dtype 3 (MXFP8), with which
 * each index query head is MX-quantised per group of 32 (oracle_mx_quantize)
 * and the dot product is that of the two dequantised vectors.
 * Only queries with want[b*T+t] != 0 are computed (want == NULL: all).
 */
int oracle_index_scores(const oracle_dims* d, const void* q_idx, const float* head_w,
                        const void* k_idx, const void* k_scale, const int32_t* seq_lens,
                        const uint8_t* want, double* scores) {
  const int B = d->batch, T = d->q_len, Hi = d->idx_heads, Di = d->idx_dim;
  const int64_t L = d->max_seq_len;
  const int kd = d->idx_key_dtype, G = (Di + 31) / 32;
  double* qd = (double*)malloc(sizeof(double) * Hi * Di);
  double* grp = (double*)malloc(sizeof(double) * 32);
  for (int b = 0; b < B; ++b) {
    for (int t = 0; t < T; ++t) {
      int64_t bt = (int64_t)b * T + t;
      double* out = scores + bt * L;
      if (want && !want[bt]) continue;
      int64_t vis = visible(d, seq_lens, b, t);
      for (int h = 0; h < Hi; ++h)
        for (int i = 0; i < Di; ++i) {
          double v = load(q_idx, d->q_idx_dtype, (bt * Hi + h) * Di + i);
          qd[h * Di + i] = kd == 2 ? oracle_e4m3_quantize(v) : v;
        }
      if (kd == 3) /* dynamic MX quantisation of the query, group by group */
        for (int h = 0; h < Hi; ++h)
          for (int g = 0; g < G; ++g) {
            const int n = (Di - 32 * g) < 32 ? (Di - 32 * g) : 32;
            uint8_t e;
            oracle_mx_quantize(qd + h * Di + 32 * g, n, &e, grp);
            for (int i = 0; i < n; ++i) qd[h * Di + 32 * g + i] = grp[i] * oracle_e8m0_value(e);
          }
#pragma omp parallel
      {
        double* k = (double*)malloc(sizeof(double) * Di);
#pragma omp for schedule(static)
        for (int64_t s = 0; s < L; ++s) {
          if (s >= vis) { out[s] = NAN; continue; }
          const int64_t r = (int64_t)b * L + s, krow = r * Di;
          double scale = kd == 2 ? (double)((const float*)k_scale)[r] : 1.0;
          for (int i = 0; i < Di; ++i) {
            k[i] = load(k_idx, kd, krow + i);
            if (kd == 3) k[i] *= oracle_e8m0_value(((const uint8_t*)k_scale)[r * G + i / 32]);
          }
          double S = 0.0;
          for (int h = 0; h < Hi; ++h) {
            double dot = 0.0;
            for (int i = 0; i < Di; ++i) dot += qd[h * Di + i] * k[i];
            dot *= scale;
            S += (double)head_w[bt * Hi + h] * (dot > 0.0 ? dot : 0.0);
          }
          out[s] = S;
        }
        free(k);
      }
    }
  }
  free(qd);
  free(grp);
  return 0;
}

/* ---------------- 2. Top-K ---------------- */

typedef struct {
  double score;
  int64_t pos;
} scored;

/* Descending score; among equal scores the lower position first. */
static int by_score_then_pos(const void* a, const void* b) {
  const scored* x = (const scored*)a;
  const scored* y = (const scored*)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->pos > y->pos) - (x->pos < y->pos);
}

static int ascending(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/*
 * idx: [B, T, K] int32, the selected positions in ascending order, padded
 * with -1; count: [B, T] = min(K, vis).  Scores are read from the fp64
 * array oracle_index_scores fills (or any [B,T,Lmax] fp64 array).
 */
int oracle_topk(const oracle_dims* d, const double* scores, const int32_t* seq_lens,
                const uint8_t* want, int32_t* idx, int32_t* count) {
  const int B = d->batch, T = d->q_len, K = d->top_k;
  const int64_t L = d->max_seq_len;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
  for (int b = 0; b < B; ++b) {
    for (int t = 0; t < T; ++t) {
      int64_t bt = (int64_t)b * T + t;
      if (want && !want[bt]) continue;
      int64_t vis = visible(d, seq_lens, b, t);
      if (vis < 0) vis = 0;
      scored* all = (scored*)malloc(sizeof(scored) * (size_t)(vis > 0 ? vis : 1));
      for (int64_t s = 0; s < vis; ++s) {
        all[s].score = scores[bt * L + s];
        all[s].pos = s;
      }
      qsort(all, (size_t)vis, sizeof(scored), by_score_then_pos);
      int64_t n = vis < K ? vis : K;
      int32_t* row = idx + bt * K;
      for (int64_t j = 0; j < n; ++j) row[j] = (int32_t)all[j].pos;
      qsort(row, (size_t)n, sizeof(int32_t), ascending);
      for (int64_t j = n; j < K; ++j) row[j] = -1;
      count[bt] = (int32_t)n;
      free(all);
    }
  }
  return 0;
}

/* ---------------- 3. sparse attention over the selected rows ---------------- */
/*
 * q: [B,T,H,Dqk]; kv: [B,Lmax,Dqk] (+ kv_scale: [B,Lmax] for dtype 2,
 * [B,Lmax,ceil(Dqk/128)] for dtype 4, else NULL);
 * idx: [B,T,K]; entries outside [0, len_b) are not selected rows.
 * out: [B,T,H,Dv] fp64; lse: [B,T,H] fp64 (natural log of the softmax
 * normaliser of the scaled logits) or NULL.  No selected row: out = 0,
 * lse = -inf.
 */
int oracle_sparse_mla(const oracle_dims* d, const void* q, const void* kv, const float* kv_scale,
                      const int32_t* idx, const int32_t* seq_lens, const uint8_t* want,
                      double* out, double* lse) {
  const int B = d->batch, T = d->q_len, H = d->heads, Dqk = d->qk_dim, Dv = d->v_dim;
  const int K = d->top_k;
  const int64_t L = d->max_seq_len;
#pragma omp parallel for schedule(dynamic, 1) collapse(3)
  for (int b = 0; b < B; ++b) {
    for (int t = 0; t < T; ++t) {
      for (int h = 0; h < H; ++h) {
        int64_t bt = (int64_t)b * T + t;
        if (want && !want[bt]) continue;
        int64_t len = seq_lens[b] < L ? seq_lens[b] : L;
        const int32_t* sel = idx + bt * K;
        double* o = out + (bt * H + h) * Dv;
        double* qv = (double*)malloc(sizeof(double) * Dqk);
        double* c = (double*)malloc(sizeof(double) * Dqk);
        double* z = (double*)malloc(sizeof(double) * (K > 0 ? K : 1));
        int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (K > 0 ? K : 1));
        int n = 0;
        for (int i = 0; i < Dqk; ++i) qv[i] = load(q, d->q_dtype, (bt * H + h) * Dqk + i);
        for (int j = 0; j < K; ++j)
          if (sel[j] >= 0 && sel[j] < len) rows[n++] = (int64_t)b * L + sel[j];
        /* logits z_j = scale * q . c_j (the row decoded: elements times their scales) */
        for (int j = 0; j < n; ++j) {
          double dot = 0.0;
          for (int i = 0; i < Dqk; ++i) dot += qv[i] * kv_value(kv, d->kv_dtype, kv_scale, rows[j], Dqk, i);
          z[j] = d->softmax_scale * dot;
        }
        for (int v = 0; v < Dv; ++v) o[v] = 0.0;
        if (n == 0) {
          if (lse) lse[bt * H + h] = -INFINITY;
        } else {
          /* pass 1: the maximum logit; pass 2: exponentials and their sum */
          double m = z[0];
          for (int j = 1; j < n; ++j) if (z[j] > m) m = z[j];
          double Z = 0.0;
          for (int j = 0; j < n; ++j) { z[j] = exp(z[j] - m); Z += z[j]; }
          /* weighted sum of the value part (first Dv columns) of each row */
          for (int j = 0; j < n; ++j) {
            double p = z[j] / Z;
            for (int v = 0; v < Dv; ++v) c[v] = kv_value(kv, d->kv_dtype, kv_scale, rows[j], Dqk, v);
            for (int v = 0; v < Dv; ++v) o[v] += p * c[v];
          }
          if (lse) lse[bt * H + h] = m + log(Z);
        }
        free(qv);
        free(c);
        free(z);
        free(rows);
      }
    }
  }
  return 0;
}

/* Softmax weights of one (b, t, h) over its selected rows, in index-list
 * order (entries that are not selected rows get weight 0).  For tests. */
int oracle_attention_weights(const oracle_dims* d, const void* q, const void* kv,
                             const float* kv_scale, const int32_t* idx, const int32_t* seq_lens,
                             int b, int t, int h, double* p_out) {
  const int T = d->q_len, H = d->heads, Dqk = d->qk_dim, K = d->top_k;
  const int64_t L = d->max_seq_len;
  int64_t bt = (int64_t)b * T + t;
  int64_t len = seq_lens[b] < L ? seq_lens[b] : L;
  const int32_t* sel = idx + bt * K;
  double m = -INFINITY, Z = 0.0;
  for (int j = 0; j < K; ++j) {
    p_out[j] = -INFINITY;
    if (sel[j] < 0 || sel[j] >= len) continue;
    int64_t r = (int64_t)b * L + sel[j];
    double dot = 0.0;
    for (int i = 0; i < Dqk; ++i)
      dot += load(q, d->q_dtype, (bt * H + h) * Dqk + i) * kv_value(kv, d->kv_dtype, kv_scale, r, Dqk, i);
    p_out[j] = d->softmax_scale * dot;
    if (p_out[j] > m) m = p_out[j];
  }
  for (int j = 0; j < K; ++j) {
    p_out[j] = (p_out[j] == -INFINITY) ? 0.0 : exp(p_out[j] - m);
    Z += p_out[j];
  }
  for (int j = 0; j < K; ++j) p_out[j] = Z > 0 ? p_out[j] / Z : 0.0;
  return 0;
}
