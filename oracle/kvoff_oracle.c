/*
 * kvoff_oracle.c - plain CPU oracle (TEST INFRASTRUCTURE; see kvoff_oracle.h
 * for the rule each function follows and for what may load it).
 *
 * Every loop runs in the plain order of its definition: no blocking, no
 * reordering, no threads.  Build flags must not enable fast-math or FMA
 * contraction.
 */
#include "kvoff_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

double oracle_widen(uint16_t bits, int dtype) {
  if (dtype == ORACLE_BF16) {
    /* bf16 is the top half of an fp32 pattern */
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  /* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits */
  int sign = (bits >> 15) & 1;
  int e = (bits >> 10) & 0x1f;
  int m = bits & 0x3ff;
  double v;
  if (e == 0) v = ldexp((double)m, -24);                 /* zero / subnormal */
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), e - 25);            /* (1 + m/1024) * 2^(e-15) */
  return sign ? -v : v;
}

int64_t oracle_kv_cache_bytes(int64_t L, int64_t Hkv, int64_t d, int64_t S, int64_t es) {
  return 2 * L * Hkv * d * S * es;
}

int64_t oracle_rec_bytes(int64_t Hkv, int64_t bs, int64_t d, int64_t es) {
  return 2 * Hkv * bs * d * es;
}

/* ---------------------------------------------------------------- digest */

void oracle_digest(const uint16_t* K, int dtype, int64_t ctx, int Hkv, int d, int bs, float* D) {
  int64_t nb = (ctx + bs - 1) / bs;
  for (int64_t b = 0; b < nb; ++b) {
    int64_t t0 = b * bs;
    int64_t n_valid = ctx - t0 < bs ? ctx - t0 : bs;
    for (int g = 0; g < Hkv; ++g) {
      for (int j = 0; j < d; ++j) {
        double sum = 0.0;
        for (int64_t t = t0; t < t0 + n_valid; ++t)
          sum += oracle_widen(K[(t * Hkv + g) * d + j], dtype);
        double mean = sum / (double)n_valid;
        D[(b * Hkv + g) * d + j] = (float)mean;
      }
    }
  }
}

/* ----------------------------------------------------------------- score */

void oracle_score(const uint16_t* q, int dtype, int Hq, int Hkv, int d,
                  const float* D, int64_t nb, double* S) {
  int G = Hq / Hkv;
  for (int64_t b = 0; b < nb; ++b) {
    double s = 0.0;
    for (int h = 0; h < Hq; ++h) {
      int g = h / G;
      for (int j = 0; j < d; ++j)
        s += oracle_widen(q[h * d + j], dtype) * (double)D[(b * Hkv + g) * d + j];
    }
    S[b] = s;
  }
}

void oracle_score_headwise(const uint16_t* q, int dtype, int Hq, int Hkv, int d,
                           const float* D, int64_t nb, double* S) {
  int G = Hq / Hkv;
  for (int g = 0; g < Hkv; ++g) {
    for (int64_t b = 0; b < nb; ++b) {
      double s = 0.0;
      for (int h = g * G; h < (g + 1) * G; ++h)
        for (int j = 0; j < d; ++j)
          s += oracle_widen(q[h * d + j], dtype) * (double)D[(b * Hkv + g) * d + j];
      S[g * nb + b] = s;
    }
  }
}

void oracle_score_consensus(const uint16_t* q, int dtype, int Hq, int Hkv, int d,
                            const float* D, int64_t nb, double lambda, double* S) {
  double* Sg = (double*)malloc((size_t)Hkv * (size_t)nb * sizeof(double));
  oracle_score_headwise(q, dtype, Hq, Hkv, d, D, nb, Sg);
  for (int64_t b = 0; b < nb; ++b) {
    double mx = Sg[b], sum = 0.0;
    for (int g = 0; g < Hkv; ++g) {
      if (Sg[g * nb + b] > mx) mx = Sg[g * nb + b];
      sum += Sg[g * nb + b];
    }
    S[b] = mx + lambda * (sum / (double)Hkv);
  }
  free(Sg);
}

void oracle_score_group_consensus(const uint16_t* q, int dtype, int Hq, int Hkv, int d,
                                  const float* D, int64_t nb, double lambda, double* S) {
  int G = Hq / Hkv;
  for (int g = 0; g < Hkv; ++g) {
    for (int64_t b = 0; b < nb; ++b) {
      double mx = -INFINITY, sum = 0.0;
      for (int h = g * G; h < (g + 1) * G; ++h) {
        double s = 0.0;
        for (int j = 0; j < d; ++j)
          s += oracle_widen(q[h * d + j], dtype) * (double)D[(b * Hkv + g) * d + j];
        if (s > mx) mx = s;
        sum += s;
      }
      S[g * nb + b] = mx + lambda * (sum / (double)G);
    }
  }
}

/* ---------------------------------------------------------------- select */

typedef struct {
  double s;
  int32_t b;
} scored_block;

/* order: higher score first; equal scores (after -0 == +0) by lower id */
static int by_score_desc(const void* pa, const void* pb) {
  const scored_block* a = (const scored_block*)pa;
  const scored_block* b = (const scored_block*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->b > b->b) - (a->b < b->b);
}

static int by_id(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

int64_t oracle_select(const double* S, int64_t nb, int64_t k, int32_t* sel) {
  if (k < 1) return -1;
  int64_t K = k < nb ? k : nb;
  scored_block* all = (scored_block*)malloc((size_t)nb * sizeof(scored_block));
  for (int64_t b = 0; b < nb; ++b) {
    all[b].s = S[b];
    all[b].b = (int32_t)b;
  }
  qsort(all, (size_t)nb, sizeof(scored_block), by_score_desc);
  for (int64_t i = 0; i < K; ++i) sel[i] = all[i].b;
  free(all);
  qsort(sel, (size_t)K, sizeof(int32_t), by_id);
  return K;
}

/* ---------------------------------------------------------------- recall */

void oracle_records(const uint16_t* K, const uint16_t* V, int64_t ctx, int Hkv, int d, int bs,
                    uint16_t* rec) {
  int64_t nb = (ctx + bs - 1) / bs;
  for (int64_t b = 0; b < nb; ++b)
    for (int g = 0; g < Hkv; ++g)
      for (int kv = 0; kv < 2; ++kv)
        for (int t = 0; t < bs; ++t)
          for (int j = 0; j < d; ++j) {
            int64_t tok = b * bs + t;
            const uint16_t* src = kv == 0 ? K : V;
            uint16_t v = tok < ctx ? src[(tok * Hkv + g) * d + j] : 0;
            rec[((((b * Hkv + g) * 2 + kv) * bs) + t) * (int64_t)d + j] = v;
          }
}

int64_t oracle_runs(const int32_t* sel, int64_t K, const uint8_t* hit,
                    int32_t* run_first_rank, int32_t* run_len) {
  int64_t n = 0;
  int64_t i = 0;
  while (i < K) {
    if (hit && hit[sel[i]]) {
      ++i;
      continue;
    }
    /* a run starts at rank i and grows while the next selected id is
       the next block and is also missing */
    int64_t j = i + 1;
    while (j < K && sel[j] == sel[j - 1] + 1 && !(hit && hit[sel[j]])) ++j;
    if (run_first_rank) run_first_rank[n] = (int32_t)i;
    if (run_len) run_len[n] = (int32_t)(j - i);
    ++n;
    i = j;
  }
  return n;
}

int64_t oracle_headwise_transfers(const int32_t* sel, const int64_t* counts, int nsets,
                                  int64_t stride, const uint8_t* hit) {
  int64_t n = 0;
  for (int s = 0; s < nsets; ++s)
    for (int64_t i = 0; i < counts[s]; ++i)
      if (!(hit && hit[sel[s * stride + i]])) ++n;
  return n;
}

int64_t oracle_union_count(const int32_t* sel, const int64_t* counts, int nsets, int64_t stride) {
  int32_t mx = -1;
  for (int s = 0; s < nsets; ++s)
    for (int64_t i = 0; i < counts[s]; ++i)
      if (sel[s * stride + i] > mx) mx = sel[s * stride + i];
  if (mx < 0) return 0;
  uint8_t* seen = (uint8_t*)calloc((size_t)mx + 1, 1);
  int64_t n = 0;
  for (int s = 0; s < nsets; ++s)
    for (int64_t i = 0; i < counts[s]; ++i) {
      int32_t b = sel[s * stride + i];
      if (!seen[b]) {
        seen[b] = 1;
        ++n;
      }
    }
  free(seen);
  return n;
}

/* ------------------------------------------------------------- attention */

/* tokens attended: the valid tokens of the selected blocks, ascending */
static int64_t gather_tokens(int64_t ctx, int bs, const int32_t* sel, int64_t nsel, int64_t* tok) {
  int64_t n = 0;
  if (!sel) {
    for (int64_t t = 0; t < ctx; ++t) tok[n++] = t;
    return n;
  }
  for (int64_t i = 0; i < nsel; ++i)
    for (int t = 0; t < bs; ++t) {
      int64_t x = (int64_t)sel[i] * bs + t;
      if (x < ctx) tok[n++] = x;
    }
  return n;
}

static void attend_head_f32(const uint16_t* qh, const uint16_t* K, const uint16_t* V, int dtype,
                            int Hkv, int d, int g, const int64_t* tok, int64_t n, float* z,
                            float* out) {
  float scale = (float)(1.0 / sqrt((double)d));
  float m = -INFINITY;
  for (int64_t i = 0; i < n; ++i) {
    float s = 0.0f;
    for (int j = 0; j < d; ++j)
      s += (float)oracle_widen(qh[j], dtype) * (float)oracle_widen(K[(tok[i] * Hkv + g) * d + j], dtype);
    z[i] = s * scale;
    if (z[i] > m) m = z[i];
  }
  float Z = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    z[i] = expf(z[i] - m);
    Z += z[i];
  }
  for (int j = 0; j < d; ++j) {
    float acc = 0.0f;
    for (int64_t i = 0; i < n; ++i)
      acc += z[i] * (float)oracle_widen(V[(tok[i] * Hkv + g) * d + j], dtype);
    out[j] = acc / Z;
  }
}

void oracle_attend_f32(const uint16_t* q, const uint16_t* K, const uint16_t* V, int dtype,
                       int64_t ctx, int Hq, int Hkv, int d, int bs,
                       const int32_t* sel, int64_t nsel, float* out) {
  int G = Hq / Hkv;
  int64_t cap = sel ? nsel * bs : ctx;
  int64_t* tok = (int64_t*)malloc((size_t)(cap > 0 ? cap : 1) * sizeof(int64_t));
  float* z = (float*)malloc((size_t)(cap > 0 ? cap : 1) * sizeof(float));
  int64_t n = gather_tokens(ctx, bs, sel, nsel, tok);
  for (int h = 0; h < Hq; ++h)
    attend_head_f32(q + (int64_t)h * d, K, V, dtype, Hkv, d, h / G, tok, n, z, out + (int64_t)h * d);
  free(z);
  free(tok);
}

void oracle_attend_headwise_f32(const uint16_t* q, const uint16_t* K, const uint16_t* V,
                                int dtype, int64_t ctx, int Hq, int Hkv, int d, int bs,
                                const int32_t* sel, int64_t nsel, int64_t stride, float* out) {
  int G = Hq / Hkv;
  int64_t cap = nsel * bs;
  int64_t* tok = (int64_t*)malloc((size_t)(cap > 0 ? cap : 1) * sizeof(int64_t));
  float* z = (float*)malloc((size_t)(cap > 0 ? cap : 1) * sizeof(float));
  for (int h = 0; h < Hq; ++h) {
    int g = h / G;
    int64_t n = gather_tokens(ctx, bs, sel + g * stride, nsel, tok);
    attend_head_f32(q + (int64_t)h * d, K, V, dtype, Hkv, d, g, tok, n, z, out + (int64_t)h * d);
  }
  free(z);
  free(tok);
}

void oracle_attend_f64(const uint16_t* q, const uint16_t* K, const uint16_t* V, int dtype,
                       int64_t ctx, int Hq, int Hkv, int d, int bs,
                       const int32_t* sel, int64_t nsel, double* out, double* wsum) {
  int G = Hq / Hkv;
  int64_t cap = sel ? nsel * bs : ctx;
  int64_t* tok = (int64_t*)malloc((size_t)(cap > 0 ? cap : 1) * sizeof(int64_t));
  double* w = (double*)malloc((size_t)(cap > 0 ? cap : 1) * sizeof(double));
  int64_t n = gather_tokens(ctx, bs, sel, nsel, tok);
  double scale = 1.0 / sqrt((double)d);
  for (int h = 0; h < Hq; ++h) {
    int g = h / G;
    double m = -INFINITY;
    for (int64_t i = 0; i < n; ++i) {
      double s = 0.0;
      for (int j = 0; j < d; ++j)
        s += oracle_widen(q[h * d + j], dtype) * oracle_widen(K[(tok[i] * Hkv + g) * d + j], dtype);
      w[i] = s * scale;
      if (w[i] > m) m = w[i];
    }
    double Z = 0.0;
    for (int64_t i = 0; i < n; ++i) {
      w[i] = exp(w[i] - m);
      Z += w[i];
    }
    if (wsum) {
      double ws = 0.0;
      for (int64_t i = 0; i < n; ++i) ws += w[i] / Z;
      wsum[h] = ws;
    }
    for (int j = 0; j < d; ++j) {
      double acc = 0.0;
      for (int64_t i = 0; i < n; ++i) acc += w[i] * oracle_widen(V[(tok[i] * Hkv + g) * d + j], dtype);
      out[h * d + j] = acc / Z;
    }
  }
  free(w);
  free(tok);
}

void oracle_dense_f64(const uint16_t* q, const uint16_t* K, const uint16_t* V, int dtype,
                      int64_t ctx, int Hq, int Hkv, int d, double* out) {
  int G = Hq / Hkv;
  double* w = (double*)malloc((size_t)(ctx > 0 ? ctx : 1) * sizeof(double));
  double scale = 1.0 / sqrt((double)d);
  for (int h = 0; h < Hq; ++h) {
    int g = h / G;
    double m = -INFINITY;
    for (int64_t t = 0; t < ctx; ++t) {
      double s = 0.0;
      for (int j = 0; j < d; ++j)
        s += oracle_widen(q[h * d + j], dtype) * oracle_widen(K[(t * Hkv + g) * d + j], dtype);
      w[t] = s * scale;
      if (w[t] > m) m = w[t];
    }
    double Z = 0.0;
    for (int64_t t = 0; t < ctx; ++t) {
      w[t] = exp(w[t] - m);
      Z += w[t];
    }
    for (int j = 0; j < d; ++j) {
      double acc = 0.0;
      for (int64_t t = 0; t < ctx; ++t) acc += w[t] * oracle_widen(V[(t * Hkv + g) * d + j], dtype);
      out[h * d + j] = acc / Z;
    }
  }
  free(w);
}

void oracle_attention_mass(const uint16_t* q, const uint16_t* K, int dtype, int64_t ctx, int Hq,
                           int Hkv, int d, int bs, const int32_t* sel, const int64_t* counts,
                           int nsets, int64_t stride, double* mass) {
  int G = Hq / Hkv;
  int64_t nb = (ctx + bs - 1) / bs;
  double* z = (double*)malloc((size_t)(ctx > 0 ? ctx : 1) * sizeof(double));
  uint8_t* chosen = (uint8_t*)malloc((size_t)(nb > 0 ? nb : 1));
  double scale = 1.0 / sqrt((double)d);
  for (int h = 0; h < Hq; ++h) {
    int g = h / G;
    int set = nsets == 1 ? 0 : g;
    for (int64_t b = 0; b < nb; ++b) chosen[b] = 0;
    for (int64_t i = 0; i < counts[set]; ++i) chosen[sel[set * stride + i]] = 1;
    double m = -INFINITY;
    for (int64_t t = 0; t < ctx; ++t) {
      double s = 0.0;
      for (int j = 0; j < d; ++j)
        s += oracle_widen(q[h * d + j], dtype) * oracle_widen(K[(t * Hkv + g) * d + j], dtype);
      z[t] = s * scale;
      if (z[t] > m) m = z[t];
    }
    double all = 0.0, kept = 0.0;
    for (int64_t t = 0; t < ctx; ++t) {
      double w = exp(z[t] - m);
      all += w;
      if (chosen[t / bs]) kept += w;
    }
    mass[h] = kept / all;
  }
  free(chosen);
  free(z);
}
