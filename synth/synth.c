/*
 * synth.c - seeded synthetic workload generator (see synth.h).
 *
 * Philox4x32-10 follows its published definition (Salmon et al., SC'11):
 * ten rounds of two 32x32->64 multiplies with multipliers 0xD2511F53 and
 * 0xCD9E8D57, the key bumped by the Weyl constants 0x9E3779B9 and 0xBB67AE85
 * between rounds.
 *
 * Counter layout used by every stream:
 *   ctr[0] = index bits 0..31, ctr[1] = index bits 32..63,
 *   ctr[2] = tag << 24 | (attempt & 0xff) << 16 | (layer & 0xffff),
 *   ctr[3] = request;   key = {seed bits 0..31, seed bits 32..63}.
 */
#include "synth.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static inline void mulhilo32(uint32_t a, uint32_t b, uint32_t* hi, uint32_t* lo) {
  uint64_t p = (uint64_t)a * (uint64_t)b;
  *hi = (uint32_t)(p >> 32);
  *lo = (uint32_t)p;
}

void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    uint32_t hi0, lo0, hi1, lo1;
    mulhilo32(0xD2511F53u, c0, &hi0, &lo0);
    mulhilo32(0xCD9E8D57u, c2, &hi1, &lo1);
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static inline void stream_block(uint64_t seed, uint32_t tag, uint32_t layer, uint32_t req,
                                uint32_t attempt, uint64_t idx, uint32_t out[4]) {
  uint32_t ctr[4] = {(uint32_t)idx, (uint32_t)(idx >> 32),
                     (tag << 24) | ((attempt & 0xffu) << 16) | (layer & 0xffffu), req};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  synth_philox4x32_10(ctr, key, out);
}

static inline double u01(uint32_t x) { return ((double)x + 0.5) * (1.0 / 4294967296.0); }

/* Box-Muller on the four words of one Philox block -> four normals. */
static inline void box_muller4(const uint32_t w[4], double z[4]) {
  const double two_pi = 6.283185307179586476925286766559;
  double r0 = sqrt(-2.0 * log(u01(w[0])));
  double t0 = two_pi * u01(w[1]);
  double r1 = sqrt(-2.0 * log(u01(w[2])));
  double t1 = two_pi * u01(w[3]);
  z[0] = r0 * cos(t0);
  z[1] = r0 * sin(t0);
  z[2] = r1 * cos(t1);
  z[3] = r1 * sin(t1);
}

void synth_normals(uint64_t seed, uint32_t tag, uint32_t layer, uint32_t req,
                   uint32_t attempt, uint64_t off, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) {
    uint64_t e = off + (uint64_t)i;
    uint32_t w[4];
    double z[4];
    stream_block(seed, tag, layer, req, attempt, e >> 2, w);
    box_muller4(w, z);
    out[i] = z[e & 3];
  }
}

uint32_t synth_u32(uint64_t seed, uint32_t tag, uint32_t layer, uint32_t req, uint64_t idx) {
  uint32_t w[4];
  stream_block(seed, tag, layer, req, 0, idx, w);
  return w[0];
}

int64_t synth_uniform_int(uint64_t seed, uint32_t tag, uint32_t layer, uint32_t req,
                          uint64_t idx, int64_t lo, int64_t hi) {
  uint64_t span = (uint64_t)(hi - lo) + 1u;
  uint64_t x = synth_u32(seed, tag, layer, req, idx);
  /* floor(x * span / 2^32); span < 2^32 for every use here */
  return lo + (int64_t)((x * span) >> 32);
}

double synth_uniform01(uint64_t seed, uint32_t tag, uint32_t layer, uint32_t req, uint64_t idx) {
  return u01(synth_u32(seed, tag, layer, req, idx));
}

/* ---- rounding to the storage types (round to nearest, ties to even) ---- */

static uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u); /* NaN */
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static uint16_t f32_to_f16(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  uint32_t sign = (x >> 16) & 0x8000u;
  uint32_t ax = x & 0x7fffffffu;
  if (ax >= 0x7f800000u) return (uint16_t)(sign | 0x7c00u | (ax > 0x7f800000u ? 0x200u : 0u));
  if (ax >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u); /* >= 65520 rounds to inf */
  if (ax < 0x38800000u) {                                    /* below 2^-14: subnormal */
    float v;
    memcpy(&v, &ax, 4);
    double scaled = (double)v * 16777216.0; /* exact: v / 2^-24 */
    return (uint16_t)(sign | (uint32_t)rint(scaled));
  }
  uint32_t odd = (ax >> 13) & 1u;
  ax += 0xc8000fffu + odd; /* exponent bias 127 -> 15, plus the rounding increment */
  return (uint16_t)(sign | (ax >> 13));
}

uint16_t synth_quantize(double x, int dtype) {
  float f = (float)x;
  return dtype == SYNTH_BF16 ? f32_to_bf16(f) : f32_to_f16(f);
}

static double decode(uint16_t h, int dtype) {
  if (dtype == SYNTH_BF16) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
  }
  uint32_t s = (h >> 15) & 1u, e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(m | 0x400u), (int)e - 25);
  return s ? -v : v;
}

void synth_q(uint64_t seed, uint32_t layer, uint32_t req, int Hq, int d, int dtype,
             uint16_t* out) {
  int64_t n = (int64_t)Hq * d;
  for (int64_t e = 0; e < n; e += 4) {
    uint32_t w[4];
    double z[4];
    stream_block(seed, SYNTH_TAG_Q, layer, req, 0, (uint64_t)e >> 2, w);
    box_muller4(w, z);
    for (int i = 0; i < 4 && e + i < n; ++i) out[e + i] = synth_quantize(z[i], dtype);
  }
}

void synth_qhat(const uint16_t* q, int dtype, int Hq, int Hkv, int d, double* out) {
  int G = Hq / Hkv;
  for (int g = 0; g < Hkv; ++g) {
    double nrm = 0.0;
    for (int j = 0; j < d; ++j) {
      double u = 0.0;
      for (int i = 0; i < G; ++i) u += decode(q[(int64_t)(g * G + i) * d + j], dtype);
      out[(int64_t)g * d + j] = u;
      nrm += u * u;
    }
    nrm = sqrt(nrm);
    for (int j = 0; j < d; ++j) out[(int64_t)g * d + j] = nrm > 0.0 ? out[(int64_t)g * d + j] / nrm : 0.0;
  }
}

/* one token row t: Hkv*d elements (a multiple of 4) */
static void kv_row(uint64_t seed, uint32_t tag, uint32_t layer, uint32_t req, int64_t t,
                   int Hkv, int d, int hot, int attempt, const double* qhat, double shift,
                   int dtype, uint16_t* row) {
  int64_t rl = (int64_t)Hkv * d;
  uint64_t base = (uint64_t)t * (uint64_t)rl;
  for (int64_t e = 0; e < rl; e += 4) {
    uint32_t w[4];
    double z[4];
    stream_block(seed, tag, layer, req, (uint32_t)attempt, (base + (uint64_t)e) >> 2, w);
    box_muller4(w, z);
    for (int i = 0; i < 4; ++i) {
      double x = z[i];
      if (hot) x += shift * qhat[e + i]; /* qhat is [Hkv][d], same flat index as the row */
      row[e + i] = synth_quantize(x, dtype);
    }
  }
}

void synth_kv(uint64_t seed, uint32_t tag, uint32_t layer, uint32_t req,
              int64_t n_tok, int Hkv, int d, int bs,
              const uint8_t* hot, const uint8_t* attempts,
              const double* qhat, double shift, int dtype, uint16_t* out) {
  int64_t rl = (int64_t)Hkv * d;
#pragma omp parallel for schedule(static, 64)
  for (int64_t t = 0; t < n_tok; ++t) {
    int64_t b = t / bs;
    int h = hot ? hot[b] != 0 : 0;
    int a = attempts ? attempts[b] : 0;
    kv_row(seed, tag, layer, req, t, Hkv, d, h, a, qhat, shift, dtype, out + t * rl);
  }
}

void synth_kv_block(uint64_t seed, uint32_t tag, uint32_t layer, uint32_t req,
                    int64_t n_tok, int Hkv, int d, int bs, int64_t b,
                    int hot, int attempt, const double* qhat, double shift,
                    int dtype, uint16_t* out) {
  int64_t rl = (int64_t)Hkv * d;
  int64_t t1 = (b + 1) * bs < n_tok ? (b + 1) * bs : n_tok;
  for (int64_t t = b * bs; t < t1; ++t)
    kv_row(seed, tag, layer, req, t, Hkv, d, hot, attempt, qhat, shift, dtype, out + t * rl);
}

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

void synth_choose(uint64_t seed, uint32_t tag, uint32_t layer, uint32_t req,
                  int64_t nb, int64_t n, int32_t* out) {
  int32_t* perm = (int32_t*)malloc((size_t)nb * sizeof(int32_t));
  for (int64_t i = 0; i < nb; ++i) perm[i] = (int32_t)i;
  for (int64_t i = 0; i < n; ++i) {
    int64_t j = synth_uniform_int(seed, tag, layer, req, (uint64_t)i, i, nb - 1);
    int32_t tmp = perm[i];
    perm[i] = perm[j];
    perm[j] = tmp;
  }
  memcpy(out, perm, (size_t)n * sizeof(int32_t));
  free(perm);
  qsort(out, (size_t)n, sizeof(int32_t), cmp_i32);
}

int64_t synth_runs(uint64_t seed, uint32_t layer, uint32_t req, int64_t nb, int64_t k,
                   int max_run, uint8_t* mask) {
  memset(mask, 0, (size_t)nb);
  if (k <= 0) return 0;
  /* run lengths: draw until they cover k, truncate the last */
  int64_t cap = k, m = 0, tot = 0;
  int64_t* len = (int64_t*)malloc((size_t)cap * sizeof(int64_t));
  while (tot < k) {
    int64_t L = synth_uniform_int(seed, SYNTH_TAG_RUNLEN, layer, req, (uint64_t)m, 1, max_run);
    if (tot + L > k) L = k - tot;
    len[m++] = L;
    tot += L;
  }
  int64_t spare = nb - k - (m - 1);
  if (spare < 0) {
    free(len);
    return -1;
  }
  /* stars and bars: m distinct bar positions among spare + m slots */
  int32_t* bars = (int32_t*)malloc((size_t)m * sizeof(int32_t));
  synth_choose(seed, SYNTH_TAG_RUNPOS, layer, req, spare + m, m, bars);
  int64_t pos = 0;
  for (int64_t i = 0; i < m; ++i) {
    int64_t extra = i == 0 ? bars[0] : bars[i] - bars[i - 1] - 1;
    pos += extra + (i > 0 ? 1 : 0); /* mandatory single gap between runs */
    for (int64_t j = 0; j < len[i]; ++j) mask[pos + j] = 1;
    pos += len[i];
  }
  free(bars);
  free(len);
  return m;
}
