/*
 * oracle_sanitize.c - every function of the CPU oracle and of the seeded
 * generator on small inputs and their edge cases, built with the address
 * and undefined-behaviour sanitizers (tests/test_host_sanitizers.py).
 * Edge cases: one-token and ragged contexts, block sizes 16 and 32, one and
 * several KV heads, k below 1, k = 1, k = nb and k past nb, empty selections,
 * pool-hit masks, every fp16/bf16 bit pattern widened.  The results are
 * checked only for the invariants that hold at any size (selection counts,
 * ascending ids, weights summing to one, finite outputs); parity with the
 * GPU and the pins live in the Python suites.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvoff_oracle.h"
#include "synth.h"

static int failures = 0;
#define CHECK(cond, ...)                        \
  do {                                          \
    if (!(cond)) {                              \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);             \
      fprintf(stderr, "\n");                    \
      ++failures;                               \
    }                                           \
  } while (0)

static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}

static void run_case(int dtype, int bs, int Hq, int Hkv, int64_t ctx, uint32_t req) {
  const int d = 128;
  const int64_t nb = (ctx + bs - 1) / bs;
  uint16_t* q = xmalloc(sizeof(uint16_t) * Hq * d);
  uint16_t* K = xmalloc(sizeof(uint16_t) * ctx * Hkv * d);
  uint16_t* V = xmalloc(sizeof(uint16_t) * ctx * Hkv * d);
  double* qhat = xmalloc(sizeof(double) * Hkv * d);
  uint8_t* hot = xmalloc(nb);
  uint8_t* att = xmalloc(nb);
  uint8_t* hit = xmalloc(nb);
  memset(att, 0, nb);
  synth_q(77, 0, req, Hq, d, dtype, q);
  synth_qhat(q, dtype, Hq, Hkv, d, qhat);
  /* hot blocks in runs when they fit, else a few chosen ones */
  if (synth_runs(77, 0, req, nb, nb / 4 > 0 ? nb / 4 : 1, 8, hot) < 0) {
    memset(hot, 0, nb);
    int32_t pick[1];
    synth_choose(77, SYNTH_TAG_HOT, 0, req, nb, 1, pick);
    hot[pick[0]] = 1;
  }
  synth_kv(77, SYNTH_TAG_K, 0, req, ctx, Hkv, d, bs, hot, att, qhat, 0.5, dtype, K);
  synth_kv(77, SYNTH_TAG_V, 0, req, ctx, Hkv, d, bs, NULL, NULL, NULL, 0.0, dtype, V);
  synth_kv_block(77, SYNTH_TAG_K, 0, req, ctx, Hkv, d, bs, nb - 1, hot[nb - 1], 1, qhat, 0.5, dtype, K);
  /* pool hits: a quarter of the blocks */
  memset(hit, 0, nb);
  if (nb / 4 > 0) {
    int32_t* res = xmalloc(sizeof(int32_t) * (nb / 4));
    synth_choose(77, SYNTH_TAG_POOL, 0, req, nb, nb / 4, res);
    for (int64_t i = 0; i < nb / 4; ++i) {
      CHECK(res[i] >= 0 && res[i] < nb, "choose out of range");
      hit[res[i]] = 1;
    }
    free(res);
  }

  float* D = xmalloc(sizeof(float) * nb * Hkv * d);
  oracle_digest(K, dtype, ctx, Hkv, d, bs, D);
  double* S = xmalloc(sizeof(double) * nb);
  double* Sg = xmalloc(sizeof(double) * Hkv * nb);
  double* Sc = xmalloc(sizeof(double) * nb);
  double* Sgc = xmalloc(sizeof(double) * Hkv * nb);
  oracle_score(q, dtype, Hq, Hkv, d, D, nb, S);
  oracle_score_headwise(q, dtype, Hq, Hkv, d, D, nb, Sg);
  oracle_score_consensus(q, dtype, Hq, Hkv, d, D, nb, 0.5, Sc);
  oracle_score_group_consensus(q, dtype, Hq, Hkv, d, D, nb, 1.0, Sgc);
  for (int64_t b = 0; b < nb; ++b) {
    double sum = 0.0;
    for (int g = 0; g < Hkv; ++g) sum += Sg[g * nb + b];
    CHECK(fabs(sum - S[b]) <= 1e-9 * (1.0 + fabs(S[b])), "headwise scores do not sum to the score");
  }

  const int64_t ks[] = {0, 1, nb / 2 > 0 ? nb / 2 : 1, nb, nb + 5};
  int32_t* sel = xmalloc(sizeof(int32_t) * (nb + 5));
  int32_t* first = xmalloc(sizeof(int32_t) * (nb + 5));
  int32_t* len = xmalloc(sizeof(int32_t) * (nb + 5));
  for (size_t i = 0; i < sizeof ks / sizeof ks[0]; ++i) {
    const int64_t K_r = oracle_select(S, nb, ks[i], sel);
    if (ks[i] < 1) {
      CHECK(K_r == -1, "k = %lld must be rejected", (long long)ks[i]);
      continue;
    }
    CHECK(K_r == (ks[i] < nb ? ks[i] : nb), "selected %lld of k %lld", (long long)K_r, (long long)ks[i]);
    for (int64_t j = 1; j < K_r; ++j) CHECK(sel[j - 1] < sel[j], "selection not ascending");
    const int64_t n_runs = oracle_runs(sel, K_r, NULL, first, len);
    int64_t covered = 0;
    for (int64_t j = 0; j < n_runs; ++j) covered += len[j];
    CHECK(covered == K_r, "runs cover %lld of %lld", (long long)covered, (long long)K_r);
    const int64_t n_hit_runs = oracle_runs(sel, K_r, hit, NULL, NULL);
    CHECK(n_hit_runs >= 0 && n_hit_runs <= K_r, "runs with hits");
    const int64_t cnt = K_r;
    const int64_t n_tr = oracle_headwise_transfers(sel, &cnt, 1, K_r, hit);
    CHECK(n_tr >= 0 && n_tr <= K_r, "headwise transfers");
    CHECK(oracle_union_count(sel, &cnt, 1, K_r) == K_r, "union of one set");

    float* o32 = xmalloc(sizeof(float) * Hq * d);
    double* o64 = xmalloc(sizeof(double) * Hq * d);
    double* wsum = xmalloc(sizeof(double) * Hq);
    oracle_attend_f32(q, K, V, dtype, ctx, Hq, Hkv, d, bs, sel, K_r, o32);
    oracle_attend_f64(q, K, V, dtype, ctx, Hq, Hkv, d, bs, sel, K_r, o64, wsum);
    for (int h = 0; h < Hq; ++h) CHECK(fabs(wsum[h] - 1.0) <= 1e-12, "weights sum to %.17g", wsum[h]);
    for (int64_t e = 0; e < (int64_t)Hq * d; ++e) CHECK(isfinite(o32[e]) && isfinite(o64[e]), "non-finite output");
    double* mass = xmalloc(sizeof(double) * Hq);
    oracle_attention_mass(q, K, dtype, ctx, Hq, Hkv, d, bs, sel, &cnt, 1, K_r, mass);
    for (int h = 0; h < Hq; ++h) CHECK(mass[h] >= 0.0 && mass[h] <= 1.0 + 1e-12, "mass %.17g", mass[h]);
    free(mass);
    free(wsum);
    free(o64);
    free(o32);
  }
  /* per-KV-head sets, the empty selection and every block */
  int32_t* selg = xmalloc(sizeof(int32_t) * Hkv * nb);
  int64_t* cnts = xmalloc(sizeof(int64_t) * Hkv);
  const int64_t kk = nb / 2 > 0 ? nb / 2 : 1;
  for (int g = 0; g < Hkv; ++g) cnts[g] = oracle_select(Sg + g * nb, nb, kk, selg + g * kk);
  CHECK(oracle_union_count(selg, cnts, Hkv, kk) <= nb, "union larger than the blocks");
  float* oh = xmalloc(sizeof(float) * Hq * d);
  oracle_attend_headwise_f32(q, K, V, dtype, ctx, Hq, Hkv, d, bs, selg, kk, kk, oh);
  double* mass = xmalloc(sizeof(double) * Hq);
  oracle_attention_mass(q, K, dtype, ctx, Hq, Hkv, d, bs, selg, cnts, Hkv, kk, mass);
  float* oall = xmalloc(sizeof(float) * Hq * d);
  oracle_attend_f32(q, K, V, dtype, ctx, Hq, Hkv, d, bs, NULL, 0, oall);
  double* dense = xmalloc(sizeof(double) * Hq * d);
  oracle_dense_f64(q, K, V, dtype, ctx, Hq, Hkv, d, dense);
  for (int64_t e = 0; e < (int64_t)Hq * d; ++e)
    CHECK(fabs((double)oall[e] - dense[e]) <= 1e-4, "all blocks vs dense");
  float* oempty = xmalloc(sizeof(float) * Hq * d);
  oracle_attend_f32(q, K, V, dtype, ctx, Hq, Hkv, d, bs, sel, 0, oempty);

  uint16_t* rec = xmalloc(sizeof(uint16_t) * nb * Hkv * 2 * bs * d);
  oracle_records(K, V, ctx, Hkv, d, bs, rec);
  CHECK(oracle_rec_bytes(Hkv, bs, d, 2) == (int64_t)2 * Hkv * bs * d * 2, "record bytes");

  free(rec);
  free(oempty);
  free(dense);
  free(oall);
  free(mass);
  free(oh);
  free(cnts);
  free(selg);
  free(len);
  free(first);
  free(sel);
  free(Sgc);
  free(Sc);
  free(Sg);
  free(S);
  free(D);
  free(hit);
  free(att);
  free(hot);
  free(qhat);
  free(V);
  free(K);
  free(q);
}

int main(void) {
  /* every 16-bit pattern widens without undefined behaviour */
  for (uint32_t b = 0; b < 65536; ++b) {
    (void)oracle_widen((uint16_t)b, ORACLE_F16);
    (void)oracle_widen((uint16_t)b, ORACLE_BF16);
  }
  CHECK(oracle_kv_cache_bytes(32, 8, 128, 131072, 2) == (int64_t)2 * 32 * 8 * 128 * 131072 * 2,
        "cache bytes");
  /* generator primitives, including extreme values for the rounding */
  uint32_t ctr[4] = {0, 0, 0, 0}, key[2] = {0, 0}, out[4];
  synth_philox4x32_10(ctr, key, out);
  double nrm[257];
  synth_normals(5, SYNTH_TAG_Q, 1, 2, 3, 1000, 257, nrm);
  for (int i = 0; i < 257; ++i) CHECK(isfinite(nrm[i]), "normal not finite");
  const double xs[] = {0.0, -0.0, 1e-40, -1e-40, 65504.0, 65520.0, 1e10, -1e10, 3.4e38, 1e300, 5.96e-8};
  for (size_t i = 0; i < sizeof xs / sizeof xs[0]; ++i) {
    (void)synth_quantize(xs[i], SYNTH_F16);
    (void)synth_quantize(xs[i], SYNTH_BF16);
  }
  for (uint64_t i = 0; i < 1000; ++i) {
    const int64_t v = synth_uniform_int(9, SYNTH_TAG_CTX, 0, 0, i, 8192, 131072);
    CHECK(v >= 8192 && v <= 131072, "uniform_int out of range");
    const double u = synth_uniform01(9, SYNTH_TAG_FRAC, 0, 0, i);
    CHECK(u >= 0.0 && u < 1.0, "uniform01 out of range");
    (void)synth_u32(9, 1, 2, 3, i);
  }
  int32_t all[40];
  synth_choose(3, SYNTH_TAG_HOT, 0, 0, 40, 40, all);
  synth_choose(3, SYNTH_TAG_HOT, 0, 0, 40, 0, all);
  uint8_t mask[40];
  CHECK(synth_runs(3, 0, 0, 40, 20, 8, mask) >= 0, "20 hot blocks fit 40 in runs");
  (void)synth_runs(3, 0, 0, 40, 40, 8, mask); /* may not fit: the return value says */

  const int dtypes[] = {SYNTH_F16, SYNTH_BF16};
  const int bss[] = {16, 32};
  const int heads[][2] = {{1, 1}, {4, 2}, {6, 3}};
  const int64_t ctxs[] = {1, 15, 16, 17, 100, 513};
  uint32_t req = 0;
  for (int a = 0; a < 2; ++a)
    for (int b = 0; b < 2; ++b)
      for (int h = 0; h < 3; ++h)
        for (int c = 0; c < 6; ++c)
          run_case(dtypes[a], bss[b], heads[h][0], heads[h][1], ctxs[c], req++);
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("PASS\n");
  return 0;
}
