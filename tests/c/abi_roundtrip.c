/*
 * abi_roundtrip.c - drives libkvoff.so through its C ABI alone (no Python)
 * and checks every stage against the plain C oracle.  Test infrastructure.
 *
 * One request, one layer: Hq = 8, Hkv = 2, d = 128, blocks of 16 tokens, a
 * ragged context of 1000 tokens (63 blocks, the last holding 8 tokens),
 * top-20, both storage types.  Inputs come from the seeded generator.
 *   digests           bit-exact against oracle_digest
 *   selection         equal to oracle_select of the oracle's fp64 scores
 *                     (the test first checks that rank 20 and rank 21 are
 *                     at least 1e-3 apart, so the decision is unambiguous)
 *   recalled records  byte-equal to oracle_records of the selected blocks
 *   transfers         equal to oracle_runs
 *   attention         within 2e-3 of oracle_attend_f32
 * Then two layers of the same shape through kvoff_step (compute stream plus
 * copy stream, recall of layer 1 under attention of layer 0): its outputs
 * must be bit-identical to the same layers run call by call on one stream,
 * and within 2e-3 of oracle_attend_f32.
 * Exit status 0 and a final "PASS" line on success.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "kvoff.h"
#include "kvoff_oracle.h"
#include "synth.h"

#define HQ 8
#define HKV 2
#define D 128
#define BS 16
#define CTX 1000
#define NB ((CTX + BS - 1) / BS)
#define TOPK 20

static int failures = 0;

#define CHECK(cond, ...)                  \
  do {                                    \
    if (!(cond)) {                        \
      fprintf(stderr, "FAIL: " __VA_ARGS__); \
      fprintf(stderr, "\n");              \
      ++failures;                         \
    }                                     \
  } while (0)

#define HIPOK(call)                                                                  \
  do {                                                                               \
    hipError_t e_ = (call);                                                          \
    if (e_ != hipSuccess) {                                                          \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));                     \
      exit(2);                                                                       \
    }                                                                                \
  } while (0)

#define KVOK(call)                                                                   \
  do {                                                                               \
    int s_ = (call);                                                                 \
    if (s_ != KVOFF_OK) {                                                            \
      fprintf(stderr, "%s: %s (%s)\n", #call, kvoff_strerror(s_), kvoff_last_error()); \
      exit(2);                                                                       \
    }                                                                                \
  } while (0)

static int by_desc(const void* a, const void* b) {
  double x = *(const double*)a, y = *(const double*)b;
  return (x < y) - (x > y);
}

static void run(int dtype) {
  const int sdt = dtype == KVOFF_BF16 ? SYNTH_BF16 : SYNTH_F16;
  const int odt = sdt; /* the oracle uses the same codes: 1 fp16, 2 bf16 */
  const uint64_t seed = 4242 + (uint64_t)dtype;
  const size_t n_kv = (size_t)CTX * HKV * D;
  uint16_t* q = malloc(sizeof(uint16_t) * HQ * D);
  uint16_t* K = malloc(sizeof(uint16_t) * n_kv);
  uint16_t* V = malloc(sizeof(uint16_t) * n_kv);
  synth_q(seed, 0, 0, HQ, D, sdt, q);
  synth_kv(seed, SYNTH_TAG_K, 0, 0, CTX, HKV, D, BS, NULL, NULL, NULL, 0.0, sdt, K);
  synth_kv(seed, SYNTH_TAG_V, 0, 0, CTX, HKV, D, BS, NULL, NULL, NULL, 0.0, sdt, V);

  /* oracle */
  float* D_ref = malloc(sizeof(float) * NB * HKV * D);
  double S_ref[NB], S_sorted[NB];
  int32_t sel_ref[TOPK];
  oracle_digest(K, odt, CTX, HKV, D, BS, D_ref);
  oracle_score(q, odt, HQ, HKV, D, D_ref, NB, S_ref);
  memcpy(S_sorted, S_ref, sizeof S_ref);
  qsort(S_sorted, NB, sizeof(double), by_desc);
  const double gap = S_sorted[TOPK - 1] - S_sorted[TOPK];
  CHECK(gap >= 1e-3, "dtype %d: boundary gap %g below 1e-3 (choose another seed)", dtype, gap);
  const int64_t k_ref = oracle_select(S_ref, NB, TOPK, sel_ref);
  CHECK(k_ref == TOPK, "oracle selected %lld", (long long)k_ref);
  float out_ref[HQ * D];
  oracle_attend_f32(q, K, V, odt, CTX, HQ, HKV, D, BS, sel_ref, TOPK, out_ref);
  uint16_t* rec_ref = malloc(sizeof(uint16_t) * (size_t)NB * HKV * 2 * BS * D);
  oracle_records(K, V, CTX, HKV, D, BS, rec_ref);
  const int64_t runs_ref = oracle_runs(sel_ref, TOPK, NULL, NULL, NULL);

  /* library */
  kvoff_config cfg = {1, HQ, HKV, D, BS, dtype, 4, KVOFF_HOST_COHERENT, NB};
  kvoff_ctx* ctx = NULL;
  KVOK(kvoff_create(&cfg, &ctx));
  int32_t rid = -1;
  KVOK(kvoff_register_request(ctx, CTX, &rid));
  const int64_t rec_bytes = kvoff_record_bytes(ctx);
  CHECK(rec_bytes == oracle_rec_bytes(HKV, BS, D, 2), "record bytes %lld", (long long)rec_bytes);

  void *dK, *dV, *dq, *pool, *ws;
  float *dD, *dout;
  double* dS;
  int32_t *dsel, *dcnt, *dtab;
  const int n_slots = TOPK;
  HIPOK(hipMalloc(&dK, n_kv * 2));
  HIPOK(hipMalloc(&dV, n_kv * 2));
  HIPOK(hipMalloc(&dq, HQ * D * 2));
  HIPOK(hipMalloc((void**)&dD, sizeof(float) * NB * HKV * D));
  HIPOK(hipMalloc((void**)&dS, sizeof(double) * NB));
  HIPOK(hipMalloc((void**)&dsel, sizeof(int32_t) * TOPK));
  HIPOK(hipMalloc((void**)&dcnt, sizeof(int32_t)));
  HIPOK(hipMalloc((void**)&dtab, sizeof(int32_t) * TOPK));
  HIPOK(hipMalloc(&pool, (size_t)n_slots * rec_bytes));
  HIPOK(hipMalloc((void**)&dout, sizeof(float) * HQ * D));
  const size_t ws_bytes = kvoff_workspace_size(ctx, KVOFF_CALL_SPARSE_DECODE, 1, TOPK, KVOFF_SOLOHEAD);
  HIPOK(hipMalloc(&ws, ws_bytes > 0 ? ws_bytes : 1));
  HIPOK(hipMemcpy(dK, K, n_kv * 2, hipMemcpyHostToDevice));
  HIPOK(hipMemcpy(dV, V, n_kv * 2, hipMemcpyHostToDevice));
  HIPOK(hipMemcpy(dq, q, HQ * D * 2, hipMemcpyHostToDevice));

  const int32_t ids[1] = {rid}, topk[1] = {TOPK};
  kvoff_stats st;
  KVOK(kvoff_offload_blocks(ctx, 0, rid, dK, dV, dD, NULL));
  KVOK(kvoff_select(ctx, 0, 1, ids, dq, dD, NB, topk, KVOFF_SOLOHEAD, dS, dsel, dcnt, TOPK, NULL));
  KVOK(kvoff_recall(ctx, 0, 1, ids, KVOFF_SOLOHEAD, dsel, dcnt, TOPK, NULL, NULL, 0, pool, n_slots,
                    0, dtab, KVOFF_ENGINE_ZEROCOPY, &st, NULL));
  KVOK(kvoff_sparse_decode(ctx, 1, ids, KVOFF_SOLOHEAD, dq, pool, n_slots, dtab, dsel, dcnt, TOPK,
                           (float)(1.0 / sqrt((double)D)), dout, ws, ws_bytes, NULL));
  HIPOK(hipDeviceSynchronize());

  float* D_got = malloc(sizeof(float) * NB * HKV * D);
  int32_t sel_got[TOPK], cnt_got = 0, tab_got[TOPK];
  float out_got[HQ * D];
  uint8_t* pool_got = malloc((size_t)n_slots * rec_bytes);
  HIPOK(hipMemcpy(D_got, dD, sizeof(float) * NB * HKV * D, hipMemcpyDeviceToHost));
  HIPOK(hipMemcpy(sel_got, dsel, sizeof sel_got, hipMemcpyDeviceToHost));
  HIPOK(hipMemcpy(&cnt_got, dcnt, sizeof cnt_got, hipMemcpyDeviceToHost));
  HIPOK(hipMemcpy(tab_got, dtab, sizeof tab_got, hipMemcpyDeviceToHost));
  HIPOK(hipMemcpy(out_got, dout, sizeof out_got, hipMemcpyDeviceToHost));
  HIPOK(hipMemcpy(pool_got, pool, (size_t)n_slots * rec_bytes, hipMemcpyDeviceToHost));

  CHECK(memcmp(D_got, D_ref, sizeof(float) * NB * HKV * D) == 0, "dtype %d: digests differ", dtype);
  CHECK(cnt_got == TOPK, "dtype %d: count %d", dtype, cnt_got);
  CHECK(memcmp(sel_got, sel_ref, sizeof sel_ref) == 0, "dtype %d: selection differs", dtype);
  for (int i = 0; i < TOPK; ++i) {
    CHECK(tab_got[i] == i, "dtype %d: table[%d] = %d", dtype, i, tab_got[i]);
    const uint8_t* want = (const uint8_t*)(rec_ref + (size_t)sel_ref[i] * HKV * 2 * BS * D);
    CHECK(memcmp(pool_got + (size_t)i * rec_bytes, want, (size_t)rec_bytes) == 0,
          "dtype %d: recalled record of block %d differs", dtype, sel_ref[i]);
  }
  CHECK(st.selected == TOPK && st.items_recalled == TOPK && st.pool_hits == 0,
        "dtype %d: stats selected %lld recalled %lld", dtype, (long long)st.selected,
        (long long)st.items_recalled);
  CHECK(st.transfers == runs_ref, "dtype %d: transfers %lld, oracle runs %lld", dtype,
        (long long)st.transfers, (long long)runs_ref);
  CHECK(st.bytes == TOPK * rec_bytes, "dtype %d: bytes %lld", dtype, (long long)st.bytes);
  double worst = 0.0;
  for (int i = 0; i < HQ * D; ++i) {
    const double e = fabs((double)out_got[i] - (double)out_ref[i]);
    if (!(e <= worst)) worst = e; /* NaN propagates */
  }
  CHECK(worst <= 2e-3, "dtype %d: attention max abs error %g", dtype, worst);
  printf("dtype %d: gap %.3g, %lld transfers, attention max abs error %.3g\n", dtype, gap,
         (long long)st.transfers, worst);

  HIPOK(hipFree(dK));
  HIPOK(hipFree(dV));
  HIPOK(hipFree(dq));
  HIPOK(hipFree(dD));
  HIPOK(hipFree(dS));
  HIPOK(hipFree(dsel));
  HIPOK(hipFree(dcnt));
  HIPOK(hipFree(dtab));
  HIPOK(hipFree(pool));
  HIPOK(hipFree(dout));
  HIPOK(hipFree(ws));
  KVOK(kvoff_destroy(ctx));
  free(q);
  free(K);
  free(V);
  free(D_ref);
  free(rec_ref);
  free(D_got);
  free(pool_got);
}

/* kvoff_step over two layers against the same layers call by call */
static void run_step(int dtype) {
  enum { L = 2 };
  const int sdt = dtype == KVOFF_BF16 ? SYNTH_BF16 : SYNTH_F16;
  const uint64_t seed = 5151 + (uint64_t)dtype;
  const size_t n_kv = (size_t)CTX * HKV * D;
  kvoff_config cfg = {L, HQ, HKV, D, BS, dtype, 4, KVOFF_HOST_COHERENT, (int64_t)NB * L};
  kvoff_ctx* ctx = NULL;
  KVOK(kvoff_create(&cfg, &ctx));
  int32_t rid = -1;
  KVOK(kvoff_register_request(ctx, CTX, &rid));
  const int64_t rec_bytes = kvoff_record_bytes(ctx);

  uint16_t* q[L];
  uint16_t* K[L];
  uint16_t* V[L];
  void *dq[L], *dK, *dV, *pool, *ws;
  float *dD[L], *dout[L], *dref[L];
  double* dS[2];
  int32_t *dsel[2], *dcnt[2], *dtab[2];
  HIPOK(hipMalloc(&dK, n_kv * 2));
  HIPOK(hipMalloc(&dV, n_kv * 2));
  for (int l = 0; l < L; ++l) {
    q[l] = malloc(sizeof(uint16_t) * HQ * D);
    K[l] = malloc(sizeof(uint16_t) * n_kv);
    V[l] = malloc(sizeof(uint16_t) * n_kv);
    synth_q(seed, l, 0, HQ, D, sdt, q[l]);
    synth_kv(seed, SYNTH_TAG_K, l, 0, CTX, HKV, D, BS, NULL, NULL, NULL, 0.0, sdt, K[l]);
    synth_kv(seed, SYNTH_TAG_V, l, 0, CTX, HKV, D, BS, NULL, NULL, NULL, 0.0, sdt, V[l]);
    HIPOK(hipMalloc(&dq[l], HQ * D * 2));
    HIPOK(hipMalloc((void**)&dD[l], sizeof(float) * NB * HKV * D));
    HIPOK(hipMalloc((void**)&dout[l], sizeof(float) * HQ * D));
    HIPOK(hipMalloc((void**)&dref[l], sizeof(float) * HQ * D));
    HIPOK(hipMemcpy(dq[l], q[l], HQ * D * 2, hipMemcpyHostToDevice));
    HIPOK(hipMemcpy(dK, K[l], n_kv * 2, hipMemcpyHostToDevice));
    HIPOK(hipMemcpy(dV, V[l], n_kv * 2, hipMemcpyHostToDevice));
    KVOK(kvoff_offload_blocks(ctx, l, rid, dK, dV, dD[l], NULL));
    HIPOK(hipDeviceSynchronize());
  }
  for (int b = 0; b < 2; ++b) {
    HIPOK(hipMalloc((void**)&dS[b], sizeof(double) * NB));
    HIPOK(hipMalloc((void**)&dsel[b], sizeof(int32_t) * TOPK));
    HIPOK(hipMalloc((void**)&dcnt[b], sizeof(int32_t)));
    HIPOK(hipMalloc((void**)&dtab[b], sizeof(int32_t) * TOPK));
  }
  const int n_slots = 2 * TOPK;  /* one recall region per buffer set */
  HIPOK(hipMalloc(&pool, (size_t)n_slots * rec_bytes));
  const size_t ws_bytes = kvoff_workspace_size(ctx, KVOFF_CALL_STEP, 1, TOPK, KVOFF_SOLOHEAD);
  HIPOK(hipMalloc(&ws, ws_bytes > 0 ? ws_bytes : 1));
  const float scale = (float)(1.0 / sqrt((double)D));
  const int32_t ids[1] = {rid}, topk[1] = {TOPK};

  /* call by call, one stream */
  for (int l = 0; l < L; ++l) {
    KVOK(kvoff_select(ctx, l, 1, ids, dq[l], dD[l], NB, topk, KVOFF_SOLOHEAD, dS[0], dsel[0], dcnt[0],
                      TOPK, NULL));
    KVOK(kvoff_recall(ctx, l, 1, ids, KVOFF_SOLOHEAD, dsel[0], dcnt[0], TOPK, NULL, NULL, 0, pool,
                      n_slots, 0, dtab[0], KVOFF_ENGINE_ZEROCOPY, NULL, NULL));
    KVOK(kvoff_sparse_decode(ctx, 1, ids, KVOFF_SOLOHEAD, dq[l], pool, n_slots, dtab[0], dsel[0], dcnt[0], TOPK,
                             scale, dref[l], ws, ws_bytes, NULL));
  }
  HIPOK(hipDeviceSynchronize());

  /* the same layers through kvoff_step, recall on its own streams */
  hipStream_t cs, xs;
  HIPOK(hipStreamCreate(&cs));
  HIPOK(hipStreamCreate(&xs));
  const void* qs[L] = {dq[0], dq[1]};
  const float* ds[L] = {dD[0], dD[1]};
  float* outs[L] = {dout[0], dout[1]};
  kvoff_step_args a;
  memset(&a, 0, sizeof a);
  a.layer_begin = 0;
  a.layer_end = L;
  a.n_req = 1;
  a.req_ids = ids;
  a.topk = topk;
  a.mode = KVOFF_SOLOHEAD;
  a.engine = KVOFF_ENGINE_ZEROCOPY;
  a.k_stride = TOPK;
  a.q_dev = qs;
  a.digest_dev = ds;
  a.digest_stride = NB;
  a.slot_pool_dev = pool;
  a.n_slots = n_slots;
  a.recall_base_slot[0] = 0;
  a.recall_base_slot[1] = TOPK;
  for (int b = 0; b < 2; ++b) {
    a.scores_dev[b] = dS[b];
    a.sel_idx_dev[b] = dsel[b];
    a.sel_cnt_dev[b] = dcnt[b];
    a.block_table_dev[b] = dtab[b];
  }
  a.scale = scale;
  a.out_dev = outs;
  a.ws_dev = ws;
  a.ws_bytes = ws_bytes;
  a.compute_stream = cs;
  a.copy_stream = xs;
  KVOK(kvoff_step(ctx, &a));
  HIPOK(hipStreamSynchronize(cs));

  for (int l = 0; l < L; ++l) {
    float got[HQ * D], ref[HQ * D], want[HQ * D];
    HIPOK(hipMemcpy(got, dout[l], sizeof got, hipMemcpyDeviceToHost));
    HIPOK(hipMemcpy(ref, dref[l], sizeof ref, hipMemcpyDeviceToHost));
    CHECK(memcmp(got, ref, sizeof got) == 0, "dtype %d layer %d: kvoff_step differs from the calls",
          dtype, l);
    /* the oracle's selection of this layer, then its attention */
    float* D_ref = malloc(sizeof(float) * NB * HKV * D);
    double S_ref[NB];
    int32_t sel_ref[TOPK];
    oracle_digest(K[l], sdt, CTX, HKV, D, BS, D_ref);
    oracle_score(q[l], sdt, HQ, HKV, D, D_ref, NB, S_ref);
    double S_sorted[NB];
    memcpy(S_sorted, S_ref, sizeof S_ref);
    qsort(S_sorted, NB, sizeof(double), by_desc);
    const double gap = S_sorted[TOPK - 1] - S_sorted[TOPK];
    /* GPU and oracle scores agree to ~1e-12: a wider gap fixes the set */
    CHECK(gap >= 1e-6, "dtype %d layer %d: boundary gap %g (choose another seed)", dtype, l, gap);
    oracle_select(S_ref, NB, TOPK, sel_ref);
    oracle_attend_f32(q[l], K[l], V[l], sdt, CTX, HQ, HKV, D, BS, sel_ref, TOPK, want);
    double worst = 0.0;
    for (int i = 0; i < HQ * D; ++i) {
      const double e = fabs((double)got[i] - (double)want[i]);
      if (!(e <= worst)) worst = e;
    }
    CHECK(worst <= 2e-3, "dtype %d layer %d: kvoff_step attention max abs error %g", dtype, l, worst);
    printf("dtype %d layer %d: kvoff_step bit-identical to the calls, attention max abs error %.3g\n",
           dtype, l, worst);
    free(D_ref);
  }

  HIPOK(hipStreamDestroy(cs));
  HIPOK(hipStreamDestroy(xs));
  for (int l = 0; l < L; ++l) {
    HIPOK(hipFree(dq[l]));
    HIPOK(hipFree(dD[l]));
    HIPOK(hipFree(dout[l]));
    HIPOK(hipFree(dref[l]));
    free(q[l]);
    free(K[l]);
    free(V[l]);
  }
  for (int b = 0; b < 2; ++b) {
    HIPOK(hipFree(dS[b]));
    HIPOK(hipFree(dsel[b]));
    HIPOK(hipFree(dcnt[b]));
    HIPOK(hipFree(dtab[b]));
  }
  HIPOK(hipFree(dK));
  HIPOK(hipFree(dV));
  HIPOK(hipFree(pool));
  HIPOK(hipFree(ws));
  KVOK(kvoff_destroy(ctx));
}

int main(void) {
  run(KVOFF_F16);
  run(KVOFF_BF16);
  run_step(KVOFF_F16);
  run_step(KVOFF_BF16);
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("PASS\n");
  return 0;
}
