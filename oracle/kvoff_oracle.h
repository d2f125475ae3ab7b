/*
 * kvoff_oracle.h - plain CPU oracle of the sparse KV-cache offloading hot path.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library; both read the same seeded
 * inputs and nothing else.
 *
 * What it follows.  The method is PulseInfer ("PulseInfer: I/O-Centric Sparse
 * KV Cache Offloading for Efficient Long-Context LLM Decoding", abstract):
 * most historical KV blocks live in CPU DRAM, a sparse selection picks the
 * blocks a decode step needs, the selection is shared across heads (SoloHead)
 * so recalls are not fragmented per head, and the recalled blocks are moved
 * with a gather engine that coalesces contiguous transfers.  The third-party
 * guide ("PulseInfer Guide: I/O-Centric Sparse KV Cache Offloading",
 * aiFetchly) supplies the mechanisms' shape:
 *   - block records of 2 * H_kv * block_size * head_dim * sizeof(dtype)
 *     bytes (its simulator's GatherScatterEngine);
 *   - one consensus block set per request instead of one per head, with
 *     top-k over block scores ("SoloHead Sparse Selection");
 *   - per-head selection as the fragmentation baseline, one transfer per
 *     head per block ("The Fallacy of Naive Offloading", Pathology 1);
 *   - the KV-cache size formula 2 * L * H_kv * d * S * sizeof(dtype)
 *     ("The Long-Context Decoding Memory Wall").
 *
 * The pages never define the per-(head, block) importance S(h, b).  The rule
 * used throughout is fixed as follows and is the same on CPU and GPU:
 *   digest   D[b][g][j] = mean over the valid tokens t of block b of K[t][g][j]
 *   score    S[b]       = sum over query heads h, dims j of q[h][j]*D[b][h/G][j]
 *   headwise S_g[b]     = the same sum restricted to the G heads of group g
 *   select   the min(k, nb) largest S, ties to the lower block id, ascending
 *   attend   softmax(scale * q.K) V over the valid tokens of the selected
 *            blocks, scale = 1/sqrt(d), GQA head h reads KV head floor(h/G).
 *
 * Precision: digests are fp64 sums of the exact widened inputs, one fp64
 * division by the valid-token count, one rounding to fp32.  Scores are fp64.
 * Attention has an fp32 form (the parity target for attention outputs) and
 * an fp64 form (for invariants).  Inputs are fp16 or bf16 bit patterns.
 */
#ifndef KVOFF_ORACLE_H
#define KVOFF_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F16 = 1, ORACLE_BF16 = 2 };

/* Exact value of an fp16 / bf16 bit pattern. */
double oracle_widen(uint16_t bits, int dtype);

/* 2 * L * Hkv * d * S * es: bytes of a full KV cache (guide, "The
 * Long-Context Decoding Memory Wall", KV cache size equation). */
int64_t oracle_kv_cache_bytes(int64_t L, int64_t Hkv, int64_t d, int64_t S, int64_t es);

/* 2 * Hkv * bs * d * es: bytes of one block record holding K and V of every
 * KV head (guide simulator, GatherScatterEngine bytes_per_block). */
int64_t oracle_rec_bytes(int64_t Hkv, int64_t bs, int64_t d, int64_t es);

/* Digest of every block: K is [ctx][Hkv][d]; D is [nb][Hkv][d] fp32 with
 * nb = ceil(ctx / bs); the last block may hold fewer than bs tokens. */
void oracle_digest(const uint16_t* K, int dtype, int64_t ctx, int Hkv, int d, int bs, float* D);

/* SoloHead score of every block: q is [Hq][d], D is [nb][Hkv][d], S is [nb]. */
void oracle_score(const uint16_t* q, int dtype, int Hq, int Hkv, int d,
                  const float* D, int64_t nb, double* S);

/* Per-KV-head score: S is [Hkv][nb]. */
void oracle_score_headwise(const uint16_t* q, int dtype, int Hq, int Hkv, int d,
                           const float* D, int64_t nb, double* S);

/* Consensus score of every block, the guide's SoloHead consensus rule
 * ("PulseInfer Guide", aiFetchly, section "SoloHead Sparse Selection",
 * consensus equation; its simulator's SoloHeadSelector applies it across KV
 * heads): S[b] = max_g S_g[b] + lambda * (sum_g S_g[b]) / Hkv, where S_g is
 * the per-KV-head score of oracle_score_headwise.  S is [nb]. */
void oracle_score_consensus(const uint16_t* q, int dtype, int Hq, int Hkv, int d,
                            const float* D, int64_t nb, double lambda, double* S);

/* Consensus score within each GQA group, the scope the guide's text gives
 * ("PulseInfer Guide", aiFetchly, section "SoloHead Sparse Selection":
 * consensus taken over the query heads of a GQA group):
 *   S[g][b] = max_{h in g} s_h[b] + lambda * (sum_{h in g} s_h[b]) / G,
 *   s_h[b]  = sum_j q[h][j] * D[b][g][j]  (the per-query-head score).
 * One ranking per KV head, as in the headwise layout.  S is [Hkv][nb]. */
void oracle_score_group_consensus(const uint16_t* q, int dtype, int Hq, int Hkv, int d,
                                  const float* D, int64_t nb, double lambda, double* S);

/* Top-k selection over nb scores: sel receives K = min(k, nb) block ids in
 * ascending order; returns K, or -1 if k < 1. */
int64_t oracle_select(const double* S, int64_t nb, int64_t k, int32_t* sel);

/* Block records rec[nb][Hkv][2][bs][d]: K then V rows of each KV head; rows
 * past the end of the context are zero. */
void oracle_records(const uint16_t* K, const uint16_t* V, int64_t ctx, int Hkv, int d, int bs,
                    uint16_t* rec);

/* Coalesced transfers of one request's shared selection: maximal runs of
 * consecutive block ids that are selected and not resident (hit == NULL:
 * none resident).  Writes the first rank and length (blocks) of each run
 * when the arrays are non-NULL; returns the number of runs. */
int64_t oracle_runs(const int32_t* sel, int64_t K, const uint8_t* hit,
                    int32_t* run_first_rank, int32_t* run_len);

/* Per-head recall of the fragmentation baseline: one transfer per selected,
 * non-resident (block, KV head) slice.  sel is [nsets][stride], counts[s]
 * entries valid.  Returns the number of slices. */
int64_t oracle_headwise_transfers(const int32_t* sel, const int64_t* counts, int nsets,
                                  int64_t stride, const uint8_t* hit);

/* Size of the union of nsets block-id sets (each sorted or not). */
int64_t oracle_union_count(const int32_t* sel, const int64_t* counts, int nsets, int64_t stride);

/* Sparse GQA decode attention in fp32 over the valid tokens of the nsel
 * selected blocks (ascending ids): q [Hq][d], K and V [ctx][Hkv][d],
 * out [Hq][d] fp32.  When sel is NULL every block is used. */
void oracle_attend_f32(const uint16_t* q, const uint16_t* K, const uint16_t* V, int dtype,
                       int64_t ctx, int Hq, int Hkv, int d, int bs,
                       const int32_t* sel, int64_t nsel, float* out);

/* The same in fp64; wsum (nullable, [Hq]) receives sum_t w_t / Z per head. */
void oracle_attend_f64(const uint16_t* q, const uint16_t* K, const uint16_t* V, int dtype,
                       int64_t ctx, int Hq, int Hkv, int d, int bs,
                       const int32_t* sel, int64_t nsel, double* out, double* wsum);

/* Headwise sparse attention in fp32: head h attends over the blocks that KV
 * head g = floor(h/G) selected, sel is [Hkv][stride] with nsel entries each. */
void oracle_attend_headwise_f32(const uint16_t* q, const uint16_t* K, const uint16_t* V,
                                int dtype, int64_t ctx, int Hq, int Hkv, int d, int bs,
                                const int32_t* sel, int64_t nsel, int64_t stride, float* out);

/* Attention mass a selection keeps (the quantity behind the guide's
 * "attention mass preserved" figure, section "SoloHead Sparse Selection"):
 * for each query head h, with fp64 logits z_t = <q_h, K_t[g]> / sqrt(d) over
 * all ctx tokens and w_t = exp(z_t - max z),
 *   mass[h] = (sum of w_t over the valid tokens of the blocks KV head
 *              g = floor(h/G) selected) / (sum of w_t over all tokens).
 * sel is [nsets][stride] with counts[s] entries in set s; nsets is 1 (one
 * set shared by every head) or Hkv (one set per KV head). */
void oracle_attention_mass(const uint16_t* q, const uint16_t* K, int dtype, int64_t ctx, int Hq,
                           int Hkv, int d, int bs, const int32_t* sel, const int64_t* counts,
                           int nsets, int64_t stride, double* mass);

/* Dense decode attention in fp64 over all ctx tokens, by token index alone
 * (no block bookkeeping): the textbook definition. */
void oracle_dense_f64(const uint16_t* q, const uint16_t* K, const uint16_t* V, int dtype,
                      int64_t ctx, int Hq, int Hkv, int d, double* out);

#ifdef __cplusplus
}
#endif
#endif
