/*
 * synth.h - seeded synthetic workload generator shared by the CPU oracle's
 * tests and by the GPU path's tests and benchmark.
 *
 * This module draws random numbers and lays them out; it holds none of the
 * sparse-offloading method's arithmetic (no digests, scores, selection,
 * recall or attention).  Every value is a pure function of
 * (seed, tag, layer, request, attempt, element index): the stream is
 * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
 * easy as 1, 2, 3", SC'11) used as a counter-based generator, so any slice
 * can be regenerated on its own and results do not depend on thread count.
 *
 * Normal variates use the Box-Muller transform on two 32-bit uniforms
 * u = (x + 0.5) / 2^32.  Values are produced in double precision, rounded to
 * float (round-to-nearest-even) and then to the storage type (bf16 or fp16,
 * round-to-nearest-even).
 */
#ifndef SYNTH_H
#define SYNTH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* storage types for generated tensors (bit patterns in uint16_t) */
enum { SYNTH_F16 = 1, SYNTH_BF16 = 2 };

/* stream tags: one independent Philox stream family per quantity */
enum {
  SYNTH_TAG_Q = 1,      /* query vectors                                 */
  SYNTH_TAG_K = 2,      /* keys                                          */
  SYNTH_TAG_V = 3,      /* values                                        */
  SYNTH_TAG_HOT = 4,    /* positions of planted hot blocks               */
  SYNTH_TAG_CTX = 5,    /* per-request context length draws              */
  SYNTH_TAG_FRAC = 6,   /* per-request top-k fraction draws               */
  SYNTH_TAG_RUNLEN = 7, /* run lengths of clustered hot blocks            */
  SYNTH_TAG_RUNPOS = 8, /* placement of clustered runs                    */
  SYNTH_TAG_POOL = 9    /* blocks already resident in the HBM block pool  */
};

/* Philox4x32-10 block function: out = philox(ctr, key). */
void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* n standard normals (double) of stream (seed, tag, layer, req, attempt),
 * elements [off, off + n). */
void synth_normals(uint64_t seed, uint32_t tag, uint32_t layer, uint32_t req,
                   uint32_t attempt, uint64_t off, int64_t n, double* out);

/* A uniform 32-bit word: element idx of stream (seed, tag, layer, req). */
uint32_t synth_u32(uint64_t seed, uint32_t tag, uint32_t layer, uint32_t req, uint64_t idx);

/* Uniform integer in [lo, hi] (inclusive), from synth_u32. */
int64_t synth_uniform_int(uint64_t seed, uint32_t tag, uint32_t layer, uint32_t req,
                          uint64_t idx, int64_t lo, int64_t hi);

/* Uniform double in (0, 1), from synth_u32. */
double synth_uniform01(uint64_t seed, uint32_t tag, uint32_t layer, uint32_t req, uint64_t idx);

/* Round a double to the storage type (via float, both steps nearest-even). */
uint16_t synth_quantize(double x, int dtype);

/* Query vectors q[Hq][d] of (layer, req): N(0,1) quantized to dtype. */
void synth_q(uint64_t seed, uint32_t layer, uint32_t req, int Hq, int d, int dtype,
             uint16_t* out);

/* Planting direction per KV head: u_g = sum of the quantized q_h over the
 * G = Hq/Hkv query heads h with floor(h/G) == g (in double), qhat_g = u_g/|u_g|.
 * out is [Hkv][d] doubles. */
void synth_qhat(const uint16_t* q, int dtype, int Hq, int Hkv, int d, double* out);

/* Keys or values of (layer, req): x[t][g][j] for t < n_tok.
 * tag is SYNTH_TAG_K or SYNTH_TAG_V.  Block b = t / bs uses attempt
 * attempts[b] (NULL = all 0).  When hot != NULL and hot[b] != 0, shift*qhat[g][j]
 * is added (in double) before quantization.  Multithreaded (OpenMP). */
void synth_kv(uint64_t seed, uint32_t tag, uint32_t layer, uint32_t req,
              int64_t n_tok, int Hkv, int d, int bs,
              const uint8_t* hot, const uint8_t* attempts,
              const double* qhat, double shift, int dtype, uint16_t* out);

/* Regenerate only the token rows of block b (rows [b*bs, min((b+1)*bs, n_tok)))
 * into out (which is the full [n_tok][Hkv][d] tensor). */
void synth_kv_block(uint64_t seed, uint32_t tag, uint32_t layer, uint32_t req,
                    int64_t n_tok, int Hkv, int d, int bs, int64_t b,
                    int hot, int attempt, const double* qhat, double shift,
                    int dtype, uint16_t* out);

/* n distinct values from [0, nb), uniform without replacement (partial
 * Fisher-Yates driven by stream (seed, tag, layer, req)); out sorted ascending. */
void synth_choose(uint64_t seed, uint32_t tag, uint32_t layer, uint32_t req,
                  int64_t nb, int64_t n, int32_t* out);

/* Clustered hot set: exactly k of nb blocks marked in mask, laid out as runs
 * whose lengths are drawn from U{1..max_run} (the last run truncated so the
 * total is k), consecutive runs separated by at least one unmarked block, and
 * the spare unmarked blocks spread uniformly over the gaps (stars and bars).
 * Returns the number of runs, or -1 if k runs cannot fit. */
int64_t synth_runs(uint64_t seed, uint32_t layer, uint32_t req, int64_t nb, int64_t k,
                   int max_run, uint8_t* mask);

#ifdef __cplusplus
}
#endif
#endif
