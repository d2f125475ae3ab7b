// select.hip - block scoring and SoloHead / headwise top-k (kvoff_select).
//
// SoloHead ("PulseInfer Guide", aiFetchly, section "SoloHead Sparse
// Selection") replaces per-head block choices with one block set shared by
// all heads.  Scores use the rule fixed in kvoff.h:
//   S[b] = sum_h sum_j q[h][j] * D[b][floor(h/G)][j]
//        = sum_g <u_g, D[b][g]>,  u_g = sum of the G query heads of group g,
// evaluated in fp64 (u_g in fp64 from the exact fp16/bf16 inputs; digests
// widened exactly).  fp64 keeps the score error near 1e-12, far below any
// gap that separates rank K from rank K+1, so the selection does not depend
// on summation order.
//
// score_kernel: HBM-bound streaming of the fp32 digests.  Each wave handles
// SCORE_BPW consecutive blocks of one request; a lane loads 16 bytes per
// 1 KiB chunk of a block's [Hkv][d] digest row (coalesced dwordx4 loads), does
// fp64 FMAs against its slice of u, and the wave reduces with DPP lane moves
// inside rows of 16 lanes and shuffles across rows.
//
// Consensus modes: across KV heads (KVOFF_CONSENSUS) the per-KV-head sums
// are combined into one shared score; within a GQA group
// (KVOFF_CONSENSUS_GROUP) each query head's sum is formed from the q rows in
// LDS and the group's max + lambda * mean is one score per KV head.
//
// Top-k: one workgroup per request (per (request, KV head) when headwise)
// runs an MSB-first radix select over order-preserving 64-bit keys of the
// fp64 scores (up to 8 passes of 8 bits, LDS histogram, stopping once the
// threshold bucket is taken whole), then an ordered compaction in block
// order that keeps every key above the threshold and the lowest-numbered
// keys equal to it.  Output is ascending block ids.  topk_regs_kernel keeps
// up to 64 keys per thread in registers (nb <= 16,384) and needs one barrier
// per pass; topk_kernel re-reads the scores for longer contexts.
#include <algorithm>
#include <cstdlib>

#include "kvoff_internal.h"

namespace kvoff {
namespace {

// blocks per wave of score_kernel (measured: 2 and 4 equal, 8 slower)
constexpr int SCORE_BPW = 2;
constexpr int SCORE_WG_BLOCKS = 4 * SCORE_BPW;

// digest loads with the nontemporal hint (KVOFF_SCORE_NT=0 turns it off)
bool score_nt() {
  static const bool v = [] {
    const char* e = std::getenv("KVOFF_SCORE_NT");
    return !(e && e[0] == '0');
  }();
  return v;
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct ScoreArgs {
  BatchIds batch;
  const ReqDev* reqs;
  const uint16_t* q;
  const float* digest;
  double* scores;
  int64_t stride;
  int64_t nb_lo;  // the fewest blocks of any request of the batch, at launch
  int32_t Hq, Hkv, G, bf16;
  double lambda;  // consensus mode only
};

enum { MODE_SOLO = 0, MODE_HEADWISE = 1, MODE_CONSENSUS = 2, MODE_GROUP = 3 };

// fp64 lane moves within a row of 16 lanes (DPP: no trip through the LDS
// crossbar that a shuffle takes)
template <int CTRL>
__device__ __forceinline__ double dpp_move(double x) {
  const int lo = __double2loint(x), hi = __double2hiint(x);
  return __hiloint2double(__builtin_amdgcn_update_dpp(hi, hi, CTRL, 0xF, 0xF, false),
                          __builtin_amdgcn_update_dpp(lo, lo, CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of 32 lanes, the result in every lane of the
// group: xor 1 and xor 2 inside quads, then the mirrored half of each 8 and
// each 16 lanes (by then every lane of a quad / of 8 lanes holds the same
// partial), then one shuffle across the two rows.  Additions commute, so
// every lane ends with the same bits.
__device__ __forceinline__ double sum32(double v) {
  v += dpp_move<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_move<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_move<0x141>(v);  // row_half_mirror
  v += dpp_move<0x140>(v);  // row_mirror
  return v + __shfl_xor(v, 16);
}

// x from lane (lane ^ m), m < 32 a constant once loops are unrolled: DPP
// quad permutes for 1 and 2, a shuffle otherwise
__device__ __forceinline__ double xor_move(double x, int m) {
  if (m == 1) return dpp_move<0xB1>(x);  // quad_perm [1,0,3,2]
  if (m == 2) return dpp_move<0x4E>(x);  // quad_perm [2,3,0,1]
  return __shfl_xor(x, m);
}

template <bool BF16>
__device__ __forceinline__ double widen_t(uint16_t h) {
  if constexpr (BF16) return (double)__uint_as_float((uint32_t)h << 16);
  else return (double)__builtin_bit_cast(_Float16, h);
}

// GG: the group size G as a constant (consensus within GQA groups only)
template <int NC, int MODE, bool BF16, bool NT, int GG>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
  __shared__ double u_s[NC * 256];
  extern __shared__ uint4 q_s[];  // the request's q rows, Hq * 16 chunks of 16 bytes
  const int r = blockIdx.y;
  const int64_t b0 = (int64_t)blockIdx.x * SCORE_WG_BLOCKS;
  // A workgroup whose blocks all lie below the batch's shortest request
  // issues its digest loads at once; only the others first wait for their
  // request's block count (and leave if they hold no block of it).  The
  // count stands in for the request's own one: every block test below is
  // against it, and all of this workgroup's blocks pass.
  int64_t nb;
  if (b0 + SCORE_WG_BLOCKS <= a.nb_lo) {
    nb = b0 + SCORE_WG_BLOCKS;
  } else {
    nb = a.reqs[a.batch.id[r]].nb;
    if (b0 >= nb) return;  // uniform over the workgroup
  }
  const int F = a.Hkv * kHeadDim;
  const int tid = threadIdx.x;

  // Load order: the digests first, then the request's q rows.  Loads retire
  // in issue order, so waiting for the q rows waits for the digests too:
  // one memory round trip covers both, and the q -> u_g preamble runs while
  // nothing else is outstanding.
  // Every load is unconditional (block index clamped to the last block,
  // column clamped inside the row) so all of them are in flight together;
  // results of clamped blocks are not stored, clamped columns meet u = 0.
  const float* dr = a.digest + (int64_t)r * a.stride * F;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t bw = b0 + wave * SCORE_BPW;
  float4 v[SCORE_BPW][NC];
#pragma unroll
  for (int k = 0; k < SCORE_BPW; ++k) {
    const int64_t b = min<int64_t>(bw + k, nb - 1);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int idx = min(c * 256 + lane * 4, F - 4);
      const f32x4_t* p = reinterpret_cast<const f32x4_t*>(dr + b * F + idx);
      f32x4_t x;
      if constexpr (NT)
        x = __builtin_nontemporal_load(p);
      else
        x = *p;
      v[k][c] = make_float4(x[0], x[1], x[2], x[3]);
    }
  }
  // q rows: 4 chunks of 16 bytes per thread (Hq <= 64 in one round); the
  // LDS copy has room for all 4, so stores are unconditional too
  const uint4* qr = reinterpret_cast<const uint4*>(a.q + (int64_t)r * a.Hq * kHeadDim);
  const int nq = a.Hq * (kHeadDim / 8);
  uint4 qw[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) qw[c] = qr[min(c * 256 + tid, nq - 1)];
#pragma unroll
  for (int c = 0; c < 4; ++c) q_s[c * 256 + tid] = qw[c];
  for (int i = 4 * 256 + tid; i < nq; i += 256) q_s[i] = qr[i];  // Hq > 64 only
  __syncthreads();

  // u_g = sum of the group's G query heads, in fp64: thread (g, 8-dim group)
  for (int t = tid; t < (MODE == MODE_GROUP ? 0 : NC * 32); t += 256) {
    const int g = t >> 4, dg = t & 15;
    double s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = 0.0;
    if (g < a.Hkv) {
      for (int i = 0; i < a.G; ++i) {
        const uint4 w = q_s[(g * a.G + i) * (kHeadDim / 8) + dg];
        const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[2 * e] += widen_t<BF16>((uint16_t)(x[e] & 0xffffu));
          s[2 * e + 1] += widen_t<BF16>((uint16_t)(x[e] >> 16));
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) u_s[t * 8 + e] = s[e];
  }
  __syncthreads();

  if constexpr (MODE == MODE_GROUP) {
    // consensus within each GQA group: per query head h of group g,
    // s_h = <q_h, D[b][g]>; S_g = max_h s_h + lambda * mean_h s_h.  Lane
    // holds dims idx..idx+3 of KV head idx/128 in chunk c (chunk c covers
    // heads 2c and 2c+1 in lanes 0-31 and 32-63); dims past the row
    // contribute nothing.  The GG per-head partials of a lane are summed over
    // its 32 lanes by a reduce-scatter: at step st (lane bit st, st < log2
    // GG) a lane keeps half of its values and adds the partner lane's copies
    // of them, so after log2 GG steps it holds one head's sum over GG lanes,
    // and the remaining steps of the 32-lane butterfly complete it.  The
    // group's head sums then sit in the lanes that differ in bits 0 .. log2
    // GG - 1, where a butterfly takes their max and their sum.  Additions
    // commute, so every lane ends with the same bits.  (Sharing each q
    // slice's widening between the wave's two blocks needs 116 VGPRs instead
    // of 72 at G = 4 and was slower: 28.3 against 23.1 us.)
    static_assert(GG >= 1 && GG <= 16 && (GG & (GG - 1)) == 0, "group size");
    constexpr int LG = GG >= 16 ? 4 : GG >= 8 ? 3 : GG >= 4 ? 2 : GG >= 2 ? 1 : 0;
    const uint16_t* q16 = reinterpret_cast<const uint16_t*>(q_s);
#pragma unroll
    for (int k = 0; k < SCORE_BPW; ++k) {
      const int64_t b = bw + k;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int idx = c * 256 + lane * 4;
        const int g = min(idx, F - 4) / kHeadDim, j0 = idx % kHeadDim;
        double p[GG];
#pragma unroll
        for (int i = 0; i < GG; ++i) {
          double acc = 0.0;
          if (idx < F) {
            const uint2 w = *reinterpret_cast<const uint2*>(q16 + (g * GG + i) * kHeadDim + j0);
            acc = fma(widen_t<BF16>((uint16_t)(w.x & 0xffffu)), (double)v[k][c].x, acc);
            acc = fma(widen_t<BF16>((uint16_t)(w.x >> 16)), (double)v[k][c].y, acc);
            acc = fma(widen_t<BF16>((uint16_t)(w.y & 0xffffu)), (double)v[k][c].z, acc);
            acc = fma(widen_t<BF16>((uint16_t)(w.y >> 16)), (double)v[k][c].w, acc);
          }
          p[i] = acc;
        }
#pragma unroll
        for (int st = 0; st < LG; ++st) {
          const int half = GG >> (st + 1);
          const bool up = (lane >> st) & 1;
#pragma unroll
          for (int j = 0; j < half; ++j) {
            const double keep = up ? p[j + half] : p[j];
            const double send = up ? p[j] : p[j + half];
            p[j] = keep + xor_move(send, 1 << st);
          }
        }
        double sum = p[0];
#pragma unroll
        for (int st = LG; st < 5; ++st) sum += xor_move(sum, 1 << st);
        double mx = sum, sm = sum;
#pragma unroll
        for (int st = 0; st < LG; ++st) {
          mx = fmax(mx, xor_move(mx, 1 << st));
          sm += xor_move(sm, 1 << st);
        }
        const int gw = (c * 256 + (lane & 32) * 4) / kHeadDim;  // the half's KV head
        if ((lane & 31) == 0 && b < nb && gw < a.Hkv)
          a.scores[((int64_t)r * a.Hkv + gw) * a.stride + b] = mx + a.lambda * (sm / (double)GG);
      }
    }
    return;
  }

  double u[NC][4];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) u[c][e] = u_s[c * 256 + lane * 4 + e];

#pragma unroll
  for (int k = 0; k < SCORE_BPW; ++k) {
    const int64_t b = bw + k;
    if constexpr (MODE == MODE_SOLO) {
      double acc = 0.0;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        acc = fma(u[c][0], (double)v[k][c].x, acc);
        acc = fma(u[c][1], (double)v[k][c].y, acc);
        acc = fma(u[c][2], (double)v[k][c].z, acc);
        acc = fma(u[c][3], (double)v[k][c].w, acc);
      }
      acc = sum32(acc);
      acc += __shfl_xor(acc, 32);
      if (lane == 0 && b < nb) a.scores[(int64_t)r * a.stride + b] = acc;
    } else {
      // per-KV-head sums: a KV head's 128 dims are 32 consecutive lanes of
      // one chunk, so chunk c holds heads 2c (lanes 0-31) and 2c+1 (32-63).
      // The NC chunk partials are summed over their 32 lanes by a
      // reduce-scatter, as in the GQA-group mode: after log2 NC halving steps
      // lane bits 0 .. log2 NC - 1 name the lane's chunk, and the rest of
      // the butterfly completes its sum.
      constexpr int LN = NC >= 8 ? 3 : NC >= 4 ? 2 : NC >= 2 ? 1 : 0;
      double p[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        double acc = 0.0;
        acc = fma(u[c][0], (double)v[k][c].x, acc);
        acc = fma(u[c][1], (double)v[k][c].y, acc);
        acc = fma(u[c][2], (double)v[k][c].z, acc);
        acc = fma(u[c][3], (double)v[k][c].w, acc);
        p[c] = acc;
      }
      int c = 0;  // the chunk whose sum this lane ends with
#pragma unroll
      for (int st = 0; st < LN; ++st) {
        const int half = NC >> (st + 1);
        const bool up = (lane >> st) & 1;
        c += up ? half : 0;
#pragma unroll
        for (int j = 0; j < half; ++j) {
          const double keep = up ? p[j + half] : p[j];
          const double send = up ? p[j] : p[j + half];
          p[j] = keep + xor_move(send, 1 << st);
        }
      }
      double sg = p[0];
#pragma unroll
      for (int st = LN; st < 5; ++st) sg += xor_move(sg, 1 << st);
      const int g = 2 * c + (lane >> 5);  // this lane's KV head
      if constexpr (MODE == MODE_HEADWISE) {
        if ((lane & 31) < NC && b < nb && g < a.Hkv)
          a.scores[((int64_t)r * a.Hkv + g) * a.stride + b] = sg;
      } else {
        // consensus: S = max_g S_g + lambda * mean_g S_g over the KV heads
        double mx = g < a.Hkv ? sg : -INFINITY, sm = g < a.Hkv ? sg : 0.0;
#pragma unroll
        for (int st = 0; st < LN; ++st) {
          mx = fmax(mx, xor_move(mx, 1 << st));
          sm += xor_move(sm, 1 << st);
        }
        mx = fmax(mx, __shfl_xor(mx, 32));
        sm += __shfl_xor(sm, 32);
        if (lane == 0 && b < nb) a.scores[(int64_t)r * a.stride + b] = mx + a.lambda * (sm / (double)a.Hkv);
      }
    }
  }
}

struct TopkArgs {
  BatchIds batch;
  const ReqDev* reqs;
  const double* scores;
  int64_t stride;
  int32_t* sel_idx;
  int32_t* sel_cnt;
  int32_t k_stride;
  int32_t Hkv;
  int32_t k[KVOFF_MAX_BATCH];
};

// order-preserving key: larger score -> larger key; -0.0 keys as +0.0
__device__ __forceinline__ uint64_t score_key(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  if ((u << 1) == 0) u = 0;
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Streaming top-k for long contexts (more blocks than topk_regs_kernel keeps
// in registers): the scores are re-read from memory in every pass.
template <bool HW>
__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_digit, s_above, s_count;
  __shared__ uint32_t w_take[4], w_eq[4];

  const int r = HW ? blockIdx.x / a.Hkv : blockIdx.x;
  const int g = HW ? blockIdx.x % a.Hkv : 0;
  const ReqDev rq = a.reqs[a.batch.id[r]];
  const int64_t row = HW ? (int64_t)r * a.Hkv + g : (int64_t)r;
  const double* S = a.scores + row * a.stride;
  int32_t* out = a.sel_idx + row * a.k_stride;
  const int nb = rq.nb;
  const int K = a.k[r] < nb ? a.k[r] : nb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunks = (nb + 255) / 256;

  auto key_at = [&](int k) -> uint64_t { return score_key(S[min(tid + 256 * k, nb - 1)]); };

  uint64_t prefix = 0, mask = 0;
  uint32_t need = (uint32_t)K;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    for (int kk = 0; kk < chunks; ++kk) {
      const uint64_t key = key_at(kk);
      if (tid + 256 * kk < nb && (key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds digits 255-4l .. 252-4l (descending order)
      uint32_t c[4], local = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[e] = hist[255 - 4 * lane - e];
        local += c[e];
      }
      uint32_t incl = local;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const uint32_t o = __shfl_up(incl, m);
        if (lane >= m) incl += o;
      }
      uint32_t run = incl - local;  // keys in higher digits
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (run < need && need <= run + c[e]) {
          s_digit = 255u - 4u * lane - e;
          s_above = run;
          s_count = c[e];
        }
        run += c[e];
      }
    }
    __syncthreads();
    prefix |= (uint64_t)s_digit << shift;
    mask |= 255ull << shift;
    need -= s_above;
    const bool whole_bucket = s_count == need;  // every key of the bucket is taken
    __syncthreads();
    if (whole_bucket) break;
  }
  // selected: masked key above the prefix, or equal to it and among the
  // `need` lowest block ids with that masked key

  uint32_t taken = 0, eq_seen = 0;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  {  // chunks of 256 keys in block order
    for (int kk = 0; kk < chunks; ++kk) {
      const int i = tid + 256 * kk;
      const bool valid = i < nb;
      const uint64_t mk = key_at(kk) & mask;
      const bool gt = valid && mk > prefix;
      const bool eq = valid && mk == prefix;
      const uint64_t eq_b = __ballot(eq);
      if (lane == 0) w_eq[wave] = (uint32_t)__popcll(eq_b);
      __syncthreads();
      uint32_t eq_before = eq_seen + (uint32_t)__popcll(eq_b & lt_mask);
      uint32_t eq_total = 0;
      for (int w = 0; w < 4; ++w) {
        if (w < wave) eq_before += w_eq[w];
        eq_total += w_eq[w];
      }
      const bool take = gt || (eq && eq_before < need);
      const uint64_t tk_b = __ballot(take);
      if (lane == 0) w_take[wave] = (uint32_t)__popcll(tk_b);
      __syncthreads();
      uint32_t pos = taken + (uint32_t)__popcll(tk_b & lt_mask);
      uint32_t tk_total = 0;
      for (int w = 0; w < 4; ++w) {
        if (w < wave) pos += w_take[w];
        tk_total += w_take[w];
      }
      if (take && pos < (uint32_t)K) out[pos] = i;  // pos < K by construction
      taken += tk_total;
      eq_seen += eq_total;
      __syncthreads();
    }
  }
  for (int i = K + tid; i < a.k_stride; i += 256) out[i] = -1;
  if (tid == 0 && g == 0) a.sel_cnt[r] = K;
}

// Register-resident top-k (nb <= 256*KPT, keys of blocks tid + 256*k): the
// same radix select and selection rule as topk_kernel, with one barrier per
// pass and one for the whole compaction.
//   passes      three histograms in rotation: pass p counts into hist[p%3]
//               and clears hist[(p+1)%3], whose last readers (the scans of
//               pass p-2) finished before the barrier of pass p-1.  After
//               the pass's barrier every wave scans hist[p%3] itself, so the
//               chosen digit needs no broadcast through LDS.
//   compaction  per 256-key chunk, ballots rank each lane's key among the
//               wave's keys above the threshold (gt) and equal to it (eq);
//               the waves' counts of every chunk cross through LDS once.  A
//               key with gt_before / eq_before such keys at lower block ids
//               is taken if gt, or if eq and eq_before < need, and lands at
//               gt_before + min(eq_before, need).
template <bool HW, int KPT>
__global__ __launch_bounds__(256) void topk_regs_kernel(TopkArgs a) {
  static_assert(KPT > 0 && KPT <= 64, "keys per thread");
  __shared__ uint32_t hist[3][256];
  __shared__ uint32_t wcnt[KPT][4];  // per chunk and wave: gt count << 16 | eq count

  const int r = HW ? blockIdx.x / a.Hkv : blockIdx.x;
  const int g = HW ? blockIdx.x % a.Hkv : 0;
  const ReqDev rq = a.reqs[a.batch.id[r]];
  const int64_t row = HW ? (int64_t)r * a.Hkv + g : (int64_t)r;
  const double* S = a.scores + row * a.stride;
  int32_t* out = a.sel_idx + row * a.k_stride;
  const int nb = rq.nb;
  const int K = a.k[r] < nb ? a.k[r] : nb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // the keys load together with the block count, not after it: indices are
  // clamped inside the row (stride entries); keys past the count are never
  // counted or taken
  uint64_t keys[KPT];
#pragma unroll
  for (int k = 0; k < KPT; ++k) keys[k] = score_key(S[min<int64_t>(tid + 256 * k, a.stride - 1)]);

  hist[0][tid] = 0;
  __syncthreads();
  uint64_t prefix = 0, mask = 0;
  uint32_t need = (uint32_t)K;  // keys still to take from the bucket of `prefix`
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    uint32_t* h = hist[pass % 3];
    hist[(pass + 1) % 3][tid] = 0;
#pragma unroll
    for (int k = 0; k < KPT; ++k)
      if (tid + 256 * k < nb && (keys[k] & mask) == prefix) atomicAdd(&h[(keys[k] >> shift) & 255u], 1u);
    __syncthreads();
    // lane l holds digits 255-4l .. 252-4l (descending order)
    uint32_t c[4], local = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c[e] = h[255 - 4 * lane - e];
      local += c[e];
    }
    uint32_t incl = local;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const uint32_t o = __shfl_up(incl, m);
      if (lane >= m) incl += o;
    }
    uint32_t run = incl - local;  // keys in higher digits
    int f_digit = -1;
    uint32_t f_above = 0, f_count = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (run < need && need <= run + c[e]) {  // one digit of one lane: the bucket holding rank `need`
        f_digit = 255 - 4 * lane - e;
        f_above = run;
        f_count = c[e];
      }
      run += c[e];
    }
    const int src = __ffsll((unsigned long long)__ballot(f_digit >= 0)) - 1;
    const uint32_t digit = (uint32_t)__shfl(f_digit, src);
    const uint32_t above = (uint32_t)__shfl((int)f_above, src);
    const uint32_t count = (uint32_t)__shfl((int)f_count, src);
    prefix |= (uint64_t)digit << shift;
    mask |= 255ull << shift;
    need -= above;
    if (count == need) break;  // every key of the bucket is taken (uniform: all waves read one histogram)
  }

  const uint64_t lt_mask = (1ull << lane) - 1ull;
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const bool valid = tid + 256 * k < nb;
    const uint64_t mk = keys[k] & mask;
    const uint64_t gt_b = __ballot(valid && mk > prefix);
    const uint64_t eq_b = __ballot(valid && mk == prefix);
    if (lane == 0) wcnt[k][wave] = (uint32_t)__popcll(gt_b) << 16 | (uint32_t)__popcll(eq_b);
  }
  __syncthreads();
  uint32_t before = 0;  // gt << 16 | eq counts of the chunks already passed
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const bool valid = tid + 256 * k < nb;
    const uint64_t mk = keys[k] & mask;
    const bool gt = valid && mk > prefix, eq = valid && mk == prefix;
    const uint64_t gt_b = __ballot(gt);
    const uint64_t eq_b = __ballot(eq);
    uint32_t base = before;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t cw = wcnt[k][w];
      if (w < wave) base += cw;
      before += cw;
    }
    const uint32_t gt_before = (base >> 16) + (uint32_t)__popcll(gt_b & lt_mask);
    const uint32_t eq_before = (base & 0xffffu) + (uint32_t)__popcll(eq_b & lt_mask);
    const uint32_t pos = gt_before + min(eq_before, need);
    if ((gt || (eq && eq_before < need)) && pos < (uint32_t)K) out[pos] = tid + 256 * k;  // pos < K by construction
  }
  for (int i = K + tid; i < a.k_stride; i += 256) out[i] = -1;
  if (tid == 0 && g == 0) a.sel_cnt[r] = K;
}

template <int KPT>
void topk_launch(const TopkArgs& a, dim3 grid, bool hw, hipStream_t s, KEv ev) {
  if constexpr (KPT > 0) {
    if (hw)
      KVOFF_LAUNCH(ev, (topk_regs_kernel<true, KPT>), grid, dim3(256), 0, s, a);
    else
      KVOFF_LAUNCH(ev, (topk_regs_kernel<false, KPT>), grid, dim3(256), 0, s, a);
  } else {
    if (hw)
      KVOFF_LAUNCH(ev, (topk_kernel<true>), grid, dim3(256), 0, s, a);
    else
      KVOFF_LAUNCH(ev, (topk_kernel<false>), grid, dim3(256), 0, s, a);
  }
}

template <int NC, int MODE, bool NT, int GG>
void score_launch_g(const ScoreArgs& a, int64_t max_nb, hipStream_t s, KEv ev) {
  const uint32_t lds = (uint32_t)std::max<size_t>((size_t)a.Hq * kHeadDim * 2, 4 * 256 * 16);  // staged q rows
  const dim3 grid((unsigned)((max_nb + SCORE_WG_BLOCKS - 1) / SCORE_WG_BLOCKS), (unsigned)a.batch.n);
  if (a.bf16)
    KVOFF_LAUNCH(ev, (score_kernel<NC, MODE, true, NT, GG>), grid, dim3(256), lds, s, a);
  else
    KVOFF_LAUNCH(ev, (score_kernel<NC, MODE, false, NT, GG>), grid, dim3(256), lds, s, a);
}

template <int NC, int MODE, bool NT>
void score_launch_b(const ScoreArgs& a, int64_t max_nb, hipStream_t s, KEv ev) {
  if constexpr (MODE == MODE_GROUP) {
    switch (a.G) {
      case 1: return score_launch_g<NC, MODE, NT, 1>(a, max_nb, s, ev);
      case 2: return score_launch_g<NC, MODE, NT, 2>(a, max_nb, s, ev);
      case 4: return score_launch_g<NC, MODE, NT, 4>(a, max_nb, s, ev);
      case 8: return score_launch_g<NC, MODE, NT, 8>(a, max_nb, s, ev);
      default: return score_launch_g<NC, MODE, NT, 16>(a, max_nb, s, ev);
    }
  } else {
    score_launch_g<NC, MODE, NT, 0>(a, max_nb, s, ev);
  }
}

template <int NC, int MODE>
void score_launch_m(const ScoreArgs& a, int64_t max_nb, hipStream_t s, KEv ev) {
  if (score_nt())
    score_launch_b<NC, MODE, true>(a, max_nb, s, ev);
  else
    score_launch_b<NC, MODE, false>(a, max_nb, s, ev);
}

template <int NC>
void score_launch(const ScoreArgs& a, int64_t max_nb, int mode, hipStream_t s, KEv ev) {
  if (mode == KVOFF_HEADWISE)
    score_launch_m<NC, MODE_HEADWISE>(a, max_nb, s, ev);
  else if (mode == KVOFF_CONSENSUS)
    score_launch_m<NC, MODE_CONSENSUS>(a, max_nb, s, ev);
  else if (mode == KVOFF_CONSENSUS_GROUP)
    score_launch_m<NC, MODE_GROUP>(a, max_nb, s, ev);
  else
    score_launch_m<NC, MODE_SOLO>(a, max_nb, s, ev);
}

}  // namespace

int launch_score(const kvoff_ctx* ctx, const BatchIds& b, int64_t min_nb, int64_t max_nb,
                 const void* q_dev, const float* digest_dev, int64_t digest_stride, int32_t mode,
                 double* scores_dev, hipStream_t stream) {
  ScoreArgs a;
  a.batch = b;
  a.reqs = ctx->d_reqs;
  a.q = (const uint16_t*)q_dev;
  a.digest = digest_dev;
  a.scores = scores_dev;
  a.stride = digest_stride;
  a.nb_lo = min_nb;
  a.Hq = ctx->cfg.num_q_heads;
  a.Hkv = ctx->cfg.num_kv_heads;
  a.G = ctx->G;
  a.bf16 = ctx->cfg.dtype == KVOFF_BF16;
  a.lambda = ctx->consensus_lambda;
  const int F = a.Hkv * kHeadDim;
  const int NC = (F + 255) / 256;
  const KEv ev = kernel_events(ctx, KT_SCORE);
  switch (NC) {
    case 1: score_launch<1>(a, max_nb, mode, stream, ev); break;
    case 2: score_launch<2>(a, max_nb, mode, stream, ev); break;
    case 3:
    case 4: score_launch<4>(a, max_nb, mode, stream, ev); break;
    default: score_launch<8>(a, max_nb, mode, stream, ev); break;
  }
  KVOFF_HIP(hipGetLastError());
  return KVOFF_OK;
}

int launch_topk(const kvoff_ctx* ctx, const BatchIds& b, const int32_t* topk_host, int32_t mode,
                const double* scores_dev, int64_t digest_stride, int32_t* sel_idx_dev,
                int32_t* sel_cnt_dev, int32_t k_stride, hipStream_t stream) {
  TopkArgs a;
  a.batch = b;
  a.reqs = ctx->d_reqs;
  a.scores = scores_dev;
  a.stride = digest_stride;
  a.sel_idx = sel_idx_dev;
  a.sel_cnt = sel_cnt_dev;
  a.k_stride = k_stride;
  a.Hkv = ctx->cfg.num_kv_heads;
  for (int i = 0; i < KVOFF_MAX_BATCH; ++i) a.k[i] = i < b.n ? topk_host[i] : 0;
  int64_t max_nb = 0;
  for (int i = 0; i < b.n; ++i) max_nb = std::max<int64_t>(max_nb, ctx->reqs[b.id[i]].nb);
  const bool hw = mode == KVOFF_HEADWISE;
  const dim3 grid((unsigned)(hw ? b.n * a.Hkv : b.n));
  const KEv ev = kernel_events(ctx, KT_TOPK);
  if (max_nb <= 1024)
    topk_launch<4>(a, grid, hw, stream, ev);
  else if (max_nb <= 4096)
    topk_launch<16>(a, grid, hw, stream, ev);
  else if (max_nb <= 16384)
    topk_launch<64>(a, grid, hw, stream, ev);
  else
    topk_launch<0>(a, grid, hw, stream, ev);
  KVOFF_HIP(hipGetLastError());
  return KVOFF_OK;
}

}  // namespace kvoff
