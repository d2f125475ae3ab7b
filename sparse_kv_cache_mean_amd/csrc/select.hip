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
// fp64 FMAs against its slice of u, and the wave reduces with lane shuffles.
//
// topk_kernel: one workgroup per request (per (request, KV head) when
// headwise) runs an MSB-first radix select over order-preserving 64-bit keys
// of the fp64 scores (8 passes of 8 bits, LDS histogram), then an ordered
// compaction in block order that keeps every key above the threshold and the
// lowest-numbered keys equal to it.  Output is ascending block ids.
#include "kvoff_internal.h"

namespace kvoff {
namespace {

constexpr int SCORE_BPW = 4;
constexpr int SCORE_WG_BLOCKS = 4 * SCORE_BPW;

struct ScoreArgs {
  BatchIds batch;
  const ReqDev* reqs;
  const uint16_t* q;
  const float* digest;
  double* scores;
  int64_t stride;
  int32_t Hq, Hkv, G, bf16;
};

__device__ __forceinline__ double widen(uint16_t h, int bf16) {
  if (bf16) return (double)__uint_as_float((uint32_t)h << 16);
  return (double)__builtin_bit_cast(_Float16, h);
}

template <int NC, bool HW>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
  __shared__ double u_s[NC * 256];
  const int r = blockIdx.y;
  const ReqDev rq = a.reqs[a.batch.id[r]];
  const int64_t b0 = (int64_t)blockIdx.x * SCORE_WG_BLOCKS;
  if (b0 >= rq.nb) return;  // uniform over the workgroup
  const int F = a.Hkv * kHeadDim;

  const uint16_t* qr = a.q + (int64_t)r * a.Hq * kHeadDim;
  for (int idx = threadIdx.x; idx < NC * 256; idx += 256) {
    double s = 0.0;
    if (idx < F) {
      const int g = idx / kHeadDim, j = idx % kHeadDim;
      for (int i = 0; i < a.G; ++i) s += widen(qr[(g * a.G + i) * kHeadDim + j], a.bf16);
    }
    u_s[idx] = s;
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double u[NC][4];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) u[c][e] = u_s[c * 256 + lane * 4 + e];

  const float* dr = a.digest + (int64_t)r * a.stride * F;
  const int64_t bw = b0 + wave * SCORE_BPW;
  float4 v[SCORE_BPW][NC];
#pragma unroll
  for (int k = 0; k < SCORE_BPW; ++k)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int idx = c * 256 + lane * 4;
      const int64_t b = bw + k;
      v[k][c] = (b < rq.nb && idx < F)
                    ? *reinterpret_cast<const float4*>(dr + b * F + idx)
                    : make_float4(0.f, 0.f, 0.f, 0.f);
    }

#pragma unroll
  for (int k = 0; k < SCORE_BPW; ++k) {
    const int64_t b = bw + k;
    if (!HW) {
      double acc = 0.0;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        acc = fma(u[c][0], (double)v[k][c].x, acc);
        acc = fma(u[c][1], (double)v[k][c].y, acc);
        acc = fma(u[c][2], (double)v[k][c].z, acc);
        acc = fma(u[c][3], (double)v[k][c].w, acc);
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
      if (lane == 0 && b < rq.nb) a.scores[(int64_t)r * a.stride + b] = acc;
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        double acc = 0.0;
        acc = fma(u[c][0], (double)v[k][c].x, acc);
        acc = fma(u[c][1], (double)v[k][c].y, acc);
        acc = fma(u[c][2], (double)v[k][c].z, acc);
        acc = fma(u[c][3], (double)v[k][c].w, acc);
        // a KV head's 128 dims are 32 consecutive lanes of one chunk
#pragma unroll
        for (int m = 16; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
        const int g = (c * 256 + lane * 4) / kHeadDim;
        if ((lane & 31) == 0 && b < rq.nb && g < a.Hkv)
          a.scores[((int64_t)r * a.Hkv + g) * a.stride + b] = acc;
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

template <bool HW>
__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_digit, s_above;
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

  uint64_t prefix = 0, mask = 0;
  uint32_t need = (uint32_t)K;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < nb; i += 256) {
      const uint64_t key = score_key(S[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
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
        }
        run += c[e];
      }
    }
    __syncthreads();
    prefix |= (uint64_t)s_digit << shift;
    mask |= 255ull << shift;
    need -= s_above;
    __syncthreads();
  }
  const uint64_t T = prefix;  // the K-th largest key; take `need` of its copies

  uint32_t taken = 0, eq_seen = 0;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  for (int base = 0; base < nb; base += 256) {
    const int i = base + tid;
    const bool valid = i < nb;
    const uint64_t key = valid ? score_key(S[i]) : 0;
    const bool gt = valid && key > T;
    const bool eq = valid && key == T;
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
  for (int i = K + tid; i < a.k_stride; i += 256) out[i] = -1;
  if (tid == 0 && g == 0) a.sel_cnt[r] = K;
}

template <int NC>
void score_launch(const ScoreArgs& a, dim3 grid, bool hw, hipStream_t s) {
  if (hw)
    hipLaunchKernelGGL((score_kernel<NC, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((score_kernel<NC, false>), grid, dim3(256), 0, s, a);
}

}  // namespace

int launch_score(const kvoff_ctx* ctx, const BatchIds& b, int64_t max_nb, const void* q_dev,
                 const float* digest_dev, int64_t digest_stride, int32_t mode, double* scores_dev,
                 hipStream_t stream) {
  ScoreArgs a;
  a.batch = b;
  a.reqs = ctx->d_reqs;
  a.q = (const uint16_t*)q_dev;
  a.digest = digest_dev;
  a.scores = scores_dev;
  a.stride = digest_stride;
  a.Hq = ctx->cfg.num_q_heads;
  a.Hkv = ctx->cfg.num_kv_heads;
  a.G = ctx->G;
  a.bf16 = ctx->cfg.dtype == KVOFF_BF16;
  const int F = a.Hkv * kHeadDim;
  const int NC = (F + 255) / 256;
  dim3 grid((unsigned)((max_nb + SCORE_WG_BLOCKS - 1) / SCORE_WG_BLOCKS), (unsigned)b.n);
  const bool hw = mode == KVOFF_HEADWISE;
  switch (NC) {
    case 1: score_launch<1>(a, grid, hw, stream); break;
    case 2: score_launch<2>(a, grid, hw, stream); break;
    case 3:
    case 4: score_launch<4>(a, grid, hw, stream); break;
    default: score_launch<8>(a, grid, hw, stream); break;
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
  if (mode == KVOFF_HEADWISE)
    hipLaunchKernelGGL(topk_kernel<true>, dim3((unsigned)(b.n * a.Hkv)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(topk_kernel<false>, dim3((unsigned)b.n), dim3(256), 0, stream, a);
  KVOFF_HIP(hipGetLastError());
  return KVOFF_OK;
}

}  // namespace kvoff
