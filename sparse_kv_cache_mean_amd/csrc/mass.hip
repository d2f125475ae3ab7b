// mass.hip - attention mass a block selection keeps (kvoff_attention_mass).
//
// The guide ("PulseInfer Guide", aiFetchly, section "SoloHead Sparse
// Selection", attention mass preservation) assesses a shared block set by the
// share of the attention weight it keeps compared with per-head sets.  For
// each request r and query head h (KV head g = floor(h/G)):
//   z_t    = scale * <q_h, K_t[g]> over all valid tokens t of the context
//   mass_h = sum of exp(z_t - max z) over the tokens of the blocks g's set
//            holds / the same sum over every token.
// The keys are read from the pinned store over the host link (this is a
// diagnostic: the full context never has to be in HBM), so the kernel is
// bound by the link like the gather.  One workgroup per (request, KV head)
// streams that head's K slices block by block; lanes form the logits of all
// G query heads in fp32 (threads of one token split its 128 dims, summed with
// lane shuffles), and one thread per query head folds the block's logits
// into a running max and two fp64 sums (all tokens, selected tokens),
// rescaled whenever the max grows.
#include "kvoff_internal.h"

namespace kvoff {
namespace {

struct MassArgs {
  BatchIds batch;
  const ReqDev* reqs;
  const uint8_t* store;  // device-mapped pinned store
  const uint16_t* q;
  const int32_t* sel_idx;
  const int32_t* sel_cnt;
  double* mass;
  int64_t rec_bytes, slice_bytes;
  int32_t layer, Hq, Hkv, G, k_stride, hw;
  float scale;
};

constexpr int MAX_G = 16;

template <bool BF16>
__device__ __forceinline__ float widen16(uint32_t h) {
  if constexpr (BF16) return __uint_as_float(h << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

template <int BS, bool BF16>
__global__ __launch_bounds__(256) void mass_kernel(MassArgs a) {
  constexpr int D = kHeadDim;
  constexpr int TPT = 256 / BS;  // threads per token: 8 (bs 32) or 16 (bs 16)
  constexpr int DPT = D / TPT;   // dims per thread: 16 or 8
  constexpr int LPT = DPT / 8;   // 16-byte loads per thread: 2 or 1
  __shared__ float q_s[MAX_G][D];
  __shared__ float z_s[BS][MAX_G];

  const int r = blockIdx.x / a.Hkv, g = blockIdx.x % a.Hkv;
  const int tid = threadIdx.x;
  const ReqDev rq = a.reqs[a.batch.id[r]];
  const uint16_t* qg = a.q + ((int64_t)r * a.Hq + (int64_t)g * a.G) * D;
  for (int i = tid; i < a.G * D; i += 256) q_s[i / D][i % D] = widen16<BF16>(qg[i]);
  __syncthreads();

  const int tok = tid / TPT, part = tid % TPT;
  const int32_t* sel = a.sel_idx + (a.hw ? (int64_t)r * a.Hkv + g : (int64_t)r) * a.k_stride;
  const int cnt = min(a.sel_cnt[r], a.k_stride);
  const uint8_t* base =
      a.store + (rq.rec_base + (int64_t)a.layer * rq.nb) * a.rec_bytes + (int64_t)g * a.slice_bytes;
  double m = -INFINITY, z_all = 0.0, z_sel = 0.0;  // thread h < G: query head g*G + h
  int p = 0;                                       // position in the ascending set

  for (int b = 0; b < rq.nb; ++b) {
    // K rows of this head: [BS][D] at the start of the slice
    const uint16_t* Kb = reinterpret_cast<const uint16_t*>(base + (int64_t)b * a.rec_bytes);
    float kf[DPT];
#pragma unroll
    for (int l = 0; l < LPT; ++l) {
      const uint4 w = *reinterpret_cast<const uint4*>(Kb + tok * D + part * DPT + l * 8);
      const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[l * 8 + 2 * e] = widen16<BF16>(x[e] & 0xffffu);
        kf[l * 8 + 2 * e + 1] = widen16<BF16>(x[e] >> 16);
      }
    }
    __syncthreads();  // the previous block's logits have been consumed
    for (int h = 0; h < a.G; ++h) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < DPT; ++e) acc = fmaf(q_s[h][part * DPT + e], kf[e], acc);
#pragma unroll
      for (int o = 1; o < TPT; o <<= 1) acc += __shfl_xor(acc, o);
      if (part == 0) z_s[tok][h] = acc * a.scale;
    }
    __syncthreads();
    if (tid < a.G) {
      const int n_valid = (int)min<int64_t>(BS, (int64_t)rq.n_tokens - (int64_t)b * BS);
      while (p < cnt && sel[p] < b) ++p;
      const bool chosen = p < cnt && sel[p] == b;
      for (int t = 0; t < n_valid; ++t) {
        const double z = z_s[t][tid];
        if (z > m) {
          const double f = exp(m - z);
          z_all *= f;
          z_sel *= f;
          m = z;
        }
        const double w = exp(z - m);
        z_all += w;
        if (chosen) z_sel += w;
      }
    }
  }
  if (tid < a.G) a.mass[(int64_t)r * a.Hq + (int64_t)g * a.G + tid] = z_sel / z_all;
}

}  // namespace

int launch_mass(const kvoff_ctx* ctx, const BatchIds& b, int32_t layer, int32_t mode,
                const void* q_dev, const int32_t* sel_idx, const int32_t* sel_cnt,
                int32_t k_stride, float scale, double* mass_dev, hipStream_t stream) {
  if (ctx->G > MAX_G) return fail(KVOFF_EINVAL, "G = %d > %d", ctx->G, MAX_G);
  MassArgs a;
  a.batch = b;
  a.reqs = ctx->d_reqs;
  a.store = ctx->store_dev;
  a.q = (const uint16_t*)q_dev;
  a.sel_idx = sel_idx;
  a.sel_cnt = sel_cnt;
  a.mass = mass_dev;
  a.rec_bytes = ctx->rec_bytes;
  a.slice_bytes = ctx->slice_bytes;
  a.layer = layer;
  a.Hq = ctx->cfg.num_q_heads;
  a.Hkv = ctx->cfg.num_kv_heads;
  a.G = ctx->G;
  a.k_stride = k_stride;
  a.hw = mode == KVOFF_HEADWISE;
  a.scale = scale;
  const dim3 grid((unsigned)(b.n * a.Hkv));
  const bool bf16 = ctx->cfg.dtype == KVOFF_BF16;
  if (ctx->cfg.block_size == 16) {
    if (bf16) hipLaunchKernelGGL((mass_kernel<16, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((mass_kernel<16, false>), grid, dim3(256), 0, stream, a);
  } else {
    if (bf16) hipLaunchKernelGGL((mass_kernel<32, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((mass_kernel<32, false>), grid, dim3(256), 0, stream, a);
  }
  KVOFF_HIP(hipGetLastError());
  return KVOFF_OK;
}

}  // namespace kvoff
