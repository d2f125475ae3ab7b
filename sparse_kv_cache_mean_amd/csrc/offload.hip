// offload.hip - digest build and block offload (kvoff_offload_blocks).
//
// PulseInfer's abstract keeps most historical KV blocks in CPU DRAM; this
// kernel produces both halves of that state for one (layer, request):
//   - the per-block key digest in HBM: D[b][g][j] = fp32 rounding of the
//     mean of K[t][g][j] over the block's valid tokens (fp64 sum in token
//     order, one fp64 division by the valid-token count);
//   - the block record in the pinned host store, written through its mapped
//     address: [Hkv][K,V][bs][d] elements, rows past the context end zero.
//
// Summation order: each (KV head, dim) is summed in fp64 over the block's
// valid tokens one after another in token order, the order of the plain
// definition, so the digest bits equal a sequential sum for every finite
// input (no reassociation: bf16 values 40 or more binades apart would round
// differently in another order).
//
// One workgroup per (block, KV head); 256 threads = 16 row groups x 16 lanes
// of 16 bytes (8 elements) across the 256-byte row move the K and V rows to
// the record and the key rows to LDS; then one thread per dim sums its
// column.
#include "kvoff_internal.h"

namespace kvoff {
namespace {

struct OffloadArgs {
  const uint16_t* K;
  const uint16_t* V;
  float* digest;
  uint8_t* rec0;  // device address of record (layer, request, block 0)
  int64_t rec_bytes;
  int64_t n_tok;
  int32_t Hkv;
  int32_t bf16;
};

__device__ __forceinline__ double widen(uint16_t h, int bf16) {
  if (bf16) return (double)__uint_as_float((uint32_t)h << 16);
  return (double)__builtin_bit_cast(_Float16, h);
}

template <int BS>
__global__ __launch_bounds__(256) void offload_kernel(OffloadArgs a) {
  constexpr int D = kHeadDim;
  constexpr int ROWS_PER_THREAD = BS / 16;
  __shared__ __align__(16) uint16_t k_s[BS][D];  // key rows of this (block, KV head)

  const int64_t b = blockIdx.x / a.Hkv;
  const int g = blockIdx.x % a.Hkv;
  const int t = threadIdx.x;
  const int dg = t & 15;       // 8-element column group
  const int rg = t >> 4;       // row group
  const int64_t tok0 = b * BS;
  const int n_valid = (int)min<int64_t>(BS, a.n_tok - tok0);

  uint8_t* rec = a.rec0 + b * a.rec_bytes + (int64_t)g * (2 * BS * D * 2);
#pragma unroll
  for (int i = 0; i < ROWS_PER_THREAD; ++i) {
    const int row = rg + 16 * i;
    const int64_t tok = tok0 + row;
    uint4 kx = make_uint4(0, 0, 0, 0), vx = make_uint4(0, 0, 0, 0);
    if (row < n_valid) {
      const int64_t off = (tok * a.Hkv + g) * D + dg * 8;
      kx = *reinterpret_cast<const uint4*>(a.K + off);
      vx = *reinterpret_cast<const uint4*>(a.V + off);
    }
    *reinterpret_cast<uint4*>(&k_s[row][dg * 8]) = kx;
    *reinterpret_cast<uint4*>(rec + (int64_t)row * D * 2 + dg * 16) = kx;
    *reinterpret_cast<uint4*>(rec + (int64_t)(BS + row) * D * 2 + dg * 16) = vx;
  }
  __syncthreads();
  if (t < D) {
    double s = 0.0;
    for (int row = 0; row < n_valid; ++row) s += widen(k_s[row][t], a.bf16);
    a.digest[(b * a.Hkv + g) * D + t] = (float)(s / (double)n_valid);
  }
}

}  // namespace

int launch_offload(const kvoff_ctx* ctx, int32_t layer, int32_t req_id, const void* k_dev,
                   const void* v_dev, float* digest_dev, hipStream_t stream) {
  const ReqHost& r = ctx->reqs[req_id];
  OffloadArgs a;
  a.K = (const uint16_t*)k_dev;
  a.V = (const uint16_t*)v_dev;
  a.digest = digest_dev;
  a.rec0 = ctx->store_dev + (size_t)(r.rec_base + (int64_t)layer * r.nb) * ctx->rec_bytes;
  a.rec_bytes = ctx->rec_bytes;
  a.n_tok = r.n_tokens;
  a.Hkv = ctx->cfg.num_kv_heads;
  a.bf16 = ctx->cfg.dtype == KVOFF_BF16;
  dim3 grid((unsigned)(r.nb * a.Hkv));
  if (ctx->cfg.block_size == 16)
    hipLaunchKernelGGL(offload_kernel<16>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(offload_kernel<32>, grid, dim3(256), 0, stream, a);
  KVOFF_HIP(hipGetLastError());
  return KVOFF_OK;
}

}  // namespace kvoff
