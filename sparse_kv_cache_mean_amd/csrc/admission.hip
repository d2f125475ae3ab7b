// admission.hip - IO-adaptive offloading admission: the calls that pin or
// release one (layer, request) in HBM ("PulseInfer Guide" (aiFetchly),
// section "Interruptible Layer-Wise Scheduling & Adaptive Admission"; the
// abstract's IO-Adaptive Offloading Admission).  The residency policy that
// decides which layers to pin is host logic, in admission_policy.cpp.

#include "kvoff_internal.h"

namespace kvoff {
namespace {

__global__ void fill_maps_kernel(uint8_t* hit, int32_t* slot, int64_t nb, int64_t first,
                                 uint8_t value) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nb) return;
  hit[b] = value;
  if (slot) slot[b] = (int32_t)(first + b);
}

}  // namespace
}  // namespace kvoff

using namespace kvoff;

extern "C" {

int kvoff_make_resident(kvoff_ctx* ctx, int32_t layer, int32_t req_id, void* slot_pool_dev,
                        int64_t n_slots, int64_t first_slot, uint8_t* pool_hit_dev,
                        int32_t* pool_slot_dev, void* stream) {
  return guarded([&]() -> int {
    if (!ctx || !slot_pool_dev || !pool_hit_dev || !pool_slot_dev)
      return fail(KVOFF_EINVAL, "NULL argument");
    if (req_id < 0 || req_id >= (int32_t)ctx->reqs.size())
      return fail(KVOFF_ESTATE, "request id %d is not registered", req_id);
    if (layer < 0 || layer >= ctx->cfg.num_layers) return fail(KVOFF_ERANGE, "layer %d", layer);
    if (!ctx->offloaded[(size_t)req_id * ctx->cfg.num_layers + layer])
      return fail(KVOFF_ESTATE, "layer %d of request %d was not offloaded", layer, req_id);
    const ReqHost& r = ctx->reqs[req_id];
    // pool_slot_dev entries are int32, and recall turns them into table
    // entries (headwise: slot * Hkv + g)
    if (n_slots > INT32_MAX / ctx->cfg.num_kv_heads)
      return fail(KVOFF_EINVAL, "n_slots %lld > %d", (long long)n_slots, INT32_MAX / ctx->cfg.num_kv_heads);
    if (first_slot < 0 || first_slot + r.nb > n_slots)
      return fail(KVOFF_ERANGE, "slots [%lld, %lld) outside the pool's %lld", (long long)first_slot,
                  (long long)(first_slot + r.nb), (long long)n_slots);
    hipStream_t s = (hipStream_t)stream;
    DeviceScope dev_scope;
    KVOFF_HIP(dev_scope.enter(ctx->device));
    const uint8_t* src = ctx->store + (size_t)(r.rec_base + (int64_t)layer * r.nb) * ctx->rec_bytes;
    uint8_t* dst = (uint8_t*)slot_pool_dev + (size_t)first_slot * ctx->rec_bytes;
    KVOFF_HIP(hipMemcpyAsync(dst, src, (size_t)r.nb * ctx->rec_bytes, hipMemcpyHostToDevice, s));
    hipLaunchKernelGGL(fill_maps_kernel, dim3((unsigned)((r.nb + 255) / 256)), dim3(256), 0, s,
                       pool_hit_dev, pool_slot_dev, (int64_t)r.nb, first_slot, (uint8_t)1);
    KVOFF_HIP(hipGetLastError());
    ctx->resident[(size_t)req_id * ctx->cfg.num_layers + layer] = 1;
    return KVOFF_OK;
  });
}

int kvoff_release_resident(kvoff_ctx* ctx, int32_t layer, int32_t req_id, uint8_t* pool_hit_dev,
                           void* stream) {
  return guarded([&]() -> int {
    if (!ctx || !pool_hit_dev) return fail(KVOFF_EINVAL, "NULL argument");
    if (req_id < 0 || req_id >= (int32_t)ctx->reqs.size())
      return fail(KVOFF_ESTATE, "request id %d is not registered", req_id);
    if (layer < 0 || layer >= ctx->cfg.num_layers) return fail(KVOFF_ERANGE, "layer %d", layer);
    const ReqHost& r = ctx->reqs[req_id];
    DeviceScope dev_scope;
    KVOFF_HIP(dev_scope.enter(ctx->device));
    hipLaunchKernelGGL(fill_maps_kernel, dim3((unsigned)((r.nb + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, pool_hit_dev, (int32_t*)nullptr, (int64_t)r.nb,
                       (int64_t)0, (uint8_t)0);
    KVOFF_HIP(hipGetLastError());
    ctx->resident[(size_t)req_id * ctx->cfg.num_layers + layer] = 0;
    return KVOFF_OK;
  });
}

}  // extern "C"
