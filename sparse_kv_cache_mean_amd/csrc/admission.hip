// admission.hip - IO-adaptive offloading admission: the layer-residency
// policy (host logic) and the calls that pin or release one (layer,
// request) in HBM.  Source: "PulseInfer Guide" (aiFetchly), section
// "Interruptible Layer-Wise Scheduling & Adaptive Admission"; the abstract's
// IO-Adaptive Offloading Admission.  The guide gives the thresholds (50%,
// 85%), the 90% offload ceiling and that the first and last layers are the
// ones kept; the pinning order between them, the step of two layers per
// decision and the rounding of the floor are this library's reading.
#include <climits>
#include <cmath>
#include <vector>

#include "kvoff_internal.h"

namespace kvoff {
namespace {

// pin order: 0, L-1, 1, L-2, ...
std::vector<int> pin_order(int L) {
  std::vector<int> o;
  for (int i = 0, j = L - 1; i <= j; ++i, --j) {
    o.push_back(i);
    if (j != i) o.push_back(j);
  }
  return o;
}

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

void kvoff_admission_defaults(kvoff_admission_policy* p) {
  if (!p) return;
  p->low = 0.50;
  p->high = 0.85;
  p->max_offload = 0.90;
  p->step_layers = 2;
  p->max_resident = INT32_MAX;
}

int kvoff_admission_plan(const kvoff_admission_policy* p, int32_t num_layers, double utilization,
                         uint8_t* resident, int32_t* n_resident) {
  return guarded([&]() -> int {
    if (!p || !resident || !n_resident || num_layers < 1)
      return fail(KVOFF_EINVAL, "admission: NULL argument or num_layers < 1");
    if (!(p->low >= 0.0 && p->low <= p->high) || !(p->max_offload >= 0.0 && p->max_offload <= 1.0) ||
        p->step_layers < 1 || p->max_resident < 0 || !(utilization >= 0.0))
      return fail(KVOFF_EINVAL, "admission: bad policy or utilization");
    const std::vector<int> order = pin_order(num_layers);
    int cur = 0;
    for (int i = 0; i < num_layers; ++i) cur += resident[i] != 0;
    const int floor_res = (int)std::ceil((1.0 - p->max_offload) * num_layers - 1e-9);
    int want = cur;
    if (utilization > p->high)
      want = cur + p->step_layers;
    else if (utilization < p->low)
      want = cur - p->step_layers;
    if (want < floor_res) want = floor_res;
    if (want > num_layers) want = num_layers;
    if (want > p->max_resident) want = p->max_resident;  // the HBM budget wins
    for (int i = 0; i < num_layers; ++i) resident[i] = 0;
    for (int i = 0; i < want; ++i) resident[order[i]] = 1;
    *n_resident = want;
    return KVOFF_OK;
  });
}

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
    if (first_slot < 0 || first_slot + r.nb > n_slots)
      return fail(KVOFF_ERANGE, "slots [%lld, %lld) outside the pool's %lld", (long long)first_slot,
                  (long long)(first_slot + r.nb), (long long)n_slots);
    hipStream_t s = (hipStream_t)stream;
    KVOFF_HIP(hipSetDevice(ctx->device));
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
    KVOFF_HIP(hipSetDevice(ctx->device));
    hipLaunchKernelGGL(fill_maps_kernel, dim3((unsigned)((r.nb + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, pool_hit_dev, (int32_t*)nullptr, (int64_t)r.nb,
                       (int64_t)0, (uint8_t)0);
    KVOFF_HIP(hipGetLastError());
    ctx->resident[(size_t)req_id * ctx->cfg.num_layers + layer] = 0;
    return KVOFF_OK;
  });
}

}  // extern "C"
