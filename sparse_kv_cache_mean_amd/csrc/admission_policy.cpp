// admission_policy.cpp - IO-adaptive offloading admission: the
// layer-residency policy, pure host logic ("PulseInfer Guide" (aiFetchly),
// section "Interruptible Layer-Wise Scheduling & Adaptive Admission"; the
// abstract's IO-Adaptive Offloading Admission).  The guide gives the
// thresholds (50%, 85%), the 90% offload ceiling and that the first and last
// layers are the ones kept; the pinning order between them, the step of two
// layers per decision and the rounding of the floor are this library's
// reading.  No HIP: it also builds and runs under the CPU sanitizers.
#include <climits>
#include <cmath>
#include <cstdint>
#include <vector>

#include "host_errors.h"

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
    const int64_t floor_res = (int64_t)std::ceil((1.0 - p->max_offload) * num_layers - 1e-9);
    // 64-bit: cur +- step_layers must not overflow for any step_layers
    int64_t want = cur;
    if (utilization > p->high)
      want = (int64_t)cur + p->step_layers;
    else if (utilization < p->low)
      want = (int64_t)cur - p->step_layers;
    if (want < floor_res) want = floor_res;
    if (want > num_layers) want = num_layers;
    if (want > p->max_resident) want = p->max_resident;  // the HBM budget wins
    for (int i = 0; i < num_layers; ++i) resident[i] = 0;
    for (int64_t i = 0; i < want; ++i) resident[order[i]] = 1;
    *n_resident = (int32_t)want;
    return KVOFF_OK;
  });
}

}  // extern "C"
