// host_policy_test.cpp - the library's host-only code (the IO-adaptive
// admission policy and the status strings) built with the address and
// undefined-behaviour sanitizers and driven over its whole input space,
// including invalid policies and extreme step sizes
// (tests/test_host_sanitizers.py).  Invariants checked on every decision:
// the plan is a prefix of the pin order 0, L-1, 1, L-2, ...; it holds at
// least the offload floor and at most the HBM budget; it moves by at most
// step_layers from the current count.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "kvoff.h"

static int failures = 0;
#define CHECK(cond, ...)                                      \
  do {                                                        \
    if (!(cond)) {                                            \
      std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);                      \
      std::fprintf(stderr, "\n");                             \
      ++failures;                                             \
    }                                                         \
  } while (0)

static std::vector<int> pin_order(int L) {
  std::vector<int> o;
  for (int i = 0, j = L - 1; i <= j; ++i, --j) {
    o.push_back(i);
    if (j != i) o.push_back(j);
  }
  return o;
}

int main() {
  for (int s = -8; s <= 1; ++s) CHECK(kvoff_strerror(s) != nullptr, "strerror %d", s);
  kvoff_admission_defaults(nullptr);
  kvoff_admission_policy p;
  kvoff_admission_defaults(&p);
  CHECK(p.low == 0.5 && p.high == 0.85 && p.max_offload == 0.9 && p.step_layers == 2 &&
            p.max_resident == INT32_MAX,
        "defaults");
  int32_t n = -1;
  uint8_t one = 0;
  CHECK(kvoff_admission_plan(nullptr, 1, 0.5, &one, &n) == KVOFF_EINVAL, "NULL policy");
  CHECK(kvoff_admission_plan(&p, 0, 0.5, &one, &n) == KVOFF_EINVAL, "no layers");
  CHECK(kvoff_admission_plan(&p, 1, NAN, &one, &n) == KVOFF_EINVAL, "NaN utilization");
  CHECK(kvoff_admission_plan(&p, 1, -1.0, &one, &n) == KVOFF_EINVAL, "negative utilization");
  CHECK(std::strlen(kvoff_last_error()) > 0, "a failure leaves a message");
  kvoff_admission_policy bad = p;
  bad.low = 0.9;
  bad.high = 0.1;
  CHECK(kvoff_admission_plan(&bad, 4, 0.5, &one, &n) == KVOFF_EINVAL, "low above high");
  bad = p;
  bad.step_layers = 0;
  CHECK(kvoff_admission_plan(&bad, 4, 0.5, &one, &n) == KVOFF_EINVAL, "zero step");
  bad = p;
  bad.max_offload = 1.5;
  CHECK(kvoff_admission_plan(&bad, 4, 0.5, &one, &n) == KVOFF_EINVAL, "offload above 1");

  std::mt19937 rng(12345);
  const double utils[] = {0.0, 0.3, 0.5, 0.6, 0.85, 0.86, 0.9, 2.0, 1e300};
  const int32_t steps[] = {1, 2, 3, 7, INT32_MAX};
  const int32_t caps[] = {0, 1, 3, 16, INT32_MAX};
  const double offl[] = {0.0, 0.5, 0.9, 1.0};
  int decisions = 0;
  for (int L = 1; L <= 70; ++L) {
    const std::vector<int> order = pin_order(L);
    for (int32_t step : steps)
      for (int32_t cap : caps)
        for (double mo : offl)
          for (double u : utils) {
            kvoff_admission_policy q = p;
            q.step_layers = step;
            q.max_resident = cap;
            q.max_offload = mo;
            std::vector<uint8_t> res(L, 0);
            int cur = 0;
            for (int i = 0; i < L; ++i)
              if (rng() % 3 == 0) {
                res[i] = 1;
                ++cur;
              }
            int32_t got = -1;
            const int st = kvoff_admission_plan(&q, L, u, res.data(), &got);
            ++decisions;
            CHECK(st == KVOFF_OK, "status %d", st);
            int cnt = 0;
            for (int i = 0; i < L; ++i) cnt += res[i] != 0;
            CHECK(cnt == got, "count %d vs %d", cnt, got);
            for (int i = 0; i < L; ++i)
              CHECK((res[order[i]] != 0) == (i < got), "not a prefix of the pin order (L %d)", L);
            const int64_t floor_res = (int64_t)std::ceil((1.0 - mo) * L - 1e-9);
            CHECK(got <= cap, "over the HBM budget");
            CHECK(got <= L, "over the layers");
            if (cap >= floor_res) CHECK(got >= floor_res, "under the offload floor");
            const int64_t lo = std::min<int64_t>((int64_t)cur - step, floor_res);
            const int64_t hi = std::max<int64_t>((int64_t)cur + step, floor_res);
            CHECK(got >= std::min<int64_t>(lo, cap) && got <= hi, "moved too far");
          }
  }
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("PASS %d decisions\n", decisions);
  return 0;
}
