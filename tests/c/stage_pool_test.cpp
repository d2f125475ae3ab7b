// stage_pool_test.cpp - the staged recall engine's host worker pool
// (StagePool, StageJob) driven the way the engine drives it, built with the
// thread sanitizer and, separately, the address and undefined-behaviour
// sanitizers (tests/test_host_sanitizers.py).  The issuing thread publishes
// one job at a time, waits for each chunk's counter to reach zero and then
// reads what the workers wrote for that chunk; some jobs follow at once
// (workers still spinning), others after a pause longer than the spin, so
// workers must be woken from the condition variable.  Pools are destroyed
// both while idle and right after a job.
#include <chrono>
#include <cstdint>
#include <cstdio>
#include <memory>
#include <random>
#include <thread>
#include <vector>

#include "stage_pool.h"

using kvoff::StageJob;
using kvoff::StagePool;

static int failures = 0;

static void one_job(StagePool& pool, std::mt19937& rng) {
  auto job = std::make_shared<StageJob>();
  const size_t n = 1 + rng() % 300;
  const size_t n_chunks = 1 + rng() % 9;
  job->n = n;
  job->chunk_of.resize(n);
  for (size_t t = 0; t < n; ++t) job->chunk_of[t] = (uint32_t)(t * n_chunks / n);
  job->left.reset(new std::atomic<int>[n_chunks]);
  for (size_t c = 0; c < n_chunks; ++c) job->left[c].store(0, std::memory_order_relaxed);
  for (size_t t = 0; t < n; ++t) job->left[job->chunk_of[t]].fetch_add(1, std::memory_order_relaxed);
  std::vector<uint64_t> out(n, 0);
  uint64_t* o = out.data();
  job->fn = [o](size_t t) { o[t] += 1000003ull * (t + 1); };
  pool.run(job);
  size_t t0 = 0;
  for (size_t c = 0; c < n_chunks; ++c) {
    while (job->left[c].load(std::memory_order_acquire) != 0) _mm_pause();
    for (; t0 < n && job->chunk_of[t0] == c; ++t0)
      if (out[t0] != 1000003ull * (t0 + 1)) {
        std::fprintf(stderr, "FAIL task %zu of chunk %zu ran %llu times\n", t0, c,
                     (unsigned long long)(out[t0] / (1000003ull * (t0 + 1))));
        ++failures;
      }
  }
}

int main() {
  std::mt19937 rng(2024);
  {
    StagePool pool(6);
    for (int i = 0; i < 400; ++i) {
      one_job(pool, rng);
      if (i % 9 == 0) std::this_thread::sleep_for(std::chrono::microseconds(1500));
    }
  }  // destroyed right after a job
  {
    StagePool pool(3);
    one_job(pool, rng);
    std::this_thread::sleep_for(std::chrono::milliseconds(3));
  }  // destroyed while its workers sleep
  {
    StagePool pool(1);  // a single worker
    for (int i = 0; i < 50; ++i) one_job(pool, rng);
  }
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("PASS\n");
  return 0;
}
