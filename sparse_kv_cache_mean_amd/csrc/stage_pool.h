// stage_pool.h - the host worker pool of the staged recall engine
// (KVOFF_ENGINE_STAGED): a fixed set of threads that take task indices of
// one job at a time.  Host code only (C++ threads and atomics, no HIP), so
// the same classes also run under the CPU thread sanitizer.
#pragma once

#include <emmintrin.h>

#include <atomic>
#include <chrono>
#include <condition_variable>
#include <cstddef>
#include <cstdint>
#include <functional>
#include <memory>
#include <mutex>
#include <thread>
#include <vector>

namespace kvoff {

// One recall's copy work: n tasks, fn(t) for each, and per chunk of the
// staging buffer the number of its tasks still to finish.  Owned jointly by
// the issuing thread and every worker that picked it up, so a worker that
// arrives after the last task was claimed still finds the counters alive.
struct StageJob {
  std::atomic<size_t> next{0};
  size_t n = 0;
  std::function<void(size_t)> fn;
  std::vector<uint32_t> chunk_of;                // task -> chunk
  std::unique_ptr<std::atomic<int>[]> left;      // chunk -> tasks not yet done
  void work() {
    for (;;) {
      const size_t t = next.fetch_add(1, std::memory_order_relaxed);
      if (t >= n) return;
      fn(t);
      left[chunk_of[t]].fetch_sub(1, std::memory_order_release);
    }
  }
};

// Fixed-size pool of host worker threads.  The issuing thread publishes one
// job at a time; workers take task indices from its counter.  Between jobs a
// worker spins for a while before it sleeps: in a decode loop the next
// layer's recall follows within a few hundred microseconds and then finds it
// awake, where a sleeping thread costs a wake-up of up to hundreds of
// microseconds before the link can start.
class StagePool {
 public:
  // throws if a thread cannot be started, after stopping the ones that did
  explicit StagePool(int n) {
    try {
      for (int i = 0; i < n; ++i) workers_.emplace_back([this] { worker(); });
    } catch (...) {
      shutdown();
      throw;
    }
  }
  ~StagePool() { shutdown(); }
  void run(std::shared_ptr<StageJob> j) {
    {
      std::lock_guard<std::mutex> g(mu_);
      job_ = std::move(j);
      gen_.fetch_add(1, std::memory_order_release);
    }
    cv_.notify_all();
  }
  int size() const { return (int)workers_.size(); }

 private:
  static constexpr std::chrono::microseconds kSpin{500};
  void shutdown() {
    {
      std::lock_guard<std::mutex> g(mu_);
      stop_.store(true);
    }
    cv_.notify_all();
    for (auto& t : workers_) t.join();
    workers_.clear();
  }
  void worker() {
    uint64_t seen = 0;
    for (;;) {
      // wait for a job newer than the last one seen: spin, then sleep
      const auto t0 = std::chrono::steady_clock::now();
      while (gen_.load(std::memory_order_acquire) == seen && !stop_.load()) {
        _mm_pause();
        if (std::chrono::steady_clock::now() - t0 > kSpin) {
          std::unique_lock<std::mutex> l(mu_);
          cv_.wait(l, [&] { return gen_.load() != seen || stop_.load(); });
        }
      }
      if (stop_.load()) return;
      std::shared_ptr<StageJob> j;
      {
        std::lock_guard<std::mutex> g(mu_);
        j = job_;
        seen = gen_.load();
      }
      if (j) j->work();
    }
  }
  std::vector<std::thread> workers_;
  std::shared_ptr<StageJob> job_;
  std::atomic<uint64_t> gen_{0};
  std::atomic<bool> stop_{false};
  std::mutex mu_;
  std::condition_variable cv_;
};

}  // namespace kvoff
