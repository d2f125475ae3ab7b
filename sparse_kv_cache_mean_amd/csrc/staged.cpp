// staged.cpp - the three-phase gather-scatter recall engine
// (KVOFF_ENGINE_STAGED) of the guide ("PulseInfer Guide", aiFetchly, section
// "The Gather-Scatter I/O Engine"): CPU worker threads gather the selected
// records from the pinned store into one contiguous pinned staging buffer,
// then bulk host->HBM copies move it across the link.
//
// Differences from the guide's description, and why:
//  - the bulk copy is cut into 4 MiB chunks issued as soon as the workers
//    have filled them, so gathering and the link transfer overlap instead of
//    running back to back;
//  - there is no scatter kernel: items are placed compactly, in selection
//    order, at the start of the recall region and the block table points at
//    them (item n of the call -> slot recall_base + n; headwise: slice
//    recall_base*Hkv + n), so the attention reads them where they land.
// The staging buffer and the block-table staging are reused by the next
// call only after an event recorded behind this call's last copy (the table
// upload when nothing is recalled) has completed; the next call may run on
// another stream, so the event, not stream order, protects them.
#include <emmintrin.h>

#include <algorithm>
#include <condition_variable>
#include <deque>
#include <cstdint>
#include <cstring>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "kvoff_internal.h"

namespace kvoff {

constexpr size_t kStageChunk = 4u << 20;

// Fixed-size pool of host worker threads running copy tasks.
class StagePool {
 public:
  explicit StagePool(int n) {
    for (int i = 0; i < n; ++i) workers_.emplace_back([this] { run(); });
  }
  ~StagePool() {
    {
      std::lock_guard<std::mutex> g(mu_);
      stop_ = true;
    }
    cv_.notify_all();
    for (auto& t : workers_) t.join();
  }
  void submit(std::function<void()> f) {
    {
      std::lock_guard<std::mutex> g(mu_);
      q_.push_back(std::move(f));
    }
    cv_.notify_one();
  }
  int size() const { return (int)workers_.size(); }

 private:
  void run() {
    for (;;) {
      std::function<void()> f;
      {
        std::unique_lock<std::mutex> l(mu_);
        cv_.wait(l, [this] { return stop_ || !q_.empty(); });
        if (stop_ && q_.empty()) return;
        f = std::move(q_.front());
        q_.pop_front();
      }
      f();
    }
  }
  std::vector<std::thread> workers_;
  std::deque<std::function<void()>> q_;
  std::mutex mu_;
  std::condition_variable cv_;
  bool stop_ = false;
};

void stage_pool_destroy(kvoff_ctx* ctx) {
  delete ctx->stage_pool;
  ctx->stage_pool = nullptr;
}

namespace {

// Copy into the staging buffer with streaming (non-temporal) stores: the
// buffer is only read again by the copy engine, so the stores skip the
// caches and the read-for-ownership of every destination line that plain
// stores cost (measured on the host: 1.4-1.5x the bandwidth of memcpy).  The
// fence makes the stores globally visible before the chunk is handed to the
// copy engine.  Falls back to memcpy for an unaligned destination.
void copy_streaming(uint8_t* dst, const uint8_t* src, size_t n) {
  if (reinterpret_cast<uintptr_t>(dst) % 16 != 0) {
    std::memcpy(dst, src, n);
    return;
  }
  size_t i = 0;
  for (; i + 64 <= n; i += 64) {
    const __m128i a = _mm_loadu_si128(reinterpret_cast<const __m128i*>(src + i));
    const __m128i b = _mm_loadu_si128(reinterpret_cast<const __m128i*>(src + i + 16));
    const __m128i c = _mm_loadu_si128(reinterpret_cast<const __m128i*>(src + i + 32));
    const __m128i d = _mm_loadu_si128(reinterpret_cast<const __m128i*>(src + i + 48));
    _mm_stream_si128(reinterpret_cast<__m128i*>(dst + i), a);
    _mm_stream_si128(reinterpret_cast<__m128i*>(dst + i + 16), b);
    _mm_stream_si128(reinterpret_cast<__m128i*>(dst + i + 32), c);
    _mm_stream_si128(reinterpret_cast<__m128i*>(dst + i + 48), d);
  }
  if (i < n) std::memcpy(dst + i, src + i, n - i);
  _mm_sfence();
}

struct Piece {  // one contiguous source range of the store
  const uint8_t* src;
  size_t bytes;
};

// Completion flags of the chunks, waited for in order by the issuing thread.
struct ChunkDone {
  std::mutex mu;
  std::condition_variable cv;
  std::vector<int> left;  // worker tasks still running, per chunk
};

int ensure_host(void** buf, size_t* cap, size_t need) {
  if (*cap >= need) return KVOFF_OK;
  if (*buf) KVOFF_HIP(hipHostFree(*buf));
  *buf = nullptr;
  *cap = 0;
  void* p = nullptr;
  hipError_t e = hipHostMalloc(&p, need, hipHostMallocDefault);
  if (e != hipSuccess) return fail(KVOFF_ENOMEM, "staging buffer of %zu bytes: %s", need, hipGetErrorString(e));
  *buf = p;
  *cap = need;
  return KVOFF_OK;
}

}  // namespace

int recall_staged(kvoff_ctx* ctx, const BatchIds& b, const RecallArgs& r, kvoff_stats* stats,
                  hipStream_t stream) {
  const bool hw = r.mode == KVOFF_HEADWISE;
  const int Hkv = ctx->cfg.num_kv_heads;
  const int sets = hw ? Hkv : 1;
  const size_t n_sel = (size_t)b.n * sets * r.k_stride;
  const int64_t item = hw ? ctx->slice_bytes : ctx->rec_bytes;

  // the previous staged call's copies must be done before its buffers are reused
  if (ctx->ev_stage_pending) {
    KVOFF_HIP(hipEventSynchronize(ctx->ev_stage));
    ctx->ev_stage_pending = false;
  }
  std::vector<int32_t> cnt(b.n), sel(n_sel);
  std::vector<uint8_t> hit;
  KVOFF_HIP(hipMemcpyAsync(cnt.data(), r.sel_cnt, sizeof(int32_t) * b.n, hipMemcpyDeviceToHost, stream));
  KVOFF_HIP(hipMemcpyAsync(sel.data(), r.sel_idx, sizeof(int32_t) * n_sel, hipMemcpyDeviceToHost, stream));
  if (r.pool_hit) {
    hit.resize((size_t)b.n * r.pool_stride);
    KVOFF_HIP(hipMemcpyAsync(hit.data(), r.pool_hit, hit.size(), hipMemcpyDeviceToHost, stream));
  }
  std::vector<int32_t> pslot;
  if (r.pool_slot) {
    pslot.resize((size_t)b.n * r.pool_stride);
    KVOFF_HIP(hipMemcpyAsync(pslot.data(), r.pool_slot, pslot.size() * sizeof(int32_t),
                             hipMemcpyDeviceToHost, stream));
  }
  KVOFF_HIP(hipStreamSynchronize(stream));

  // plan: compact order of the missing items, their block-table entries and
  // the source pieces (consecutive blocks of one request coalesced)
  int st = ensure_host(&ctx->table_host, &ctx->table_cap, n_sel * sizeof(int32_t));
  if (st) return st;
  int32_t* table = (int32_t*)ctx->table_host;
  std::vector<Piece> pieces;
  int64_t n_items = 0, n_hits = 0, n_selected = 0;
  for (int ri = 0; ri < b.n; ++ri) {
    const ReqHost& rq = ctx->reqs[b.id[ri]];
    const uint8_t* rec_l = ctx->store + (size_t)(rq.rec_base + (int64_t)r.layer * rq.nb) * ctx->rec_bytes;
    const int K = cnt[ri];
    for (int g = 0; g < sets; ++g) {
      const size_t row = ((size_t)ri * sets + g) * r.k_stride;
      for (int i = 0; i < r.k_stride; ++i) {
        const int32_t blk = i < K ? sel[row + i] : -1;
        if (blk < 0 || blk >= rq.nb) {  // unused entry (or an id outside the request)
          table[row + i] = -1;
          continue;
        }
        ++n_selected;
        if (r.pool_hit && hit[(size_t)ri * r.pool_stride + blk]) {
          const int64_t ps = pslot[(size_t)ri * r.pool_stride + blk];
          table[row + i] = (int32_t)(hw ? ps * Hkv + g : ps);
          ++n_hits;
          continue;
        }
        table[row + i] = (int32_t)(hw ? r.recall_base_slot * Hkv + n_items : r.recall_base_slot + n_items);
        const uint8_t* src = rec_l + (size_t)blk * ctx->rec_bytes + (hw ? (size_t)g * item : 0);
        if (!pieces.empty() && pieces.back().src + pieces.back().bytes == src)
          pieces.back().bytes += item;
        else
          pieces.push_back({src, (size_t)item});
        ++n_items;
      }
    }
  }
  const size_t total = (size_t)n_items * item;
  KVOFF_HIP(hipMemcpyAsync(r.table, table, n_sel * sizeof(int32_t), hipMemcpyHostToDevice, stream));
  if (total == 0) {
    // the upload reads the block-table staging: the next call (possibly on
    // another stream) waits for this event before rewriting it
    KVOFF_HIP(hipEventRecord(ctx->ev_stage, stream));
    ctx->ev_stage_pending = true;
    if (stats) {
      KVOFF_HIP(hipStreamSynchronize(stream));
      *stats = kvoff_stats{n_selected, n_hits, 0, 0, 0};
    }
    return KVOFF_OK;
  }
  if ((st = ensure_host(&ctx->stage_buf, &ctx->stage_cap, total))) return st;
  if (!ctx->stage_pool) {
    const unsigned hc = std::thread::hardware_concurrency();
    ctx->stage_pool = new StagePool((int)std::max(1u, std::min(16u, hc ? hc : 4u)));
  }

  // one worker task per 1 MiB of staging (kStageChunk / 4): it copies every
  // piece, or part of a piece, that lands in its range.  A chunk's bulk copy
  // is issued once its four tasks are done.
  constexpr size_t kTask = kStageChunk / 4;  // measured: 256 KiB to 2 MiB, 1 MiB is best
  const size_t n_chunks = (total + kStageChunk - 1) / kStageChunk;
  const size_t n_tasks = (total + kTask - 1) / kTask;
  ChunkDone done;
  done.left.assign(n_chunks, 0);
  for (size_t t = 0; t < n_tasks; ++t) ++done.left[t * kTask / kStageChunk];
  std::vector<size_t> piece_off(pieces.size() + 1, 0);
  for (size_t i = 0; i < pieces.size(); ++i) piece_off[i + 1] = piece_off[i] + pieces[i].bytes;
  uint8_t* stage = (uint8_t*)ctx->stage_buf;
  const Piece* pc = pieces.data();
  const size_t* po = piece_off.data();
  const size_t n_pieces = pieces.size();
  for (size_t t = 0; t < n_tasks; ++t) {
    ctx->stage_pool->submit([t, total, stage, pc, po, n_pieces, &done] {
      const size_t lo = t * kTask, hi = std::min(total, lo + kTask);
      // first piece overlapping [lo, hi)
      size_t i = std::upper_bound(po, po + n_pieces + 1, lo) - po - 1;
      for (; i < n_pieces && po[i] < hi; ++i) {
        const size_t a = std::max(lo, po[i]), b = std::min(hi, po[i + 1]);
        copy_streaming(stage + a, pc[i].src + (a - po[i]), b - a);
      }
      std::lock_guard<std::mutex> g(done.mu);
      if (--done.left[t * kTask / kStageChunk] == 0) done.cv.notify_all();
    });
  }
  // issue each chunk's copy as soon as it is filled, in order
  uint8_t* dst0 = r.pool + (size_t)r.recall_base_slot * ctx->rec_bytes;
  int64_t n_transfers = 0;
  int err = KVOFF_OK;
  for (size_t c = 0; c < n_chunks; ++c) {
    {
      std::unique_lock<std::mutex> l(done.mu);
      done.cv.wait(l, [&] { return done.left[c] == 0; });
    }
    const size_t o = c * kStageChunk;
    const size_t n = std::min(kStageChunk, total - o);
    if (err == KVOFF_OK) {
      hipError_t e = hipMemcpyAsync(dst0 + o, stage + o, n, hipMemcpyHostToDevice, stream);
      if (e != hipSuccess) err = fail(KVOFF_EHIP, "staged copy: %s", hipGetErrorString(e));
      ++n_transfers;
    }
  }
  if (err) {
    (void)hipStreamSynchronize(stream);
    return err;
  }
  KVOFF_HIP(hipEventRecord(ctx->ev_stage, stream));
  ctx->ev_stage_pending = true;
  if (stats) {
    KVOFF_HIP(hipStreamSynchronize(stream));
    *stats = kvoff_stats{n_selected, n_hits, n_items, n_transfers, n_items * item};
  }
  return KVOFF_OK;
}

}  // namespace kvoff
