// staged.cpp - the three-phase gather-scatter recall engine
// (KVOFF_ENGINE_STAGED) of the guide ("PulseInfer Guide", aiFetchly, section
// "The Gather-Scatter I/O Engine"): CPU worker threads gather the selected
// records from the pinned store into one contiguous pinned staging buffer,
// then bulk host->HBM copies move it across the link.
//
// Differences from the guide's description, and why:
//  - the bulk copy is cut into chunks (1 MiB, 3 MiB, then 16 MiB) issued
//    as soon as the workers have filled them, so gathering and the link
//    transfer overlap instead of running back to back;
//  - there is no scatter kernel: items are placed compactly, in selection
//    order, at the start of the recall region and the block table points at
//    them (item n of the call -> slot recall_base + n; headwise: slice
//    recall_base*Hkv + n), so the attention reads them where they land.
// The context keeps two sets of pinned buffers (staging, block-table
// staging, selection read-back) and the calls use them by turns.  A set is
// reused only after an event recorded behind its last copy has completed;
// the next call may run on another stream, so the event, not stream order,
// protects it.  With two sets a call gathers while the previous call's copies
// still run (when the two calls are on different streams, as kvoff_step's
// consecutive layers are), so the link does not wait for the read-back, the
// plan and the first chunk.  Measured on the Llama-3-8B-shaped layer in
// kvoff_step: 384-388 layer-steps/s with one set, 411-413 with two.
// Optionally (KVOFF_STAGE_STREAMS=2) a call's odd chunks go to a copy stream
// of the context, so that one copy's start overlaps the previous one's end:
// alone, a recall then runs at 53.7-53.9 GB/s instead of 52.2-52.7, but
// kvoff_step loses 3 layer-steps/s, so one stream is the default.
#include <emmintrin.h>
#include <sched.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <condition_variable>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <memory>
#include <mutex>
#include <thread>
#include <vector>

#include "kvoff_internal.h"
#include "stage_pool.h"

namespace kvoff {

// steady chunk size (measured over 4, 8, 16 and 32 MiB: 16 MiB is best on the
// variable-recall layer and level with 8 MiB on the Llama-3-8B layer);
// KVOFF_STAGE_CHUNK_MIB (4..64) overrides it for tuning
constexpr size_t kStageChunk = 16u << 20;

size_t stage_chunk() {
  static const size_t c = [] {
    const char* e = std::getenv("KVOFF_STAGE_CHUNK_MIB");
    const long v = e ? std::atol(e) : 0;
    return v >= 4 && v <= 64 ? (size_t)v << 20 : kStageChunk;
  }();
  return c;
}

// sets of staging buffers used by turns, and streams the chunk copies of a
// call alternate over (measured defaults; KVOFF_STAGE_SETS and
// KVOFF_STAGE_STREAMS, 1 or 2 each, override them for tuning)
int stage_env(const char* name, int dflt) {
  const char* e = std::getenv(name);
  const int v = e ? std::atoi(e) : 0;
  return v == 1 || v == 2 ? v : dflt;
}
int stage_sets() {
  static const int n = stage_env("KVOFF_STAGE_SETS", 2);
  return n;
}
int stage_streams() {
  static const int n = stage_env("KVOFF_STAGE_STREAMS", 1);
  return n;
}

// hardware threads this process may run on (its affinity mask), else the
// machine's
int usable_cpus() {
  cpu_set_t set;
  CPU_ZERO(&set);
  if (sched_getaffinity(0, sizeof set, &set) == 0) {
    const int n = CPU_COUNT(&set);
    if (n > 0) return n;
  }
  const int hc = (int)std::thread::hardware_concurrency();
  return hc > 0 ? hc : 4;
}

// worker threads of the pool: at most 10, and three usable hardware threads
// left beside them (the issuing thread, which spins on the chunk counters
// while the workers copy, and the HIP runtime's own threads).  Measured on
// 16 hardware threads, kvoff_step on the Llama-3-8B-shaped layer: 6 workers
// 408-411 layer-steps/s, 10 412-413, 15 (all but the issuing thread) 332-402
// and erratic.  KVOFF_STAGE_THREADS (1..64) overrides the count for tuning.
int stage_threads() {
  static const int n = [] {
    const char* e = std::getenv("KVOFF_STAGE_THREADS");
    const int v = e ? std::atoi(e) : 0;
    if (v >= 1 && v <= 64) return v;
    return std::max(1, std::min(10, usable_cpus() - 3));
  }();
  return n;
}

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

// the call's status once its work is enqueued: ESTATE when pool hits named
// slots outside the pool (their table entries are -1)
// the context's first copy stream beside the caller's (shared with the DMA
// engine; created on first use, non-blocking, default priority) and the
// event recorded behind its last copy
int side_stream(kvoff_ctx* ctx, hipStream_t* s, hipEvent_t* done) {
  if (!ctx->dma_done[0]) KVOFF_HIP(hipEventCreateWithFlags(&ctx->dma_done[0], hipEventDisableTiming));
  if (!ctx->dma_stream[0]) KVOFF_HIP(hipStreamCreateWithFlags(&ctx->dma_stream[0], hipStreamNonBlocking));
  *s = ctx->dma_stream[0];
  *done = ctx->dma_done[0];
  return KVOFF_OK;
}

int bad_slots(int64_t n_bad, int64_t n_slots) {
  if (!n_bad) return KVOFF_OK;
  return fail(KVOFF_ESTATE, "%lld pool hits name a slot outside [0, %lld): table entries -1",
              (long long)n_bad, (long long)n_slots);
}

int ensure_host(void** buf, size_t* cap, size_t need, bool staging = false) {
  if (*cap >= need) return KVOFF_OK;
  if (*buf) KVOFF_HIP(hipHostFree(*buf));
  *buf = nullptr;
  *cap = 0;
  void* p = nullptr;
  hipError_t e = staging && test_fail_alloc("staging") ? hipErrorOutOfMemory
                                                      : hipHostMalloc(&p, need, hipHostMallocDefault);
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

  // this call's set: the copies of the call that used it last must be done
  // before its buffers are rewritten
  const int set = stage_sets() > 1 ? ctx->stage_next : 0;
  StageSet& ss = ctx->stage[set];
  if (ss.pending) {
    KVOFF_HIP(hipEventSynchronize(ss.done));
    ss.pending = false;
  }
  // once this call's work is enqueued: the set's event, and the other set next
  auto enqueued = [&]() -> int {
    KVOFF_HIP(hipEventRecord(ss.done, stream));
    ss.pending = true;
    ctx->stage_next = set ^ 1;
    return KVOFF_OK;
  };
  // read the selection (and the pool maps) back into pinned memory
  const size_t n_map = r.pool_hit || r.pool_slot ? (size_t)b.n * r.pool_stride : 0;
  const size_t o_sel = ((size_t)b.n * sizeof(int32_t) + 255) & ~(size_t)255;
  const size_t o_slot = (o_sel + n_sel * sizeof(int32_t) + 255) & ~(size_t)255;
  const size_t o_hit = (o_slot + (r.pool_slot ? n_map * sizeof(int32_t) : 0) + 255) & ~(size_t)255;
  int st = ensure_host(&ss.sel, &ss.sel_cap, o_hit + (r.pool_hit ? n_map : 0) + 1);
  if (st) return st;
  uint8_t* rb = (uint8_t*)ss.sel;
  const int32_t* cnt = (const int32_t*)rb;
  const int32_t* sel = (const int32_t*)(rb + o_sel);
  const int32_t* pslot = (const int32_t*)(rb + o_slot);
  const uint8_t* hit = rb + o_hit;
  KVOFF_HIP(hipMemcpyAsync(rb, r.sel_cnt, sizeof(int32_t) * b.n, hipMemcpyDeviceToHost, stream));
  KVOFF_HIP(hipMemcpyAsync(rb + o_sel, r.sel_idx, sizeof(int32_t) * n_sel, hipMemcpyDeviceToHost, stream));
  if (r.pool_hit)
    KVOFF_HIP(hipMemcpyAsync(rb + o_hit, r.pool_hit, n_map, hipMemcpyDeviceToHost, stream));
  if (r.pool_slot)
    KVOFF_HIP(hipMemcpyAsync(rb + o_slot, r.pool_slot, n_map * sizeof(int32_t), hipMemcpyDeviceToHost,
                             stream));
  KVOFF_HIP(hipStreamSynchronize(stream));

  // plan: compact order of the missing items, their block-table entries and
  // the source pieces (consecutive blocks of one request coalesced)
  st = ensure_host(&ss.table, &ss.table_cap, n_sel * sizeof(int32_t));
  if (st) return st;
  int32_t* table = (int32_t*)ss.table;
  std::vector<Piece> pieces;
  int64_t n_items = 0, n_hits = 0, n_selected = 0, n_bad = 0;
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
        if (r.pool_hit && hit[(size_t)ri * r.pool_stride + blk]) {
          const int64_t ps = pslot[(size_t)ri * r.pool_stride + blk];
          if (ps < 0 || ps >= r.n_slots) {  // a resident copy outside the pool: never read
            table[row + i] = -1;
            ++n_bad;
            continue;
          }
          table[row + i] = (int32_t)(hw ? ps * Hkv + g : ps);
          ++n_selected;
          ++n_hits;
          continue;
        }
        ++n_selected;
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
  if (total == 0) {
    KVOFF_HIP(hipMemcpyAsync(r.table, table, n_sel * sizeof(int32_t), hipMemcpyHostToDevice, stream));
    // the upload reads the block-table staging: the set's event covers it
    if ((st = enqueued())) return st;
    if (stats) {
      KVOFF_HIP(hipStreamSynchronize(stream));
      *stats = kvoff_stats{n_selected, n_hits, 0, 0, 0};
    }
    return bad_slots(n_bad, r.n_slots);
  }

  // Chunks of the staging buffer, each one bulk copy: 1 MiB, then 3 MiB,
  // then 16 MiB each, so the link starts as soon as the first megabyte is
  // gathered, and later copies are long enough that the copy engine's
  // per-copy cost stays small.  Worker tasks: 256 KiB in the first two
  // chunks, so that every worker helps fill them, then 1 MiB (measured:
  // smaller tasks throughout cost more in hand-offs than they gain).  A task
  // copies every piece, or part of a piece, that lands in its range.
  std::vector<size_t> chunk_lo{0};
  for (size_t o = 0; o < total;) {
    const size_t c = chunk_lo.size() - 1;
    o = std::min(total, o + (c == 0 ? (1u << 20) : c == 1 ? (3u << 20) : stage_chunk()));
    chunk_lo.push_back(o);
  }
  const size_t n_chunks = chunk_lo.size() - 1;
  auto job = std::make_shared<StageJob>();
  std::vector<size_t> task_lo;
  for (size_t c = 0; c < n_chunks; ++c) {
    const size_t step = c < 2 ? (256u << 10) : (1u << 20);
    for (size_t o = chunk_lo[c]; o < chunk_lo[c + 1]; o += step) {
      task_lo.push_back(o);
      job->chunk_of.push_back((uint32_t)c);
    }
  }
  task_lo.push_back(total);
  job->n = task_lo.size() - 1;
  job->left.reset(new std::atomic<int>[n_chunks]);
  for (size_t c = 0; c < n_chunks; ++c) job->left[c].store(0, std::memory_order_relaxed);
  for (size_t t = 0; t < job->n; ++t) job->left[job->chunk_of[t]].fetch_add(1, std::memory_order_relaxed);
  std::vector<size_t> piece_off(pieces.size() + 1, 0);
  for (size_t i = 0; i < pieces.size(); ++i) piece_off[i + 1] = piece_off[i] + pieces[i].bytes;
  // Everything this call allocates or creates is done before the first copy
  // is enqueued, so a failure leaves no copy in flight that reads the staging
  // the next call rewrites.
  if ((st = ensure_host(&ss.buf, &ss.cap, total, true))) return st;
  // odd chunks go to a copy stream of the context: every earlier command of
  // `stream` has completed (the read-back waited for them), so it may start
  // at once, and `stream` waits for its last copy below
  hipStream_t side = nullptr;
  hipEvent_t side_done = nullptr;
  const bool two = stage_streams() > 1 && n_chunks > 1;
  if (two && (st = side_stream(ctx, &side, &side_done))) return st;
  if (!ctx->stage_pool) ctx->stage_pool = new StagePool(stage_threads());
  uint8_t* stage = (uint8_t*)ss.buf;
  const Piece* pc = pieces.data();
  const size_t* po = piece_off.data();
  const size_t* tl = task_lo.data();
  const size_t n_pieces = pieces.size();
  // fn runs only for claimed tasks, all of which finish before this call
  // returns, so it may refer to this frame's vectors
  job->fn = [stage, pc, po, tl, n_pieces](size_t t) {
    const size_t lo = tl[t], hi = tl[t + 1];
    // first piece overlapping [lo, hi)
    size_t i = std::upper_bound(po, po + n_pieces + 1, lo) - po - 1;
    for (; i < n_pieces && po[i] < hi; ++i) {
      const size_t a = std::max(lo, po[i]), b = std::min(hi, po[i + 1]);
      copy_streaming(stage + a, pc[i].src + (a - po[i]), b - a);
    }
  };
  ctx->stage_pool->run(job);
  // issue each chunk's copy as soon as it is filled, in order; every chunk
  // is waited for, also after an error, so no task outlives this call
  uint8_t* dst0 = r.pool + (size_t)r.recall_base_slot * ctx->rec_bytes;
  int64_t n_transfers = 0;
  int err = KVOFF_OK;
  for (size_t c = 0; c < n_chunks; ++c) {
    while (job->left[c].load(std::memory_order_acquire) != 0) _mm_pause();
    const size_t o = chunk_lo[c];
    const size_t n = chunk_lo[c + 1] - o;
    if (err == KVOFF_OK) {
      hipError_t e = hipMemcpyAsync(dst0 + o, stage + o, n, hipMemcpyHostToDevice,
                                    two && (c & 1) ? side : stream);
      if (e != hipSuccess) err = fail(KVOFF_EHIP, "staged copy: %s", hipGetErrorString(e));
      ++n_transfers;
    }
  }
  // the block table last: the first chunk does not wait for its upload
  if (err == KVOFF_OK) {
    hipError_t e = hipMemcpyAsync(r.table, table, n_sel * sizeof(int32_t), hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) err = fail(KVOFF_EHIP, "block-table upload: %s", hipGetErrorString(e));
  }
  if (two && err == KVOFF_OK) {
    hipError_t e = hipEventRecord(side_done, side);
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, side_done, 0);
    if (e != hipSuccess) err = fail(KVOFF_EHIP, "copy-stream join: %s", hipGetErrorString(e));
  }
  if (err) {
    // nothing may still read this set's buffers when the call returns
    if (two) (void)hipStreamSynchronize(side);
    (void)hipStreamSynchronize(stream);
    return err;
  }
  if ((st = enqueued())) return st;
  if (stats) {
    KVOFF_HIP(hipStreamSynchronize(stream));
    *stats = kvoff_stats{n_selected, n_hits, n_items, n_transfers, n_items * item};
  }
  return bad_slots(n_bad, r.n_slots);
}

}  // namespace kvoff
