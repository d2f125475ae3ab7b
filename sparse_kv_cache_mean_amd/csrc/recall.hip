// recall.hip - host -> HBM recall of the selected blocks (kvoff_recall).
//
// The pages put the decode bottleneck on recall I/O and fix it by sending
// few large transfers instead of many per-head fragments ("PulseInfer
// Guide", aiFetchly, sections "The Fallacy of Naive Offloading" and "The
// Gather-Scatter I/O Engine"; abstract: SoloHead selection plus a
// gather-scatter I/O engine coalesce fragmented transfers).  Two engines:
//
//  ZEROCOPY  One kernel.  Every (request, rank) item of the selection is a
//            record (headwise: a (block, KV head) slice) copied from the
//            mapped pinned store straight into its HBM slot with 16-byte
//            lane loads; each workgroup moves pieces of up to 16 KiB so tens
//            of MB of reads are in flight over the link.  The block table is
//            written by the same kernel; the plan never leaves the GPU.
//            A pool hit whose slot lies outside [0, n_slots) gets the table
//            entry -1 (attention skips it) and is counted in a sticky
//            counter that the next call filling stats reports.
//  DMA       The host reads the selection back, finds the maximal runs of
//            consecutive missing blocks and issues one hipMemcpyAsync per
//            run (per slice when headwise), round robin over the caller's
//            stream and up to three copy streams of the context, which the
//            copy engines execute; the caller's stream then waits for all.
// A third engine, STAGED (the guide's CPU gather into pinned staging plus
// bulk copies), is in staged.cpp.  Every engine ignores a selected block id
// outside its request, as if the entry were unused.
//
// Slot layout: rank i of request r goes to slot base + r*k_stride + i, so a
// run of consecutive block ids is contiguous in the store and in the pool.
#include <algorithm>
#include <cstdlib>
#include <vector>

#include "kvoff_internal.h"

namespace kvoff {
namespace {

constexpr int GATHER_THREADS = 256;
constexpr int64_t GATHER_PIECE = 16384;  // bytes per workgroup task

struct GatherArgs {
  BatchIds batch;
  const ReqDev* reqs;
  const uint8_t* store;
  uint8_t* pool;
  const int32_t* sel_idx;
  const int32_t* sel_cnt;
  const uint8_t* pool_hit;
  const int32_t* pool_slot;
  int32_t* table;
  unsigned long long* counters;
  int64_t rec_bytes;
  int64_t item_bytes;   // rec_bytes, or slice bytes when headwise
  int64_t piece_bytes;  // the largest power of two <= GATHER_PIECE dividing item_bytes
  int64_t pool_stride;
  int64_t base_slot;
  int64_t n_slots;
  int64_t n_pieces;
  int32_t pieces_per_item;
  int32_t layer, Hkv, k_stride, hw, count;
  int32_t flag_bad;  // count out-of-range hit slots in counters[kBadSlots]
};

struct Item {
  int r, g, i, b;
  bool active, hit;
  int64_t slot;
};

__device__ __forceinline__ Item decode_item(const GatherArgs& a, int64_t item) {
  Item it;
  it.i = (int)(item % a.k_stride);
  const int64_t rg = item / a.k_stride;
  it.r = a.hw ? (int)(rg / a.Hkv) : (int)rg;
  it.g = a.hw ? (int)(rg % a.Hkv) : 0;
  it.active = it.i < a.sel_cnt[it.r];
  it.b = it.active ? a.sel_idx[item] : -1;
  // a block id outside the request is never dereferenced
  if (it.active && (it.b < 0 || it.b >= a.reqs[a.batch.id[it.r]].nb)) it.active = false;
  it.hit = it.active && a.pool_hit && a.pool_hit[(int64_t)it.r * a.pool_stride + it.b];
  it.slot = a.base_slot + (int64_t)it.r * a.k_stride + it.i;
  return it;
}

__device__ __forceinline__ void write_table_and_count(const GatherArgs& a, int64_t item,
                                                      const Item& it) {
  if (!it.active) {
    a.table[item] = -1;
    return;
  }
  int64_t entry;
  if (it.hit) {
    const int64_t ps = a.pool_slot[(int64_t)it.r * a.pool_stride + it.b];
    if (ps < 0 || ps >= a.n_slots) {  // a resident copy outside the pool: never read
      a.table[item] = -1;
      if (a.flag_bad) atomicAdd(&a.counters[kBadSlots], 1ull);
      return;
    }
    entry = a.hw ? ps * a.Hkv + it.g : ps;
  } else {
    entry = a.hw ? it.slot * a.Hkv + it.g : it.slot;
  }
  a.table[item] = (int32_t)entry;
  if (a.count) {
    atomicAdd(&a.counters[0], 1ull);
    if (it.hit) {
      atomicAdd(&a.counters[1], 1ull);
    } else {
      atomicAdd(&a.counters[2], 1ull);
      // a transfer starts here unless the previous rank is the previous,
      // also-missing block (headwise: every slice is its own transfer)
      bool cont = false;
      if (!a.hw && it.i > 0) {
        const int pb = a.sel_idx[item - 1];
        if (pb >= 0 && pb == it.b - 1) {  // then pb is inside the request too
          const bool phit = a.pool_hit && a.pool_hit[(int64_t)it.r * a.pool_stride + pb];
          cont = !phit;
        }
      }
      if (!cont) atomicAdd(&a.counters[3], 1ull);
    }
  }
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u32x4_t ld16(const u32x4_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT>
__device__ __forceinline__ void st16(u32x4_t* p, u32x4_t v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// NTL / NTS: nontemporal hint on the host-link loads / the HBM stores
template <bool NTL, bool NTS>
__global__ __launch_bounds__(GATHER_THREADS) void gather_kernel(GatherArgs a) {
  const int tid = threadIdx.x;
  for (int64_t p = blockIdx.x; p < a.n_pieces; p += gridDim.x) {
    const int64_t item = p / a.pieces_per_item;
    const int piece = (int)(p % a.pieces_per_item);
    const Item it = decode_item(a, item);
    if (piece == 0 && tid == 0) write_table_and_count(a, item, it);
    if (!it.active || it.hit) continue;
    const ReqDev rq = a.reqs[a.batch.id[it.r]];
    const uint8_t* src = a.store + (rq.rec_base + (int64_t)a.layer * rq.nb + it.b) * a.rec_bytes +
                         (a.hw ? (int64_t)it.g * a.item_bytes : 0) + (int64_t)piece * a.piece_bytes;
    uint8_t* dst = a.pool + (a.hw ? (it.slot * a.Hkv + it.g) * a.item_bytes : it.slot * a.rec_bytes) +
                   (int64_t)piece * a.piece_bytes;
    const u32x4_t* s4 = reinterpret_cast<const u32x4_t*>(src);
    u32x4_t* d4 = reinterpret_cast<u32x4_t*>(dst);
    const int n16 = (int)(a.piece_bytes / 16);  // 1024, 512 or 256 (a multiple of 256)
    if (n16 == 1024) {
      const u32x4_t x0 = ld16<NTL>(s4 + tid), x1 = ld16<NTL>(s4 + tid + 256),
                    x2 = ld16<NTL>(s4 + tid + 512), x3 = ld16<NTL>(s4 + tid + 768);
      st16<NTS>(d4 + tid, x0);
      st16<NTS>(d4 + tid + 256, x1);
      st16<NTS>(d4 + tid + 512, x2);
      st16<NTS>(d4 + tid + 768, x3);
    } else {
      for (int k = tid; k < n16; k += GATHER_THREADS) st16<NTS>(d4 + k, ld16<NTL>(s4 + k));
    }
  }
}

__global__ void table_kernel(GatherArgs a, int64_t n_items) {
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= n_items) return;
  GatherArgs b = a;
  b.count = 0;
  write_table_and_count(b, item, decode_item(a, item));
}

// clears the per-call statistics (counters 0..3), or with `sticky` the
// out-of-range slot count once it has been reported
__global__ void zero_counters_kernel(unsigned long long* c, int sticky) {
  if (sticky) {
    if (threadIdx.x == 0) c[kBadSlots] = 0ull;
  } else if (threadIdx.x < 4) {
    c[threadIdx.x] = 0ull;
  }
}

__global__ __launch_bounds__(256) void probe_kernel(const uint4* src, int64_t n16, uint32_t* sink) {
  uint32_t acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * 1024; base < n16; base += (int64_t)gridDim.x * 1024) {
    uint4 x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t idx = base + threadIdx.x + 256 * k;
      x[k] = idx < n16 ? src[idx] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) acc ^= x[k].x ^ x[k].y ^ x[k].z ^ x[k].w;
  }
  sink[threadIdx.x] = acc;
}

// KVOFF_GATHER_NT: bit 0 = nontemporal host loads, bit 1 = nontemporal HBM
// stores; unset = decided per call (see launch_gather).  Neither changes the
// link rate (56.9 GB/s measured either way).
int gather_nt() {
  static int v = [] {
    const char* e = std::getenv("KVOFF_GATHER_NT");
    return e ? (std::atoi(e) & 3) : -1;
  }();
  return v;
}

// Above this many bytes a recall cannot stay in the 256 MB MALL for the
// attention that reads it next.
constexpr int64_t kMallBytes = 256ll << 20;

int gather_grid_cap() {
  static int cap = [] {
    const char* e = std::getenv("KVOFF_GATHER_WG");
    int v = e ? std::atoi(e) : 0;
    return v > 0 ? v : 128;  // measured: 32..256 saturate the link, more congest it
  }();
  return cap;
}

GatherArgs make_args(const kvoff_ctx* ctx, const BatchIds& b, const RecallArgs& r) {
  GatherArgs a;
  a.batch = b;
  a.reqs = ctx->d_reqs;
  a.store = ctx->store_dev;
  a.pool = r.pool;
  a.sel_idx = r.sel_idx;
  a.sel_cnt = r.sel_cnt;
  a.pool_hit = r.pool_hit;
  a.pool_slot = r.pool_slot;
  a.table = r.table;
  a.counters = ctx->d_counters;
  a.rec_bytes = ctx->rec_bytes;
  a.hw = r.mode == KVOFF_HEADWISE;
  a.item_bytes = a.hw ? ctx->slice_bytes : ctx->rec_bytes;
  // Pieces tile the item exactly.  A record is Hkv slices of 2*bs*d*es
  // bytes (8 KiB at 16-token blocks, 16 KiB at 32), so a record of an odd
  // number of 8 KiB slices (Hkv = 3 at 16-token blocks: 24 KiB) is moved in
  // 8 KiB pieces, not in one 16 KiB piece that would leave its tail behind.
  a.piece_bytes = GATHER_PIECE;
  while (a.piece_bytes > GATHER_THREADS * 16 && a.item_bytes % a.piece_bytes != 0) a.piece_bytes /= 2;
  a.pieces_per_item = (int32_t)(a.item_bytes / a.piece_bytes);
  a.pool_stride = r.pool_stride;
  a.base_slot = r.recall_base_slot;
  a.n_slots = r.n_slots;
  a.flag_bad = 1;
  a.layer = r.layer;
  a.Hkv = ctx->cfg.num_kv_heads;
  a.k_stride = r.k_stride;
  a.count = 0;
  const int64_t n_items = (int64_t)b.n * (a.hw ? a.Hkv : 1) * r.k_stride;
  a.n_pieces = n_items * a.pieces_per_item;
  return a;
}

}  // namespace

int launch_zero_counters(const kvoff_ctx* ctx, bool sticky, hipStream_t stream) {
  hipLaunchKernelGGL(zero_counters_kernel, dim3(1), dim3(64), 0, stream, ctx->d_counters,
                     sticky ? 1 : 0);
  KVOFF_HIP(hipGetLastError());
  return KVOFF_OK;
}

int launch_gather(const kvoff_ctx* ctx, const BatchIds& b, const RecallArgs& r, bool count,
                  hipStream_t stream) {
  GatherArgs a = make_args(ctx, b, r);
  a.count = count ? 1 : 0;
  if (a.item_bytes % a.piece_bytes != 0 || a.piece_bytes % (GATHER_THREADS * 16) != 0)
    return fail(KVOFF_ESTATE, "gather: %lld-byte items do not split into whole pieces",
                (long long)a.item_bytes);
  if (a.n_pieces == 0) return KVOFF_OK;
  const int64_t cap = gather_grid_cap();
  const unsigned grid = (unsigned)(a.n_pieces < cap ? a.n_pieces : cap);
  int nt = gather_nt();
  if (nt < 0) {
    // Plain stores leave the recalled records in the caches for the
    // attention that follows, which pays off while they fit the MALL
    // (Llama-3-8B layer, 128 MiB: attention 32 us, 36 us after nontemporal
    // stores).  A larger recall evicts its own dirty lines, and the
    // attention pays for the write-backs: nontemporal stores then (the
    // variable-recall layer, 968 MB: attention 245 -> 220 us).  The bound
    // is every entry missing.
    nt = a.n_pieces * a.piece_bytes > kMallBytes ? 2 : 0;
  }
  switch (nt) {
    case 1: hipLaunchKernelGGL((gather_kernel<true, false>), dim3(grid), dim3(GATHER_THREADS), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((gather_kernel<false, true>), dim3(grid), dim3(GATHER_THREADS), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((gather_kernel<true, true>), dim3(grid), dim3(GATHER_THREADS), 0, stream, a); break;
    default: hipLaunchKernelGGL((gather_kernel<false, false>), dim3(grid), dim3(GATHER_THREADS), 0, stream, a); break;
  }
  KVOFF_HIP(hipGetLastError());
  return KVOFF_OK;
}

int launch_table(const kvoff_ctx* ctx, const BatchIds& b, const RecallArgs& r,
                 hipStream_t stream) {
  GatherArgs a = make_args(ctx, b, r);
  a.flag_bad = 0;  // the host engines check the hit slots themselves
  const int64_t n_items = a.n_pieces / a.pieces_per_item;
  if (n_items == 0) return KVOFF_OK;
  hipLaunchKernelGGL(table_kernel, dim3((unsigned)((n_items + 255) / 256)), dim3(256), 0, stream,
                     a, n_items);
  KVOFF_HIP(hipGetLastError());
  return KVOFF_OK;
}

// Copy streams of the DMA engine: the caller's stream plus up to three the
// context owns (non-blocking, default priority), which the box's four
// hardware queues per process can all serve.  KVOFF_DMA_STREAMS (1..4)
// overrides the count for measurements.
int dma_streams() {
  static const int n = [] {
    const char* e = std::getenv("KVOFF_DMA_STREAMS");
    const int v = e ? std::atoi(e) : 0;
    return v >= 1 && v <= 1 + kDmaSideStreams ? v : 1 + kDmaSideStreams;
  }();
  return n;
}

int recall_dma(kvoff_ctx* ctx, const BatchIds& b, const RecallArgs& r, kvoff_stats* stats,
               hipStream_t stream) {
  const bool hw = r.mode == KVOFF_HEADWISE;
  const int Hkv = ctx->cfg.num_kv_heads;
  const int sets = hw ? Hkv : 1;
  const size_t n_sel = (size_t)b.n * sets * r.k_stride;
  std::vector<int32_t> cnt(b.n), sel(n_sel), pslot;
  std::vector<uint8_t> hit;
  // the selection must be complete before the host can plan the copies
  // (read back on the same stream, so no other stream is waited for)
  KVOFF_HIP(hipMemcpyAsync(cnt.data(), r.sel_cnt, sizeof(int32_t) * b.n, hipMemcpyDeviceToHost,
                           stream));
  KVOFF_HIP(hipMemcpyAsync(sel.data(), r.sel_idx, sizeof(int32_t) * n_sel, hipMemcpyDeviceToHost,
                           stream));
  if (r.pool_hit) {
    hit.resize((size_t)b.n * r.pool_stride);
    pslot.resize(hit.size());
    KVOFF_HIP(hipMemcpyAsync(hit.data(), r.pool_hit, hit.size(), hipMemcpyDeviceToHost, stream));
    KVOFF_HIP(hipMemcpyAsync(pslot.data(), r.pool_slot, pslot.size() * sizeof(int32_t),
                             hipMemcpyDeviceToHost, stream));
  }
  KVOFF_HIP(hipStreamSynchronize(stream));
  // every earlier command of `stream` has completed, so the side streams may
  // start at once; `stream` waits for their last copies below
  const int n_streams = dma_streams();
  for (int k = 0; k + 1 < n_streams; ++k) {
    if (!ctx->dma_stream[k]) {
      KVOFF_HIP(hipStreamCreateWithFlags(&ctx->dma_stream[k], hipStreamNonBlocking));
      KVOFF_HIP(hipEventCreateWithFlags(&ctx->dma_done[k], hipEventDisableTiming));
    }
  }
  int st = launch_table(ctx, b, r, stream);
  if (st) return st;
  const int64_t item = hw ? ctx->slice_bytes : ctx->rec_bytes;
  int64_t n_selected = 0, n_hits = 0, n_items = 0, n_transfers = 0, n_bad = 0;
  bool used[1 + kDmaSideStreams] = {};
  for (int ri = 0; ri < b.n; ++ri) {
    const ReqHost& rq = ctx->reqs[b.id[ri]];
    const uint8_t* rec_l = ctx->store + (size_t)(rq.rec_base + (int64_t)r.layer * rq.nb) * ctx->rec_bytes;
    const int K = std::min(cnt[ri], r.k_stride);
    for (int g = 0; g < sets; ++g) {
      const int32_t* s = sel.data() + ((size_t)ri * sets + g) * r.k_stride;
      auto is_hit = [&](int32_t blk) { return r.pool_hit && hit[(size_t)ri * r.pool_stride + blk]; };
      auto valid = [&](int32_t blk) { return blk >= 0 && blk < rq.nb; };
      int i = 0;
      while (i < K) {
        if (!valid(s[i])) {  // an id outside the request: an unused entry
          ++i;
          continue;
        }
        if (is_hit(s[i])) {
          const int64_t ps = pslot[(size_t)ri * r.pool_stride + s[i]];
          if (ps < 0 || ps >= r.n_slots) {
            ++n_bad;  // table entry -1 (table_kernel): neither read nor moved
          } else {
            ++n_selected;
            ++n_hits;
          }
          ++i;
          continue;
        }
        int j = i + 1;
        if (!hw)
          while (j < K && valid(s[j]) && s[j] == s[j - 1] + 1 && !is_hit(s[j])) ++j;
        n_selected += j - i;
        const int64_t slot = r.recall_base_slot + (int64_t)ri * r.k_stride + i;
        const uint8_t* src = rec_l + (size_t)s[i] * ctx->rec_bytes + (hw ? (size_t)g * item : 0);
        uint8_t* dst = r.pool + (hw ? (slot * Hkv + g) * item : slot * ctx->rec_bytes);
        const size_t bytes = (size_t)(j - i) * item;
        const int k = (int)(n_transfers % n_streams);  // round robin over the copy streams
        used[k] = true;
        KVOFF_HIP(hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice,
                                 k == 0 ? stream : ctx->dma_stream[k - 1]));
        n_items += j - i;
        ++n_transfers;
        i = j;
      }
    }
  }
  for (int k = 1; k < n_streams; ++k) {
    if (!used[k]) continue;
    KVOFF_HIP(hipEventRecord(ctx->dma_done[k - 1], ctx->dma_stream[k - 1]));
    KVOFF_HIP(hipStreamWaitEvent(stream, ctx->dma_done[k - 1], 0));
  }
  if (stats) {
    KVOFF_HIP(hipStreamSynchronize(stream));
    stats->selected = n_selected;
    stats->pool_hits = n_hits;
    stats->items_recalled = n_items;
    stats->transfers = n_transfers;
    stats->bytes = n_items * item;
  }
  if (n_bad)
    return fail(KVOFF_ESTATE, "%lld pool hits name a slot outside [0, %lld): table entries -1",
                (long long)n_bad, (long long)r.n_slots);
  return KVOFF_OK;
}

int launch_probe(const void* host_ptr, int64_t n_bytes, void* sink, int32_t n_wg,
                 hipStream_t stream) {
  const int64_t n16 = n_bytes / 16;
  const int64_t max_wg = (n16 + 1023) / 1024;
  int64_t wg = n_wg > 0 ? n_wg : 1024;
  if (wg > max_wg) wg = max_wg;
  hipLaunchKernelGGL(probe_kernel, dim3((unsigned)wg), dim3(256), 0, stream,
                     (const uint4*)host_ptr, n16, (uint32_t*)sink);
  KVOFF_HIP(hipGetLastError());
  return KVOFF_OK;
}

}  // namespace kvoff
