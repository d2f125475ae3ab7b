// api.cpp - extern "C" entry points of kvoff.h: argument checks, the
// context, the pinned host block store and the request table.  Kernels live
// in the .hip files; this file only validates and dispatches.
#include <cstdlib>
#include <cstring>
#include <new>

#include "kvoff_internal.h"

namespace kvoff {

bool test_fail_alloc(const char* what) {
  const char* e = std::getenv("KVOFF_TEST_FAIL_ALLOC");
  return e && std::strcmp(e, what) == 0;
}

int make_batch(const kvoff_ctx* ctx, int32_t n_req, const int32_t* req_ids, BatchIds* out) {
  if (n_req < 0) return fail(KVOFF_EINVAL, "n_req %d < 0", n_req);
  if (n_req > KVOFF_MAX_BATCH)
    return fail(KVOFF_ERANGE, "n_req %d exceeds KVOFF_MAX_BATCH %d", n_req, KVOFF_MAX_BATCH);
  if (n_req > 0 && !req_ids) return fail(KVOFF_EINVAL, "req_ids is NULL");
  out->n = n_req;
  for (int i = 0; i < n_req; ++i) {
    int32_t id = req_ids[i];
    if (id < 0 || id >= (int32_t)ctx->reqs.size())
      return fail(KVOFF_ESTATE, "request id %d is not registered", id);
    out->id[i] = id;
  }
  for (int i = n_req; i < KVOFF_MAX_BATCH; ++i) out->id[i] = 0;
  return KVOFF_OK;
}

// reads the n oldest in-use event sets of a kernel slot into its sums
static int read_pending_sets(kvoff_ctx* ctx, int slot, int n) {
  for (; n > 0; --n) {
    const int set = (ctx->kt_next[slot] - ctx->kt_pending[slot] + KT_RING) % KT_RING;
    const size_t i = 2 * ((size_t)slot * KT_RING + (size_t)set);
    float ms = 0.f;
    KVOFF_HIP(hipEventSynchronize(ctx->kt_ev[i + 1]));
    KVOFF_HIP(hipEventElapsedTime(&ms, ctx->kt_ev[i], ctx->kt_ev[i + 1]));
    ctx->kt_sum_ms[slot] += ms;
    ++ctx->kt_count[slot];
    --ctx->kt_pending[slot];
  }
  return KVOFF_OK;
}

int kernel_timing_advance(kvoff_ctx* ctx, int slot) {
  if (!ctx->kernel_timing) return KVOFF_OK;
  ctx->kt_next[slot] = (ctx->kt_next[slot] + 1) % KT_RING;
  ++ctx->kt_pending[slot];
  // the next launch reuses the oldest set once every set is in use
  return ctx->kt_pending[slot] == KT_RING ? read_pending_sets(ctx, slot, 1) : KVOFF_OK;
}

}  // namespace kvoff

using namespace kvoff;

extern "C" {

int kvoff_create(const kvoff_config* cfg, kvoff_ctx** out) {
  return guarded([&]() -> int {
    if (!cfg || !out) return fail(KVOFF_EINVAL, "cfg and out must be non-NULL");
    *out = nullptr;
    const kvoff_config& c = *cfg;
    if (c.num_layers < 1) return fail(KVOFF_EINVAL, "num_layers %d < 1", c.num_layers);
    if (c.num_kv_heads < 1 || c.num_q_heads < c.num_kv_heads || c.num_q_heads % c.num_kv_heads)
      return fail(KVOFF_EINVAL, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                  c.num_q_heads, c.num_kv_heads);
    int G = c.num_q_heads / c.num_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
      return fail(KVOFF_EINVAL, "group size %d must be 1, 2, 4, 8 or 16", G);
    if (c.num_kv_heads > 16) return fail(KVOFF_EINVAL, "num_kv_heads %d > 16", c.num_kv_heads);
    if (c.head_dim != kHeadDim) return fail(KVOFF_EINVAL, "head_dim %d must be 128", c.head_dim);
    if (c.block_size != 16 && c.block_size != 32)
      return fail(KVOFF_EINVAL, "block_size %d must be 16 or 32", c.block_size);
    if (c.dtype != KVOFF_F16 && c.dtype != KVOFF_BF16)
      return fail(KVOFF_EINVAL, "dtype %d must be KVOFF_F16 or KVOFF_BF16", c.dtype);
    if (c.max_requests < 1) return fail(KVOFF_EINVAL, "max_requests %d < 1", c.max_requests);
    if (c.host_capacity_blocks < 1)
      return fail(KVOFF_EINVAL, "host_capacity_blocks %lld < 1", (long long)c.host_capacity_blocks);
    if (c.host_mem_kind != KVOFF_HOST_COHERENT && c.host_mem_kind != KVOFF_HOST_NONCOHERENT)
      return fail(KVOFF_EINVAL, "host_mem_kind %d", c.host_mem_kind);

    int ndev = 0;
    hipError_t e = hipGetDeviceCount(&ndev);
    if (e != hipSuccess || ndev < 1)
      return fail(KVOFF_ENODEV, "no GPU visible (%s)", e == hipSuccess ? "0 devices" : hipGetErrorString(e));

    kvoff_ctx* ctx = new (std::nothrow) kvoff_ctx();
    if (!ctx) return fail(KVOFF_ENOMEM, "context allocation failed");
    ctx->cfg = c;
    ctx->G = G;
    const int64_t es = 2;
    ctx->slice_bytes = 2LL * c.block_size * c.head_dim * es;
    ctx->rec_bytes = ctx->slice_bytes * c.num_kv_heads;
    int status = KVOFF_OK;
    do {
      if (hipGetDevice(&ctx->device) != hipSuccess) {
        status = fail(KVOFF_EHIP, "hipGetDevice failed");
        break;
      }
      // kvoff_sparse_decode_noalloc's scratch: its address on this device
      if ((status = attend_scratch_address(ctx->device, &ctx->noalloc_scratch)) != KVOFF_OK) break;
      size_t bytes = (size_t)c.host_capacity_blocks * (size_t)ctx->rec_bytes;
      unsigned flags = hipHostMallocMapped | hipHostMallocPortable |
                       (c.host_mem_kind == KVOFF_HOST_COHERENT ? hipHostMallocCoherent
                                                               : hipHostMallocNonCoherent);
      void* p = nullptr;
      e = test_fail_alloc("store") ? hipErrorOutOfMemory : hipHostMalloc(&p, bytes, flags);
      if (e != hipSuccess || !p) {
        status = fail(KVOFF_ENOMEM, "pinned store of %zu bytes: %s", bytes, hipGetErrorString(e));
        break;
      }
      ctx->store = (uint8_t*)p;
      void* dp = nullptr;
      e = hipHostGetDevicePointer(&dp, p, 0);
      if (e != hipSuccess) {
        status = fail(KVOFF_EHIP, "hipHostGetDevicePointer: %s", hipGetErrorString(e));
        break;
      }
      ctx->store_dev = (uint8_t*)dp;
      // a device allocation that fails is a HIP error (EHIP), after the
      // store was allocated: the teardown below frees it
      e = test_fail_alloc("table") ? hipErrorOutOfMemory
                                   : hipMalloc(&ctx->d_reqs, sizeof(ReqDev) * (size_t)c.max_requests);
      if (e == hipSuccess) e = hipMalloc(&ctx->d_counters, 8 * sizeof(unsigned long long));
      for (int i = 0; i < 2 && e == hipSuccess; ++i)
        e = hipEventCreateWithFlags(&ctx->stage[i].done, hipEventDisableTiming);
      for (int i = 0; i < 2 && e == hipSuccess; ++i)
        e = hipEventCreateWithFlags(&ctx->ev_sel[i], hipEventDisableTiming);
      if (e != hipSuccess) {
        status = fail(KVOFF_EHIP, "context setup: %s", hipGetErrorString(e));
        break;
      }
    } while (0);
    if (status != KVOFF_OK) {
      kvoff_destroy(ctx);
      return status;
    }
    *out = ctx;
    return KVOFF_OK;
  });
}

int kvoff_destroy(kvoff_ctx* ctx) {
  return guarded([&]() -> int {
    if (!ctx) return KVOFF_OK;
    // best-effort teardown: errors here cannot be acted on
    int dev = 0;
    (void)hipGetDevice(&dev);
    (void)hipSetDevice(ctx->device);
    (void)hipDeviceSynchronize();
    for (int i = 0; i < 2; ++i) {
      if (ctx->ev_sel[i]) (void)hipEventDestroy(ctx->ev_sel[i]);
    }
    stage_pool_destroy(ctx);
    for (hipEvent_t e : ctx->ev_group) (void)hipEventDestroy(e);
    for (hipEvent_t e : ctx->ev_timing) (void)hipEventDestroy(e);
    if (ctx->copy2) (void)hipStreamDestroy(ctx->copy2);
    for (int k = 0; k < kDmaSideStreams; ++k) {
      if (ctx->dma_stream[k]) (void)hipStreamDestroy(ctx->dma_stream[k]);
      if (ctx->dma_done[k]) (void)hipEventDestroy(ctx->dma_done[k]);
    }
    for (hipEvent_t e : ctx->kt_ev)
      if (e) (void)hipEventDestroy(e);
    for (StageSet& ss : ctx->stage) {
      if (ss.done) (void)hipEventDestroy(ss.done);
      if (ss.buf) (void)hipHostFree(ss.buf);
      if (ss.table) (void)hipHostFree(ss.table);
      if (ss.sel) (void)hipHostFree(ss.sel);
    }
    if (ctx->d_counters) (void)hipFree(ctx->d_counters);
    if (ctx->d_reqs) (void)hipFree(ctx->d_reqs);
    if (ctx->store) (void)hipHostFree(ctx->store);
    (void)hipSetDevice(dev);
    delete ctx;
    return KVOFF_OK;
  });
}

int64_t kvoff_record_bytes(const kvoff_ctx* ctx) { return ctx ? ctx->rec_bytes : 0; }

int kvoff_set_consensus_lambda(kvoff_ctx* ctx, double lambda) {
  return guarded([&]() -> int {
    if (!ctx) return fail(KVOFF_EINVAL, "ctx is NULL");
    if (!(lambda >= 0.0) || lambda > 1e6) return fail(KVOFF_EINVAL, "lambda %g outside [0, 1e6]", lambda);
    ctx->consensus_lambda = lambda;
    return KVOFF_OK;
  });
}

int kvoff_set_attention_qk(kvoff_ctx* ctx, int32_t qk) {
  return guarded([&]() -> int {
    if (!ctx) return fail(KVOFF_EINVAL, "ctx is NULL");
    if (qk != KVOFF_QK_MFMA && qk != KVOFF_QK_VALU) return fail(KVOFF_EINVAL, "unknown QK engine %d", qk);
    if (qk == KVOFF_QK_VALU && ctx->G > 8)
      return fail(KVOFF_EINVAL, "the VALU QK needs G <= 8 (G = %d)", ctx->G);
    ctx->attn_qk = qk;
    return KVOFF_OK;
  });
}

int kvoff_register_request(kvoff_ctx* ctx, int64_t n_tokens, int32_t* req_id) {
  return guarded([&]() -> int {
    if (!ctx || !req_id) return fail(KVOFF_EINVAL, "ctx and req_id must be non-NULL");
    if (n_tokens < 1) return fail(KVOFF_EINVAL, "n_tokens %lld < 1", (long long)n_tokens);
    if ((int64_t)ctx->reqs.size() >= ctx->cfg.max_requests)
      return fail(KVOFF_ERANGE, "request table full (%d)", ctx->cfg.max_requests);
    int64_t nb = (n_tokens + ctx->cfg.block_size - 1) / ctx->cfg.block_size;
    if (nb > INT32_MAX / 2) return fail(KVOFF_ERANGE, "n_tokens %lld too large", (long long)n_tokens);
    int64_t need = nb * ctx->cfg.num_layers;
    if (ctx->store_used + need > ctx->cfg.host_capacity_blocks)
      return fail(KVOFF_ERANGE, "store full: %lld of %lld records used, request needs %lld",
                  (long long)ctx->store_used, (long long)ctx->cfg.host_capacity_blocks,
                  (long long)need);
    ReqHost h{ctx->store_used, n_tokens, nb};
    ReqDev d{h.rec_base, (int32_t)n_tokens, (int32_t)nb};
    int32_t id = (int32_t)ctx->reqs.size();
    DeviceScope dev_scope;
    KVOFF_HIP(dev_scope.enter(ctx->device));
    KVOFF_HIP(hipMemcpy(ctx->d_reqs + id, &d, sizeof d, hipMemcpyHostToDevice));
    ctx->reqs.push_back(h);
    ctx->offloaded.resize(ctx->reqs.size() * (size_t)ctx->cfg.num_layers, 0);
    ctx->resident.resize(ctx->reqs.size() * (size_t)ctx->cfg.num_layers, 0);
    ctx->store_used += need;
    *req_id = id;
    return KVOFF_OK;
  });
}

int kvoff_host_record(kvoff_ctx* ctx, int32_t layer, int32_t req_id, int64_t block,
                      const void** ptr) {
  return guarded([&]() -> int {
    if (!ctx || !ptr) return fail(KVOFF_EINVAL, "ctx and ptr must be non-NULL");
    if (req_id < 0 || req_id >= (int32_t)ctx->reqs.size())
      return fail(KVOFF_ESTATE, "request id %d is not registered", req_id);
    if (layer < 0 || layer >= ctx->cfg.num_layers) return fail(KVOFF_ERANGE, "layer %d", layer);
    const ReqHost& r = ctx->reqs[req_id];
    if (block < 0 || block >= r.nb) return fail(KVOFF_ERANGE, "block %lld", (long long)block);
    *ptr = ctx->store + (size_t)(r.rec_base + (int64_t)layer * r.nb + block) * ctx->rec_bytes;
    return KVOFF_OK;
  });
}

int kvoff_offload_blocks(kvoff_ctx* ctx, int32_t layer, int32_t req_id, const void* k_dev,
                         const void* v_dev, float* digest_dev, void* stream) {
  return guarded([&]() -> int {
    if (!ctx || !k_dev || !v_dev || !digest_dev)
      return fail(KVOFF_EINVAL, "ctx, k_dev, v_dev and digest_dev must be non-NULL");
    if (layer < 0 || layer >= ctx->cfg.num_layers)
      return fail(KVOFF_ERANGE, "layer %d outside [0, %d)", layer, ctx->cfg.num_layers);
    if (req_id < 0 || req_id >= (int32_t)ctx->reqs.size())
      return fail(KVOFF_ESTATE, "request id %d is not registered", req_id);
    DeviceScope dev_scope;
    KVOFF_HIP(dev_scope.enter(ctx->device));
    int st = launch_offload(ctx, layer, req_id, k_dev, v_dev, digest_dev, (hipStream_t)stream);
    if (st == KVOFF_OK) ctx->offloaded[(size_t)req_id * ctx->cfg.num_layers + layer] = 1;
    return st;
  });
}

static int check_layer_offloaded(const kvoff_ctx* ctx, int32_t layer, const BatchIds& b) {
  if (layer < 0 || layer >= ctx->cfg.num_layers)
    return fail(KVOFF_ERANGE, "layer %d outside [0, %d)", layer, ctx->cfg.num_layers);
  for (int i = 0; i < b.n; ++i)
    if (!ctx->offloaded[(size_t)b.id[i] * ctx->cfg.num_layers + layer])
      return fail(KVOFF_ESTATE, "layer %d of request %d was not offloaded", layer, b.id[i]);
  return KVOFF_OK;
}

int kvoff_select(kvoff_ctx* ctx, int32_t layer, int32_t n_req, const int32_t* req_ids,
                 const void* q_dev, const float* digest_dev, int64_t digest_stride,
                 const int32_t* topk, int32_t mode, double* scores_dev, int32_t* sel_idx_dev,
                 int32_t* sel_cnt_dev, int32_t k_stride, void* stream) {
  return guarded([&]() -> int {
    if (!ctx) return fail(KVOFF_EINVAL, "ctx is NULL");
    BatchIds b;
    int st = make_batch(ctx, n_req, req_ids, &b);
    if (st) return st;
    if (n_req == 0) return KVOFF_OK;
    if (layer < 0 || layer >= ctx->cfg.num_layers)
      return fail(KVOFF_ERANGE, "layer %d outside [0, %d)", layer, ctx->cfg.num_layers);
    if (!q_dev || !digest_dev || !topk || !scores_dev || !sel_idx_dev || !sel_cnt_dev)
      return fail(KVOFF_EINVAL, "NULL buffer argument");
    if (layout_of(mode) < 0) return fail(KVOFF_EINVAL, "mode %d", mode);
    if (k_stride < 1) return fail(KVOFF_EINVAL, "k_stride %d < 1", k_stride);
    int64_t max_nb = 0, min_nb = INT64_MAX;
    for (int i = 0; i < n_req; ++i) {
      const ReqHost& r = ctx->reqs[b.id[i]];
      if (topk[i] < 1) return fail(KVOFF_EINVAL, "topk[%d] = %d < 1", i, topk[i]);
      int64_t K = topk[i] < r.nb ? topk[i] : r.nb;
      if (K > k_stride)
        return fail(KVOFF_ERANGE, "K of request %d is %lld > k_stride %d", i, (long long)K, k_stride);
      if (r.nb > digest_stride)
        return fail(KVOFF_EINVAL, "digest_stride %lld < nb %lld of request %d",
                    (long long)digest_stride, (long long)r.nb, i);
      if (r.nb > max_nb) max_nb = r.nb;
      if (r.nb < min_nb) min_nb = r.nb;
    }
    DeviceScope dev_scope;
    KVOFF_HIP(dev_scope.enter(ctx->device));
    hipStream_t s = (hipStream_t)stream;
    st = launch_score(ctx, b, min_nb, max_nb, q_dev, digest_dev, digest_stride, mode, scores_dev, s);
    if (st) return st;
    if ((st = kernel_timing_advance(ctx, KT_SCORE))) return st;
    // consensus selections use the layout of their scope (shared or per KV head)
    st = launch_topk(ctx, b, topk, layout_of(mode), scores_dev, digest_stride, sel_idx_dev, sel_cnt_dev,
                     k_stride, s);
    if (st) return st;
    if ((st = kernel_timing_advance(ctx, KT_TOPK))) return st;
    return KVOFF_OK;
  });
}

static int read_counters(kvoff_ctx* ctx, const BatchIds& b, const RecallArgs& a,
                         kvoff_stats* stats, hipStream_t s) {
  unsigned long long c[8] = {0};
  KVOFF_HIP(hipMemcpyAsync(c, ctx->d_counters, sizeof c, hipMemcpyDeviceToHost, s));
  KVOFF_HIP(hipStreamSynchronize(s));
  int64_t item = a.mode == KVOFF_HEADWISE ? ctx->slice_bytes : ctx->rec_bytes;
  stats->selected = (int64_t)c[0];
  stats->pool_hits = (int64_t)c[1];
  stats->items_recalled = (int64_t)c[2];
  stats->transfers = (int64_t)c[3];
  stats->bytes = (int64_t)c[2] * item;
  (void)b;
  if (c[kBadSlots]) {
    // reported once: cleared for the calls that follow
    int st = launch_zero_counters(ctx, true, s);
    if (st) return st;
    return fail(KVOFF_ESTATE,
                "%llu pool hits (this call and earlier ones without stats) named a slot outside "
                "the pool: table entries -1",
                c[kBadSlots]);
  }
  return KVOFF_OK;
}

static int recall_impl(kvoff_ctx* ctx, const BatchIds& b, const RecallArgs& a, int32_t engine,
                       kvoff_stats* stats, hipStream_t s) {
  if (a.recall_base_slot < 0 ||
      a.recall_base_slot + (int64_t)b.n * a.k_stride > a.n_slots)
    return fail(KVOFF_ERANGE, "recall region [%lld, %lld) exceeds the pool's %lld slots",
                (long long)a.recall_base_slot,
                (long long)(a.recall_base_slot + (int64_t)b.n * a.k_stride), (long long)a.n_slots);
  if (engine == KVOFF_ENGINE_DMA) return recall_dma(ctx, b, a, stats, s);
  if (engine == KVOFF_ENGINE_STAGED) return recall_staged(ctx, b, a, stats, s);
  if (engine != KVOFF_ENGINE_ZEROCOPY) return fail(KVOFF_EINVAL, "engine %d", engine);
  int st;
  if (stats && (st = launch_zero_counters(ctx, false, s))) return st;
  if ((st = launch_gather(ctx, b, a, stats != nullptr, s))) return st;
  if (stats) return read_counters(ctx, b, a, stats, s);
  return KVOFF_OK;
}

int kvoff_recall(kvoff_ctx* ctx, int32_t layer, int32_t n_req, const int32_t* req_ids,
                 int32_t mode, const int32_t* sel_idx_dev, const int32_t* sel_cnt_dev,
                 int32_t k_stride, const uint8_t* pool_hit_dev, const int32_t* pool_slot_dev,
                 int64_t pool_stride, void* slot_pool_dev, int64_t n_slots,
                 int64_t recall_base_slot, int32_t* block_table_dev, int32_t engine,
                 kvoff_stats* stats, void* stream) {
  return guarded([&]() -> int {
    if (!ctx) return fail(KVOFF_EINVAL, "ctx is NULL");
    BatchIds b;
    int st = make_batch(ctx, n_req, req_ids, &b);
    if (st) return st;
    if (stats) memset(stats, 0, sizeof *stats);
    if (n_req == 0) return KVOFF_OK;
    if ((st = check_layer_offloaded(ctx, layer, b))) return st;
    if (!sel_idx_dev || !sel_cnt_dev || !slot_pool_dev || !block_table_dev)
      return fail(KVOFF_EINVAL, "NULL buffer argument");
    mode = layout_of(mode);  // consensus modes use the layout of their scope
    if (mode < 0) return fail(KVOFF_EINVAL, "unknown mode");
    if (k_stride < 1) return fail(KVOFF_EINVAL, "k_stride %d < 1", k_stride);
    // table entries are int32 slot (headwise: slice) indices
    if (n_slots < 1 || n_slots > INT32_MAX / ctx->cfg.num_kv_heads)
      return fail(KVOFF_EINVAL, "n_slots %lld outside [1, %d]", (long long)n_slots,
                  INT32_MAX / ctx->cfg.num_kv_heads);
    if ((pool_hit_dev == nullptr) != (pool_slot_dev == nullptr))
      return fail(KVOFF_EINVAL, "pool_hit_dev and pool_slot_dev must both be given or both NULL");
    if (pool_hit_dev) {
      for (int i = 0; i < n_req; ++i)
        if (ctx->reqs[b.id[i]].nb > pool_stride)
          return fail(KVOFF_EINVAL, "pool_stride %lld < nb of request %d", (long long)pool_stride, i);
    }
    DeviceScope dev_scope;
    KVOFF_HIP(dev_scope.enter(ctx->device));
    RecallArgs a{layer,       mode,         sel_idx_dev, sel_cnt_dev,
                 k_stride,    pool_hit_dev, pool_slot_dev, pool_stride,
                 (uint8_t*)slot_pool_dev, n_slots, recall_base_slot, block_table_dev};
    return recall_impl(ctx, b, a, engine, stats, (hipStream_t)stream);
  });
}

size_t kvoff_workspace_size(const kvoff_ctx* ctx, int32_t call, int32_t n_req, int32_t k_stride,
                            int32_t mode) {
  (void)mode;
  if (!ctx || n_req < 0 || k_stride < 1) return 0;
  if (call == KVOFF_CALL_SPARSE_DECODE || call == KVOFF_CALL_STEP)
    return attend_ws_bytes(ctx, n_req, k_stride);
  return 0;
}

}  // extern "C"

// kvoff_sparse_decode and its no-alloc form: ws_dev is the caller's
// workspace or the library's scratch array (noalloc), ws_bytes its size
static int sparse_decode_impl(kvoff_ctx* ctx, int32_t n_req, const int32_t* req_ids, int32_t mode,
                              const void* q_dev, const void* slot_pool_dev, int64_t n_slots,
                              const int32_t* block_table_dev, const int32_t* sel_idx_dev,
                              const int32_t* sel_cnt_dev, int32_t k_stride, float scale,
                              float* out_dev, void* ws_dev, size_t ws_bytes, bool noalloc,
                              void* stream) {
  if (!ctx) return fail(KVOFF_EINVAL, "ctx is NULL");
  BatchIds b;
  int st = make_batch(ctx, n_req, req_ids, &b);
  if (st) return st;
  if (n_req == 0) return KVOFF_OK;
  if (!q_dev || !slot_pool_dev || !block_table_dev || !sel_idx_dev || !sel_cnt_dev || !out_dev)
    return fail(KVOFF_EINVAL, "NULL buffer argument");
  mode = layout_of(mode);  // consensus modes use the layout of their scope
  if (mode < 0) return fail(KVOFF_EINVAL, "unknown mode");
  if (k_stride < 1) return fail(KVOFF_EINVAL, "k_stride %d < 1", k_stride);
  if (n_slots < 1 || n_slots > INT32_MAX / ctx->cfg.num_kv_heads)
    return fail(KVOFF_EINVAL, "n_slots %lld outside [1, %d]", (long long)n_slots,
                INT32_MAX / ctx->cfg.num_kv_heads);
  size_t need = attend_ws_bytes(ctx, n_req, k_stride);
  if (noalloc && need > ws_bytes)
    return fail(KVOFF_ERANGE, "split partials of %zu bytes exceed the %zu-byte scratch array",
                need, ws_bytes);
  if (need > 0 && (!ws_dev || ws_bytes < need))
    return fail(KVOFF_ERANGE, "workspace of %zu bytes < %zu needed", ws_bytes, need);
  DeviceScope dev_scope;
  KVOFF_HIP(dev_scope.enter(ctx->device));
  st = launch_attend(ctx, b, mode, q_dev, slot_pool_dev, n_slots, block_table_dev, sel_idx_dev,
                     sel_cnt_dev, k_stride, scale, out_dev, ws_dev, (hipStream_t)stream);
  if (st) return st;
  if ((st = kernel_timing_advance(ctx, KT_ATTEND))) return st;
  if ((st = kernel_timing_advance(ctx, KT_COMBINE))) return st;
  return KVOFF_OK;
}

extern "C" {

int kvoff_sparse_decode(kvoff_ctx* ctx, int32_t n_req, const int32_t* req_ids, int32_t mode,
                        const void* q_dev, const void* slot_pool_dev, int64_t n_slots,
                        const int32_t* block_table_dev, const int32_t* sel_idx_dev,
                        const int32_t* sel_cnt_dev, int32_t k_stride, float scale,
                        float* out_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  return guarded([&]() -> int {
    return sparse_decode_impl(ctx, n_req, req_ids, mode, q_dev, slot_pool_dev, n_slots,
                              block_table_dev, sel_idx_dev, sel_cnt_dev, k_stride, scale, out_dev,
                              ws_dev, ws_bytes, false, stream);
  });
}

int kvoff_sparse_decode_noalloc(kvoff_ctx* ctx, int32_t n_req, const int32_t* req_ids,
                                int32_t mode, const void* q_dev, const void* slot_pool_dev,
                                int64_t n_slots, const int32_t* block_table_dev,
                                const int32_t* sel_idx_dev, const int32_t* sel_cnt_dev,
                                int32_t k_stride, float scale, float* out_dev, void* stream) {
  return guarded([&]() -> int {
    if (!ctx) return fail(KVOFF_EINVAL, "ctx is NULL");
    if (!ctx->noalloc_scratch) return fail(KVOFF_ESTATE, "the context has no scratch address");
    return sparse_decode_impl(ctx, n_req, req_ids, mode, q_dev, slot_pool_dev, n_slots,
                              block_table_dev, sel_idx_dev, sel_cnt_dev, k_stride, scale, out_dev,
                              ctx->noalloc_scratch, KVOFF_NOALLOC_SCRATCH_BYTES, true, stream);
  });
}

int kvoff_attention_mass(kvoff_ctx* ctx, int32_t layer, int32_t n_req, const int32_t* req_ids,
                         int32_t mode, const void* q_dev, const int32_t* sel_idx_dev,
                         const int32_t* sel_cnt_dev, int32_t k_stride, float scale,
                         double* mass_dev, void* stream) {
  return guarded([&]() -> int {
    if (!ctx) return fail(KVOFF_EINVAL, "ctx is NULL");
    BatchIds b;
    int st = make_batch(ctx, n_req, req_ids, &b);
    if (st) return st;
    if (n_req == 0) return KVOFF_OK;
    if (layer < 0 || layer >= ctx->cfg.num_layers)
      return fail(KVOFF_ERANGE, "layer %d outside [0, %d)", layer, ctx->cfg.num_layers);
    if (!q_dev || !sel_idx_dev || !sel_cnt_dev || !mass_dev)
      return fail(KVOFF_EINVAL, "NULL buffer argument");
    mode = layout_of(mode);
    if (mode < 0) return fail(KVOFF_EINVAL, "unknown mode");
    if (k_stride < 1) return fail(KVOFF_EINVAL, "k_stride %d < 1", k_stride);
    if ((st = check_layer_offloaded(ctx, layer, b))) return st;
    DeviceScope dev_scope;
    KVOFF_HIP(dev_scope.enter(ctx->device));
    return launch_mass(ctx, b, layer, mode, q_dev, sel_idx_dev, sel_cnt_dev, k_stride, scale,
                       mass_dev, (hipStream_t)stream);
  });
}

int kvoff_set_kernel_timing(kvoff_ctx* ctx, int32_t on) {
  return guarded([&]() -> int {
    if (!ctx) return fail(KVOFF_EINVAL, "ctx is NULL");
    if (on && ctx->kt_ev.empty()) {
      DeviceScope dev_scope;
      KVOFF_HIP(dev_scope.enter(ctx->device));
      ctx->kt_ev.reserve(2 * (size_t)KT_N * KT_RING);
      while (ctx->kt_ev.size() < 2 * (size_t)KT_N * KT_RING) {
        hipEvent_t e;
        KVOFF_HIP(hipEventCreate(&e));
        ctx->kt_ev.push_back(e);
      }
    }
    ctx->kernel_timing = on != 0;
    for (int k = 0; k < KT_N; ++k) {
      ctx->kt_next[k] = ctx->kt_pending[k] = 0;
      ctx->kt_sum_ms[k] = 0.0;
      ctx->kt_count[k] = 0;
    }
    return KVOFF_OK;
  });
}

int kvoff_get_kernel_times(kvoff_ctx* ctx, kvoff_kernel_times* t) {
  return guarded([&]() -> int {
    if (!ctx || !t) return fail(KVOFF_EINVAL, "ctx and t must be non-NULL");
    for (int k = 0; k < KT_N; ++k) {
      int st = read_pending_sets(ctx, k, ctx->kt_pending[k]);
      if (st) return st;
    }
    double ms[KT_N];
    for (int k = 0; k < KT_N; ++k)
      ms[k] = ctx->kt_count[k] ? ctx->kt_sum_ms[k] / (double)ctx->kt_count[k] : 0.0;
    t->score_ms = ms[KT_SCORE];
    t->topk_ms = ms[KT_TOPK];
    t->attend_ms = ms[KT_ATTEND];
    t->combine_ms = ms[KT_COMBINE];
    t->select_calls = ctx->kt_count[KT_SCORE];
    t->decode_calls = ctx->kt_count[KT_ATTEND];
    return KVOFF_OK;
  });
}

int kvoff_probe_read(const void* ptr, int64_t n_bytes, void* dev_sink, int32_t n_wg,
                     void* stream) {
  return guarded([&]() -> int {
    if (!ptr || !dev_sink) return fail(KVOFF_EINVAL, "NULL pointer");
    if (n_bytes <= 0 || n_bytes % 4096)
      return fail(KVOFF_EINVAL, "n_bytes must be a positive multiple of 4096");
    hipPointerAttribute_t attr;
    KVOFF_HIP(hipPointerGetAttributes(&attr, ptr));
    const void* dp = ptr;
    if (attr.type == hipMemoryTypeHost) {
      void* mapped = nullptr;
      KVOFF_HIP(hipHostGetDevicePointer(&mapped, const_cast<void*>(ptr), 0));
      dp = mapped;
    } else if (attr.type != hipMemoryTypeDevice) {
      return fail(KVOFF_EINVAL, "probe pointer is neither device memory nor pinned host memory");
    }
    return launch_probe(dp, n_bytes, dev_sink, n_wg, (hipStream_t)stream);
  });
}

}  // extern "C"
