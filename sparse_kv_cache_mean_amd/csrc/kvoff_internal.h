// kvoff_internal.h - context, error plumbing and kernel launchers shared by
// the library's translation units.  Not part of the ABI.
#pragma once

#include <exception>
#include <new>
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/kvoff.h"
#include "host_errors.h"

namespace kvoff {

constexpr int kHeadDim = 128;

// device statistics counters of the context (d_counters[8]): 0..3 the
// per-call recall statistics (selected, pool hits, items, transfers), and
// the sticky count of pool hits whose slot lay outside the pool
constexpr int kBadSlots = 4;

// copy streams the DMA engine owns beside the caller's
constexpr int kDmaSideStreams = 3;

// Per-request entry of the device request table.  The record of
// (layer, request, block) sits at store + (rec_base + layer*nb + block) * rec_bytes.
struct ReqDev {
  int64_t rec_base;
  int32_t n_tokens;
  int32_t nb;
};

// Request ids of one call, passed by value in kernel arguments.
struct BatchIds {
  int32_t n;
  int32_t id[KVOFF_MAX_BATCH];
};

struct ReqHost {
  int64_t rec_base;
  int64_t n_tokens;
  int64_t nb;
};

class StagePool;

// One set of the staged engine's pinned host buffers and the event behind
// the last copy that reads them.  The context holds two, used by turns, so
// that a call can gather into one set while the previous call's copies
// still read the other.
struct StageSet {
  void* buf = nullptr;    // staging buffer, grown on demand
  size_t cap = 0;
  void* table = nullptr;  // block-table staging
  size_t table_cap = 0;
  void* sel = nullptr;    // read-back of the selection and pool maps
  size_t sel_cap = 0;
  hipEvent_t done = nullptr;  // behind the set's last copy
  bool pending = false;       // `done` recorded and not yet waited for
};

// kernels timed by kvoff_set_kernel_timing, in kvoff_kernel_times order,
// and the event sets each keeps in its ring
enum KernelSlot { KT_SCORE = 0, KT_TOPK, KT_ATTEND, KT_COMBINE, KT_N };
constexpr int KT_RING = 64;

// start/stop events of one kernel launch; both null: an untimed launch
struct KEv {
  hipEvent_t start = nullptr, stop = nullptr;
};

}  // namespace kvoff

struct kvoff_ctx {
  kvoff_config cfg;
  int device = 0;
  int G = 1;
  double consensus_lambda = 0.5;  // KVOFF_CONSENSUS mode
  int32_t attn_qk = KVOFF_QK_MFMA;  // what computes the attention's QK^T
  int64_t rec_bytes = 0;    // 2 * Hkv * bs * d * es
  int64_t slice_bytes = 0;  // 2 * bs * d * es (K and V of one KV head)
  uint8_t* store = nullptr; // pinned host store (mapped into the GPU's address space)
  uint8_t* store_dev = nullptr;  // device-side address of the store
  int64_t store_used = 0;   // records reserved so far
  std::vector<kvoff::ReqHost> reqs;
  std::vector<uint8_t> offloaded;  // [req][layer]: offload enqueued
  std::vector<uint8_t> resident;   // [req][layer]: pinned in HBM by kvoff_make_resident
  kvoff::ReqDev* d_reqs = nullptr; // device copy of the request table
  unsigned long long* d_counters = nullptr;  // recall statistics (device)
  hipEvent_t ev_sel[2] = {nullptr, nullptr};  // selection -> recall hand-off per buffer set
  // staged (CPU gather + bulk copy) recall engine
  kvoff::StagePool* stage_pool = nullptr;  // host worker threads, created on first use
  kvoff::StageSet stage[2];                 // pinned buffers, used by turns
  int stage_next = 0;                       // the set the next staged call uses
  std::vector<hipEvent_t> ev_group;         // per request group (interruptible step)
  std::vector<hipEvent_t> ev_timing;        // timing events of kvoff_step (on request)
  void* noalloc_scratch = nullptr;          // device address of the attention scratch array
  hipStream_t copy2 = nullptr;              // kvoff_step's own second copy stream (lazy)
  hipStream_t dma_stream[kvoff::kDmaSideStreams] = {};  // DMA engine's copy streams (lazy)
  hipEvent_t dma_done[kvoff::kDmaSideStreams] = {};     // behind each one's last copy
  // per-kernel timing (kvoff_set_kernel_timing): per kernel slot a ring of
  // KT_RING (start, stop) event pairs, [slot][set][start|stop]; sets in use
  // are the `pending` ones before `next`; their durations, once read, go to
  // the sums
  bool kernel_timing = false;
  std::vector<hipEvent_t> kt_ev;
  int kt_next[kvoff::KT_N] = {};
  int kt_pending[kvoff::KT_N] = {};
  double kt_sum_ms[kvoff::KT_N] = {};
  int64_t kt_count[kvoff::KT_N] = {};
};

namespace kvoff {

// Test switch for the allocation-failure paths: true when the environment
// variable KVOFF_TEST_FAIL_ALLOC names `what` ("store": the pinned store of
// kvoff_create; "table": the device request table, allocated after the
// store; "staging": the staged engine's pinned staging buffer).  Read at
// each of those allocations, which are rare, so a test can set and clear it
// between calls.
bool test_fail_alloc(const char* what);

// Makes `dev` the calling thread's current device for the life of the
// object and, if it was another one, restores that one after: a call into
// the library leaves the caller's current device as it found it.
class DeviceScope {
 public:
  hipError_t enter(int dev) {
    hipError_t e = hipGetDevice(&prev_);
    if (e != hipSuccess || prev_ == dev) return e;
    e = hipSetDevice(dev);
    switched_ = e == hipSuccess;
    return e;
  }
  ~DeviceScope() {
    if (switched_) (void)hipSetDevice(prev_);
  }

 private:
  int prev_ = -1;
  bool switched_ = false;
};

#define KVOFF_HIP(call)                                                            \
  do {                                                                             \
    hipError_t e_ = (call);                                                        \
    if (e_ != hipSuccess)                                                          \
      return ::kvoff::fail(KVOFF_EHIP, "%s failed: %s (%s:%d)", #call,             \
                           hipGetErrorString(e_), __FILE__, __LINE__);             \
  } while (0)

// selection layout of a mode: one set per KV head (KVOFF_HEADWISE) or one
// shared set (KVOFF_SOLOHEAD); -1 for an unknown mode
inline int32_t layout_of(int32_t mode) {
  switch (mode) {
    case KVOFF_SOLOHEAD:
    case KVOFF_CONSENSUS: return KVOFF_SOLOHEAD;
    case KVOFF_HEADWISE:
    case KVOFF_CONSENSUS_GROUP: return KVOFF_HEADWISE;
    default: return -1;
  }
}

// the next events of a kernel slot while per-kernel timing is on, else none
inline KEv kernel_events(const kvoff_ctx* ctx, int slot) {
  KEv e;
  if (ctx->kernel_timing) {
    const size_t i = 2 * ((size_t)slot * KT_RING + (size_t)ctx->kt_next[slot]);
    e.start = ctx->kt_ev[i];
    e.stop = ctx->kt_ev[i + 1];
  }
  return e;
}

// after a launch that used kernel_events(ctx, slot): moves the slot's ring
// on, first reading the oldest set when the ring is full
int kernel_timing_advance(kvoff_ctx* ctx, int slot);

// Launch of `kernel` on `stream`: with the start/stop events bound to the
// dispatch itself (hipExtLaunchKernelGGL) when `ev` holds them, else plain.
#define KVOFF_LAUNCH(ev, kernel, grid, block, lds, stream, ...)                             \
  do {                                                                                     \
    if ((ev).start)                                                                        \
      hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, (ev).start, (ev).stop, 0,     \
                            __VA_ARGS__);                                                  \
    else                                                                                   \
      hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);                   \
  } while (0)

// check a batch and fill BatchIds; ESTATE for an unknown id
int make_batch(const kvoff_ctx* ctx, int32_t n_req, const int32_t* req_ids, BatchIds* out);

// ---- launchers (each returns a kvoff status) ----

int launch_offload(const kvoff_ctx* ctx, int32_t layer, int32_t req_id, const void* k_dev,
                   const void* v_dev, float* digest_dev, hipStream_t stream);

int launch_score(const kvoff_ctx* ctx, const BatchIds& b, int64_t min_nb, int64_t max_nb,
                 const void* q_dev, const float* digest_dev, int64_t digest_stride, int32_t mode,
                 double* scores_dev, hipStream_t stream);

int launch_topk(const kvoff_ctx* ctx, const BatchIds& b, const int32_t* topk_host,
                int32_t mode, const double* scores_dev, int64_t digest_stride,
                int32_t* sel_idx_dev, int32_t* sel_cnt_dev, int32_t k_stride,
                hipStream_t stream);

struct RecallArgs {
  int32_t layer;
  int32_t mode;
  const int32_t* sel_idx;
  const int32_t* sel_cnt;
  int32_t k_stride;
  const uint8_t* pool_hit;
  const int32_t* pool_slot;
  int64_t pool_stride;
  uint8_t* pool;
  int64_t n_slots;
  int64_t recall_base_slot;
  int32_t* table;
};

int launch_gather(const kvoff_ctx* ctx, const BatchIds& b, const RecallArgs& a, bool count,
                  hipStream_t stream);
int launch_table(const kvoff_ctx* ctx, const BatchIds& b, const RecallArgs& a,
                 hipStream_t stream);
// sticky = false: clear the per-call statistics; true: clear the
// out-of-range slot count
int launch_zero_counters(const kvoff_ctx* ctx, bool sticky, hipStream_t stream);

int recall_dma(kvoff_ctx* ctx, const BatchIds& b, const RecallArgs& a, kvoff_stats* stats,
               hipStream_t stream);
int recall_staged(kvoff_ctx* ctx, const BatchIds& b, const RecallArgs& a, kvoff_stats* stats,
                  hipStream_t stream);
void stage_pool_destroy(kvoff_ctx* ctx);

int launch_mass(const kvoff_ctx* ctx, const BatchIds& b, int32_t layer, int32_t mode,
                const void* q_dev, const int32_t* sel_idx, const int32_t* sel_cnt,
                int32_t k_stride, float scale, double* mass_dev, hipStream_t stream);

// device address of the attention's file-scope scratch array on `device`
// (which must be current), looked up once per device
int attend_scratch_address(int device, void** out);

// split policy of the attention kernel: number of splits per (request, KV head)
int attend_splits(int32_t n_req, int32_t Hkv, int32_t k_stride, int G);
size_t attend_ws_bytes(const kvoff_ctx* ctx, int32_t n_req, int32_t k_stride);

int launch_attend(const kvoff_ctx* ctx, const BatchIds& b, int32_t mode, const void* q_dev,
                  const void* pool, int64_t n_slots, const int32_t* table, const int32_t* sel_idx,
                  const int32_t* sel_cnt, int32_t k_stride, float scale, float* out,
                  void* ws, hipStream_t stream);

int launch_probe(const void* host_ptr, int64_t n_bytes, void* sink, int32_t n_wg,
                 hipStream_t stream);

}  // namespace kvoff
