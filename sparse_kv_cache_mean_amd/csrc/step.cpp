// step.cpp - kvoff_step: select, recall and attend over a range of layers
// with recall of layer l+1 overlapped with attention of layer l.
//
// The guide's analysis ("PulseInfer Guide", aiFetchly, section "The Fallacy
// of Naive Offloading", prefetching mismatch; section "Interruptible
// Layer-Wise Scheduling") is that recall must run while the GPU computes.
// On one GPU this is a compute stream, two copy streams and two buffer sets:
//   compute stream:  select(0) select(1) attend(0) select(2) attend(1) ...
//   copy stream:     recall(0) recall(2) recall(4) ...
//   copy stream 2:   recall(1) recall(3) recall(5) ...
// recall(l) waits for the event recorded after select(l); attend(l) waits
// for the event recorded after recall(l).  Buffer set l%2 is rewritten by
// select(l+2) and recall(l+2) only after attend(l) completed, because
// select(l+2) is enqueued on the compute stream after attend(l) and
// recall(l+2) waits for select(l+2).  Every kernel reads exactly the data a
// serial run would, so outputs are bit-identical to the serial order.
//
// Recalls of even and odd layers use different copy streams: a recall then
// starts as soon as its own dependencies are met instead of queueing behind
// the previous layer's recall and a cross-stream wait (measured when chosen:
// 11 us per layer on one copy stream; with the current select and attention
// kernels the two forms run within 0.2% of each other on the
// Llama-3-8B-shaped layer).  Two recalls then share the link for most of
// their length, and the link idles while the next selection waits for the
// attention ahead of it on the compute stream: 10-75 us per pair of layers
// in a kernel trace.
//
// With group_requests > 0 each layer's recall and attention are issued per
// contiguous request group, every group's attention waiting only for its own
// recall: the per-request form of the guide's interruptible layer-wise
// scheduling.  Within a layer the groups go in ascending order of the blocks
// they must transfer (selected blocks of requests not pinned in HBM for that
// layer by kvoff_make_resident), so groups already in HBM are attended while
// the others are still crossing the link.
#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "kvoff_internal.h"

using namespace kvoff;

extern "C" int kvoff_step(kvoff_ctx* ctx, const kvoff_step_args* A) {
  return guarded([&]() -> int {
    if (!ctx || !A) return fail(KVOFF_EINVAL, "ctx and args must be non-NULL");
    const int L = A->layer_end - A->layer_begin;
    if (L < 0 || A->layer_begin < 0 || A->layer_end > ctx->cfg.num_layers)
      return fail(KVOFF_ERANGE, "layers [%d, %d) outside [0, %d)", A->layer_begin, A->layer_end,
                  ctx->cfg.num_layers);
    if (A->stats) memset(A->stats, 0, sizeof *A->stats);
    if (A->timing) memset(A->timing, 0, sizeof *A->timing);
    if (L == 0 || A->n_req == 0) return KVOFF_OK;
    if (!A->q_dev || !A->digest_dev || !A->out_dev || !A->req_ids || !A->topk)
      return fail(KVOFF_EINVAL, "q_dev, digest_dev, out_dev, req_ids and topk must be non-NULL");
    for (int i = 0; i < 2; ++i)
      if (!A->scores_dev[i] || !A->sel_idx_dev[i] || !A->sel_cnt_dev[i] || !A->block_table_dev[i])
        return fail(KVOFF_EINVAL, "buffer set %d has a NULL buffer", i);
    // every per-layer pointer up front, so a bad one never leaves a step half enqueued
    for (int li = 0; li < L; ++li) {
      if (!A->q_dev[li] || !A->digest_dev[li] || !A->out_dev[li])
        return fail(KVOFF_EINVAL, "layer %d: NULL q, digest or out", A->layer_begin + li);
      if (A->pool_hit_dev && (!A->pool_hit_dev[li] != !(A->pool_slot_dev && A->pool_slot_dev[li])))
        return fail(KVOFF_EINVAL, "layer %d: pool hit and slot maps must both be given or both NULL",
                    A->layer_begin + li);
    }
    if (!A->pool_hit_dev != !A->pool_slot_dev)
      return fail(KVOFF_EINVAL, "pool_hit_dev and pool_slot_dev must both be given or both NULL");
    // overlapped layers write one buffer set's recall region while attention
    // reads the other's: the two regions of n_req * k_stride slots must not
    // share a slot
    const int64_t region = (int64_t)A->n_req * A->k_stride;
    const int64_t gap = A->recall_base_slot[0] > A->recall_base_slot[1]
                            ? A->recall_base_slot[0] - A->recall_base_slot[1]
                            : A->recall_base_slot[1] - A->recall_base_slot[0];
    if (L > 1 && A->copy_stream != A->compute_stream && gap < region)
      return fail(KVOFF_EINVAL,
                  "overlapped layers need disjoint recall regions: bases %lld and %lld are %lld "
                  "slots apart, a region is %lld",
                  (long long)A->recall_base_slot[0], (long long)A->recall_base_slot[1],
                  (long long)gap, (long long)region);

    hipStream_t cs = (hipStream_t)A->compute_stream;
    hipStream_t xs0 = (hipStream_t)A->copy_stream;
    DeviceScope dev_scope;
    KVOFF_HIP(dev_scope.enter(ctx->device));
    // odd layers recall on a second copy stream (the caller's, or the
    // context's own), so consecutive recalls do not queue behind each other
    hipStream_t xs1 = xs0;
    if (xs0 != cs && L > 1) {
      if (A->copy_stream2) {
        xs1 = (hipStream_t)A->copy_stream2;
      } else {
        if (!ctx->copy2) KVOFF_HIP(hipStreamCreateWithFlags(&ctx->copy2, hipStreamNonBlocking));
        xs1 = ctx->copy2;
      }
    }
    auto xs_of = [&](int li) { return (li & 1) ? xs1 : xs0; };

    auto select_l = [&](int li) -> int {
      const int buf = li & 1;
      int st = kvoff_select(ctx, A->layer_begin + li, A->n_req, A->req_ids, A->q_dev[li],
                            A->digest_dev[li], A->digest_stride, A->topk, A->mode,
                            A->scores_dev[buf], A->sel_idx_dev[buf], A->sel_cnt_dev[buf],
                            A->k_stride, cs);
      if (st) return st;
      KVOFF_HIP(hipEventRecord(ctx->ev_sel[buf], cs));
      return KVOFF_OK;
    };
    // request groups (one group = the whole batch unless group_requests > 0)
    struct Group {
      int r0, n;
    };
    std::vector<Group> groups;
    const int gsz = A->group_requests > 0 ? A->group_requests : A->n_req;
    for (int r0 = 0; r0 < A->n_req; r0 += gsz) {
      groups.push_back(Group{r0, std::min(gsz, A->n_req - r0)});
      for (int r = r0; r < r0 + groups.back().n; ++r)
        if (A->req_ids[r] < 0 || A->req_ids[r] >= (int)ctx->reqs.size())
          return fail(KVOFF_ESTATE, "request id %d is not registered", A->req_ids[r]);
    }
    // every (layer, request) offloaded, so that the only ESTATE a recall
    // below can return is the pool-slot report, after enqueuing its work
    for (int li = 0; li < L; ++li)
      for (int r = 0; r < A->n_req; ++r)
        if (!ctx->offloaded[(size_t)A->req_ids[r] * ctx->cfg.num_layers + A->layer_begin + li])
          return fail(KVOFF_ESTATE, "layer %d of request %d was not offloaded", A->layer_begin + li,
                      A->req_ids[r]);
    // issue order of the groups for layer li: fewest blocks to transfer first
    // (stable, so equal groups keep batch order)
    auto order_for = [&](int li) {
      const int layer = A->layer_begin + li;
      std::vector<int64_t> key(groups.size(), 0);
      for (size_t gi = 0; gi < groups.size(); ++gi)
        for (int r = groups[gi].r0; r < groups[gi].r0 + groups[gi].n; ++r) {
          const int id = A->req_ids[r];
          if (!ctx->resident[(size_t)id * ctx->cfg.num_layers + layer])
            key[gi] += std::min<int64_t>(A->topk[r], ctx->reqs[id].nb);
        }
      std::vector<int> ord(groups.size());
      for (size_t gi = 0; gi < groups.size(); ++gi) ord[gi] = (int)gi;
      std::stable_sort(ord.begin(), ord.end(), [&](int a, int b) { return key[a] < key[b]; });
      return ord;
    };
    const size_t n_ev = 2 * groups.size();
    while (ctx->ev_group.size() < n_ev) {
      hipEvent_t e;
      KVOFF_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
      ctx->ev_group.push_back(e);
    }
    // timing events (on request): the step's start, then per (layer, group)
    // before the wait for its recall, after it, after its attention, and on
    // the copy stream before and after its recall call
    const size_t NG = groups.size();
    auto tev = [&](int li, size_t gi, int k) { return ctx->ev_timing[1 + ((size_t)li * NG + gi) * 5 + k]; };
    if (A->timing) {
      while (ctx->ev_timing.size() < 1 + 5 * (size_t)L * NG) {
        hipEvent_t e;
        KVOFF_HIP(hipEventCreate(&e));
        ctx->ev_timing.push_back(e);
      }
    }
    const int sets = layout_of(A->mode) == KVOFF_HEADWISE ? ctx->cfg.num_kv_heads : 1;
    const int64_t q_row = (int64_t)ctx->cfg.num_q_heads * ctx->cfg.head_dim;  // elements per request

    // a recall that reports pool hits outside the pool (ESTATE, only known
    // when stats are filled) has still enqueued its work: the step goes on
    // and returns that status at the end
    int deferred = KVOFF_OK;
    std::string deferred_msg;
    auto recall_l = [&](int li) -> int {
      const int buf = li & 1;
      // this layer's pool maps (a layer may have none)
      const uint8_t* hit_l = A->pool_hit_dev ? A->pool_hit_dev[li] : nullptr;
      const int32_t* slot_l = A->pool_slot_dev ? A->pool_slot_dev[li] : nullptr;
      hipStream_t xs = xs_of(li);
      KVOFF_HIP(hipStreamWaitEvent(xs, ctx->ev_sel[buf], 0));
      for (int gi : order_for(li)) {
        const Group& g = groups[gi];
        const int64_t sel_off = (int64_t)g.r0 * sets * A->k_stride;
        kvoff_stats st_l;
        if (A->timing) KVOFF_HIP(hipEventRecord(tev(li, gi, 3), xs));
        int st = kvoff_recall(
            ctx, A->layer_begin + li, g.n, A->req_ids + g.r0, A->mode, A->sel_idx_dev[buf] + sel_off,
            A->sel_cnt_dev[buf] + g.r0, A->k_stride,
            hit_l ? hit_l + (int64_t)g.r0 * A->pool_stride : nullptr,
            slot_l ? slot_l + (int64_t)g.r0 * A->pool_stride : nullptr,
            A->pool_stride, A->slot_pool_dev, A->n_slots,
            A->recall_base_slot[buf] + (int64_t)g.r0 * A->k_stride, A->block_table_dev[buf] + sel_off,
            A->engine, A->stats ? &st_l : nullptr, xs);
        if (st == KVOFF_ESTATE && deferred == KVOFF_OK) {
          deferred = st;
          deferred_msg = kvoff_last_error();
          st = KVOFF_OK;
        }
        if (st) return st;
        if (A->timing) KVOFF_HIP(hipEventRecord(tev(li, gi, 4), xs));
        if (A->stats) {
          A->stats->selected += st_l.selected;
          A->stats->pool_hits += st_l.pool_hits;
          A->stats->items_recalled += st_l.items_recalled;
          A->stats->transfers += st_l.transfers;
          A->stats->bytes += st_l.bytes;
        }
        KVOFF_HIP(hipEventRecord(ctx->ev_group[buf * groups.size() + gi], xs));
      }
      return KVOFF_OK;
    };
    auto attend_l = [&](int li) -> int {
      const int buf = li & 1;
      for (int gi : order_for(li)) {
        const Group& g = groups[gi];
        const int64_t sel_off = (int64_t)g.r0 * sets * A->k_stride;
        if (A->timing) KVOFF_HIP(hipEventRecord(tev(li, gi, 0), cs));
        KVOFF_HIP(hipStreamWaitEvent(cs, ctx->ev_group[buf * groups.size() + gi], 0));
        if (A->timing) KVOFF_HIP(hipEventRecord(tev(li, gi, 1), cs));
        int st = kvoff_sparse_decode(
            ctx, g.n, A->req_ids + g.r0, A->mode,
            (const uint8_t*)A->q_dev[li] + g.r0 * q_row * 2, A->slot_pool_dev, A->n_slots,
            A->block_table_dev[buf] + sel_off, A->sel_idx_dev[buf] + sel_off,
            A->sel_cnt_dev[buf] + g.r0, A->k_stride, A->scale, A->out_dev[li] + g.r0 * q_row,
            A->ws_dev, A->ws_bytes, cs);
        if (st) return st;
        if (A->timing) KVOFF_HIP(hipEventRecord(tev(li, gi, 2), cs));
      }
      return KVOFF_OK;
    };

    int st;
    if (A->timing) KVOFF_HIP(hipEventRecord(ctx->ev_timing[0], cs));
    if ((st = select_l(0)) || (st = recall_l(0))) return st;
    for (int li = 0; li < L; ++li) {
      if (li + 1 < L && ((st = select_l(li + 1)) || (st = recall_l(li + 1)))) return st;
      if ((st = attend_l(li))) return st;
    }
    if (A->timing) {
      KVOFF_HIP(hipStreamSynchronize(cs));
      kvoff_step_timing& T = *A->timing;
      float ms;
      for (int li = 0; li < L; ++li)
        for (size_t gi = 0; gi < NG; ++gi) {
          KVOFF_HIP(hipEventElapsedTime(&ms, tev(li, gi, 0), tev(li, gi, 1)));
          T.compute_wait_ms += ms;
          KVOFF_HIP(hipEventSynchronize(tev(li, gi, 4)));
          KVOFF_HIP(hipEventElapsedTime(&ms, tev(li, gi, 3), tev(li, gi, 4)));
          T.recall_ms += ms;
          ++T.recalls;
        }
      for (size_t gi = 0; gi < NG; ++gi) {  // requests finish with their last layer
        KVOFF_HIP(hipEventElapsedTime(&ms, ctx->ev_timing[0], tev(L - 1, gi, 2)));
        T.mean_request_done_ms += (double)ms * groups[gi].n / A->n_req;
        T.max_request_done_ms = std::max(T.max_request_done_ms, (double)ms);
      }
      T.step_ms = T.max_request_done_ms;
    }
    if (deferred) return fail(deferred, "%s", deferred_msg.c_str());
    return KVOFF_OK;
  });
}
