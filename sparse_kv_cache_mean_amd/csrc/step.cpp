// step.cpp - kvoff_step: select, recall and attend over a range of layers
// with recall of layer l+1 overlapped with attention of layer l.
//
// The guide's analysis ("PulseInfer Guide", aiFetchly, section "The Fallacy
// of Naive Offloading", prefetching mismatch; section "Interruptible
// Layer-Wise Scheduling") is that recall must run while the GPU computes.
// On one GPU this is two HIP streams and two buffer sets:
//   compute stream:  select(0) select(1) attend(0) select(2) attend(1) ...
//   copy stream:     recall(0) recall(1) recall(2) ...
// recall(l) waits for the event recorded after select(l); attend(l) waits
// for the event recorded after recall(l).  Buffer set l%2 is rewritten by
// select(l+2) and recall(l+2) only after attend(l) completed, because
// select(l+2) is enqueued on the compute stream after attend(l) and
// recall(l+2) waits for select(l+2).  Every kernel reads exactly the data a
// serial run would, so outputs are bit-identical to the serial order.
#include <cstring>

#include "kvoff_internal.h"

using namespace kvoff;

extern "C" int kvoff_step(kvoff_ctx* ctx, const kvoff_step_args* A) {
  if (!ctx || !A) return fail(KVOFF_EINVAL, "ctx and args must be non-NULL");
  const int L = A->layer_end - A->layer_begin;
  if (L < 0 || A->layer_begin < 0 || A->layer_end > ctx->cfg.num_layers)
    return fail(KVOFF_ERANGE, "layers [%d, %d) outside [0, %d)", A->layer_begin, A->layer_end,
                ctx->cfg.num_layers);
  if (A->stats) memset(A->stats, 0, sizeof *A->stats);
  if (L == 0 || A->n_req == 0) return KVOFF_OK;
  if (!A->q_dev || !A->digest_dev || !A->out_dev)
    return fail(KVOFF_EINVAL, "q_dev, digest_dev and out_dev arrays must be non-NULL");
  for (int i = 0; i < 2; ++i)
    if (!A->scores_dev[i] || !A->sel_idx_dev[i] || !A->sel_cnt_dev[i] || !A->block_table_dev[i])
      return fail(KVOFF_EINVAL, "buffer set %d has a NULL buffer", i);
  if (L > 1 && A->recall_base_slot[0] == A->recall_base_slot[1] && A->copy_stream != A->compute_stream)
    return fail(KVOFF_EINVAL, "overlapped layers need two distinct recall regions");

  hipStream_t cs = (hipStream_t)A->compute_stream;
  hipStream_t xs = (hipStream_t)A->copy_stream;
  KVOFF_HIP(hipSetDevice(ctx->device));

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
  auto recall_l = [&](int li) -> int {
    const int buf = li & 1;
    KVOFF_HIP(hipStreamWaitEvent(xs, ctx->ev_sel[buf], 0));
    kvoff_stats st_l;
    int st = kvoff_recall(ctx, A->layer_begin + li, A->n_req, A->req_ids, A->mode,
                          A->sel_idx_dev[buf], A->sel_cnt_dev[buf], A->k_stride,
                          A->pool_hit_dev ? A->pool_hit_dev[li] : nullptr,
                          A->pool_slot_dev ? A->pool_slot_dev[li] : nullptr, A->pool_stride,
                          A->slot_pool_dev, A->n_slots, A->recall_base_slot[buf],
                          A->block_table_dev[buf], A->engine, A->stats ? &st_l : nullptr, xs);
    if (st) return st;
    if (A->stats) {
      A->stats->selected += st_l.selected;
      A->stats->pool_hits += st_l.pool_hits;
      A->stats->items_recalled += st_l.items_recalled;
      A->stats->transfers += st_l.transfers;
      A->stats->bytes += st_l.bytes;
    }
    KVOFF_HIP(hipEventRecord(ctx->ev_rec[buf], xs));
    return KVOFF_OK;
  };
  auto attend_l = [&](int li) -> int {
    const int buf = li & 1;
    KVOFF_HIP(hipStreamWaitEvent(cs, ctx->ev_rec[buf], 0));
    return kvoff_sparse_decode(ctx, A->n_req, A->req_ids, A->mode, A->q_dev[li], A->slot_pool_dev,
                               A->block_table_dev[buf], A->sel_idx_dev[buf], A->sel_cnt_dev[buf],
                               A->k_stride, A->scale, A->out_dev[li], A->ws_dev, A->ws_bytes, cs);
  };

  int st;
  if ((st = select_l(0)) || (st = recall_l(0))) return st;
  for (int li = 0; li < L; ++li) {
    if (li + 1 < L && ((st = select_l(li + 1)) || (st = recall_l(li + 1)))) return st;
    if ((st = attend_l(li))) return st;
  }
  return KVOFF_OK;
}
