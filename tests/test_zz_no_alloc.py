"""kvoff_sparse_decode_noalloc, the attention entry point that allocates
nothing (its split partials go to the library's file-scope scratch array),
against kvoff_sparse_decode with a caller workspace on the same inputs: two
calls in a row, the second with a smaller batch and selection, each bit for
bit equal to the workspace form and within the attention tolerance of the
oracle; a call whose partials exceed the array is rejected."""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_kv_cache_mean_amd as kv
import synth
from tests import gpu_harness as H
from tests import parity as P
from tests import workloads

pytestmark = pytest.mark.gpu


def _both(c, ids, rows, mode, bufs, k_stride):
    """Both entry points on the first `rows` requests and `k_stride` ranks;
    returns (workspace form, no-alloc form) outputs, each NaN-filled before
    its call, and whether the device's free memory was the same before and
    after the no-alloc call (every buffer is allocated before it)."""
    s = c.s
    out_ws = torch.full((rows, s.Hq, s.d), float("nan"), device="cuda")
    out_na = torch.full((rows, s.Hq, s.d), float("nan"), device="cuda")
    wsb = kv.kvoff_workspace_size(c.ctx, kv.KVOFF_CALL_SPARSE_DECODE, rows, k_stride, mode)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(s.d)
    q = c.q[0][:rows].contiguous()
    sel = bufs.sel_idx[:rows, :, :k_stride].contiguous()
    tab = bufs.table[:rows, :, :k_stride].contiguous()
    cnt = bufs.sel_cnt[:rows].clamp(max=k_stride).contiguous()
    kv.kvoff_sparse_decode(c.ctx, ids, mode, q, c.pool, c.n_slots, tab, sel, cnt, k_stride, scale,
                           out_ws, ws)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    kv.kvoff_sparse_decode_noalloc(c.ctx, ids, mode, q, c.pool, c.n_slots, tab, sel, cnt, k_stride,
                                   scale, out_na)
    torch.cuda.synchronize()
    same_free = torch.cuda.mem_get_info()[0] == free0
    return out_ws.cpu().numpy(), out_na.cpu().numpy(), same_free


@pytest.mark.parametrize("mode", [kv.KVOFF_SOLOHEAD, kv.KVOFF_HEADWISE])
def test_noalloc_decode_matches_workspace_decode(mode):
    s = synth.spec(2, B=4, ctx=6000, k=40, hot=8, headwise=True)
    H.log(f"[noalloc] mode {mode}")
    reqs = synth.request_draws(s)
    sl = {(0, r): workloads.make_slice(s, 0, r, rq) for r, rq in enumerate(reqs)}
    c = H.build_case(s, {k: v.lr for k, v in sl.items()}, [0], reqs)
    try:
        bufs = H.make_buffers(c, mode)
        H.run_layer(c, 0, mode, bufs)
        torch.cuda.synchronize()
        # first call: the whole batch
        got_ws, got_na, _ = _both(c, c.rids, c.B, mode, bufs, c.k_stride)
        assert np.array_equal(got_na.view(np.uint32), got_ws.view(np.uint32))
        P.check_attention_close(got_na, P.oracle_attention(c, 0, mode, sl), "noalloc, batch 4")
        # second call: two requests and the first 24 ranks of each selection,
        # so fewer partials than the first call left in the array
        k2 = 24
        got_ws, got_na, same_free = _both(c, c.rids[:2], 2, mode, bufs, k2)
        assert same_free, "device memory changed across the no-alloc call"
        assert np.array_equal(got_na.view(np.uint32), got_ws.view(np.uint32))
        ref = np.empty((2, s.Hq, s.d), np.float32)
        for r in range(2):
            x = sl[(0, r)]
            if P.per_head(mode):
                ref[r] = oracle.attend_headwise_f32(x.lr.q, x.lr.K, x.lr.V, s.dtype, s.bs,
                                                    np.ascontiguousarray(x.sel_g[:, :k2]))
            else:
                ref[r] = oracle.attend_f32(x.lr.q, x.lr.K, x.lr.V, s.dtype, s.bs, x.sel[:k2])
        P.check_attention_close(got_na, ref, "noalloc, batch 2, 24 ranks")
    finally:
        H.destroy(c)


def test_noalloc_decode_rejects_partials_past_the_array():
    """8 requests x 32 heads x 128 splits (k_stride 4096, 8 blocks per wave)
    of 520-byte partials is 17.0 MB, past the 16 MiB array: ERANGE before
    any launch."""
    s = synth.spec(2, B=1, ctx=2048, k=8, hot=2)
    reqs = synth.request_draws(s)
    c = H.build_case(s, lambda key: synth.gen_layer_request(s, key[0], key[1], reqs[key[1]]), [0],
                     reqs)
    try:
        k_stride, n = 4096, 8
        need = kv.kvoff_workspace_size(c.ctx, kv.KVOFF_CALL_SPARSE_DECODE, n, k_stride,
                                       kv.KVOFF_SOLOHEAD)
        assert need > kv.KVOFF_NOALLOC_SCRATCH_BYTES, need
        sel = torch.zeros((n, k_stride), dtype=torch.int32, device="cuda")
        cnt = torch.zeros((n,), dtype=torch.int32, device="cuda")
        out = torch.empty((n, s.Hq, s.d), dtype=torch.float32, device="cuda")
        ids = [c.rids[0]] * n
        with pytest.raises(kv.KvoffError) as e:
            kv.kvoff_sparse_decode_noalloc(c.ctx, ids, kv.KVOFF_SOLOHEAD, c.q[0].repeat(n, 1, 1),
                                           c.pool, c.n_slots, sel, sel, cnt, k_stride, 0.1, out)
        assert e.value.status == kv.KVOFF_ERANGE
    finally:
        H.destroy(c)
