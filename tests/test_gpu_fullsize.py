"""GPU parity at the workloads' full sizes, in the launch configuration
bench.py times (same context, batch, k_stride, kernels).

Digests, selections and recalled bytes are compared for every block; the
oracle computes attention for every (request, head) row where that is cheap
(Llama-3-8B-shaped layer) and for one sampled KV group per request elsewhere
(its G heads, computed one group at a time by the same oracle call on that
group's keys and values).
"""
import math
import time

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


def _conditioned(s, layers, reqs, lam=None, group_lam=None):
    sl = {}
    for l in layers:
        for r, rq in enumerate(reqs):
            sl[(l, r)] = workloads.make_slice(s, l, r, rq, lam=lam, group_lam=group_lam)
    return sl


def _sampled_attention(c, l, mode, bufs, slices, groups):
    """Compare the G heads of KV group groups[r] of every request r."""
    s = c.s
    G = s.G
    got = bufs.out.cpu().numpy()
    worst = (0.0, 0.0)
    for r in range(c.B):
        g = groups[r]
        sl = slices[(l, r)]
        lr = sl.lr
        Kg = np.ascontiguousarray(lr.K[:, g:g + 1, :])
        Vg = np.ascontiguousarray(lr.V[:, g:g + 1, :])
        qg = lr.q[g * G:(g + 1) * G]
        sel = P.head_sets(sl, mode)[g] if P.per_head(mode) else P.shared_set(sl, mode)
        ref = oracle.attend_f32(qg, Kg, Vg, s.dtype, s.bs, sel)
        err = P.check_attention_close(got[r, g * G:(g + 1) * G], ref, f"(layer {l} req {r} group {g})")
        worst = (max(worst[0], err[0]), max(worst[1], err[1]))
    return worst


def test_llama3_8b_layer_full_size():
    t0 = time.time()
    s = synth.spec(2)  # batch 16, 32/8 heads, 32768 tokens, block 32, top-64, bf16
    reqs = synth.request_draws(s)
    H.log(f"[full llama3-8b-layer] conditioning inputs")
    sl = _conditioned(s, [0], reqs)
    H.log(f"  built in {time.time() - t0:.1f} s; offloading")
    c = H.build_case(s, {k: v.lr for k, v in sl.items()}, [0], reqs, two_regions=False)
    try:
        bufs = H.make_buffers(c, kv.KVOFF_SOLOHEAD)
        H.log("  zero-copy layer step")
        st = H.run_layer(c, 0, kv.KVOFF_SOLOHEAD, bufs, want_stats=True)
        torch.cuda.synchronize()
        P.check_digests(c, 0, sl)
        P.check_selection(c, 0, kv.KVOFF_SOLOHEAD, bufs, sl)
        P.check_recall(c, 0, kv.KVOFF_SOLOHEAD, bufs, sl, stats=st)
        err = P.check_attention(c, 0, kv.KVOFF_SOLOHEAD, bufs, sl)
        H.log(f"  stats {st}; attention max abs {err[0]:.2e} row rel {err[1]:.2e}")
        hot_hit = np.mean([len(set(np.flatnonzero(sl[(0, r)].lr.hot)) & set(sl[(0, r)].sel.tolist()))
                           / max(1, sl[(0, r)].lr.hot.sum()) for r in range(c.B)])
        H.log(f"  planted hot blocks recovered: {hot_hit:.3f}")
        H.log("  DMA recall")
        c.pool.zero_()
        st2 = H.run_layer(c, 0, kv.KVOFF_SOLOHEAD, bufs, engine=kv.KVOFF_ENGINE_DMA, want_stats=True)
        torch.cuda.synchronize()
        P.check_recall(c, 0, kv.KVOFF_SOLOHEAD, bufs, sl, stats=st2)
        P.check_attention(c, 0, kv.KVOFF_SOLOHEAD, bufs, sl)
        H.log("  staged recall")
        c.pool.zero_()
        st3 = H.run_layer(c, 0, kv.KVOFF_SOLOHEAD, bufs, engine=kv.KVOFF_ENGINE_STAGED,
                          want_stats=True)
        torch.cuda.synchronize()
        P.check_recall(c, 0, kv.KVOFF_SOLOHEAD, bufs, sl, stats=st3, engine=kv.KVOFF_ENGINE_STAGED)
        P.check_attention(c, 0, kv.KVOFF_SOLOHEAD, bufs, sl)
    finally:
        H.destroy(c)
    H.log(f"  done in {time.time() - t0:.1f} s")


def test_variable_contexts_full_size():
    t0 = time.time()
    s = synth.spec(4)  # batch 32, 64/8 heads, contexts U[8K,128K], k 2-15%, runs of hot blocks
    reqs = synth.request_draws(s)
    H.log(f"[full llama3-70b-variable] {sum(rq.ctx for rq in reqs)} tokens, "
          f"k {min(rq.k for rq in reqs)}..{max(rq.k for rq in reqs)}")
    sl = _conditioned(s, [0], reqs)
    H.log(f"  built in {time.time() - t0:.1f} s; offloading")
    c = H.build_case(s, {k: v.lr for k, v in sl.items()}, [0], reqs, two_regions=False)
    try:
        bufs = H.make_buffers(c, kv.KVOFF_SOLOHEAD)
        st = H.run_layer(c, 0, kv.KVOFF_SOLOHEAD, bufs, want_stats=True)
        torch.cuda.synchronize()
        P.check_digests(c, 0, sl)
        P.check_selection(c, 0, kv.KVOFF_SOLOHEAD, bufs, sl)
        P.check_recall(c, 0, kv.KVOFF_SOLOHEAD, bufs, sl, stats=st)
        err = _sampled_attention(c, 0, kv.KVOFF_SOLOHEAD, bufs, sl, [r % s.Hkv for r in range(c.B)])
        mean_run = st["items_recalled"] / st["transfers"]
        H.log(f"  stats {st}; mean run {mean_run:.2f} blocks; attention {err}")
        assert mean_run > 2.0  # clustered hot runs were coalesced
    finally:
        H.destroy(c)
    H.log(f"  done in {time.time() - t0:.1f} s")


def test_headwise_vs_solohead_full_size():
    t0 = time.time()
    s = synth.spec(5)  # llama3-8b shapes, per-KV-head top-64 vs shared, 25% pool hits
    reqs = synth.request_draws(s)
    H.log("[full headwise-vs-solohead] conditioning (SoloHead, 8 per-head, consensus and "
          "8 per-group consensus rankings)")
    sl = _conditioned(s, [0], reqs, lam=0.5, group_lam=0.5)
    H.log(f"  built in {time.time() - t0:.1f} s; offloading")
    c = H.build_case(s, {k: v.lr for k, v in sl.items()}, [0], reqs, with_pool_hits=True,
                     two_regions=False)
    try:
        report = {}
        for mode in (kv.KVOFF_SOLOHEAD, kv.KVOFF_HEADWISE):
            for engine in (kv.KVOFF_ENGINE_ZEROCOPY, kv.KVOFF_ENGINE_DMA):
                bufs = H.make_buffers(c, mode)
                st = H.run_layer(c, 0, mode, bufs, engine=engine, with_pool_hits=True,
                                 want_stats=True)
                torch.cuda.synchronize()
                P.check_selection(c, 0, mode, bufs, sl)
                P.check_recall(c, 0, mode, bufs, sl, with_pool_hits=True, stats=st)
                _sampled_attention(c, 0, mode, bufs, sl, [(3 * r) % s.Hkv for r in range(c.B)])
                report[(mode, engine)] = st
                H.log(f"  mode {mode} engine {engine}: {st}, mean transfer "
                      f"{st['bytes'] / max(1, st['transfers']) / 1024:.1f} KiB")
        for mode in (kv.KVOFF_CONSENSUS, kv.KVOFF_CONSENSUS_GROUP):  # lambda 0.5 (default)
            bufs = H.make_buffers(c, mode)
            st = H.run_layer(c, 0, mode, bufs, with_pool_hits=True, want_stats=True)
            torch.cuda.synchronize()
            P.check_selection(c, 0, mode, bufs, sl)
            P.check_recall(c, 0, mode, bufs, sl, with_pool_hits=True, stats=st)
            _sampled_attention(c, 0, mode, bufs, sl, [(5 * r + 1) % s.Hkv for r in range(c.B)])
            # attention mass of two sampled requests against the oracle
            mass = torch.empty((c.B, s.Hq), dtype=torch.float64, device="cuda")
            kv.kvoff_attention_mass(c.ctx, 0, c.rids, mode, c.q[0], bufs.sel_idx, bufs.sel_cnt,
                                    c.k_stride, 1.0 / math.sqrt(s.d), mass)
            torch.cuda.synchronize()
            got = mass.cpu().numpy()
            for r in (0, c.B - 1):
                x = sl[(0, r)]
                sets = P.block_sets(x, mode)
                ref = oracle.attention_mass(x.lr.q, x.lr.K, s.dtype, s.bs,
                                            np.stack(sets) if len(sets) > 1 else sets[0])
                assert np.abs(got[r] - ref).max() <= 1e-4, (mode, r)
            H.log(f"  mode {mode}: {st}; mean mass {got.mean():.4f}")
        solo, hw = report[(0, 0)], report[(1, 0)]
        assert hw["transfers"] > 4 * solo["transfers"]  # per-head recall fragments
        unions = [oracle.union_count(sl[(0, r)].sel_g, [sl[(0, r)].K] * s.Hkv) for r in range(c.B)]
        H.log(f"  per-head sets cover {np.mean(unions):.1f} distinct blocks per request "
              f"vs {s.k} shared")
    finally:
        H.destroy(c)
    H.log(f"  done in {time.time() - t0:.1f} s")


def test_32_layer_step_full_size():
    """All 32 layers of the 8-request decode step offloaded (about 34 GB of
    pinned host KV); the overlapped kvoff_step must equal the serial order bit
    for bit on every layer, and three layers are checked against the oracle."""
    t0 = time.time()
    s = synth.spec(3)
    reqs = synth.request_draws(s)
    checked = (0, 15, 31)
    H.log(f"[full llama3-8b-32layer] conditioning checked layers {checked}")
    sl = _conditioned(s, checked, reqs)

    def get(key):
        l, r = key
        return sl[key].lr if l in checked else synth.gen_layer_request(s, l, r, reqs[r])

    H.log(f"  offloading 32 layers (built checked layers in {time.time() - t0:.1f} s)")
    layers = list(range(s.L))
    c = H.build_case(s, get, layers, reqs, keep=lambda l, r: l in checked)
    H.log(f"  offloaded in {time.time() - t0:.1f} s")
    try:
        mode = kv.KVOFF_SOLOHEAD
        sets = [H.make_buffers(c, mode) for _ in range(2)]
        outs = [torch.empty((c.B, s.Hq, s.d), dtype=torch.float32, device="cuda") for _ in layers]
        compute, copy = torch.cuda.Stream(), torch.cuda.Stream()

        def step(copy_stream):
            return kv.kvoff_step(
                c.ctx, layer_begin=0, layer_end=s.L, req_ids=c.rids, topk=[rq.k for rq in reqs],
                mode=mode, engine=kv.KVOFF_ENGINE_ZEROCOPY, k_stride=c.k_stride,
                q=[c.q[l] for l in layers], digest=[c.digest[l] for l in layers],
                digest_stride=c.nb_max, slot_pool=c.pool, n_slots=c.n_slots,
                recall_base_slot=c.recall_base, scores=[b.scores for b in sets],
                sel_idx=[b.sel_idx for b in sets], sel_cnt=[b.sel_cnt for b in sets],
                block_table=[b.table for b in sets], scale=1.0 / math.sqrt(s.d), out=outs,
                ws=sets[0].ws, compute_stream=compute, copy_stream=copy_stream)

        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(compute)
        step(copy)
        ev[1].record(compute)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1])
        H.log(f"  overlapped 32-layer step {ms:.2f} ms ({32e3 / ms:.0f} layer-steps/s)")
        over = [o.cpu().numpy().copy() for o in outs]
        step(compute)
        torch.cuda.synchronize()
        for l in layers:
            assert np.array_equal(outs[l].cpu().numpy().view(np.uint32), over[l].view(np.uint32)), l
        for l in checked:
            P.check_attention_close(over[l], P.oracle_attention(c, l, mode, sl), f"layer {l}")
            bufs = H.make_buffers(c, mode)
            st = H.run_layer(c, l, mode, bufs, want_stats=True)
            torch.cuda.synchronize()
            P.check_digests(c, l, sl)
            P.check_selection(c, l, mode, bufs, sl)
            P.check_recall(c, l, mode, bufs, sl, stats=st)
    finally:
        H.destroy(c)
    H.log(f"  done in {time.time() - t0:.1f} s")
