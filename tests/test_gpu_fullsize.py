"""GPU parity at the workloads' full sizes, in the launch configuration
bench.py times (same context, batch, k_stride, kernels).

Digests, selections and recalled bytes are compared for every block, and
attention for every (request, head) row of every compared layer: all 32
layers of the decode step, all requests and heads of the variable-recall
layer and of the headwise-vs-SoloHead workload in each selection mode.  The
oracle runs one call per (layer, request) on a pool of threads.
"""
import math
import os
import time
from concurrent.futures import ThreadPoolExecutor

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

THREADS = max(1, min(16, os.cpu_count() or 1))


def _conditioned(s, layers, reqs, lam=None, group_lam=None):
    """Gap-conditioned slices of every (layer, request), built on a pool of
    threads (generation and the oracle's scoring release the interpreter
    lock)."""
    keys = [(l, r) for l in layers for r in range(len(reqs))]

    def one(key):
        return workloads.make_slice(s, key[0], key[1], reqs[key[1]], lam=lam, group_lam=group_lam)

    with ThreadPoolExecutor(THREADS) as ex:
        return dict(zip(keys, ex.map(one, keys)))


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
        ref = P.oracle_attention(c, 0, kv.KVOFF_SOLOHEAD, sl)
        H.log("  zero-copy layer step")
        st = H.run_layer(c, 0, kv.KVOFF_SOLOHEAD, bufs, want_stats=True)
        torch.cuda.synchronize()
        P.check_digests(c, 0, sl)
        P.check_selection(c, 0, kv.KVOFF_SOLOHEAD, bufs, sl)
        P.check_recall(c, 0, kv.KVOFF_SOLOHEAD, bufs, sl, stats=st)
        err = P.check_attention(c, 0, kv.KVOFF_SOLOHEAD, bufs, sl, ref)
        H.log(f"  stats {st}; attention max abs {err[0]:.2e} row rel {err[1]:.2e}")
        hot_hit = np.mean([len(set(np.flatnonzero(sl[(0, r)].lr.hot)) & set(sl[(0, r)].sel.tolist()))
                           / max(1, sl[(0, r)].lr.hot.sum()) for r in range(c.B)])
        H.log(f"  planted hot blocks recovered: {hot_hit:.3f}")
        for engine in (kv.KVOFF_ENGINE_DMA, kv.KVOFF_ENGINE_STAGED):
            H.log(f"  engine {engine}")
            c.pool.zero_()
            st2 = H.run_layer(c, 0, kv.KVOFF_SOLOHEAD, bufs, engine=engine, want_stats=True)
            torch.cuda.synchronize()
            P.check_recall(c, 0, kv.KVOFF_SOLOHEAD, bufs, sl, stats=st2, engine=engine)
            P.check_attention(c, 0, kv.KVOFF_SOLOHEAD, bufs, sl, ref)
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
        t1 = time.time()
        err = P.check_attention(c, 0, kv.KVOFF_SOLOHEAD, bufs, sl)
        mean_run = st["items_recalled"] / st["transfers"]
        H.log(f"  stats {st}; mean run {mean_run:.2f} blocks; attention (all {c.B} x {s.Hq} rows, "
              f"oracle {time.time() - t1:.1f} s) max abs {err[0]:.2e} row rel {err[1]:.2e}")
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
            ref = P.oracle_attention(c, 0, mode, sl)
            for engine in (kv.KVOFF_ENGINE_ZEROCOPY, kv.KVOFF_ENGINE_DMA):
                bufs = H.make_buffers(c, mode)
                st = H.run_layer(c, 0, mode, bufs, engine=engine, with_pool_hits=True,
                                 want_stats=True)
                torch.cuda.synchronize()
                P.check_selection(c, 0, mode, bufs, sl)
                P.check_recall(c, 0, mode, bufs, sl, with_pool_hits=True, stats=st)
                err = P.check_attention(c, 0, mode, bufs, sl, ref)
                report[(mode, engine)] = st
                H.log(f"  mode {mode} engine {engine}: {st}, mean transfer "
                      f"{st['bytes'] / max(1, st['transfers']) / 1024:.1f} KiB, attention {err}")
        for mode in (kv.KVOFF_CONSENSUS, kv.KVOFF_CONSENSUS_GROUP):  # lambda 0.5 (default)
            bufs = H.make_buffers(c, mode)
            st = H.run_layer(c, 0, mode, bufs, with_pool_hits=True, want_stats=True)
            torch.cuda.synchronize()
            P.check_selection(c, 0, mode, bufs, sl)
            P.check_recall(c, 0, mode, bufs, sl, with_pool_hits=True, stats=st)
            err = P.check_attention(c, 0, mode, bufs, sl)
            # attention mass of every request against the oracle
            mass = torch.empty((c.B, s.Hq), dtype=torch.float64, device="cuda")
            kv.kvoff_attention_mass(c.ctx, 0, c.rids, mode, c.q[0], bufs.sel_idx, bufs.sel_cnt,
                                    c.k_stride, 1.0 / math.sqrt(s.d), mass)
            torch.cuda.synchronize()
            got = mass.cpu().numpy()

            def mass_ref(r):
                x = sl[(0, r)]
                sets = P.block_sets(x, mode)
                return oracle.attention_mass(x.lr.q, x.lr.K, s.dtype, s.bs,
                                             np.stack(sets) if len(sets) > 1 else sets[0])

            with ThreadPoolExecutor(THREADS) as ex:
                ref_mass = np.stack(list(ex.map(mass_ref, range(c.B))))
            assert np.abs(got - ref_mass).max() <= 1e-4, mode
            H.log(f"  mode {mode}: {st}; attention {err}; mean mass {got.mean():.4f}")
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
    pinned host KV).  The overlapped kvoff_step must equal the serial order
    bit for bit on every layer and the oracle on every layer, request and
    head; every layer's digests and selections are compared too, and three
    layers' recalled bytes.  The inputs are generated, gap-conditioned and
    run through the oracle one layer at a time on a pool of threads; only the
    three byte-checked layers keep their keys and values afterwards."""
    t0 = time.time()
    s = synth.spec(3)
    reqs = synth.request_draws(s)
    B, layers = len(reqs), list(range(s.L))
    byte_checked = (0, 15, 31)
    sl, ref, pending = {}, {}, {}
    mode = kv.KVOFF_SOLOHEAD

    def prepare(key):
        x = workloads.make_slice(s, key[0], key[1], reqs[key[1]])
        return x, P.oracle_attention_one(s, x, mode)

    def get(key):
        l, r = key
        if key not in pending:  # the first request of a layer: build the whole layer
            keys = [(l, rr) for rr in range(B)]
            with ThreadPoolExecutor(THREADS) as ex:
                pending.update(zip(keys, ex.map(prepare, keys)))
        x, ref[key] = pending.pop(key)
        sl[key] = x
        lr = x.lr
        if l not in byte_checked:  # keep the digests and selections, drop the inputs
            x.lr = synth.LayerRequest(lr.layer, lr.req, lr.rq, lr.q, lr.qhat, lr.hot, lr.attempts,
                                      None, None, lr.pool)
        return lr

    H.log(f"[full llama3-8b-32layer] generating, conditioning and offloading 32 layers")
    c = H.build_case(s, get, layers, reqs, keep=lambda l, r: False)
    H.log(f"  offloaded, oracle done in {time.time() - t0:.1f} s")
    try:
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
        worst = (0.0, 0.0)
        for l in layers:
            assert np.array_equal(outs[l].cpu().numpy().view(np.uint32), over[l].view(np.uint32)), l
            want = np.stack([ref[(l, r)] for r in range(B)])
            err = P.check_attention_close(over[l], want, f"layer {l}")
            worst = (max(worst[0], err[0]), max(worst[1], err[1]))
            P.check_digests(c, l, sl)
            bufs = sets[0]
            if l in byte_checked:
                st = H.run_layer(c, l, mode, bufs, want_stats=True)
                torch.cuda.synchronize()
                P.check_selection(c, l, mode, bufs, sl)
                P.check_recall(c, l, mode, bufs, sl, stats=st)
            else:
                kv.kvoff_select(c.ctx, l, c.rids, c.q[l], c.digest[l], c.nb_max,
                                [rq.k for rq in reqs], mode, bufs.scores, bufs.sel_idx,
                                bufs.sel_cnt, c.k_stride)
                torch.cuda.synchronize()
                P.check_selection(c, l, mode, bufs, sl)
        H.log(f"  all 32 layers x {B} requests x {s.Hq} heads: max abs {worst[0]:.2e}, "
              f"row rel {worst[1]:.2e}")
    finally:
        H.destroy(c)
    H.log(f"  done in {time.time() - t0:.1f} s")
