"""GPU parity: the HIP path through the C ABI against the oracle, element by
element, at sizes the oracle finishes in seconds (several tiles, ragged
tails).  Full-size workloads are in test_gpu_fullsize.py."""
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


def _slices(s, layers, reqs=None, lam=None, group_lam=None):
    reqs = reqs or synth.request_draws(s)
    out = {}
    for l in layers:
        for r, rq in enumerate(reqs):
            out[(l, r)] = workloads.make_slice(s, l, r, rq, lam=lam, group_lam=group_lam)
    return reqs, out


def _case(s, layers, with_pool_hits=False, host_kind=kv.KVOFF_HOST_COHERENT, reqs=None, lam=None,
          group_lam=None):
    reqs, sl = _slices(s, layers, reqs, lam, group_lam)
    inputs = {k: v.lr for k, v in sl.items()}
    c = H.build_case(s, inputs, layers, reqs, host_kind=host_kind, with_pool_hits=with_pool_hits)
    return c, sl


def _full_check(c, sl, l, mode, engine, with_pool_hits=False):
    bufs = H.make_buffers(c, mode)
    H.log(f"  run layer {l} mode {mode} engine {engine} hits {with_pool_hits}")
    stats = H.run_layer(c, l, mode, bufs, engine=engine, with_pool_hits=with_pool_hits,
                        want_stats=True)
    torch.cuda.synchronize()
    P.check_digests(c, l, sl)
    P.check_selection(c, l, mode, bufs, sl)
    P.check_recall(c, l, mode, bufs, sl, with_pool_hits=with_pool_hits, stats=stats, engine=engine)
    err = P.check_attention(c, l, mode, bufs, sl)
    return stats, err


TINY = synth.spec(1)  # 1 request, 8/2 heads, 4096 tokens, bs 16, k 32, fp16


@pytest.mark.parametrize("engine", [kv.KVOFF_ENGINE_ZEROCOPY, kv.KVOFF_ENGINE_DMA, kv.KVOFF_ENGINE_STAGED])
def test_tiny_config_full_parity(engine):
    H.log(f"[tiny] engine {engine}")
    c, sl = _case(TINY, [0])
    try:
        stats, err = _full_check(c, sl, 0, kv.KVOFF_SOLOHEAD, engine)
        H.log(f"  stats {stats} attention err {err}")
    finally:
        H.destroy(c)


@pytest.mark.parametrize("engine", [kv.KVOFF_ENGINE_ZEROCOPY, kv.KVOFF_ENGINE_DMA, kv.KVOFF_ENGINE_STAGED])
def test_tiny_config_noncoherent_store(engine):
    H.log(f"[tiny] noncoherent host store, engine {engine}")
    c, sl = _case(TINY, [0], host_kind=kv.KVOFF_HOST_NONCOHERENT)
    try:
        _full_check(c, sl, 0, kv.KVOFF_SOLOHEAD, engine)
    finally:
        H.destroy(c)


def test_offloaded_records_in_pinned_store():
    H.log("[records] pinned store contents")
    import ctypes
    s = synth.spec(1, ctx=1000)  # 63 blocks, last one holds 8 of 16 tokens
    c, sl = _case(s, [0])
    try:
        rec = kv.kvoff_record_bytes(c.ctx)
        for b in (0, 5, 62):
            buf = np.empty(rec, np.uint8)
            ctypes.memmove(buf.ctypes.data, kv.kvoff_host_record(c.ctx, 0, c.rids[0], b), rec)
            want = workloads.block_records(sl[(0, 0)], [b])[0].reshape(-1).view(np.uint8)
            assert np.array_equal(buf, want), b
    finally:
        H.destroy(c)


# ragged contexts, variable k, G = 8, bf16, clustered hot runs (the variable
# workload's recipe at reduced context lengths)
RAGGED = synth.spec(4, B=6, ctx_range=(700, 5000))


@pytest.mark.parametrize("engine", [kv.KVOFF_ENGINE_ZEROCOPY, kv.KVOFF_ENGINE_DMA, kv.KVOFF_ENGINE_STAGED])
def test_ragged_variable_parity(engine):
    H.log(f"[ragged] engine {engine}")
    c, sl = _case(RAGGED, [0])
    try:
        assert any(rq.ctx % RAGGED.bs for rq in c.reqs)
        stats, err = _full_check(c, sl, 0, kv.KVOFF_SOLOHEAD, engine)
        H.log(f"  stats {stats} attention err {err}")
        assert stats["transfers"] < stats["items_recalled"]  # runs were coalesced
    finally:
        H.destroy(c)


# headwise vs SoloHead with a quarter of the blocks resident in the HBM pool
HW = synth.spec(5, B=3, ctx=4096, k=16, hot=6)


@pytest.mark.parametrize("mode", [kv.KVOFF_SOLOHEAD, kv.KVOFF_HEADWISE])
@pytest.mark.parametrize("engine", [kv.KVOFF_ENGINE_ZEROCOPY, kv.KVOFF_ENGINE_DMA, kv.KVOFF_ENGINE_STAGED])
def test_headwise_and_pool_hits(mode, engine):
    H.log(f"[headwise] mode {mode} engine {engine}")
    c, sl = _case(HW, [0], with_pool_hits=True)
    try:
        stats, _ = _full_check(c, sl, 0, mode, engine, with_pool_hits=True)
        H.log(f"  stats {stats}")
        assert stats["pool_hits"] > 0
    finally:
        H.destroy(c)


@pytest.mark.parametrize("lam", [0.5, 1.0])
@pytest.mark.parametrize("engine", [kv.KVOFF_ENGINE_ZEROCOPY, kv.KVOFF_ENGINE_DMA, kv.KVOFF_ENGINE_STAGED])
def test_consensus_rule(lam, engine):
    """The guide's max + lambda * mean consensus across KV heads as the shared set."""
    H.log(f"[consensus] lambda {lam} engine {engine}")
    c, sl = _case(HW, [0], with_pool_hits=True, lam=lam)
    try:
        kv.kvoff_set_consensus_lambda(c.ctx, lam)
        stats, _ = _full_check(c, sl, 0, kv.KVOFF_CONSENSUS, engine, with_pool_hits=True)
        H.log(f"  stats {stats}")
        diff = sum(len(set(sl[(0, r)].sel_c.tolist()) ^ set(sl[(0, r)].sel.tolist()))
                   for r in range(c.B))
        H.log(f"  blocks differing from the summed-score set: {diff}")
    finally:
        H.destroy(c)


@pytest.mark.parametrize("lam", [0.5, 1.0])
@pytest.mark.parametrize("engine", [kv.KVOFF_ENGINE_ZEROCOPY, kv.KVOFF_ENGINE_DMA, kv.KVOFF_ENGINE_STAGED])
def test_group_consensus_rule(lam, engine):
    """The consensus rule with the GQA-group scope: one set per KV head from
    max + lambda * mean over the group's query heads, recalled and attended
    in the headwise layout."""
    H.log(f"[group consensus] lambda {lam} engine {engine}")
    c, sl = _case(HW, [0], with_pool_hits=True, group_lam=lam)
    try:
        kv.kvoff_set_consensus_lambda(c.ctx, lam)
        stats, _ = _full_check(c, sl, 0, kv.KVOFF_CONSENSUS_GROUP, engine, with_pool_hits=True)
        H.log(f"  stats {stats}")
        diff = sum(len(set(sl[(0, r)].sel_gc[g].tolist()) ^ set(sl[(0, r)].sel_g[g].tolist()))
                   for r in range(c.B) for g in range(HW.Hkv))
        H.log(f"  blocks differing from the headwise sets: {diff}")
    finally:
        H.destroy(c)


@pytest.mark.parametrize("Hq,Hkv", [(16, 1), (32, 2), (16, 16), (64, 4), (12, 3), (40, 5)])
def test_group_sizes(Hq, Hkv):
    H.log(f"[groups] Hq {Hq} Hkv {Hkv}")
    s = synth.spec(2, B=2, Hq=Hq, Hkv=Hkv, ctx=2000, k=12, hot=5, headwise=Hkv > 1)
    c, sl = _case(s, [0], lam=0.5, group_lam=0.5)  # the context's default lambda
    try:
        _full_check(c, sl, 0, kv.KVOFF_SOLOHEAD, kv.KVOFF_ENGINE_ZEROCOPY)
        if Hkv > 1:
            _full_check(c, sl, 0, kv.KVOFF_HEADWISE, kv.KVOFF_ENGINE_ZEROCOPY)
        # consensus across KV heads (also for a single KV head: (1 + lambda) * S)
        _full_check(c, sl, 0, kv.KVOFF_CONSENSUS, kv.KVOFF_ENGINE_ZEROCOPY)
        # consensus within each GQA group (a group of one head: (1 + lambda) * S_g)
        _full_check(c, sl, 0, kv.KVOFF_CONSENSUS_GROUP, kv.KVOFF_ENGINE_ZEROCOPY)
    finally:
        H.destroy(c)


@pytest.mark.parametrize("spec_args", [
    dict(wl=1),                                              # fp16, bs 16, G 4
    dict(wl=2, B=2, Hq=8, Hkv=8, ctx=2000, k=12, hot=5),     # bf16, bs 32, G 1
    dict(wl=2, B=2, Hq=16, Hkv=8, ctx=2000, k=12, hot=5),    # G 2
    dict(wl=4, B=4, ctx_range=(700, 5000)),                  # G 8, ragged contexts
    dict(wl=5, B=2, ctx=4096, k=16, hot=6, headwise=True),   # G 4, headwise
])
def test_attention_qk_on_vector_alus(spec_args):
    """The v_dot2 QK^T matches the oracle to the same bar as the MFMA one, in
    SoloHead and headwise layouts, over ragged last blocks."""
    args = dict(spec_args)
    wl = args.pop("wl")
    s = synth.spec(wl, **args)
    H.log(f"[qk valu] {s.name} Hq {s.Hq} Hkv {s.Hkv} bs {s.bs}")
    c, sl = _case(s, [0])
    try:
        modes = [kv.KVOFF_SOLOHEAD] + ([kv.KVOFF_HEADWISE] if s.headwise else [])
        for mode in modes:
            kv.kvoff_set_attention_qk(c.ctx, kv.KVOFF_QK_MFMA)
            bufs = H.make_buffers(c, mode)
            H.run_layer(c, 0, mode, bufs)
            torch.cuda.synchronize()
            mfma_out = bufs.out.cpu().numpy().copy()
            kv.kvoff_set_attention_qk(c.ctx, kv.KVOFF_QK_VALU)
            bufs.out.fill_(float("nan"))
            H.run_layer(c, 0, mode, bufs)
            torch.cuda.synchronize()
            err = P.check_attention(c, 0, mode, bufs, sl)
            H.log(f"  mode {mode} attention err {err} "
                  f"max |valu - mfma| {np.abs(bufs.out.cpu().numpy() - mfma_out).max():.3g}")
    finally:
        H.destroy(c)


def test_attention_qk_valu_rejects_large_groups():
    s = synth.spec(2, B=1, Hq=32, Hkv=2, ctx=512, k=4, hot=1)
    c, _ = _case(s, [0])
    try:
        with pytest.raises(kv.KvoffError) as e:
            kv.kvoff_set_attention_qk(c.ctx, kv.KVOFF_QK_VALU)
        assert e.value.status == kv.KVOFF_EINVAL
        with pytest.raises(kv.KvoffError):
            kv.kvoff_set_attention_qk(c.ctx, 7)
    finally:
        H.destroy(c)


# fp32 logits differ from the oracle's fp64 ones by at most about
# 128 * 2^-24 * sum_j |q_j K_j| / sqrt(d) (~5e-5 at unit-variance inputs);
# the kept share moves by at most about twice that.
MASS_ATOL = 1e-4


@pytest.mark.parametrize("which", ["tiny", "hw", "ragged"])
def test_attention_mass_matches_oracle(which):
    """kvoff_attention_mass against the oracle for shared and per-KV-head
    sets, including partial last blocks."""
    s = {"tiny": TINY, "hw": HW, "ragged": RAGGED}[which]
    H.log(f"[mass] {which}")
    lam = 0.5
    c, sl = _case(s, [0], lam=lam, group_lam=lam)
    try:
        modes = [kv.KVOFF_SOLOHEAD, kv.KVOFF_CONSENSUS, kv.KVOFF_CONSENSUS_GROUP] + \
            ([kv.KVOFF_HEADWISE] if s.headwise else [])
        for mode in modes:
            bufs = H.make_buffers(c, mode)
            kv.kvoff_select(c.ctx, 0, c.rids, c.q[0], c.digest[0], c.nb_max,
                            [rq.k for rq in c.reqs], mode, bufs.scores, bufs.sel_idx,
                            bufs.sel_cnt, c.k_stride)
            mass = torch.full((c.B, s.Hq), float("nan"), dtype=torch.float64, device="cuda")
            kv.kvoff_attention_mass(c.ctx, 0, c.rids, mode, c.q[0], bufs.sel_idx, bufs.sel_cnt,
                                    c.k_stride, 1.0 / math.sqrt(s.d), mass)
            torch.cuda.synchronize()
            got = mass.cpu().numpy()
            worst = 0.0
            for r in range(c.B):
                x = sl[(0, r)]
                sets = P.block_sets(x, mode)
                ref = oracle.attention_mass(x.lr.q, x.lr.K, s.dtype, s.bs,
                                            np.stack(sets) if len(sets) > 1 else sets[0])
                err = np.abs(got[r] - ref).max()
                worst = max(worst, err)
                assert err <= MASS_ATOL, (mode, r, err)
            H.log(f"  mode {mode}: mean mass {got.mean():.4f}, max |err| {worst:.2e}")
    finally:
        H.destroy(c)


def test_very_long_context_takes_the_streaming_topk():
    """More than 16384 blocks in one request: the top-k re-reads the scores
    each pass instead of holding them in registers; k above 128 uses four
    blocks per attention wave."""
    s = synth.spec(1, B=2, ctx=300_000, k=300, hot=40)  # bs 16: 18750 blocks per request
    H.log(f"[long context] {s.ctx} tokens, {-(-s.ctx // s.bs)} blocks, k {s.k}")
    c, sl = _case(s, [0])
    try:
        assert c.nb_max > 16384
        stats, err = _full_check(c, sl, 0, kv.KVOFF_SOLOHEAD, kv.KVOFF_ENGINE_ZEROCOPY)
        H.log(f"  stats {stats} attention err {err}")
    finally:
        H.destroy(c)


def test_largest_batch_and_one_past_it():
    """KVOFF_MAX_BATCH (128) requests in one call, mixed short contexts; 129
    is rejected before anything is enqueued."""
    s = synth.spec(4, B=kv.KVOFF_MAX_BATCH, ctx_range=(40, 400), k_frac_range=(0.1, 0.6), hot=0)
    H.log(f"[max batch] {s.B} requests")
    c, sl = _case(s, [0])
    try:
        _full_check(c, sl, 0, kv.KVOFF_SOLOHEAD, kv.KVOFF_ENGINE_ZEROCOPY)
        bufs = H.make_buffers(c, kv.KVOFF_SOLOHEAD)
        with pytest.raises(kv.KvoffError) as e:
            kv.kvoff_select(c.ctx, 0, c.rids + [c.rids[0]], c.q[0], c.digest[0], c.nb_max,
                            [1] * (s.B + 1), kv.KVOFF_SOLOHEAD, bufs.scores, bufs.sel_idx,
                            bufs.sel_cnt, c.k_stride)
        assert e.value.status == kv.KVOFF_ERANGE
    finally:
        H.destroy(c)


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
@pytest.mark.parametrize("bs", [16, 32])
def test_dtype_and_block_size_grid(dtype, bs):
    """Every (storage type, block size) pair of the kernels, SoloHead and
    headwise, with a ragged last block."""
    s = synth.spec(2, B=2, dtype=dtype, bs=bs, ctx=2500, k=14, hot=6, headwise=True)
    H.log(f"[dtype/bs] dtype {dtype} bs {bs}")
    c, sl = _case(s, [0])
    try:
        for mode in (kv.KVOFF_SOLOHEAD, kv.KVOFF_HEADWISE):
            _, err = _full_check(c, sl, 0, mode, kv.KVOFF_ENGINE_ZEROCOPY)
            H.log(f"  mode {mode} attention err {err}")
    finally:
        H.destroy(c)


# 4 and 8 blocks per attention wave (selections of 64 blocks and up; 8 when
# the grid still has 256 workgroups) at G = 4, with counts that leave waves
# partly filled and whole splits empty: K is 70, 47 (every block of a
# 47-block request) and 66, so the splits end inside a wave and the short
# request's last split holds no block.
BPW_CASES = [
    dict(wl=2, dtype=synth.BF16, bs=32, reqs=[(5000, 70), (1500, 70), (3000, 66)]),
    dict(wl=1, dtype=synth.F16, bs=16, reqs=[(2500, 70), (752, 70), (1500, 66)]),
    dict(wl=2, dtype=synth.BF16, bs=32, reqs=[(3000, 70), (1500, 70), (2200, 66)] * 5 + [(1200, 70)]),
]


@pytest.mark.parametrize("case", BPW_CASES, ids=["bf16-bs32-4", "fp16-bs16-4", "bf16-bs32-8"])
def test_blocks_per_wave_with_partial_and_empty_splits(case):
    n = len(case["reqs"])
    s = synth.spec(case["wl"], B=n, dtype=case["dtype"], bs=case["bs"], ctx=5000, k=70, hot=8,
                   headwise=True)
    reqs = [synth.Request(ctx=ctx, nb=-(-ctx // s.bs), k=k) for ctx, k in case["reqs"]]
    H.log(f"[blocks per wave] dtype {case['dtype']} bs {case['bs']} {n} requests")
    c, sl = _case(s, [0], reqs=reqs)
    try:
        assert c.k_stride == 70 and s.Hq // s.Hkv == 4
        assert min(min(rq.k, rq.nb) for rq in reqs) <= 48  # a request with an empty split
        # 8 blocks per wave when 8-block splits still give 256 workgroups
        assert (n * s.Hkv * 3 >= 256) == (n == 16)
        for mode in (kv.KVOFF_SOLOHEAD, kv.KVOFF_HEADWISE):
            _, err = _full_check(c, sl, 0, mode, kv.KVOFF_ENGINE_ZEROCOPY)
            H.log(f"  mode {mode} attention err {err}")
    finally:
        H.destroy(c)


def test_degenerate_sizes():
    """k >= nb (take every block), k = 1, one-token and one-block contexts."""
    H.log("[degenerate]")
    s = synth.spec(2, B=4, ctx=100, k=1, hot=1, headwise=True)
    reqs = [synth.Request(ctx=1, nb=1, k=1), synth.Request(ctx=33, nb=2, k=5),
            synth.Request(ctx=100, nb=4, k=1), synth.Request(ctx=96, nb=3, k=3)]
    c, sl = _case(s, [0], reqs=reqs)
    try:
        _full_check(c, sl, 0, kv.KVOFF_SOLOHEAD, kv.KVOFF_ENGINE_ZEROCOPY)
        _full_check(c, sl, 0, kv.KVOFF_HEADWISE, kv.KVOFF_ENGINE_DMA)
        _full_check(c, sl, 0, kv.KVOFF_SOLOHEAD, kv.KVOFF_ENGINE_STAGED)
        _full_check(c, sl, 0, kv.KVOFF_HEADWISE, kv.KVOFF_ENGINE_STAGED)
    finally:
        H.destroy(c)


# Exact score ties across the top-k boundary.  Every key of block b of
# request r is the constant c = (7b + r) mod 3 (the last request: 0
# everywhere) and the queries are positive, so blocks with one constant get
# bit-identical scores on either side, ordered by the constant; the boundary
# falls inside a tie group, which the selection must cut at the lower block
# ids.  The three cases take the register top-k with 4 and 16 keys per thread
# and the streaming top-k past 16,384 blocks.
TIE_CASES = [
    dict(wl=2, B=3, ctx=8192, k=100),                        # bf16, 32-token blocks, 256 blocks
    dict(wl=2, B=3, ctx=65536, k=900),                       # 2,048 blocks
    dict(wl=1, B=2, ctx=300000, k=300),                      # fp16, 16-token blocks, 18,750 blocks
]


@pytest.mark.parametrize("case", TIE_CASES, ids=["256-blocks", "2048-blocks", "18750-blocks"])
def test_topk_exact_ties_take_the_lower_block_ids(case):
    args = dict(case)
    s = synth.spec(args.pop("wl"), headwise=True, **args)
    H.log(f"[ties] {s.name} ctx {s.ctx} k {s.k}")
    one, two = (0x3F80, 0x4000) if s.dtype == synth.BF16 else (0x3C00, 0x4000)
    reqs = synth.request_draws(s)
    sl = {}
    for r, rq in enumerate(reqs):
        lr = synth.gen_layer_request(s, 0, r, rq)
        lr.q &= np.uint16(0x7FFF)
        for b in range(rq.nb):
            c = 0 if r == len(reqs) - 1 else (7 * b + r) % 3
            lr.K[b * s.bs:(b + 1) * s.bs] = (0, one, two)[c]
        sl[(0, r)] = workloads.condition(s, lr, enforce=False)
        assert sl[(0, r)].gap == 0.0  # the boundary is a tie in every ranking
    c = H.build_case(s, {k: v.lr for k, v in sl.items()}, [0], reqs)
    try:
        for mode in (kv.KVOFF_SOLOHEAD, kv.KVOFF_HEADWISE):
            _full_check(c, sl, 0, mode, kv.KVOFF_ENGINE_ZEROCOPY)
        zero = sl[(0, len(reqs) - 1)]
        assert zero.sel.tolist() == list(range(zero.K))
    finally:
        H.destroy(c)


# several layers: overlapped kvoff_step must equal the serial order bit for bit
MULTI = synth.spec(3, B=2, L=4, ctx=3000, k=20, hot=8)


@pytest.mark.parametrize("engine", [kv.KVOFF_ENGINE_ZEROCOPY, kv.KVOFF_ENGINE_DMA, kv.KVOFF_ENGINE_STAGED])
def test_step_overlap_matches_serial_and_oracle(engine):
    H.log(f"[step] engine {engine}")
    layers = list(range(MULTI.L))
    c, sl = _case(MULTI, layers)
    try:
        mode = kv.KVOFF_SOLOHEAD
        sets = [H.make_buffers(c, mode) for _ in range(2)]
        outs = {l: torch.empty((c.B, MULTI.Hq, MULTI.d), dtype=torch.float32, device="cuda")
                for l in layers}
        compute = torch.cuda.Stream()
        copy = torch.cuda.Stream()

        def step(copy_stream, want_stats=False, copy2=None):
            return kv.kvoff_step(
                c.ctx, layer_begin=0, layer_end=len(layers), req_ids=c.rids,
                topk=[rq.k for rq in c.reqs], mode=mode, engine=engine, k_stride=c.k_stride,
                q=[c.q[l] for l in layers], digest=[c.digest[l] for l in layers],
                digest_stride=c.nb_max, slot_pool=c.pool, n_slots=c.n_slots,
                recall_base_slot=c.recall_base, scores=[b.scores for b in sets],
                sel_idx=[b.sel_idx for b in sets], sel_cnt=[b.sel_cnt for b in sets],
                block_table=[b.table for b in sets], scale=1.0 / math.sqrt(MULTI.d),
                out=[outs[l] for l in layers], ws=sets[0].ws, compute_stream=compute,
                copy_stream=copy_stream, want_stats=want_stats, copy_stream2=copy2)

        step(copy)  # odd layers on the context's own second copy stream
        torch.cuda.synchronize()
        overlapped = {l: outs[l].cpu().numpy().copy() for l in layers}
        for o in outs.values():
            o.fill_(float("nan"))
        step(copy, copy2=torch.cuda.Stream())  # the caller's second copy stream
        torch.cuda.synchronize()
        for l in layers:
            assert np.array_equal(outs[l].cpu().numpy().view(np.uint32),
                                  overlapped[l].view(np.uint32)), l
        stats = step(compute, want_stats=True)  # serial: one stream
        torch.cuda.synchronize()
        for l in layers:
            serial = outs[l].cpu().numpy()
            assert np.array_equal(serial.view(np.uint32), overlapped[l].view(np.uint32)), l
            P.check_attention_close(serial, P.oracle_attention(c, l, mode, sl), f"layer {l}")
        exp = [P.expected_transfers(c, l, mode, sl, False) for l in layers]
        rec = kv.kvoff_record_bytes(c.ctx)
        if engine == kv.KVOFF_ENGINE_STAGED:  # transfers are the bulk staging copies
            want_tr = sum(P.staged_copies(e["items_recalled"] * rec) for e in exp)
        else:
            want_tr = sum(e["transfers"] for e in exp)
        assert stats["transfers"] == want_tr
        assert stats["items_recalled"] == sum(e["items_recalled"] for e in exp)
    finally:
        H.destroy(c)


RAGGED_LAYERS = synth.spec(4, B=6, L=2, ctx_range=(700, 5000))


@pytest.mark.parametrize("engine", [kv.KVOFF_ENGINE_ZEROCOPY, kv.KVOFF_ENGINE_DMA, kv.KVOFF_ENGINE_STAGED])
def test_step_request_groups_match_whole_batch(engine):
    """Interruptible per-request-group scheduling gives the same bits as one
    recall and one attention per layer, and both match the oracle."""
    H.log(f"[step groups] engine {engine}")
    s = RAGGED_LAYERS
    layers = [0, 1]
    c, sl = _case(s, layers)
    try:
        mode = kv.KVOFF_SOLOHEAD
        sets = [H.make_buffers(c, mode) for _ in range(2)]
        compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
        results = {}
        for grp in (0, 1, 4):
            outs = [torch.full((c.B, s.Hq, s.d), float("nan"), device="cuda") for _ in layers]
            st = kv.kvoff_step(
                c.ctx, layer_begin=0, layer_end=2, req_ids=c.rids, topk=[rq.k for rq in c.reqs],
                mode=mode, engine=engine, k_stride=c.k_stride, q=[c.q[l] for l in layers],
                digest=[c.digest[l] for l in layers], digest_stride=c.nb_max, slot_pool=c.pool,
                n_slots=c.n_slots, recall_base_slot=c.recall_base,
                scores=[b.scores for b in sets], sel_idx=[b.sel_idx for b in sets],
                sel_cnt=[b.sel_cnt for b in sets], block_table=[b.table for b in sets],
                scale=1.0 / math.sqrt(s.d), out=outs, ws=sets[0].ws, compute_stream=compute,
                copy_stream=copy, want_stats=True, group_requests=grp)
            torch.cuda.synchronize()
            results[grp] = ([o.cpu().numpy() for o in outs], st)
        for grp in (1, 4):
            for l in layers:
                assert np.array_equal(results[grp][0][l].view(np.uint32),
                                      results[0][0][l].view(np.uint32)), (grp, l)
            assert results[grp][1]["items_recalled"] == results[0][1]["items_recalled"]
        for l in layers:
            P.check_attention_close(results[0][0][l], P.oracle_attention(c, l, mode, sl), f"layer {l}")
    finally:
        H.destroy(c)


@pytest.mark.parametrize("engine", [kv.KVOFF_ENGINE_ZEROCOPY, kv.KVOFF_ENGINE_DMA, kv.KVOFF_ENGINE_STAGED])
def test_step_groups_with_resident_requests(engine):
    """Request groups reordered by residency (resident groups first, a
    different order per layer) still give the whole-batch bits, and pinned
    (layer, request) pairs recall nothing.  With groups of one request, a
    resident request's recall moves nothing at all (for the staged engine:
    only its block table goes up), on alternating copy streams."""
    H.log(f"[step groups] resident requests, engine {engine}")
    s = RAGGED_LAYERS
    layers = [0, 1]
    reqs, sl = _slices(s, layers)
    nb_tot = sum(rq.nb for rq in reqs)
    c = H.build_case(s, {k: v.lr for k, v in sl.items()}, layers, reqs, extra_slots=2 * nb_tot)
    try:
        mode = kv.KVOFF_SOLOHEAD
        sets = [H.make_buffers(c, mode) for _ in range(2)]
        compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
        hit = [torch.zeros((c.B, c.nb_max), dtype=torch.uint8, device="cuda") for _ in layers]
        slot = [torch.full((c.B, c.nb_max), -1, dtype=torch.int32, device="cuda") for _ in layers]
        pinned = {0: [4, 5], 1: [1, 3]}  # layer -> requests made resident
        first = c.extra_base
        for l, rs in pinned.items():
            for r in rs:
                kv.kvoff_make_resident(c.ctx, l, c.rids[r], c.pool, c.n_slots, first, hit[l][r],
                                       slot[l][r])
                first += reqs[r].nb
        torch.cuda.synchronize()
        results = {}
        for grp in (0, 1, 2):
            outs = [torch.full((c.B, s.Hq, s.d), float("nan"), device="cuda") for _ in layers]
            st = kv.kvoff_step(
                c.ctx, layer_begin=0, layer_end=2, req_ids=c.rids, topk=[rq.k for rq in reqs],
                mode=mode, engine=engine, k_stride=c.k_stride,
                q=[c.q[l] for l in layers], digest=[c.digest[l] for l in layers],
                digest_stride=c.nb_max, slot_pool=c.pool, n_slots=c.n_slots,
                recall_base_slot=c.recall_base, scores=[b.scores for b in sets],
                sel_idx=[b.sel_idx for b in sets], sel_cnt=[b.sel_cnt for b in sets],
                block_table=[b.table for b in sets], scale=1.0 / math.sqrt(s.d), out=outs,
                ws=sets[0].ws, pool_hit=hit, pool_slot=slot, pool_stride=c.nb_max,
                compute_stream=compute, copy_stream=copy, want_stats=True, group_requests=grp,
                want_timing=True)
            torch.cuda.synchronize()
            results[grp] = ([o.cpu().numpy() for o in outs], st)
            t = st["timing"]
            H.log(f"  groups of {grp}: {t}")
            assert 0 < t["mean_request_done_ms"] <= t["max_request_done_ms"] == t["step_ms"]
            assert 0 <= t["compute_wait_ms"] < t["step_ms"]
            if grp == 0:
                assert t["mean_request_done_ms"] == t["max_request_done_ms"]
            n_groups = 1 if grp == 0 else -(-c.B // grp)
            assert t["recalls"] == len(layers) * n_groups and t["recall_ms"] > 0
        want_items = sum(min(reqs[r].k, reqs[r].nb) for l in layers for r in range(c.B)
                         if r not in pinned[l])
        for grp in (0, 1, 2):
            assert results[grp][1]["items_recalled"] == want_items, grp
            for l in layers:
                assert np.array_equal(results[grp][0][l].view(np.uint32),
                                      results[0][0][l].view(np.uint32)), (grp, l)
        for l in layers:
            P.check_attention_close(results[0][0][l], P.oracle_attention(c, l, mode, sl), f"layer {l}")
    finally:
        H.destroy(c)


def test_resident_layer_is_not_recalled():
    """IO-adaptive admission: a layer made resident in HBM recalls nothing and
    attends to the same bytes; releasing it brings the recall back."""
    H.log("[admission] resident layer")
    s = synth.spec(2, B=3, ctx=3000, k=20, hot=8)
    reqs, sl = _slices(s, [0])
    nb_tot = sum(rq.nb for rq in reqs)
    c = H.build_case(s, {k: v.lr for k, v in sl.items()}, [0], reqs, extra_slots=nb_tot)
    try:
        mode = kv.KVOFF_SOLOHEAD
        bufs = H.make_buffers(c, mode)
        st0 = H.run_layer(c, 0, mode, bufs, want_stats=True)
        torch.cuda.synchronize()
        out0 = bufs.out.cpu().numpy().copy()
        hit = torch.zeros((c.B, c.nb_max), dtype=torch.uint8, device="cuda")
        slot = torch.full((c.B, c.nb_max), -1, dtype=torch.int32, device="cuda")
        first = c.extra_base
        for r, rq in enumerate(reqs):
            kv.kvoff_make_resident(c.ctx, 0, c.rids[r], c.pool, c.n_slots, first, hit[r], slot[r])
            first += rq.nb
        c.pool_hit[0], c.pool_slot[0] = hit, slot
        st1 = H.run_layer(c, 0, mode, bufs, with_pool_hits=True, want_stats=True)
        torch.cuda.synchronize()
        assert st1["items_recalled"] == 0 and st1["bytes"] == 0
        assert st1["pool_hits"] == st0["selected"]
        assert np.array_equal(bufs.out.cpu().numpy().view(np.uint32), out0.view(np.uint32))
        for r in range(c.B):
            kv.kvoff_release_resident(c.ctx, 0, c.rids[r], hit[r])
        st2 = H.run_layer(c, 0, mode, bufs, with_pool_hits=True, want_stats=True)
        torch.cuda.synchronize()
        assert st2["items_recalled"] == st0["items_recalled"]
        assert np.array_equal(bufs.out.cpu().numpy().view(np.uint32), out0.view(np.uint32))
        with pytest.raises(kv.KvoffError) as e:  # slots past the pool
            kv.kvoff_make_resident(c.ctx, 0, c.rids[0], c.pool, c.n_slots, c.n_slots - 1, hit[0], slot[0])
        assert e.value.status == kv.KVOFF_ERANGE
    finally:
        H.destroy(c)


def test_error_paths_on_device():
    H.log("[errors]")
    s = synth.spec(1, ctx=512, k=8, hot=2)
    c, sl = _case(s, [0])
    try:
        bufs = H.make_buffers(c, kv.KVOFF_SOLOHEAD)
        with pytest.raises(kv.KvoffError) as e:  # k_stride smaller than K
            kv.kvoff_select(c.ctx, 0, c.rids, c.q[0], c.digest[0], c.nb_max, [8],
                            kv.KVOFF_SOLOHEAD, bufs.scores, bufs.sel_idx, bufs.sel_cnt, 4)
        assert e.value.status == kv.KVOFF_ERANGE
        with pytest.raises(kv.KvoffError) as e:  # k < 1
            kv.kvoff_select(c.ctx, 0, c.rids, c.q[0], c.digest[0], c.nb_max, [0],
                            kv.KVOFF_SOLOHEAD, bufs.scores, bufs.sel_idx, bufs.sel_cnt, 8)
        assert e.value.status == kv.KVOFF_EINVAL
        with pytest.raises(kv.KvoffError) as e:  # unknown request id
            kv.kvoff_select(c.ctx, 0, [5], c.q[0], c.digest[0], c.nb_max, [8],
                            kv.KVOFF_SOLOHEAD, bufs.scores, bufs.sel_idx, bufs.sel_cnt, 8)
        assert e.value.status == kv.KVOFF_ESTATE
        with pytest.raises(kv.KvoffError) as e:  # store is full
            kv.kvoff_register_request(c.ctx, 512)
        assert e.value.status == kv.KVOFF_ERANGE
        with pytest.raises(kv.KvoffError) as e:  # recall region past the pool
            kv.kvoff_recall(c.ctx, 0, c.rids, kv.KVOFF_SOLOHEAD, bufs.sel_idx, bufs.sel_cnt,
                            c.k_stride, None, None, 0, c.pool, c.n_slots, c.n_slots,
                            bufs.table)
        assert e.value.status == kv.KVOFF_ERANGE
        # a pool whose slot (headwise: slice) indices would not fit the int32
        # table and pool-slot entries
        too_many = (2**31 - 1) // s.Hkv + 1
        with pytest.raises(kv.KvoffError) as e:
            kv.kvoff_recall(c.ctx, 0, c.rids, kv.KVOFF_SOLOHEAD, bufs.sel_idx, bufs.sel_cnt,
                            c.k_stride, None, None, 0, c.pool, too_many, 0, bufs.table)
        assert e.value.status == kv.KVOFF_EINVAL
        hit = torch.zeros(c.nb_max, dtype=torch.uint8, device="cuda")
        slot = torch.zeros(c.nb_max, dtype=torch.int32, device="cuda")
        with pytest.raises(kv.KvoffError) as e:
            kv.kvoff_make_resident(c.ctx, 0, c.rids[0], c.pool, too_many, 0, hit, slot)
        assert e.value.status == kv.KVOFF_EINVAL
        with pytest.raises(kv.KvoffError) as e:  # workspace too small
            kv.kvoff_sparse_decode(c.ctx, c.rids, kv.KVOFF_SOLOHEAD, c.q[0], c.pool, c.n_slots, bufs.table,
                                   bufs.sel_idx, bufs.sel_cnt, c.k_stride, 0.1, bufs.out,
                                   bufs.ws[:4])
        assert e.value.status == kv.KVOFF_ERANGE
        # an empty batch is a no-op
        kv.kvoff_select(c.ctx, 0, [], c.q[0], c.digest[0], c.nb_max, [], kv.KVOFF_SOLOHEAD,
                        bufs.scores, bufs.sel_idx, bufs.sel_cnt, 8)
        torch.cuda.synchronize()
    finally:
        H.destroy(c)


def test_attention_mass_error_paths():
    H.log("[mass errors]")
    s = synth.spec(1, ctx=512, k=8, hot=2)
    c, sl = _case(s, [0])
    try:
        bufs = H.make_buffers(c, kv.KVOFF_SOLOHEAD)
        mass = torch.empty((c.B, s.Hq), dtype=torch.float64, device="cuda")
        args = (c.q[0], bufs.sel_idx, bufs.sel_cnt, c.k_stride, 0.1, mass)
        with pytest.raises(kv.KvoffError) as e:  # unknown mode
            kv.kvoff_attention_mass(c.ctx, 0, c.rids, 9, *args)
        assert e.value.status == kv.KVOFF_EINVAL
        with pytest.raises(kv.KvoffError) as e:  # layer outside the store
            kv.kvoff_attention_mass(c.ctx, 1, c.rids, kv.KVOFF_SOLOHEAD, *args)
        assert e.value.status == kv.KVOFF_ERANGE
        with pytest.raises(kv.KvoffError) as e:  # unknown request
            kv.kvoff_attention_mass(c.ctx, 0, [7], kv.KVOFF_SOLOHEAD, *args)
        assert e.value.status == kv.KVOFF_ESTATE
        with pytest.raises(kv.KvoffError) as e:  # k_stride < 1
            kv.kvoff_attention_mass(c.ctx, 0, c.rids, kv.KVOFF_SOLOHEAD, c.q[0], bufs.sel_idx,
                                    bufs.sel_cnt, 0, 0.1, mass)
        assert e.value.status == kv.KVOFF_EINVAL
        kv.kvoff_attention_mass(c.ctx, 0, [], kv.KVOFF_SOLOHEAD, *args)  # empty batch: no-op
    finally:
        H.destroy(c)


@pytest.mark.parametrize("engine", [kv.KVOFF_ENGINE_ZEROCOPY, kv.KVOFF_ENGINE_DMA, kv.KVOFF_ENGINE_STAGED])
def test_out_of_range_block_ids_are_unused_entries(engine):
    """A selection entry outside its request (too large or negative) is
    treated as unused by every recall engine and by the attention: no bytes
    move for it, its table entry is -1, and attention covers the rest."""
    H.log(f"[bad ids] engine {engine}")
    s = synth.spec(2, B=2, ctx=3000, k=12, hot=5)
    c, sl = _case(s, [0])
    try:
        bufs = H.make_buffers(c, kv.KVOFF_SOLOHEAD)
        kv.kvoff_select(c.ctx, 0, c.rids, c.q[0], c.digest[0], c.nb_max, [rq.k for rq in c.reqs],
                        kv.KVOFF_SOLOHEAD, bufs.scores, bufs.sel_idx, bufs.sel_cnt, c.k_stride)
        torch.cuda.synchronize()
        nb = [rq.nb for rq in c.reqs]
        bad = {(0, 2): nb[0] + 5, (1, 0): -7}
        for (r, i), v in bad.items():
            bufs.sel_idx[r, 0, i] = v
        st = kv.kvoff_recall(c.ctx, 0, c.rids, kv.KVOFF_SOLOHEAD, bufs.sel_idx, bufs.sel_cnt,
                             c.k_stride, None, None, 0, c.pool, c.n_slots, c.recall_base[0],
                             bufs.table, engine, want_stats=True)
        kv.kvoff_sparse_decode(c.ctx, c.rids, kv.KVOFF_SOLOHEAD, c.q[0], c.pool, c.n_slots, bufs.table,
                               bufs.sel_idx, bufs.sel_cnt, c.k_stride, 1.0 / math.sqrt(s.d),
                               bufs.out, bufs.ws)
        torch.cuda.synchronize()
        table = bufs.table.cpu().numpy()
        for (r, i) in bad:
            assert table[r, 0, i] == -1, (r, i)
        K = sum(x.K for x in sl.values())
        assert st["selected"] == K - len(bad) and st["items_recalled"] == K - len(bad)
        got = bufs.out.cpu().numpy()
        for r in range(c.B):
            x = sl[(0, r)]
            keep = np.array([b for i, b in enumerate(x.sel.tolist()) if (r, i) not in bad], np.int32)
            ref = oracle.attend_f32(x.lr.q, x.lr.K, x.lr.V, s.dtype, s.bs, keep)
            P.check_attention_close(got[r], ref, f"request {r}")
    finally:
        H.destroy(c)


def test_step_error_paths():
    """kvoff_step rejects bad layer ranges, shared recall regions when
    overlapping, unknown requests and NULL buffers (also a later layer's)
    before enqueuing any work."""
    H.log("[step errors]")
    layers = list(range(MULTI.L))
    c, sl = _case(MULTI, layers)
    try:
        sets = [H.make_buffers(c, kv.KVOFF_SOLOHEAD) for _ in range(2)]
        outs = [torch.empty((c.B, MULTI.Hq, MULTI.d), dtype=torch.float32, device="cuda")
                for _ in layers]
        compute, copy = torch.cuda.Stream(), torch.cuda.Stream()

        def step(**kw):
            args = dict(layer_begin=0, layer_end=len(layers), req_ids=c.rids,
                        topk=[rq.k for rq in c.reqs], mode=kv.KVOFF_SOLOHEAD,
                        engine=kv.KVOFF_ENGINE_ZEROCOPY, k_stride=c.k_stride,
                        q=[c.q[l] for l in layers], digest=[c.digest[l] for l in layers],
                        digest_stride=c.nb_max, slot_pool=c.pool, n_slots=c.n_slots,
                        recall_base_slot=c.recall_base, scores=[b.scores for b in sets],
                        sel_idx=[b.sel_idx for b in sets], sel_cnt=[b.sel_cnt for b in sets],
                        block_table=[b.table for b in sets], scale=0.1, out=outs, ws=sets[0].ws,
                        compute_stream=compute, copy_stream=copy)
            args.update(kw)
            return kv.kvoff_step(c.ctx, **args)

        for kw, status in ((dict(layer_end=len(layers) + 1), kv.KVOFF_ERANGE),
                           (dict(layer_begin=-1), kv.KVOFF_ERANGE),
                           (dict(recall_base_slot=(0, 0)), kv.KVOFF_EINVAL),
                           # regions of B * k_stride slots that overlap by one slot
                           (dict(recall_base_slot=(0, c.B * c.k_stride - 1)), kv.KVOFF_EINVAL),
                           (dict(recall_base_slot=(c.B * c.k_stride - 1, 0)), kv.KVOFF_EINVAL),
                           (dict(req_ids=[c.rids[0], 99]), kv.KVOFF_ESTATE),
                           (dict(q=[c.q[l] for l in layers[:-1]] + [None]), kv.KVOFF_EINVAL)):
            with pytest.raises(kv.KvoffError) as e:
                step(**kw)
            assert e.value.status == status, kw
        with pytest.raises(kv.KvoffError) as e:  # a hit map without its slot map
            step(pool_hit=[None] + [torch.zeros((c.B, c.nb_max), dtype=torch.uint8, device="cuda")]
                 * (len(layers) - 1), pool_slot=[None] * len(layers), pool_stride=c.nb_max)
        assert e.value.status == kv.KVOFF_EINVAL
        # one stream for both roles may share a recall region (serial order)
        step(recall_base_slot=(0, 0), copy_stream=compute)
        step(layer_end=0)  # an empty layer range is a no-op
        # maps for some layers only: the others recall everything
        step()
        torch.cuda.synchronize()
        ref = [o.cpu().numpy().copy() for o in outs]
        hits = [None] + [torch.zeros((c.B, c.nb_max), dtype=torch.uint8, device="cuda")
                         for _ in layers[1:]]
        slots = [None] + [torch.full((c.B, c.nb_max), -1, dtype=torch.int32, device="cuda")
                          for _ in layers[1:]]
        step(pool_hit=hits, pool_slot=slots, pool_stride=c.nb_max)
        torch.cuda.synchronize()
        for l in layers:
            assert np.array_equal(outs[l].cpu().numpy().view(np.uint32), ref[l].view(np.uint32)), l
    finally:
        H.destroy(c)


def test_recall_before_offload_is_rejected():
    H.log("[errors] recall before offload")
    ctx = kv.kvoff_create(num_layers=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                          block_size=16, dtype=kv.KVOFF_F16, max_requests=1,
                          host_capacity_blocks=64)
    try:
        rid = kv.kvoff_register_request(ctx, 256)
        sel = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
        cnt = torch.ones((1,), dtype=torch.int32, device="cuda")
        pool = torch.zeros(4 * kv.kvoff_record_bytes(ctx), dtype=torch.uint8, device="cuda")
        table = torch.empty((1, 4), dtype=torch.int32, device="cuda")
        with pytest.raises(kv.KvoffError) as e:
            kv.kvoff_recall(ctx, 1, [rid], kv.KVOFF_SOLOHEAD, sel, cnt, 4, None, None, 0, pool, 4,
                            0, table)
        assert e.value.status == kv.KVOFF_ESTATE
    finally:
        kv.kvoff_destroy(ctx)


@pytest.mark.parametrize("mode", [kv.KVOFF_SOLOHEAD, kv.KVOFF_HEADWISE])
def test_staged_recall_back_to_back_calls(mode):
    """Many staged recalls in a row, alternating between two streams, two
    layers and batches of one to four requests (3 to 4 bulk copies each),
    every one checked byte for byte and for compact placement: the worker
    pool hands each call's job over without mixing calls, and the staging
    buffers are reused only after the previous call's copies."""
    # 256 blocks, top-64: 8 MiB per request (per-head sets generated too)
    s = synth.spec(2, B=4, L=2, ctx=8192, headwise=True)
    H.log(f"[staged back to back] mode {mode}")
    c, sl = _case(s, [0, 1])
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    subsets = [[0, 1, 2, 3], [2], [1, 3], [0], [3, 2, 1, 0], [0, 2, 3], [1]]
    rec = kv.kvoff_record_bytes(c.ctx)
    hw = P.per_head(mode)
    item = rec // s.Hkv if hw else rec
    base = c.recall_base[0]
    try:
        for call in range(14):
            sub = subsets[call % len(subsets)]
            l = call % 2
            st = streams[call % 2]
            rids = [c.rids[r] for r in sub]
            idx = torch.tensor(sub, device="cuda")
            q = c.q[l].index_select(0, idx).contiguous()
            dg = c.digest[l].index_select(0, idx).contiguous()
            sets = s.Hkv if hw else 1
            scores = torch.empty((len(sub), sets, c.nb_max), dtype=torch.float64, device="cuda")
            sel = torch.empty((len(sub), sets, c.k_stride), dtype=torch.int32, device="cuda")
            cnt = torch.empty((len(sub),), dtype=torch.int32, device="cuda")
            table = torch.empty((len(sub), sets, c.k_stride), dtype=torch.int32, device="cuda")
            topk = [c.reqs[r].k for r in sub]
            kv.kvoff_select(c.ctx, l, rids, q, dg, c.nb_max, topk, mode, scores, sel, cnt,
                            c.k_stride, stream=st)
            stats = kv.kvoff_recall(c.ctx, l, rids, mode, sel, cnt, c.k_stride, None, None, 0,
                                    c.pool, c.n_slots, base, table, kv.KVOFF_ENGINE_STAGED,
                                    want_stats=True, stream=st)
            torch.cuda.synchronize()
            tab = table.cpu().numpy()
            pool = c.pool.cpu().numpy()
            n = 0
            for i, r in enumerate(sub):
                for g, bset in enumerate(P.block_sets(sl[(l, r)], mode)):
                    want = workloads.block_records(sl[(l, r)], bset.tolist())
                    for j in range(len(bset)):
                        ent = int(tab[i, g, j])
                        assert ent == (base * s.Hkv if hw else base) + n, (call, r, g, j, ent)
                        n += 1
                        got = pool[ent * item:(ent + 1) * item]
                        exp = (want[j, g] if hw else want[j]).reshape(-1).view(np.uint8)
                        assert np.array_equal(got, exp), (call, r, g, j)
            assert stats["items_recalled"] == n and stats["bytes"] == n * item
            assert stats["transfers"] == P.staged_copies(n * item), (call, stats)
        H.log(f"  {call + 1} calls checked")
    finally:
        H.destroy(c)


@pytest.mark.parametrize("mode", [kv.KVOFF_SOLOHEAD, kv.KVOFF_HEADWISE])
def test_staged_recall_overlapping_calls(mode):
    """Staged recalls issued on two streams with nothing waited for in
    between: each call reads back its selection and gathers while the
    previous call's copies are still in flight on the other stream, so the
    engine's two staging sets alternate under load, and one of them grows
    (a one-request call, then a three-request one, on the same set) while
    the other set's copies run.  Every call writes its own pool region and
    block table; all are checked byte for byte once both streams are done."""
    s = synth.spec(2, B=4, L=2, ctx=8192, headwise=True)
    H.log(f"[staged overlapping calls] mode {mode}")
    c, sl = _case(s, [0, 1])
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    subsets = [[0, 1, 2, 3], [2], [1, 3], [0], [3, 2, 1, 0], [0, 2, 3], [1]]
    n_calls = 14
    rec = kv.kvoff_record_bytes(c.ctx)
    hw = P.per_head(mode)
    item = rec // s.Hkv if hw else rec
    sets = s.Hkv if hw else 1
    region = 4 * c.k_stride  # slots of one call's recall region (at most 4 requests)
    n_slots = n_calls * region
    pool = torch.zeros(n_slots * rec, dtype=torch.uint8, device="cuda")
    calls = []
    for call in range(n_calls):
        sub = subsets[call % len(subsets)]
        l = call % 2
        idx = torch.tensor(sub, device="cuda")
        calls.append(dict(
            sub=sub, l=l, st=streams[call % 2], base=call * region,
            q=c.q[l].index_select(0, idx).contiguous(),
            dg=c.digest[l].index_select(0, idx).contiguous(),
            scores=torch.empty((len(sub), sets, c.nb_max), dtype=torch.float64, device="cuda"),
            sel=torch.empty((len(sub), sets, c.k_stride), dtype=torch.int32, device="cuda"),
            cnt=torch.empty((len(sub),), dtype=torch.int32, device="cuda"),
            table=torch.full((len(sub), sets, c.k_stride), -7, dtype=torch.int32, device="cuda")))
    torch.cuda.synchronize()
    try:
        for k in calls:
            rids = [c.rids[r] for r in k["sub"]]
            topk = [c.reqs[r].k for r in k["sub"]]
            kv.kvoff_select(c.ctx, k["l"], rids, k["q"], k["dg"], c.nb_max, topk, mode, k["scores"],
                            k["sel"], k["cnt"], c.k_stride, stream=k["st"])
            kv.kvoff_recall(c.ctx, k["l"], rids, mode, k["sel"], k["cnt"], c.k_stride, None, None, 0,
                            pool, n_slots, k["base"], k["table"], kv.KVOFF_ENGINE_STAGED,
                            stream=k["st"])
        torch.cuda.synchronize()
        pool_h = pool.cpu().numpy()
        for call, k in enumerate(calls):
            tab = k["table"].cpu().numpy()
            base = k["base"] * s.Hkv if hw else k["base"]
            n = 0
            for i, r in enumerate(k["sub"]):
                for g, bset in enumerate(P.block_sets(sl[(k["l"], r)], mode)):
                    want = workloads.block_records(sl[(k["l"], r)], bset.tolist())
                    for j in range(len(bset)):
                        ent = int(tab[i, g, j])
                        assert ent == base + n, (call, r, g, j, ent)
                        n += 1
                        got = pool_h[ent * item:(ent + 1) * item]
                        exp = (want[j, g] if hw else want[j]).reshape(-1).view(np.uint8)
                        assert np.array_equal(got, exp), (call, r, g, j)
                    assert (tab[i, g, len(bset):] == -1).all(), (call, r, g)
        H.log(f"  {n_calls} calls checked")
    finally:
        H.destroy(c)


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
@pytest.mark.parametrize("Hq", [64, 128])
def test_attention_pv_on_matrix_cores(dtype, Hq):
    """P V on the matrix cores (8 and 16 query heads per KV head, 32-token
    blocks) in both storage types, SoloHead and headwise, with a ragged last
    block; then a selection of every block of a 12,000-token context, whose
    many small softmax weights are what the fp16 operand's 2^15 scaling
    keeps from underflowing."""
    H.log(f"[pv mfma] dtype {dtype} Hq {Hq}")
    s = synth.spec(2, B=2, Hq=Hq, Hkv=8, dtype=dtype, ctx=2500, k=14, hot=6, headwise=True)
    c, sl = _case(s, [0])
    try:
        for mode in (kv.KVOFF_SOLOHEAD, kv.KVOFF_HEADWISE):
            _, err = _full_check(c, sl, 0, mode, kv.KVOFF_ENGINE_ZEROCOPY)
            H.log(f"  mode {mode} attention err {err}")
    finally:
        H.destroy(c)
    s = synth.spec(2, B=1, Hq=Hq, Hkv=8, dtype=dtype, ctx=12000, k=400, hot=6)
    c, sl = _case(s, [0])
    try:
        _, err = _full_check(c, sl, 0, kv.KVOFF_SOLOHEAD, kv.KVOFF_ENGINE_ZEROCOPY)
        H.log(f"  every block of 12,000 tokens: attention err {err}")
    finally:
        H.destroy(c)


def test_kernel_timing_leaves_results_unchanged():
    """Per-kernel timing: with it on, the selection, block table, recalled
    bytes and attention output equal an untimed run's bit for bit, every
    timed kernel reports a positive mean duration, and the call counts cover
    more calls than the 64-set event ring holds (so the ring wraps).
    Switching timing off clears the times, and calls made while it is off
    record none."""
    H.log("[kernel timing]")
    s = synth.spec(2, B=3, ctx=3000, k=20, hot=6)
    c, sl = _case(s, [0])
    zeros = dict(score_ms=0.0, topk_ms=0.0, attend_ms=0.0, combine_ms=0.0, select_calls=0,
                 decode_calls=0)
    try:
        mode = kv.KVOFF_SOLOHEAD
        ref = H.make_buffers(c, mode)
        H.run_layer(c, 0, mode, ref)
        torch.cuda.synchronize()
        kv.kvoff_set_kernel_timing(c.ctx, True)
        assert kv.kvoff_get_kernel_times(c.ctx) == zeros
        bufs = H.make_buffers(c, mode)
        n_calls = 70
        for _ in range(n_calls):
            H.run_layer(c, 0, mode, bufs)
        t = kv.kvoff_get_kernel_times(c.ctx)
        torch.cuda.synchronize()
        H.log(f"  kernel times {t}")
        assert t["select_calls"] == t["decode_calls"] == n_calls, t
        assert all(0.0 < t[k] < 1000.0 for k in ("score_ms", "topk_ms", "attend_ms", "combine_ms")), t
        for a, b in ((ref.sel_idx, bufs.sel_idx), (ref.sel_cnt, bufs.sel_cnt),
                     (ref.table, bufs.table)):
            assert torch.equal(a, b)
        assert torch.equal(ref.out.view(torch.int32), bufs.out.view(torch.int32))
        P.check_selection(c, 0, mode, bufs, sl)
        P.check_recall(c, 0, mode, bufs, sl)
        P.check_attention(c, 0, mode, bufs, sl)
        kv.kvoff_set_kernel_timing(c.ctx, False)
        H.run_layer(c, 0, mode, bufs)
        torch.cuda.synchronize()
        assert kv.kvoff_get_kernel_times(c.ctx) == zeros
    finally:
        torch.cuda.synchronize()
        H.destroy(c)


def test_step_graph_replay():
    """kvoff_step (zero-copy recall, no stats or timing) captured into a HIP
    graph on its compute stream; its two copy streams join the capture
    through the step's own events.  Four replays, each after eager work on
    the same buffers and a synchronisation, each give the eager outputs bit
    for bit."""
    H.log("[step graph]")
    layers = list(range(MULTI.L))
    c, sl = _case(MULTI, layers)
    try:
        mode = kv.KVOFF_SOLOHEAD
        sets = [H.make_buffers(c, mode) for _ in range(2)]
        outs = {l: torch.empty((c.B, MULTI.Hq, MULTI.d), dtype=torch.float32, device="cuda")
                for l in layers}
        compute, copy, copy2 = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()

        def step(n_layers):
            return kv.kvoff_step(
                c.ctx, layer_begin=0, layer_end=n_layers, req_ids=c.rids,
                topk=[rq.k for rq in c.reqs], mode=mode, engine=kv.KVOFF_ENGINE_ZEROCOPY,
                k_stride=c.k_stride, q=[c.q[l] for l in layers],
                digest=[c.digest[l] for l in layers], digest_stride=c.nb_max, slot_pool=c.pool,
                n_slots=c.n_slots, recall_base_slot=c.recall_base,
                scores=[b.scores for b in sets], sel_idx=[b.sel_idx for b in sets],
                sel_cnt=[b.sel_cnt for b in sets], block_table=[b.table for b in sets],
                scale=1.0 / math.sqrt(MULTI.d), out=[outs[l] for l in layers], ws=sets[0].ws,
                compute_stream=compute, copy_stream=copy, copy_stream2=copy2)

        step(len(layers))
        torch.cuda.synchronize()
        eager = {l: outs[l].cpu().numpy().copy() for l in layers}
        for l in layers:
            P.check_attention_close(eager[l], P.oracle_attention(c, l, mode, sl), f"layer {l}")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=compute):
            step(len(layers))
        torch.cuda.synchronize()
        for rep in range(4):
            # eager work between replays: a shorter step over the same
            # buffers, then the outputs poisoned
            step(2)
            torch.cuda.synchronize()
            for o in outs.values():
                o.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for l in layers:
                assert np.array_equal(outs[l].cpu().numpy().view(np.uint32),
                                      eager[l].view(np.uint32)), (rep, l)
        H.log("  4 replays bit-identical to the eager step")
        del g
    finally:
        torch.cuda.synchronize()
        H.destroy(c)
