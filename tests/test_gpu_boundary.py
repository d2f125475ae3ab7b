"""GPU tests of the boundary's checks and of shapes at the edges of the
kernels' assumptions, each against the oracle:

- records made of an odd number of 8 KiB slices (16-token blocks with 3 or
  5 KV heads) are recalled whole by every engine;
- pool hits naming a slot outside the pool, and table entries outside it,
  are never read: their table entries are -1, the attention covers the other
  blocks, and the call reports KVOFF_ESTATE;
- digests of bf16 keys whose values span more than 40 binades, where the
  order of an fp64 sum decides its bits, equal the oracle's sequential sums.
"""
import ctypes
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

ENGINES = [kv.KVOFF_ENGINE_ZEROCOPY, kv.KVOFF_ENGINE_DMA, kv.KVOFF_ENGINE_STAGED]


def _case(s, layers=(0,), with_pool_hits=False, reqs=None):
    reqs = reqs or synth.request_draws(s)
    sl = {(l, r): workloads.make_slice(s, l, r, rq) for l in layers for r, rq in enumerate(reqs)}
    c = H.build_case(s, {k: v.lr for k, v in sl.items()}, list(layers), reqs,
                     with_pool_hits=with_pool_hits)
    return c, sl


@pytest.mark.parametrize("Hq,Hkv", [(12, 3), (40, 5)])
@pytest.mark.parametrize("engine", ENGINES)
def test_records_of_odd_slice_counts_move_whole(Hq, Hkv, engine):
    """16-token fp16 blocks: a slice is 8 KiB and a record Hkv slices (24 or
    40 KiB, not a multiple of the gather's 16 KiB piece)."""
    s = synth.spec(1, B=2, Hq=Hq, Hkv=Hkv, ctx=2000, k=12, hot=5, headwise=True)
    H.log(f"[odd slices] Hq {Hq} Hkv {Hkv} engine {engine}: record {s.rec_bytes} bytes")
    c, sl = _case(s)
    try:
        for mode in (kv.KVOFF_SOLOHEAD, kv.KVOFF_HEADWISE):
            c.pool.zero_()
            bufs = H.make_buffers(c, mode)
            st = H.run_layer(c, 0, mode, bufs, engine=engine, want_stats=True)
            torch.cuda.synchronize()
            P.check_digests(c, 0, sl)
            P.check_selection(c, 0, mode, bufs, sl)
            P.check_recall(c, 0, mode, bufs, sl, stats=st, engine=engine)
            err = P.check_attention(c, 0, mode, bufs, sl)
            H.log(f"  mode {mode}: {st}, attention {err}")
    finally:
        H.destroy(c)


def _select(c, mode, bufs):
    kv.kvoff_select(c.ctx, 0, c.rids, c.q[0], c.digest[0], c.nb_max, [rq.k for rq in c.reqs],
                    mode, bufs.scores, bufs.sel_idx, bufs.sel_cnt, c.k_stride)
    torch.cuda.synchronize()


def _recall(c, mode, bufs, hit, slot, engine, want_stats):
    return kv.kvoff_recall(c.ctx, 0, c.rids, mode, bufs.sel_idx, bufs.sel_cnt, c.k_stride, hit,
                           slot, c.nb_max, c.pool, c.n_slots, c.recall_base[0], bufs.table, engine,
                           want_stats=want_stats)


def _decode(c, mode, bufs, n_slots=None):
    kv.kvoff_sparse_decode(c.ctx, c.rids, mode, c.q[0], c.pool,
                           c.n_slots if n_slots is None else n_slots, bufs.table, bufs.sel_idx,
                           bufs.sel_cnt, c.k_stride, 1.0 / math.sqrt(c.s.d), bufs.out, bufs.ws)
    torch.cuda.synchronize()


def _oracle_without(c, sl, dropped):
    """Oracle attention over each request's SoloHead selection minus the
    dropped (request, 0, rank) entries."""
    s = c.s
    out = np.empty((c.B, s.Hq, s.d), np.float32)
    for r in range(c.B):
        x = sl[(0, r)]
        kept = np.array([b for i, b in enumerate(x.sel.tolist()) if (r, 0, i) not in dropped],
                        np.int32)
        out[r] = oracle.attend_f32(x.lr.q, x.lr.K, x.lr.V, s.dtype, s.bs, kept)
    return out


@pytest.mark.parametrize("engine", ENGINES)
def test_pool_hits_outside_the_pool_are_never_read(engine):
    """Two pool hits of request 0 are re-pointed, one at slot -1 and one at
    n_slots.  Their table entries become -1, the other entries are as usual,
    the attention equals the oracle over the selection without those two
    blocks, and the call (with stats) returns KVOFF_ESTATE."""
    s = synth.spec(2, B=2, ctx=4000, k=24, hot=6, pool_frac=0.5)
    H.log(f"[bad pool slots] engine {engine}")
    c, sl = _case(s, with_pool_hits=True)
    try:
        mode = kv.KVOFF_SOLOHEAD
        bufs = H.make_buffers(c, mode)
        _select(c, mode, bufs)
        sel0 = sl[(0, 0)].sel.tolist()
        hit0 = sl[(0, 0)].lr.pool
        hit_ranks = [i for i, b in enumerate(sel0) if hit0[b]]
        assert len(hit_ranks) >= 2, "the workload must select two pool hits of request 0"
        bad = {hit_ranks[0]: -1, hit_ranks[-1]: c.n_slots}
        slot = c.pool_slot[0].clone()
        for i, v in bad.items():
            slot[0, sel0[i]] = v
        with pytest.raises(kv.KvoffError) as e:
            _recall(c, mode, bufs, c.pool_hit[0], slot, engine, want_stats=True)
        assert e.value.status == kv.KVOFF_ESTATE, e.value
        torch.cuda.synchronize()
        table = bufs.table.cpu().numpy()
        ps = c.pool_slot[0].cpu().numpy()
        for i, b in enumerate(sel0):
            if i in bad:
                assert table[0, 0, i] == -1, (i, table[0, 0, i])
            elif hit0[b]:
                assert table[0, 0, i] == ps[0, b], (i, table[0, 0, i], ps[0, b])
        _decode(c, mode, bufs)
        ref = _oracle_without(c, sl, {(0, 0, i) for i in bad})
        P.check_attention_close(bufs.out.cpu().numpy(), ref, "without the two bad hits")
        # the same maps without the bad entries: no error, the usual result
        st = _recall(c, mode, bufs, c.pool_hit[0], c.pool_slot[0], engine, want_stats=True)
        torch.cuda.synchronize()
        P.check_recall(c, 0, mode, bufs, sl, with_pool_hits=True, stats=st, engine=engine)
        _decode(c, mode, bufs)
        P.check_attention(c, 0, mode, bufs, sl)
    finally:
        H.destroy(c)


def test_zero_copy_reports_bad_slots_at_the_next_stats_call():
    """Without stats the zero-copy engine cannot report at once: the table
    entry is -1 and the next call that fills stats returns KVOFF_ESTATE once;
    the one after it succeeds."""
    s = synth.spec(2, B=2, ctx=4000, k=24, hot=6, pool_frac=0.5)
    H.log("[bad pool slots, sticky report]")
    c, sl = _case(s, with_pool_hits=True)
    try:
        mode = kv.KVOFF_SOLOHEAD
        bufs = H.make_buffers(c, mode)
        _select(c, mode, bufs)
        sel1 = sl[(0, 1)].sel.tolist()
        hit1 = sl[(0, 1)].lr.pool
        i_bad = next(i for i, b in enumerate(sel1) if hit1[b])
        slot = c.pool_slot[0].clone()
        slot[1, sel1[i_bad]] = -1
        _recall(c, mode, bufs, c.pool_hit[0], slot, kv.KVOFF_ENGINE_ZEROCOPY, want_stats=False)
        torch.cuda.synchronize()
        assert bufs.table[1, 0, i_bad].item() == -1
        with pytest.raises(kv.KvoffError) as e:  # good maps, but the earlier call's report
            _recall(c, mode, bufs, c.pool_hit[0], c.pool_slot[0], kv.KVOFF_ENGINE_ZEROCOPY, True)
        assert e.value.status == kv.KVOFF_ESTATE
        st = _recall(c, mode, bufs, c.pool_hit[0], c.pool_slot[0], kv.KVOFF_ENGINE_ZEROCOPY, True)
        torch.cuda.synchronize()
        P.check_recall(c, 0, mode, bufs, sl, with_pool_hits=True, stats=st)
        _decode(c, mode, bufs)
        P.check_attention(c, 0, mode, bufs, sl)
    finally:
        H.destroy(c)


@pytest.mark.parametrize("mode", [kv.KVOFF_SOLOHEAD, kv.KVOFF_HEADWISE])
def test_attention_skips_table_entries_outside_the_pool(mode):
    """Table entries at or past n_slots (headwise: slice index at or past
    n_slots * Hkv) are skipped like negative ones; n_slots < 1 is EINVAL."""
    s = synth.spec(2, B=2, ctx=3000, k=12, hot=5, headwise=True)
    H.log(f"[table outside the pool] mode {mode}")
    c, sl = _case(s)
    try:
        bufs = H.make_buffers(c, mode)
        H.run_layer(c, 0, mode, bufs)
        torch.cuda.synchronize()
        hw = P.per_head(mode)
        edge = c.n_slots * (s.Hkv if hw else 1)
        dropped = {(0, 0, 3): edge, (1, (s.Hkv - 1) if hw else 0, 0): edge + 1000}
        for (r, g, i), v in dropped.items():
            bufs.table[r, g, i] = v
        _decode(c, mode, bufs)
        if hw:  # per-head sets of unequal length: compare head group by head group
            got = bufs.out.cpu().numpy()
            for r in range(c.B):
                x = sl[(0, r)]
                for g in range(s.Hkv):
                    keep = np.array([b for i, b in enumerate(x.sel_g[g].tolist())
                                     if (r, g, i) not in dropped], np.int32)
                    Kg = np.ascontiguousarray(x.lr.K[:, g:g + 1])
                    Vg = np.ascontiguousarray(x.lr.V[:, g:g + 1])
                    qg = x.lr.q[g * s.G:(g + 1) * s.G]
                    P.check_attention_close(got[r, g * s.G:(g + 1) * s.G],
                                            oracle.attend_f32(qg, Kg, Vg, s.dtype, s.bs, keep),
                                            f"request {r} KV head {g}")
        else:
            P.check_attention_close(bufs.out.cpu().numpy(), _oracle_without(c, sl, set(dropped)),
                                    "entries past the pool dropped")
        with pytest.raises(kv.KvoffError) as e:
            _decode(c, mode, bufs, n_slots=0)
        assert e.value.status == kv.KVOFF_EINVAL
    finally:
        H.destroy(c)


def _wide_keys(rng, ctx, Hkv, d, bs):
    """bf16 key bits: random signs, exponents in [-60, 60] (120 binades);
    in every other (KV head, dim) column each full block opens with a value
    near 2^60 whose exact negation sits half a block later, all its other
    values near 1 (the last, ragged block takes random values).  A sequential
    sum loses the values between the two big ones; summing the row pairs
    (t, t + bs/2) first keeps them."""
    n = ctx * Hkv * d
    mant = rng.integers(0, 128, n, dtype=np.uint32)
    expo = rng.integers(-60, 61, n).astype(np.uint32) + 127
    sign = rng.integers(0, 2, n, dtype=np.uint32)
    K = ((sign << 15) | (expo << 7) | mant).astype(np.uint16).reshape(ctx, Hkv, d)
    h = bs // 2
    for b in range(ctx // bs):
        t0 = b * bs
        small = rng.integers(0, 128, (bs, Hkv, d // 2), dtype=np.uint32) | \
            ((rng.integers(-4, 5, (bs, Hkv, d // 2)) + 127).astype(np.uint32) << 7) | \
            (rng.integers(0, 2, (bs, Hkv, d // 2), dtype=np.uint32) << 15)
        big = (rng.integers(0, 128, (Hkv, d // 2), dtype=np.uint32) | (np.uint32(127 + 60) << 7))
        K[t0:t0 + bs, :, 0::2] = small.astype(np.uint16)
        K[t0, :, 0::2] = big.astype(np.uint16)
        K[t0 + h, :, 0::2] = (big | np.uint32(1 << 15)).astype(np.uint16)
    return K


@pytest.mark.parametrize("bs", [16, 32])
def test_digests_of_keys_spanning_many_binades(bs):
    """bf16 keys spanning 120 binades with a ragged last block: the order of
    an fp64 sum decides many digests' bits here, and the GPU digests must
    equal the oracle's sequential sums."""
    rng = np.random.default_rng(7000 + bs)
    Hkv, d, ctx = 2, 128, 20 * bs + 7
    K = _wide_keys(rng, ctx, Hkv, d, bs)
    V = rng.integers(0, 1 << 16, K.size, dtype=np.uint32).astype(np.uint16).reshape(K.shape)
    V &= np.uint16(0xBFFF)  # finite values only (exponent field below all ones)
    want = oracle.digest(K, synth.BF16, bs)
    # the input has teeth: summing the row pairs (t, t + bs/2) first changes
    # the bits of many digests
    vals = synth.decode(K, synth.BF16)
    nb = -(-ctx // bs)
    tree = np.empty_like(want)
    for b in range(nb):
        rows = vals[b * bs:min((b + 1) * bs, ctx)]
        h = bs // 2
        acc = np.zeros((Hkv, d))
        for t in range(min(h, len(rows))):
            acc = acc + (rows[t] + rows[t + h] if t + h < len(rows) else rows[t])
        tree[b] = (acc / len(rows)).astype(np.float32)
    n_diff = int(np.count_nonzero(tree.view(np.uint32) != want.view(np.uint32)))
    H.log(f"[wide digests] bs {bs}: a pairwise order changes {n_diff} of {want.size} digests")
    assert n_diff > want.size // 8
    ctx_h = kv.kvoff_create(num_layers=1, num_q_heads=2 * Hkv, num_kv_heads=Hkv, head_dim=d,
                            block_size=bs, dtype=kv.KVOFF_BF16, max_requests=1,
                            host_capacity_blocks=nb)
    try:
        rid = kv.kvoff_register_request(ctx_h, ctx)
        dig = torch.empty((nb, Hkv, d), dtype=torch.float32, device="cuda")
        kv.kvoff_offload_blocks(ctx_h, 0, rid, H.to_dev(K), H.to_dev(V), dig)
        torch.cuda.synchronize()
        got = dig.cpu().numpy()
        diff = np.argwhere(got.view(np.uint32) != want.view(np.uint32))
        assert diff.size == 0, f"digest bits differ at {diff[:5]}"
        # the records are the input bits, rows past the context zero
        rec = oracle.records(K, V, bs)
        for b in (0, nb - 1):
            addr = kv.kvoff_host_record(ctx_h, 0, rid, b)
            buf = np.empty(rec[b].size, np.uint16)
            ctypes.memmove(buf.ctypes.data, addr, buf.nbytes)
            assert np.array_equal(buf, rec[b].reshape(-1)), b
    finally:
        kv.kvoff_destroy(ctx_h)


def _vm(field="VmSize"):
    """A field of /proc/self/status in bytes.  Pinned host memory from
    hipHostMalloc is mapped into the process's address space (VmSize) but
    not counted as resident (VmRSS)."""
    with open("/proc/self/status") as f:
        for line in f:
            if line.startswith(field + ":"):
                return int(line.split()[1]) * 1024
    return -1


def _vm_all():
    return {k: _vm(k) >> 20 for k in ("VmSize", "VmRSS", "VmLck", "VmPin")}


def test_allocation_failures_are_reported_and_leak_nothing(monkeypatch):
    """Allocation failures forced through KVOFF_TEST_FAIL_ALLOC:
    - the pinned store of kvoff_create: KVOFF_ENOMEM;
    - the device request table, after a 1 GiB store was allocated: KVOFF_EHIP,
      with the store freed (the process's resident memory does not keep it,
      while a context that succeeds does hold it);
    - the staged engine's staging buffer: KVOFF_ENOMEM with nothing enqueued,
      and the next staged recall on the context is whole and correct."""
    cfg = dict(num_layers=1, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
               dtype=kv.KVOFF_F16, max_requests=4, host_capacity_blocks=(1 << 30) // 16384)
    monkeypatch.setenv("KVOFF_TEST_FAIL_ALLOC", "store")
    with pytest.raises(kv.KvoffError) as e:
        kv.kvoff_create(**cfg)
    assert e.value.status == kv.KVOFF_ENOMEM, e.value
    vm0, all0 = _vm(), _vm_all()
    monkeypatch.setenv("KVOFF_TEST_FAIL_ALLOC", "table")
    for _ in range(3):
        with pytest.raises(kv.KvoffError) as e:
            kv.kvoff_create(**cfg)
        assert e.value.status == kv.KVOFF_EHIP, e.value
    monkeypatch.delenv("KVOFF_TEST_FAIL_ALLOC")
    vm1, all1 = _vm(), _vm_all()
    ctx = kv.kvoff_create(**cfg)
    vm2, all2 = _vm(), _vm_all()
    kv.kvoff_destroy(ctx)
    vm3, all3 = _vm(), _vm_all()
    H.log(f"[alloc failures] MiB: start {all0}, after 3 failed creates {all1}, with a 1 GiB "
          f"store {all2}, after destroying it {all3}")
    assert vm2 - vm1 > (768 << 20), "a held store shows in the mapped address space"
    assert vm1 - vm0 < (256 << 20), "failed creates kept their stores"
    assert vm3 - vm1 < (256 << 20)

    s = synth.spec(2, B=2, ctx=4000, k=24, hot=6)
    c, sl = _case(s)
    try:
        mode = kv.KVOFF_SOLOHEAD
        bufs = H.make_buffers(c, mode)
        _select(c, mode, bufs)
        bufs.table.fill_(-7)
        monkeypatch.setenv("KVOFF_TEST_FAIL_ALLOC", "staging")
        with pytest.raises(kv.KvoffError) as e:
            _recall(c, mode, bufs, None, None, kv.KVOFF_ENGINE_STAGED, want_stats=False)
        assert e.value.status == kv.KVOFF_ENOMEM, e.value
        torch.cuda.synchronize()
        assert bool((bufs.table == -7).all()), "a failed staged recall enqueued its table upload"
        monkeypatch.delenv("KVOFF_TEST_FAIL_ALLOC")
        st = _recall(c, mode, bufs, None, None, kv.KVOFF_ENGINE_STAGED, want_stats=True)
        torch.cuda.synchronize()
        P.check_recall(c, 0, mode, bufs, sl, stats=st, engine=kv.KVOFF_ENGINE_STAGED)
        _decode(c, mode, bufs)
        P.check_attention(c, 0, mode, bufs, sl)
    finally:
        H.destroy(c)
