"""Parity checks of the GPU path against the oracle (shared by the GPU tests
and the smoke check).

Bars:
  digests            bit-exact (fp32 bits)
  scores             |gpu - oracle| <= 1e-9 * (1 + |S|)   (both fp64)
  selection          bit-exact ids and counts; unused entries -1
  recalled records   bit-exact bytes; table entries point at the right slots
  transfer counts    equal to the oracle's coalesced-run / slice counts
  attention          max |gpu - oracle_fp32| <= 2e-3 and, per (request, head)
                     row, max|err| / max|oracle| <= 1e-2
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import sparse_kv_cache_mean_amd as kv
from tests import workloads

ATOL = 2e-3
ROW_RTOL = 1e-2


def check_digests(c, l, slices):
    D = c.digest[l].cpu().numpy()
    for r in range(c.B):
        sl = slices[(l, r)]
        nb = sl.lr.rq.nb
        got = D[r, :nb]
        assert np.array_equal(got.view(np.uint32), sl.D.view(np.uint32)), \
            f"digest mismatch layer {l} req {r}: {np.argwhere(got != sl.D)[:5]}"


def shared_set(sl, mode):
    """The one block set of a shared-set mode (SoloHead or consensus)."""
    return sl.sel_c if mode == kv.KVOFF_CONSENSUS else sl.sel


def per_head(mode) -> bool:
    """Modes with one block set per KV head (headwise layout)."""
    return mode in (kv.KVOFF_HEADWISE, kv.KVOFF_CONSENSUS_GROUP)


def head_sets(sl, mode):
    """[Hkv][K] block sets of a per-KV-head mode."""
    return sl.sel_gc if mode == kv.KVOFF_CONSENSUS_GROUP else sl.sel_g


def block_sets(sl, mode):
    return list(head_sets(sl, mode)) if per_head(mode) else [shared_set(sl, mode)]


def check_selection(c, l, mode, bufs, slices):
    sel = bufs.sel_idx.cpu().numpy()
    cnt = bufs.sel_cnt.cpu().numpy()
    sc = bufs.scores.cpu().numpy()
    for r in range(c.B):
        sl = slices[(l, r)]
        K, nb = sl.K, sl.lr.rq.nb
        assert cnt[r] == K, (l, r, cnt[r], K)
        if mode in (kv.KVOFF_SOLOHEAD, kv.KVOFF_CONSENSUS):
            S = sl.Sc if mode == kv.KVOFF_CONSENSUS else sl.S
            assert np.allclose(sc[r, 0, :nb], S, rtol=0, atol=1e-9 * (1 + np.abs(S).max()))
            assert sel[r, 0, :K].tolist() == shared_set(sl, mode).tolist(), (l, r)
            assert np.all(sel[r, 0, K:] == -1)
        else:
            Sh = sl.Sgc if mode == kv.KVOFF_CONSENSUS_GROUP else sl.Sg
            for g in range(c.s.Hkv):
                assert np.allclose(sc[r, g, :nb], Sh[g], rtol=0,
                                   atol=1e-9 * (1 + np.abs(Sh[g]).max()))
                assert sel[r, g, :K].tolist() == head_sets(sl, mode)[g].tolist(), (l, r, g)
                assert np.all(sel[r, g, K:] == -1)


def expected_transfers(c, l, mode, slices, with_pool_hits):
    n_tr = n_items = n_hits = n_sel = 0
    for r in range(c.B):
        sl = slices[(l, r)]
        hit = sl.lr.pool if with_pool_hits else None
        for s in block_sets(sl, mode):
            n_sel += len(s)
            miss = [b for b in s.tolist() if not (hit is not None and hit[b])]
            n_items += len(miss)
            n_hits += len(s) - len(miss)
            if not per_head(mode):
                n_tr += len(oracle.runs(s, hit)[0])
            else:
                n_tr += oracle.headwise_transfers(s[None, :], [len(s)], hit)
    return dict(selected=n_sel, pool_hits=n_hits, items_recalled=n_items, transfers=n_tr)


def staged_copies(total_bytes: int) -> int:
    """Bulk copies the staged engine issues for total_bytes of staging: one
    of 1 MiB, one of 3 MiB, then one per 16 MiB (the last one partial)."""
    if total_bytes <= 0:
        return 0
    if total_bytes <= 1 << 20:
        return 1
    if total_bytes <= 4 << 20:
        return 2
    return 2 + -(-(total_bytes - (4 << 20)) // (16 << 20))


def check_recall(c, l, mode, bufs, slices, with_pool_hits=False, region=0, stats=None,
                 engine=kv.KVOFF_ENGINE_ZEROCOPY):
    """Recalled bytes and table entries.  Placement: the zero-copy and DMA
    engines put rank i of request r at slot base + r*k_stride + i; the staged
    engine puts the n-th recalled item of the call at slot base + n (slice
    base*Hkv + n when headwise).  Resident blocks point at their pool slot."""
    s = c.s
    compact = engine == kv.KVOFF_ENGINE_STAGED
    rec = kv.kvoff_record_bytes(c.ctx)
    slice_b = rec // s.Hkv
    pool = c.pool.cpu().numpy()
    table = bufs.table.cpu().numpy()
    base = c.recall_base[region]
    ps = c.pool_slot[l].cpu().numpy() if with_pool_hits else None
    n_item = 0
    for r in range(c.B):
        sl = slices[(l, r)]
        K = sl.K
        hit = sl.lr.pool if with_pool_hits else np.zeros(sl.lr.rq.nb, np.uint8)
        for g, sset in enumerate(block_sets(sl, mode)):
            want = workloads.block_records(sl, sset.tolist())  # [K][Hkv][2][bs][d]
            for i, b in enumerate(sset.tolist()):
                ent = int(table[r, g, i])
                hw = per_head(mode)
                if hit[b]:
                    exp = int(ps[r, b]) * (s.Hkv if hw else 1) + (g if hw else 0)
                elif compact:
                    exp = base * (s.Hkv if hw else 1) + n_item
                    n_item += 1
                else:
                    exp = (base + r * c.k_stride + i) * (s.Hkv if hw else 1) + (g if hw else 0)
                assert ent == exp, (l, r, g, i, ent, exp)
                if not hw:
                    got = pool[ent * rec:(ent + 1) * rec]
                    assert np.array_equal(got, want[i].reshape(-1).view(np.uint8)), (l, r, i, b)
                else:
                    got = pool[ent * slice_b:(ent + 1) * slice_b]
                    assert np.array_equal(got, want[i, g].reshape(-1).view(np.uint8)), (l, r, g, i)
            assert np.all(table[r, g, K:] == -1)
    if stats is not None:
        exp = expected_transfers(c, l, mode, slices, with_pool_hits)
        item = slice_b if per_head(mode) else rec
        if compact:  # bulk copies of the staging buffer
            exp["transfers"] = staged_copies(exp["items_recalled"] * item)
        for k, v in exp.items():
            assert stats[k] == v, (k, stats[k], v)
        assert stats["bytes"] == exp["items_recalled"] * item


def oracle_attention_one(s, sl, mode):
    """The oracle's fp32 attention of one (layer, request) slice, [Hq][d]."""
    lr = sl.lr
    if per_head(mode):
        return oracle.attend_headwise_f32(lr.q, lr.K, lr.V, s.dtype, s.bs, head_sets(sl, mode))
    return oracle.attend_f32(lr.q, lr.K, lr.V, s.dtype, s.bs, shared_set(sl, mode))


def oracle_attention(c, l, mode, slices):
    """The oracle's attention of every request of layer l, [B][Hq][d]: one
    oracle call per request, run on a pool of threads (the calls share no
    state and release the interpreter lock), each writing its own row."""
    s = c.s
    out = np.empty((c.B, s.Hq, s.d), np.float32)

    def one(r):
        out[r] = oracle_attention_one(s, slices[(l, r)], mode)

    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        list(ex.map(one, range(c.B)))
    return out


def check_attention_close(got: np.ndarray, ref: np.ndarray, what=""):
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    assert np.isfinite(got).all(), f"non-finite attention output {what}"
    mx = float(err.max())
    rows = err.reshape(-1, ref.shape[-1]).max(axis=1) / \
        np.maximum(np.abs(ref).reshape(-1, ref.shape[-1]).max(axis=1), 1e-30)
    assert mx <= ATOL, f"max abs error {mx} > {ATOL} {what}"
    assert float(rows.max()) <= ROW_RTOL, f"row relative error {rows.max()} > {ROW_RTOL} {what}"
    return mx, float(rows.max())


def check_attention(c, l, mode, bufs, slices, ref=None):
    if ref is None:
        ref = oracle_attention(c, l, mode, slices)
    got = bufs.out.cpu().numpy()
    return check_attention_close(got, ref, f"(layer {l})")
