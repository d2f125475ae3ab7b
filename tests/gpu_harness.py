"""Drives the C ABI on the GPU for tests, the smoke check and the benchmark.

Data movement and buffer bookkeeping only: every computation goes through the
``sparse_kv_cache_mean_amd`` binding into libkvoff.so.  This module does not
import the oracle.
"""
from __future__ import annotations

import ctypes
import math
import sys
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

import sparse_kv_cache_mean_amd as kv
import synth


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    """uint16 bits -> int16 device tensor (same bytes)."""
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@dataclass
class Case:
    """One context with a batch of requests offloaded for a set of layers."""
    s: synth.Spec
    layers: list
    reqs: list                     # synth.Request per batch position
    inputs: dict                   # (layer, r) -> synth.LayerRequest
    k_stride: int
    ctx: int = 0
    rids: list = field(default_factory=list)
    nb_max: int = 0
    digest: dict = field(default_factory=dict)   # layer -> [B][nb_max][Hkv][d] f32
    q: dict = field(default_factory=dict)        # layer -> [B][Hq][d] int16
    pool: Optional[torch.Tensor] = None
    n_slots: int = 0
    recall_base: tuple = (0, 0)
    resident_base: int = 0
    extra_base: int = 0            # first slot after the recall regions and pool hits
    pool_hit: dict = field(default_factory=dict)   # layer -> [B][nb_max] uint8
    pool_slot: dict = field(default_factory=dict)  # layer -> [B][nb_max] int32

    @property
    def B(self) -> int:
        return len(self.reqs)


def build_case(s: synth.Spec, inputs, layers, reqs, k_stride: Optional[int] = None,
               host_kind: int = kv.KVOFF_HOST_COHERENT, two_regions: bool = True,
               with_pool_hits: bool = False, n_layers_ctx: Optional[int] = None,
               stream=None, keep=None, extra_slots: int = 0) -> Case:
    """Create a context, register the batch, upload and offload every (layer, request).

    `inputs` is a dict (layer, r) -> synth.LayerRequest, or a function of
    (layer, r) returning one; with a function, only the slices for which
    keep(layer, r) is true are kept in Case.inputs after offloading."""
    layers = list(layers)
    if callable(inputs):
        get, inputs = inputs, {}
    else:
        get = inputs.__getitem__
    B = len(reqs)
    nb_max = max(rq.nb for rq in reqs)
    Kmax = max(min(rq.k, rq.nb) for rq in reqs)
    k_stride = k_stride or Kmax
    L_ctx = n_layers_ctx or (max(layers) + 1)
    cap = sum(rq.nb for rq in reqs) * L_ctx
    dt = kv.KVOFF_BF16 if s.dtype == synth.BF16 else kv.KVOFF_F16
    ctx = kv.kvoff_create(num_layers=L_ctx, num_q_heads=s.Hq, num_kv_heads=s.Hkv,
                          head_dim=s.d, block_size=s.bs, dtype=dt, max_requests=max(B, 1),
                          host_capacity_blocks=cap, host_mem_kind=host_kind)
    c = Case(s, layers, reqs, inputs, k_stride, ctx=ctx, nb_max=nb_max)
    c.rids = [kv.kvoff_register_request(ctx, rq.ctx) for rq in reqs]
    pools = {}
    for l in layers:
        c.digest[l] = torch.empty((B, nb_max, s.Hkv, s.d), dtype=torch.float32, device="cuda")
        qs = []
        for r in range(B):
            lr = get((l, r))
            qs.append(lr.q)
            pools[(l, r)] = lr.pool
            kd, vd = to_dev(lr.K), to_dev(lr.V)
            kv.kvoff_offload_blocks(ctx, l, c.rids[r], kd, vd, c.digest[l][r], stream=stream)
            torch.cuda.synchronize()
            del kd, vd
            if keep is None or keep(l, r):
                inputs[(l, r)] = lr
        c.q[l] = to_dev(np.stack(qs))
    c.inputs = inputs
    torch.cuda.synchronize()
    # slot pool: recall region(s) first, then the resident blocks of pool hits
    regions = 2 if two_regions else 1
    n_recall = B * k_stride
    c.recall_base = (0, n_recall if two_regions else 0)
    c.resident_base = regions * n_recall
    n_res = 0
    if with_pool_hits:
        for l in layers:
            for r in range(B):
                n_res += int(pools[(l, r)].sum())
    c.n_slots = regions * n_recall + n_res + extra_slots
    c.extra_base = regions * n_recall + n_res
    rec = kv.kvoff_record_bytes(ctx)
    c.pool = torch.zeros(c.n_slots * rec, dtype=torch.uint8, device="cuda")
    if with_pool_hits:
        nxt = c.resident_base
        for l in layers:
            hit = np.zeros((B, nb_max), np.uint8)
            slot = np.full((B, nb_max), -1, np.int32)
            for r in range(B):
                for b in np.flatnonzero(pools[(l, r)]):
                    hit[r, b] = 1
                    slot[r, b] = nxt
                    # the resident copy is the same record bytes as the store's
                    addr = kv.kvoff_host_record(ctx, l, c.rids[r], int(b))
                    buf = np.empty(rec, np.uint8)
                    ctypes.memmove(buf.ctypes.data, addr, rec)
                    c.pool[nxt * rec:(nxt + 1) * rec].copy_(torch.from_numpy(buf))
                    nxt += 1
            c.pool_hit[l] = torch.from_numpy(hit).cuda()
            c.pool_slot[l] = torch.from_numpy(slot).cuda()
    torch.cuda.synchronize()
    return c


@dataclass
class Buffers:
    scores: torch.Tensor
    sel_idx: torch.Tensor
    sel_cnt: torch.Tensor
    table: torch.Tensor
    out: torch.Tensor
    ws: Optional[torch.Tensor]


def make_buffers(c: Case, mode: int) -> Buffers:
    s, B = c.s, c.B
    sets = s.Hkv if mode in (kv.KVOFF_HEADWISE, kv.KVOFF_CONSENSUS_GROUP) else 1
    scores = torch.empty((B, sets, c.nb_max), dtype=torch.float64, device="cuda")
    sel_idx = torch.empty((B, sets, c.k_stride), dtype=torch.int32, device="cuda")
    sel_cnt = torch.empty((B,), dtype=torch.int32, device="cuda")
    table = torch.empty((B, sets, c.k_stride), dtype=torch.int32, device="cuda")
    out = torch.empty((B, s.Hq, s.d), dtype=torch.float32, device="cuda")
    wsb = kv.kvoff_workspace_size(c.ctx, kv.KVOFF_CALL_SPARSE_DECODE, B, c.k_stride, mode)
    ws = torch.empty((max(wsb, 1),), dtype=torch.uint8, device="cuda") if wsb else None
    return Buffers(scores, sel_idx, sel_cnt, table, out, ws)


def run_layer(c: Case, l: int, mode: int, bufs: Buffers, engine: int = kv.KVOFF_ENGINE_ZEROCOPY,
              region: int = 0, with_pool_hits: bool = False, want_stats: bool = False,
              stream=None):
    """select -> recall -> sparse decode for one layer on one stream."""
    topk = [rq.k for rq in c.reqs]
    kv.kvoff_select(c.ctx, l, c.rids, c.q[l], c.digest[l], c.nb_max, topk, mode, bufs.scores,
                    bufs.sel_idx, bufs.sel_cnt, c.k_stride, stream=stream)
    stats = kv.kvoff_recall(c.ctx, l, c.rids, mode, bufs.sel_idx, bufs.sel_cnt, c.k_stride,
                            c.pool_hit.get(l) if with_pool_hits else None,
                            c.pool_slot.get(l) if with_pool_hits else None, c.nb_max,
                            c.pool, c.n_slots, c.recall_base[region], bufs.table, engine,
                            want_stats=want_stats, stream=stream)
    kv.kvoff_sparse_decode(c.ctx, c.rids, mode, c.q[l], c.pool, c.n_slots, bufs.table, bufs.sel_idx,
                           bufs.sel_cnt, c.k_stride, 1.0 / math.sqrt(c.s.d), bufs.out, bufs.ws,
                           stream=stream)
    return stats


def destroy(c: Case) -> None:
    if c.ctx:
        kv.kvoff_destroy(c.ctx)
        c.ctx = 0
