"""Seeded workloads conditioned for bit-exact selection checks.

``synth`` draws the inputs; this module (test infrastructure, so it may use
the oracle) enforces the minimum top-k score gap: for every ranking that a
test compares (the shared SoloHead ranking, plus each per-KV-head ranking
when the workload is headwise), the score at rank K must exceed the score at
rank K+1 by at least ``min_gap``.  A violating ranking has the keys of its
rank-(K+1) block re-drawn with the next attempt number of that block's
Philox stream, up to 64 times.  Scores here are the oracle's fp64 scores.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

import oracle
import synth

MIN_GAP = 1e-3
MAX_ATTEMPTS = 64


@dataclass
class Slice:
    """One (layer, request): generated inputs plus the oracle's view of them."""
    s: synth.Spec
    lr: synth.LayerRequest
    D: np.ndarray                 # [nb][Hkv][d] float32 digests
    S: np.ndarray                 # [nb] float64 SoloHead scores
    Sg: Optional[np.ndarray]      # [Hkv][nb] float64 per-KV-head scores
    sel: np.ndarray               # [K] ascending SoloHead selection
    sel_g: Optional[np.ndarray]   # [Hkv][K] ascending per-KV-head selections
    gap: float                    # smallest boundary gap over compared rankings
    redraws: int
    Sc: Optional[np.ndarray] = None    # [nb] consensus scores (when lam is given)
    sel_c: Optional[np.ndarray] = None  # [K] consensus selection
    lam: Optional[float] = None
    Sgc: Optional[np.ndarray] = None    # [Hkv][nb] GQA-group consensus scores (group_lam)
    sel_gc: Optional[np.ndarray] = None  # [Hkv][K] GQA-group consensus selections

    @property
    def K(self) -> int:
        return int(self.sel.shape[0])


def boundary(S: np.ndarray, K: int):
    """(gap between rank K and K+1, block id at rank K+1); inf/None if K >= nb."""
    nb = S.shape[0]
    if K >= nb:
        return float("inf"), None
    order = np.lexsort((np.arange(nb), -S))  # score desc, id asc
    return float(S[order[K - 1]] - S[order[K]]), int(order[K])


def condition(s: synth.Spec, lr: synth.LayerRequest, min_gap: float = MIN_GAP,
              headwise: Optional[bool] = None, enforce: bool = True,
              lam: Optional[float] = None, group_lam: Optional[float] = None) -> Slice:
    """lam: also condition and select the consensus ranking with that lambda;
    group_lam: also the per-KV-head GQA-group consensus rankings."""
    headwise = s.headwise if headwise is None else headwise
    rq = lr.rq
    K = min(rq.k, rq.nb)
    D = oracle.digest(lr.K, s.dtype, s.bs)
    redraws = 0
    while True:
        S = oracle.score(lr.q, s.dtype, D)
        Sg = oracle.score_headwise(lr.q, s.dtype, D) if headwise else None
        Sc = oracle.score_consensus(lr.q, s.dtype, D, lam) if lam is not None else None
        Sgc = (oracle.score_group_consensus(lr.q, s.dtype, D, group_lam)
               if group_lam is not None else None)
        rankings = [S] + ([Sg[g] for g in range(s.Hkv)] if headwise else []) + \
            ([Sc] if Sc is not None else []) + \
            ([Sgc[g] for g in range(s.Hkv)] if Sgc is not None else [])
        worst, bad = float("inf"), None
        for R in rankings:
            gap, b = boundary(R, K)
            worst = min(worst, gap)
            if enforce and gap < min_gap and bad is None:
                bad = b
        if bad is None:
            break
        lr.attempts[bad] += 1
        if lr.attempts[bad] >= MAX_ATTEMPTS:
            raise RuntimeError(f"gap enforcement failed for block {bad} of "
                               f"(layer {lr.layer}, request {lr.req})")
        redraws += 1
        synth.regen_block(s, synth.TAG_K, lr.layer, lr.req, rq.ctx, bad, bool(lr.hot[bad]),
                          int(lr.attempts[bad]), lr.qhat, lr.K)
        t0, t1 = bad * s.bs, min((bad + 1) * s.bs, rq.ctx)
        D[bad] = oracle.digest(lr.K[t0:t1], s.dtype, s.bs)[0]
    sel = oracle.select(S, rq.k)
    sel_g = np.stack([oracle.select(Sg[g], rq.k) for g in range(s.Hkv)]) if headwise else None
    sel_c = oracle.select(Sc, rq.k) if Sc is not None else None
    sel_gc = (np.stack([oracle.select(Sgc[g], rq.k) for g in range(s.Hkv)])
              if Sgc is not None else None)
    return Slice(s, lr, D, S, Sg, sel, sel_g, worst, redraws, Sc, sel_c, lam, Sgc, sel_gc)


def make_slice(s: synth.Spec, layer: int, req: int, rq: Optional[synth.Request] = None,
               enforce: bool = True, lam: Optional[float] = None,
               group_lam: Optional[float] = None) -> Slice:
    if rq is None:
        rq = synth.request_draws(s)[req]
    lr = synth.gen_layer_request(s, layer, req, rq)
    return condition(s, lr, enforce=enforce, lam=lam, group_lam=group_lam)


def block_records(sl: Slice, blocks) -> np.ndarray:
    """Oracle block records of the given block ids: [n][Hkv][2][bs][d] bits."""
    s, lr = sl.s, sl.lr
    out = np.empty((len(blocks), s.Hkv, 2, s.bs, s.d), np.uint16)
    for i, b in enumerate(blocks):
        t0, t1 = b * s.bs, min((b + 1) * s.bs, lr.rq.ctx)
        out[i] = oracle.records(lr.K[t0:t1], lr.V[t0:t1], s.bs)[0]
    return out
