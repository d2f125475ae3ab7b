"""Seeded synthetic workloads for the sparse KV-offloading hot path.

This package draws inputs only: query/key/value tensors, context lengths,
per-request top-k budgets, planted hot blocks and HBM-pool hit maps.  It holds
none of the method's arithmetic; both the CPU oracle's tests and the GPU path
consume what it produces.

Workload shapes follow the pages' setting (PulseInfer, aiFetchly guide,
"PulseInfer Architectural Foundations" and the simulator's ``PulseInferConfig``:
32 query / 8 KV heads, head_dim 128, a 64-block sparse budget; abstract:
"storing most historical KV blocks in CPU DRAM and recalling only selected
blocks"), scaled to five named workloads below.

Planting: in a hot block every token's key in every KV head g is shifted by
+0.5 * qhat_g before rounding, where qhat_g is the unit vector of the sum of
the (rounded) query heads of group g.  Context lengths for the variable-recall
workload are U{8192..131072}; its top-k fraction is U[0.02, 0.15].
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")

F16 = 1
BF16 = 2

TAG_Q, TAG_K, TAG_V, TAG_HOT, TAG_CTX, TAG_FRAC, TAG_RUNLEN, TAG_RUNPOS, TAG_POOL = range(1, 10)


def build(verbose: bool = False) -> str:
    """Compile libsynth.so with gcc (OpenMP for the bulk K/V fill)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
           os.path.join(_HERE, "synth.c"), "-o", LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        u64, u32, i64, i32, vp = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                   ctypes.c_int32, ctypes.c_void_p)
        dbl = ctypes.c_double
        L.synth_philox4x32_10.argtypes = [vp, vp, vp]
        L.synth_normals.argtypes = [u64, u32, u32, u32, u32, u64, i64, vp]
        L.synth_u32.argtypes = [u64, u32, u32, u32, u64]
        L.synth_u32.restype = u32
        L.synth_uniform_int.argtypes = [u64, u32, u32, u32, u64, i64, i64]
        L.synth_uniform_int.restype = i64
        L.synth_uniform01.argtypes = [u64, u32, u32, u32, u64]
        L.synth_uniform01.restype = dbl
        L.synth_quantize.argtypes = [dbl, ctypes.c_int]
        L.synth_quantize.restype = ctypes.c_uint16
        L.synth_q.argtypes = [u64, u32, u32, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
        L.synth_qhat.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
        L.synth_kv.argtypes = [u64, u32, u32, u32, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               vp, vp, vp, dbl, ctypes.c_int, vp]
        L.synth_kv_block.argtypes = [u64, u32, u32, u32, i64, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, i64, ctypes.c_int, ctypes.c_int, vp, dbl,
                                     ctypes.c_int, vp]
        L.synth_choose.argtypes = [u64, u32, u32, u32, i64, i64, vp]
        L.synth_runs.argtypes = [u64, u32, u32, i64, i64, ctypes.c_int, vp]
        L.synth_runs.restype = i64
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- raw draws

def philox(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, np.uint32)
    lib().synth_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def normals(seed, tag, layer, req, n, off=0, attempt=0) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().synth_normals(seed, tag, layer, req, attempt, off, n, _p(out))
    return out


def quantize(x: float, dtype: int) -> int:
    return int(lib().synth_quantize(float(x), dtype))


def uniform_int(seed, tag, layer, req, idx, lo, hi) -> int:
    return int(lib().synth_uniform_int(seed, tag, layer, req, idx, lo, hi))


def uniform01(seed, tag, layer, req, idx) -> float:
    return float(lib().synth_uniform01(seed, tag, layer, req, idx))


def choose(seed, tag, layer, req, nb, n) -> np.ndarray:
    out = np.empty(n, np.int32)
    lib().synth_choose(seed, tag, layer, req, nb, n, _p(out))
    return out


def runs_mask(seed, layer, req, nb, k, max_run=8) -> tuple[np.ndarray, int]:
    mask = np.zeros(nb, np.uint8)
    m = lib().synth_runs(seed, layer, req, nb, k, max_run, _p(mask))
    if m < 0:
        raise ValueError(f"cannot fit {k} hot blocks in runs into {nb} blocks")
    return mask, int(m)


def decode(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Storage bits (uint16) -> float64 values (exact widening)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


# ---------------------------------------------------------------- workloads

@dataclass(frozen=True)
class Spec:
    """Shape and draw recipe of one workload."""
    name: str
    B: int
    L: int
    Hq: int
    Hkv: int
    d: int
    bs: int
    dtype: int
    ctx: int = 0                       # fixed context length (tokens) ...
    ctx_range: tuple = ()              # ... or U{lo..hi} per request
    k: int = 0                         # fixed top-k (blocks) ...
    k_frac_range: tuple = ()           # ... or round-half-even(U[lo,hi] * nb), at least 1
    hot: int = 0                       # planted hot blocks per request (uniform positions) ...
    hot_runs: bool = False             # ... or k_r hot blocks in runs of U{1..max_run}
    max_run: int = 8
    pool_frac: float = 0.0             # fraction of blocks resident in the HBM pool
    headwise: bool = False             # compare per-KV-head selection with the shared set
    shift: float = 0.5
    seed: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def es(self) -> int:
        return 2

    @property
    def rec_bytes(self) -> int:
        """Bytes of one block record: K and V of every KV head."""
        return 2 * self.Hkv * self.bs * self.d * self.es


def _seed(number: int) -> int:
    return 1000 + number


# the five workloads, by number; each also has a name
WORKLOADS = {
    1: Spec("tiny", B=1, L=1, Hq=8, Hkv=2, d=128, bs=16, dtype=F16, ctx=4096, k=32, hot=32,
            seed=_seed(1)),
    2: Spec("llama3-8b-layer", B=16, L=1, Hq=32, Hkv=8, d=128, bs=32, dtype=BF16, ctx=32768,
            k=64, hot=51, seed=_seed(2)),
    3: Spec("llama3-8b-32layer", B=8, L=32, Hq=32, Hkv=8, d=128, bs=32, dtype=BF16, ctx=32768,
            k=64, hot=51, seed=_seed(3)),
    4: Spec("llama3-70b-variable", B=32, L=1, Hq=64, Hkv=8, d=128, bs=32, dtype=BF16,
            ctx_range=(8192, 131072), k_frac_range=(0.02, 0.15), hot_runs=True, seed=_seed(4)),
    5: Spec("headwise-vs-solohead", B=16, L=1, Hq=32, Hkv=8, d=128, bs=32, dtype=BF16,
            ctx=32768, k=64, hot=51, pool_frac=0.25, headwise=True, seed=_seed(5)),
}


def spec(workload, **overrides) -> Spec:
    """The workload by number (1-5) or name, with fields overridden."""
    if isinstance(workload, str):
        matches = [w for w in WORKLOADS.values() if w.name == workload]
        if not matches:
            raise KeyError(f"no workload named {workload!r}")
        return replace(matches[0], **overrides)
    return replace(WORKLOADS[workload], **overrides)


@dataclass
class Request:
    ctx: int
    nb: int
    k: int


def request_draws(s: Spec) -> list[Request]:
    """Context length and top-k of every request (layer independent)."""
    out = []
    for r in range(s.B):
        if s.ctx_range:
            ctx = uniform_int(s.seed, TAG_CTX, 0, r, 0, s.ctx_range[0], s.ctx_range[1])
        else:
            ctx = s.ctx
        nb = -(-ctx // s.bs)
        if s.k_frac_range:
            f = s.k_frac_range[0] + (s.k_frac_range[1] - s.k_frac_range[0]) * \
                uniform01(s.seed, TAG_FRAC, 0, r, 0)
            k = max(1, int(np.rint(f * nb)))  # numpy rint: half to even
        else:
            k = s.k
        out.append(Request(ctx=ctx, nb=nb, k=k))
    return out


def hot_mask(s: Spec, layer: int, req: int, rq: Request) -> np.ndarray:
    if s.hot_runs:
        m, _ = runs_mask(s.seed, layer, req, rq.nb, min(rq.k, rq.nb), s.max_run)
        return m
    mask = np.zeros(rq.nb, np.uint8)
    n = min(s.hot, rq.nb)
    if n:
        mask[choose(s.seed, TAG_HOT, layer, req, rq.nb, n)] = 1
    return mask


def pool_hits(s: Spec, layer: int, req: int, rq: Request) -> np.ndarray:
    """uint8 [nb]: 1 where the block is already resident in the HBM pool."""
    mask = np.zeros(rq.nb, np.uint8)
    n = int(np.floor(s.pool_frac * rq.nb))
    if n:
        mask[choose(s.seed, TAG_POOL, layer, req, rq.nb, n)] = 1
    return mask


def gen_q(s: Spec, layer: int, req: int) -> np.ndarray:
    out = np.empty((s.Hq, s.d), np.uint16)
    lib().synth_q(s.seed, layer, req, s.Hq, s.d, s.dtype, _p(out))
    return out


def gen_qhat(s: Spec, q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint16)
    out = np.empty((s.Hkv, s.d), np.float64)
    lib().synth_qhat(_p(q), s.dtype, s.Hq, s.Hkv, s.d, _p(out))
    return out


def gen_kv(s: Spec, tag: int, layer: int, req: int, n_tok: int,
           hot: Optional[np.ndarray] = None, attempts: Optional[np.ndarray] = None,
           qhat: Optional[np.ndarray] = None, out: Optional[np.ndarray] = None) -> np.ndarray:
    """K (tag TAG_K, planted where hot) or V (tag TAG_V) as [n_tok][Hkv][d] bits."""
    if out is None:
        out = np.empty((n_tok, s.Hkv, s.d), np.uint16)
    assert out.shape == (n_tok, s.Hkv, s.d) and out.dtype == np.uint16 and out.flags.c_contiguous
    if hot is not None:
        hot = np.ascontiguousarray(hot, dtype=np.uint8)
        assert qhat is not None
        qhat = np.ascontiguousarray(qhat, dtype=np.float64)
    if attempts is not None:
        attempts = np.ascontiguousarray(attempts, dtype=np.uint8)
    lib().synth_kv(s.seed, tag, layer, req, n_tok, s.Hkv, s.d, s.bs, _p(hot), _p(attempts),
                   _p(qhat), s.shift, s.dtype, _p(out))
    return out


def regen_block(s: Spec, tag: int, layer: int, req: int, n_tok: int, b: int, hot: bool,
                attempt: int, qhat: Optional[np.ndarray], out: np.ndarray) -> None:
    """Redraw the token rows of block b in place (used to re-draw a block)."""
    qp = None
    if hot:
        qhat = np.ascontiguousarray(qhat, dtype=np.float64)
        qp = _p(qhat)
    lib().synth_kv_block(s.seed, tag, layer, req, n_tok, s.Hkv, s.d, s.bs, b, int(hot),
                         int(attempt), qp, s.shift, s.dtype, _p(out))


@dataclass
class LayerRequest:
    """All inputs of one (layer, request) slice."""
    layer: int
    req: int
    rq: Request
    q: np.ndarray          # [Hq][d] uint16 bits
    qhat: np.ndarray       # [Hkv][d] float64
    hot: np.ndarray        # [nb] uint8
    attempts: np.ndarray   # [nb] uint8 (per-block re-draw counters)
    K: np.ndarray          # [ctx][Hkv][d] uint16 bits
    V: np.ndarray          # [ctx][Hkv][d] uint16 bits
    pool: np.ndarray       # [nb] uint8


def gen_layer_request(s: Spec, layer: int, req: int, rq: Request,
                      attempts: Optional[np.ndarray] = None) -> LayerRequest:
    q = gen_q(s, layer, req)
    qhat = gen_qhat(s, q)
    hot = hot_mask(s, layer, req, rq)
    if attempts is None:
        attempts = np.zeros(rq.nb, np.uint8)
    K = gen_kv(s, TAG_K, layer, req, rq.ctx, hot=hot, attempts=attempts, qhat=qhat)
    V = gen_kv(s, TAG_V, layer, req, rq.ctx)
    return LayerRequest(layer, req, rq, q, qhat, hot, attempts, K, V, pool_hits(s, layer, req, rq))
