"""Python binding of the plain CPU oracle (TEST INFRASTRUCTURE).

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  It marshals numpy arrays into
``libkvoff_oracle.so`` (plain single-threaded C, built with gcc) and does no
arithmetic of its own.  See ``kvoff_oracle.h`` for the rule each call follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvoff_oracle.so")

F16 = 1
BF16 = 2


def build(verbose: bool = False) -> str:
    """Compile the oracle (no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", os.path.join(_HERE, "kvoff_oracle.c"), "-o", LIB_PATH + ".tmp", "-lm"]
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
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.oracle_widen.argtypes = [ctypes.c_uint16, ci]
        L.oracle_widen.restype = ctypes.c_double
        L.oracle_kv_cache_bytes.argtypes = [i64] * 5
        L.oracle_kv_cache_bytes.restype = i64
        L.oracle_rec_bytes.argtypes = [i64] * 4
        L.oracle_rec_bytes.restype = i64
        L.oracle_digest.argtypes = [vp, ci, i64, ci, ci, ci, vp]
        L.oracle_score.argtypes = [vp, ci, ci, ci, ci, vp, i64, vp]
        L.oracle_score_headwise.argtypes = [vp, ci, ci, ci, ci, vp, i64, vp]
        L.oracle_score_consensus.argtypes = [vp, ci, ci, ci, ci, vp, i64, ctypes.c_double, vp]
        L.oracle_score_group_consensus.argtypes = [vp, ci, ci, ci, ci, vp, i64, ctypes.c_double,
                                                    vp]
        L.oracle_attention_mass.argtypes = [vp, vp, ci, i64, ci, ci, ci, ci, vp, vp, ci, i64, vp]
        L.oracle_select.argtypes = [vp, i64, i64, vp]
        L.oracle_select.restype = i64
        L.oracle_records.argtypes = [vp, vp, i64, ci, ci, ci, vp]
        L.oracle_runs.argtypes = [vp, i64, vp, vp, vp]
        L.oracle_runs.restype = i64
        L.oracle_headwise_transfers.argtypes = [vp, vp, ci, i64, vp]
        L.oracle_headwise_transfers.restype = i64
        L.oracle_union_count.argtypes = [vp, vp, ci, i64]
        L.oracle_union_count.restype = i64
        L.oracle_attend_f32.argtypes = [vp, vp, vp, ci, i64, ci, ci, ci, ci, vp, i64, vp]
        L.oracle_attend_f64.argtypes = [vp, vp, vp, ci, i64, ci, ci, ci, ci, vp, i64, vp, vp]
        L.oracle_attend_headwise_f32.argtypes = [vp, vp, vp, ci, i64, ci, ci, ci, ci, vp, i64,
                                                 i64, vp]
        L.oracle_dense_f64.argtypes = [vp, vp, vp, ci, i64, ci, ci, ci, vp]
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a):
    return np.ascontiguousarray(a, dtype=np.uint16)


def widen(bits: int, dtype: int) -> float:
    return float(lib().oracle_widen(bits, dtype))


def kv_cache_bytes(L, Hkv, d, S, es) -> int:
    return int(lib().oracle_kv_cache_bytes(L, Hkv, d, S, es))


def rec_bytes(Hkv, bs, d, es) -> int:
    return int(lib().oracle_rec_bytes(Hkv, bs, d, es))


def digest(K: np.ndarray, dtype: int, bs: int) -> np.ndarray:
    """K [ctx][Hkv][d] bits -> D [nb][Hkv][d] float32."""
    K = _u16(K)
    ctx, Hkv, d = K.shape
    nb = -(-ctx // bs)
    D = np.empty((nb, Hkv, d), np.float32)
    lib().oracle_digest(_p(K), dtype, ctx, Hkv, d, bs, _p(D))
    return D


def score(q: np.ndarray, dtype: int, D: np.ndarray) -> np.ndarray:
    q = _u16(q)
    D = np.ascontiguousarray(D, dtype=np.float32)
    Hq, d = q.shape
    nb, Hkv, _ = D.shape
    S = np.empty(nb, np.float64)
    lib().oracle_score(_p(q), dtype, Hq, Hkv, d, _p(D), nb, _p(S))
    return S


def score_headwise(q: np.ndarray, dtype: int, D: np.ndarray) -> np.ndarray:
    q = _u16(q)
    D = np.ascontiguousarray(D, dtype=np.float32)
    Hq, d = q.shape
    nb, Hkv, _ = D.shape
    S = np.empty((Hkv, nb), np.float64)
    lib().oracle_score_headwise(_p(q), dtype, Hq, Hkv, d, _p(D), nb, _p(S))
    return S


def score_consensus(q: np.ndarray, dtype: int, D: np.ndarray, lam: float) -> np.ndarray:
    q = _u16(q)
    D = np.ascontiguousarray(D, dtype=np.float32)
    Hq, d = q.shape
    nb, Hkv, _ = D.shape
    S = np.empty(nb, np.float64)
    lib().oracle_score_consensus(_p(q), dtype, Hq, Hkv, d, _p(D), nb, lam, _p(S))
    return S


def score_group_consensus(q: np.ndarray, dtype: int, D: np.ndarray, lam: float) -> np.ndarray:
    """-> [Hkv][nb] per-GQA-group consensus scores."""
    q = _u16(q)
    D = np.ascontiguousarray(D, dtype=np.float32)
    Hq, d = q.shape
    nb, Hkv, _ = D.shape
    S = np.empty((Hkv, nb), np.float64)
    lib().oracle_score_group_consensus(_p(q), dtype, Hq, Hkv, d, _p(D), nb, lam, _p(S))
    return S


def attention_mass(q, K, dtype: int, bs: int, sel, counts=None) -> np.ndarray:
    """sel: [K] shared by every head, or [Hkv][stride] per KV head (counts
    entries each; default: the full rows).  -> mass [Hq] float64."""
    q, K = _u16(q), _u16(K)
    Hq, d = q.shape
    ctx, Hkv, _ = K.shape
    s = np.ascontiguousarray(sel, dtype=np.int32)
    if s.ndim == 1:
        s = s[None, :]
    nsets, stride = s.shape
    c = np.full(nsets, stride, np.int64) if counts is None else np.ascontiguousarray(counts, np.int64)
    out = np.empty(Hq, np.float64)
    lib().oracle_attention_mass(_p(q), _p(K), dtype, ctx, Hq, Hkv, d, bs, _p(s), _p(c), nsets,
                                stride, _p(out))
    return out


def select(S: np.ndarray, k: int) -> np.ndarray:
    S = np.ascontiguousarray(S, dtype=np.float64)
    nb = S.shape[0]
    sel = np.empty(max(min(k, nb), 1), np.int32)
    n = lib().oracle_select(_p(S), nb, k, _p(sel))
    if n < 0:
        raise ValueError("k must be at least 1")
    return sel[:n].copy()


def records(K: np.ndarray, V: np.ndarray, bs: int) -> np.ndarray:
    K, V = _u16(K), _u16(V)
    ctx, Hkv, d = K.shape
    nb = -(-ctx // bs)
    rec = np.empty((nb, Hkv, 2, bs, d), np.uint16)
    lib().oracle_records(_p(K), _p(V), ctx, Hkv, d, bs, _p(rec))
    return rec


def runs(sel: np.ndarray, hit: Optional[np.ndarray] = None):
    """-> (first_rank[n], length[n]) of the coalesced transfers."""
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    K = sel.shape[0]
    first = np.empty(max(K, 1), np.int32)
    ln = np.empty(max(K, 1), np.int32)
    h = None if hit is None else np.ascontiguousarray(hit, dtype=np.uint8)
    n = lib().oracle_runs(_p(sel), K, _p(h), _p(first), _p(ln))
    return first[:n].copy(), ln[:n].copy()


def headwise_transfers(sel: np.ndarray, counts, hit: Optional[np.ndarray] = None) -> int:
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    nsets, stride = sel.shape
    c = np.ascontiguousarray(counts, dtype=np.int64)
    h = None if hit is None else np.ascontiguousarray(hit, dtype=np.uint8)
    return int(lib().oracle_headwise_transfers(_p(sel), _p(c), nsets, stride, _p(h)))


def union_count(sel: np.ndarray, counts) -> int:
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    nsets, stride = sel.shape
    c = np.ascontiguousarray(counts, dtype=np.int64)
    return int(lib().oracle_union_count(_p(sel), _p(c), nsets, stride))


def attend_f32(q, K, V, dtype: int, bs: int, sel: Optional[np.ndarray]) -> np.ndarray:
    q, K, V = _u16(q), _u16(K), _u16(V)
    Hq, d = q.shape
    ctx, Hkv, _ = K.shape
    out = np.empty((Hq, d), np.float32)
    s = None if sel is None else np.ascontiguousarray(sel, dtype=np.int32)
    lib().oracle_attend_f32(_p(q), _p(K), _p(V), dtype, ctx, Hq, Hkv, d, bs, _p(s),
                            0 if s is None else s.shape[0], _p(out))
    return out


def attend_f64(q, K, V, dtype: int, bs: int, sel: Optional[np.ndarray], want_wsum=False):
    q, K, V = _u16(q), _u16(K), _u16(V)
    Hq, d = q.shape
    ctx, Hkv, _ = K.shape
    out = np.empty((Hq, d), np.float64)
    ws = np.empty(Hq, np.float64) if want_wsum else None
    s = None if sel is None else np.ascontiguousarray(sel, dtype=np.int32)
    lib().oracle_attend_f64(_p(q), _p(K), _p(V), dtype, ctx, Hq, Hkv, d, bs, _p(s),
                            0 if s is None else s.shape[0], _p(out), _p(ws))
    return (out, ws) if want_wsum else out


def attend_headwise_f32(q, K, V, dtype: int, bs: int, sel: np.ndarray) -> np.ndarray:
    """sel [Hkv][K] (same count per KV head)."""
    q, K, V = _u16(q), _u16(K), _u16(V)
    Hq, d = q.shape
    ctx, Hkv, _ = K.shape
    s = np.ascontiguousarray(sel, dtype=np.int32)
    out = np.empty((Hq, d), np.float32)
    lib().oracle_attend_headwise_f32(_p(q), _p(K), _p(V), dtype, ctx, Hq, Hkv, d, bs, _p(s),
                                     s.shape[1], s.shape[1], _p(out))
    return out


def dense_f64(q, K, V, dtype: int) -> np.ndarray:
    q, K, V = _u16(q), _u16(K), _u16(V)
    Hq, d = q.shape
    ctx, Hkv, _ = K.shape
    out = np.empty((Hq, d), np.float64)
    lib().oracle_dense_f64(_p(q), _p(K), _p(V), dtype, ctx, Hq, Hkv, d, _p(out))
    return out
