"""Python binding of libkvoff.so, the MI355X sparse KV-cache offloading hot path.

Argument marshalling only: every function below has the name of the C entry
point it calls (``include/kvoff.h``), turns torch tensors into device
pointers and raises ``KvoffError`` on a negative status.  All computation
runs in the HIP kernels of the library; there is no fallback path.  If the
library is not built, importing this package raises.

torch is imported first so that the library binds to the HIP runtime torch
already loaded (same SONAME), which lets the two share streams and memory.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch  # noqa: F401  (loads the HIP runtime before libkvoff.so)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvoff.so")

KVOFF_OK = 0
KVOFF_EINVAL, KVOFF_ENOMEM, KVOFF_ENODEV, KVOFF_EHIP, KVOFF_ERANGE, KVOFF_ESTATE = range(-1, -7, -1)
KVOFF_F16, KVOFF_BF16 = 1, 2
KVOFF_SOLOHEAD, KVOFF_HEADWISE, KVOFF_CONSENSUS, KVOFF_CONSENSUS_GROUP = 0, 1, 2, 3
KVOFF_QK_MFMA, KVOFF_QK_VALU = 0, 1
KVOFF_ENGINE_ZEROCOPY, KVOFF_ENGINE_DMA, KVOFF_ENGINE_STAGED = 0, 1, 2
KVOFF_HOST_COHERENT, KVOFF_HOST_NONCOHERENT = 0, 1
KVOFF_CALL_SPARSE_DECODE, KVOFF_CALL_STEP = 1, 2
KVOFF_MAX_BATCH = 128
KVOFF_NOALLOC_SCRATCH_BYTES = 16 << 20

EXPORTS = (
    "kvoff_create", "kvoff_destroy", "kvoff_record_bytes", "kvoff_set_consensus_lambda",
    "kvoff_set_attention_qk", "kvoff_attention_mass",
    "kvoff_register_request",
    "kvoff_host_record", "kvoff_offload_blocks", "kvoff_select", "kvoff_recall",
    "kvoff_sparse_decode", "kvoff_workspace_size", "kvoff_step", "kvoff_probe_read",
    "kvoff_strerror", "kvoff_last_error", "kvoff_admission_defaults", "kvoff_admission_plan",
    "kvoff_make_resident", "kvoff_release_resident", "kvoff_set_kernel_timing",
    "kvoff_get_kernel_times", "kvoff_sparse_decode_noalloc",
)


class KvoffError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"kvoff status {status}: {message}")
        self.status = status


class kvoff_config(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("max_requests", ctypes.c_int32), ("host_mem_kind", ctypes.c_int32),
        ("host_capacity_blocks", ctypes.c_int64),
    ]


class kvoff_admission_policy(ctypes.Structure):
    _fields_ = [("low", ctypes.c_double), ("high", ctypes.c_double),
                ("max_offload", ctypes.c_double), ("step_layers", ctypes.c_int32),
                ("max_resident", ctypes.c_int32)]


class kvoff_stats(ctypes.Structure):
    _fields_ = [("selected", ctypes.c_int64), ("pool_hits", ctypes.c_int64),
                ("items_recalled", ctypes.c_int64), ("transfers", ctypes.c_int64),
                ("bytes", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {k: int(getattr(self, k)) for k, _ in self._fields_}


_vp = ctypes.c_void_p


class kvoff_step_args(ctypes.Structure):
    _fields_ = [
        ("layer_begin", ctypes.c_int32), ("layer_end", ctypes.c_int32),
        ("n_req", ctypes.c_int32), ("req_ids", _vp), ("topk", _vp),
        ("mode", ctypes.c_int32), ("engine", ctypes.c_int32), ("k_stride", ctypes.c_int32),
        ("q_dev", _vp), ("digest_dev", _vp), ("digest_stride", ctypes.c_int64),
        ("pool_hit_dev", _vp), ("pool_slot_dev", _vp), ("pool_stride", ctypes.c_int64),
        ("slot_pool_dev", _vp), ("n_slots", ctypes.c_int64),
        ("recall_base_slot", ctypes.c_int64 * 2),
        ("scores_dev", _vp * 2), ("sel_idx_dev", _vp * 2), ("sel_cnt_dev", _vp * 2),
        ("block_table_dev", _vp * 2),
        ("scale", ctypes.c_float), ("out_dev", _vp),
        ("ws_dev", _vp), ("ws_bytes", ctypes.c_size_t),
        ("compute_stream", _vp), ("copy_stream", _vp), ("stats", _vp),
        ("group_requests", ctypes.c_int32), ("timing", _vp), ("copy_stream2", _vp),
    ]


class kvoff_step_timing(ctypes.Structure):
    _fields_ = [("step_ms", ctypes.c_double), ("compute_wait_ms", ctypes.c_double),
                ("mean_request_done_ms", ctypes.c_double),
                ("max_request_done_ms", ctypes.c_double), ("recall_ms", ctypes.c_double),
                ("recalls", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {k: (int if k == "recalls" else float)(getattr(self, k)) for k, _ in self._fields_}


class kvoff_kernel_times(ctypes.Structure):
    _fields_ = [("score_ms", ctypes.c_double), ("topk_ms", ctypes.c_double),
                ("attend_ms", ctypes.c_double), ("combine_ms", ctypes.c_double),
                ("select_calls", ctypes.c_int64), ("decode_calls", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {k: (int if k.endswith("_calls") else float)(getattr(self, k)) for k, _ in self._fields_}


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                           "(the HIP library is required; there is no fallback)")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, sz, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    P = ctypes.POINTER
    L.kvoff_create.argtypes = [P(kvoff_config), P(_vp)]
    L.kvoff_destroy.argtypes = [_vp]
    L.kvoff_record_bytes.argtypes = [_vp]
    L.kvoff_record_bytes.restype = i64
    L.kvoff_register_request.argtypes = [_vp, i64, P(i32)]
    L.kvoff_set_consensus_lambda.argtypes = [_vp, ctypes.c_double]
    L.kvoff_set_attention_qk.argtypes = [_vp, i32]
    L.kvoff_host_record.argtypes = [_vp, i32, i32, i64, P(_vp)]
    L.kvoff_offload_blocks.argtypes = [_vp, i32, i32, _vp, _vp, _vp, _vp]
    L.kvoff_select.argtypes = [_vp, i32, i32, _vp, _vp, _vp, i64, _vp, i32, _vp, _vp, _vp, i32, _vp]
    L.kvoff_recall.argtypes = [_vp, i32, i32, _vp, i32, _vp, _vp, i32, _vp, _vp, i64, _vp, i64,
                               i64, _vp, i32, _vp, _vp]
    L.kvoff_sparse_decode.argtypes = [_vp, i32, _vp, i32, _vp, _vp, i64, _vp, _vp, _vp, i32, f32,
                                      _vp, _vp, sz, _vp]
    L.kvoff_sparse_decode_noalloc.argtypes = [_vp, i32, _vp, i32, _vp, _vp, i64, _vp, _vp, _vp,
                                              i32, f32, _vp, _vp]
    L.kvoff_workspace_size.argtypes = [_vp, i32, i32, i32, i32]
    L.kvoff_workspace_size.restype = sz
    L.kvoff_step.argtypes = [_vp, P(kvoff_step_args)]
    L.kvoff_probe_read.argtypes = [_vp, i64, _vp, i32, _vp]
    L.kvoff_attention_mass.argtypes = [_vp, i32, i32, _vp, i32, _vp, _vp, _vp, i32, f32, _vp, _vp]
    L.kvoff_admission_defaults.argtypes = [P(kvoff_admission_policy)]
    L.kvoff_admission_defaults.restype = None
    L.kvoff_admission_plan.argtypes = [P(kvoff_admission_policy), i32, ctypes.c_double, _vp, P(i32)]
    L.kvoff_make_resident.argtypes = [_vp, i32, i32, _vp, i64, i64, _vp, _vp, _vp]
    L.kvoff_release_resident.argtypes = [_vp, i32, i32, _vp, _vp]
    L.kvoff_set_kernel_timing.argtypes = [_vp, i32]
    L.kvoff_get_kernel_times.argtypes = [_vp, P(kvoff_kernel_times)]
    L.kvoff_strerror.argtypes = [ctypes.c_int]
    L.kvoff_strerror.restype = ctypes.c_char_p
    L.kvoff_last_error.argtypes = []
    L.kvoff_last_error.restype = ctypes.c_char_p
    for name in ("kvoff_create", "kvoff_destroy", "kvoff_register_request", "kvoff_host_record",
                 "kvoff_set_consensus_lambda", "kvoff_set_attention_qk",
                 "kvoff_offload_blocks", "kvoff_select", "kvoff_recall", "kvoff_sparse_decode",
                 "kvoff_sparse_decode_noalloc",
                 "kvoff_step", "kvoff_probe_read", "kvoff_attention_mass", "kvoff_admission_plan", "kvoff_make_resident",
                 "kvoff_release_resident", "kvoff_set_kernel_timing", "kvoff_get_kernel_times"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int) -> None:
    if status != KVOFF_OK:
        msg = lib().kvoff_last_error().decode(errors="replace")
        raise KvoffError(status, msg or lib().kvoff_strerror(status).decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _i32_array(values: Sequence[int]):
    return (ctypes.c_int32 * len(values))(*[int(v) for v in values])


def kvoff_strerror(status: int) -> str:
    return lib().kvoff_strerror(status).decode()


def kvoff_last_error() -> str:
    return lib().kvoff_last_error().decode(errors="replace")


def kvoff_create(*, num_layers: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 block_size: int, dtype: int, max_requests: int, host_capacity_blocks: int,
                 host_mem_kind: int = KVOFF_HOST_COHERENT) -> int:
    cfg = kvoff_config(num_layers, num_q_heads, num_kv_heads, head_dim, block_size, dtype,
                       max_requests, host_mem_kind, host_capacity_blocks)
    out = _vp()
    _check(lib().kvoff_create(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def kvoff_destroy(ctx: int) -> None:
    _check(lib().kvoff_destroy(ctx))


def kvoff_record_bytes(ctx: int) -> int:
    return int(lib().kvoff_record_bytes(ctx))


def kvoff_set_consensus_lambda(ctx: int, lam: float) -> None:
    _check(lib().kvoff_set_consensus_lambda(ctx, lam))


def kvoff_set_attention_qk(ctx: int, qk: int) -> None:
    _check(lib().kvoff_set_attention_qk(ctx, qk))


def kvoff_set_kernel_timing(ctx: int, on: bool) -> None:
    _check(lib().kvoff_set_kernel_timing(ctx, 1 if on else 0))


def kvoff_get_kernel_times(ctx: int) -> dict:
    t = kvoff_kernel_times()
    _check(lib().kvoff_get_kernel_times(ctx, ctypes.byref(t)))
    return t.as_dict()


def kvoff_register_request(ctx: int, n_tokens: int) -> int:
    rid = ctypes.c_int32()
    _check(lib().kvoff_register_request(ctx, n_tokens, ctypes.byref(rid)))
    return rid.value


def kvoff_host_record(ctx: int, layer: int, req_id: int, block: int) -> int:
    p = _vp()
    _check(lib().kvoff_host_record(ctx, layer, req_id, block, ctypes.byref(p)))
    return p.value


def kvoff_offload_blocks(ctx: int, layer: int, req_id: int, k, v, digest, stream=None) -> None:
    _check(lib().kvoff_offload_blocks(ctx, layer, req_id, _ptr(k), _ptr(v), _ptr(digest),
                                      _stream(stream)))


def kvoff_select(ctx: int, layer: int, req_ids: Sequence[int], q, digest, digest_stride: int,
                 topk: Sequence[int], mode: int, scores, sel_idx, sel_cnt, k_stride: int,
                 stream=None) -> None:
    ids, tk = _i32_array(req_ids), _i32_array(topk)
    _check(lib().kvoff_select(ctx, layer, len(req_ids), ids, _ptr(q), _ptr(digest), digest_stride,
                              tk, mode, _ptr(scores), _ptr(sel_idx), _ptr(sel_cnt), k_stride,
                              _stream(stream)))


def kvoff_recall(ctx: int, layer: int, req_ids: Sequence[int], mode: int, sel_idx, sel_cnt,
                 k_stride: int, pool_hit, pool_slot, pool_stride: int, slot_pool, n_slots: int,
                 recall_base_slot: int, block_table, engine: int = KVOFF_ENGINE_ZEROCOPY,
                 want_stats: bool = False, stream=None) -> Optional[dict]:
    ids = _i32_array(req_ids)
    st = kvoff_stats() if want_stats else None
    _check(lib().kvoff_recall(ctx, layer, len(req_ids), ids, mode, _ptr(sel_idx), _ptr(sel_cnt),
                              k_stride, _ptr(pool_hit), _ptr(pool_slot), pool_stride,
                              _ptr(slot_pool), n_slots, recall_base_slot, _ptr(block_table),
                              engine, ctypes.byref(st) if st is not None else None,
                              _stream(stream)))
    return st.as_dict() if st is not None else None


def kvoff_workspace_size(ctx: int, call: int, n_req: int, k_stride: int, mode: int) -> int:
    return int(lib().kvoff_workspace_size(ctx, call, n_req, k_stride, mode))


def kvoff_sparse_decode(ctx: int, req_ids: Sequence[int], mode: int, q, slot_pool, n_slots: int,
                        block_table, sel_idx, sel_cnt, k_stride: int, scale: float, out, ws,
                        stream=None) -> None:
    ids = _i32_array(req_ids)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().kvoff_sparse_decode(ctx, len(req_ids), ids, mode, _ptr(q), _ptr(slot_pool),
                                     n_slots, _ptr(block_table), _ptr(sel_idx), _ptr(sel_cnt), k_stride,
                                     scale, _ptr(out), _ptr(ws), ws_bytes, _stream(stream)))


def kvoff_sparse_decode_noalloc(ctx: int, req_ids: Sequence[int], mode: int, q, slot_pool,
                                n_slots: int, block_table, sel_idx, sel_cnt, k_stride: int,
                                scale: float, out, stream=None) -> None:
    ids = _i32_array(req_ids)
    _check(lib().kvoff_sparse_decode_noalloc(ctx, len(req_ids), ids, mode, _ptr(q),
                                             _ptr(slot_pool), n_slots, _ptr(block_table),
                                             _ptr(sel_idx), _ptr(sel_cnt), k_stride, scale,
                                             _ptr(out), _stream(stream)))


def kvoff_step(ctx: int, *, layer_begin: int, layer_end: int, req_ids: Sequence[int],
               topk: Sequence[int], mode: int, engine: int, k_stride: int, q: Sequence,
               digest: Sequence, digest_stride: int, slot_pool, n_slots: int,
               recall_base_slot: Sequence[int], scores: Sequence, sel_idx: Sequence,
               sel_cnt: Sequence, block_table: Sequence, scale: float, out: Sequence, ws,
               pool_hit: Optional[Sequence] = None, pool_slot: Optional[Sequence] = None,
               pool_stride: int = 0, compute_stream=None, copy_stream=None,
               want_stats: bool = False, group_requests: int = 0,
               want_timing: bool = False, copy_stream2=None) -> Optional[dict]:
    """Returns None, or the summed kvoff_stats fields (want_stats) and/or
    the compute-stream timing under "timing" (want_timing)."""
    n_layers = layer_end - layer_begin
    ids, tk = _i32_array(req_ids), _i32_array(topk)
    # one pointer per layer, NULL-padded: the library checks the layer range
    # and rejects missing per-layer buffers itself
    arr = lambda ts: (_vp * max(n_layers, len(ts), 1))(*[_ptr(t) for t in ts])
    a = kvoff_step_args()
    a.layer_begin, a.layer_end, a.n_req = layer_begin, layer_end, len(req_ids)
    a.req_ids = ctypes.cast(ids, _vp)
    a.topk = ctypes.cast(tk, _vp)
    a.mode, a.engine, a.k_stride = mode, engine, k_stride
    keep = [ids, tk, arr(q), arr(digest), arr(out)]
    a.q_dev = ctypes.cast(keep[2], _vp)
    a.digest_dev = ctypes.cast(keep[3], _vp)
    a.out_dev = ctypes.cast(keep[4], _vp)
    a.digest_stride = digest_stride
    if pool_hit is not None:
        keep += [arr(pool_hit), arr(pool_slot)]
        a.pool_hit_dev = ctypes.cast(keep[-2], _vp)
        a.pool_slot_dev = ctypes.cast(keep[-1], _vp)
    a.pool_stride = pool_stride
    a.slot_pool_dev = _ptr(slot_pool)
    a.n_slots = n_slots
    for i in range(2):
        a.recall_base_slot[i] = recall_base_slot[i]
        a.scores_dev[i] = _ptr(scores[i])
        a.sel_idx_dev[i] = _ptr(sel_idx[i])
        a.sel_cnt_dev[i] = _ptr(sel_cnt[i])
        a.block_table_dev[i] = _ptr(block_table[i])
    a.scale = scale
    a.ws_dev = _ptr(ws)
    a.ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    cs = _stream(compute_stream)
    a.compute_stream = cs
    a.copy_stream = _stream(copy_stream) if copy_stream is not None else cs
    a.copy_stream2 = _stream(copy_stream2) if copy_stream2 is not None else None
    st = kvoff_stats() if want_stats else None
    a.stats = ctypes.cast(ctypes.pointer(st), _vp) if st is not None else None
    a.group_requests = group_requests
    tm = kvoff_step_timing() if want_timing else None
    a.timing = ctypes.cast(ctypes.pointer(tm), _vp) if tm is not None else None
    _check(lib().kvoff_step(ctx, ctypes.byref(a)))
    if st is None and tm is None:
        return None
    res = st.as_dict() if st is not None else {}
    if tm is not None:
        res["timing"] = tm.as_dict()
    return res


def kvoff_attention_mass(ctx: int, layer: int, req_ids: Sequence[int], mode: int, q, sel_idx,
                         sel_cnt, k_stride: int, scale: float, mass, stream=None) -> None:
    ids = _i32_array(req_ids)
    _check(lib().kvoff_attention_mass(ctx, layer, len(req_ids), ctypes.cast(ids, _vp), mode,
                                      _ptr(q), _ptr(sel_idx), _ptr(sel_cnt), k_stride, scale,
                                      _ptr(mass), _stream(stream)))


def kvoff_probe_read(ptr, n_bytes: int, sink, n_wg: int = 0, stream=None) -> None:
    _check(lib().kvoff_probe_read(_ptr(ptr), n_bytes, _ptr(sink), n_wg, _stream(stream)))


def kvoff_admission_defaults() -> kvoff_admission_policy:
    p = kvoff_admission_policy()
    lib().kvoff_admission_defaults(ctypes.byref(p))
    return p


def kvoff_admission_plan(policy: kvoff_admission_policy, utilization: float, resident) -> int:
    """resident: numpy uint8 [num_layers], updated in place; returns the count."""
    n = ctypes.c_int32()
    _check(lib().kvoff_admission_plan(ctypes.byref(policy), len(resident), utilization,
                                      resident.ctypes.data_as(ctypes.c_void_p), ctypes.byref(n)))
    return n.value


def kvoff_make_resident(ctx: int, layer: int, req_id: int, slot_pool, n_slots: int,
                        first_slot: int, pool_hit, pool_slot, stream=None) -> None:
    _check(lib().kvoff_make_resident(ctx, layer, req_id, _ptr(slot_pool), n_slots, first_slot,
                                     _ptr(pool_hit), _ptr(pool_slot), _stream(stream)))


def kvoff_release_resident(ctx: int, layer: int, req_id: int, pool_hit, stream=None) -> None:
    _check(lib().kvoff_release_resident(ctx, layer, req_id, _ptr(pool_hit), _stream(stream)))
