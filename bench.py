"""Benchmark of the sparse KV-offloading hot path on one MI355X.

One step = one layer-step of the Llama-3-8B-shaped workload (batch 16, 32
query / 8 KV heads, head_dim 128, 32,768-token contexts in 32-token blocks,
top-64 blocks, bf16, 5% planted hot blocks): score + SoloHead top-k, recall
of the selected blocks from the pinned host store into HBM, sparse GQA decode
attention.  Steps cycle through `--layers` distinct layers (separate digests
and host records) so no step finds its digests in the 256 MB Infinity Cache
from the previous one.  Inputs are synthetic (seeded generator, no gap
conditioning: that only matters for parity checks) and are resident in HBM /
the pinned store before timing starts.

Prints one JSON line.  `--gpus N` with N > 1 exits: the benchmark measures one GPU.
"""
from __future__ import annotations

import argparse
import glob
import json
import math
import os
import platform
import sys
import time

# Idle OpenMP threads (the input generator's bulk fill, torch's CPU ops) go to
# sleep instead of spinning, so they leave the host's cores to the timed run
# that follows setup.  Set before numpy and torch load the OpenMP runtime.
os.environ.setdefault("OMP_WAIT_POLICY", "PASSIVE")

import numpy as np  # noqa: E402
import torch  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import sparse_kv_cache_mean_amd as kv  # noqa: E402
import synth  # noqa: E402
from tests import gpu_harness as H  # noqa: E402

METRIC = "sparse decode layer-steps/s; recall GB/s host→HBM vs link peak; HBM GB/s"

# Counter traffic of the dominant kernel (gather_kernel) per launch on this
# workload, from two rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE; summary
# and calibration in profiles/llama3-8b-layer_pmc_traffic.md).  Valid only for
# the recall source it was taken with: reported as null once that changes.
GATHER_PMC = {"workload": ("llama3-8b-layer", 4), "fetch_kib": 65605.2, "write_kib": 131082.5,
              "fetch_scale": 1.9999, "write_scale": 1.0000,
              "recall_src_sha256": "b79e692fb4abc5059c50b5a54cce73825f65cab820a3bc4647a8387842908398"}


def gather_traffic_bytes(workload, layers):
    import hashlib
    if (workload, layers) != GATHER_PMC["workload"]:
        return None
    src = os.path.join(ROOT, "sparse_kv_cache_mean_amd", "csrc", "recall.hip")
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != GATHER_PMC["recall_src_sha256"]:
            return None
    return int(GATHER_PMC["fetch_kib"] * 1024 * GATHER_PMC["fetch_scale"] +
               GATHER_PMC["write_kib"] * 1024 * GATHER_PMC["write_scale"])
HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, published
PCIE_PEAK_GBPS = 64.0       # PCIe 5.0 x16, one direction, published


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=40)
    p.add_argument("--warmup", type=int, default=8)
    p.add_argument("--workload", default="llama3-8b-layer",
                   choices=[w.name for w in synth.WORKLOADS.values()])
    p.add_argument("--config", type=int, default=None, help=argparse.SUPPRESS)  # by number
    p.add_argument("--layers", type=int, default=4)
    p.add_argument("--engine", choices=["zerocopy", "dma", "staged"], default="zerocopy")
    p.add_argument("--host-mem", choices=["coherent", "noncoherent"], default="coherent")
    p.add_argument("--attn-qk", choices=["mfma", "valu"], default="mfma",
                   help="what computes the attention's QK^T")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="oracle time on host cores for the headline workload's baseline")
    p.add_argument("--configs", default="1,3,4,5",
                   help="other workloads measured after the headline, by number (or 'none'); "
                        "each adds an entry to the line's configs object")
    p.add_argument("--config-cpu-seconds", type=float, default=6.0,
                   help="oracle time on host cores for each other workload's baseline")
    p.add_argument("--no-overlap", action="store_true",
                   help="time the serial order on one stream as the value instead of "
                        "kvoff_step (every gather then runs alone: clean kernel traces)")
    p.add_argument("--report", choices=["fragmentation", "admission", "groups", "mass", "decode32",
                                        "attention-cache", "attention-heads", "select-modes"],
                   default=None,
                   help="instead of the bench line: fragmentation = recall of the "
                        "headwise-vs-SoloHead workload with every engine; admission = the "
                        "admission policy as a control loop over the multi-layer step; groups = "
                        "interruptible per-request scheduling on the variable-recall layer; "
                        "mass = attention mass kept and recall volume of every selection mode; "
                        "decode32 = the overlapped 32-layer decode step; attention-cache = "
                        "sparse attention with its input warm, after a 1 GiB read and after "
                        "a 1 GiB write; attention-heads = sparse attention with 4, 8 and 16 "
                        "query heads per KV head over the same records; select-modes = score "
                        "and top-k kernel times of every selection mode")
    args = p.parse_args()
    if args.steps < 1 or args.warmup < 0:
        p.error("--steps must be at least 1 and --warmup at least 0")
    if args.configs.strip().lower() in ("", "none"):
        args.config_list = []
    else:
        try:
            args.config_list = [int(x) for x in args.configs.split(",")]
        except ValueError:
            p.error("--configs takes workload numbers such as 1,3,4,5, or none")
        if any(n not in CONFIG_LAYERS for n in args.config_list):
            p.error(f"--configs: workloads {sorted(CONFIG_LAYERS)} (2 is the headline)")
    return args


def step_calls(n: int, per_call: int) -> list[int]:
    """Layers per kvoff_step call for exactly n layer-steps: whole passes of
    per_call layers, then one shorter call over the first n mod per_call."""
    full, rem = divmod(n, per_call)
    return [per_call] * full + ([rem] if rem else [])


def link_peaks(case):
    """Measured host->HBM peaks: one 1 GiB pinned hipMemcpyAsync (best of 5)
    and the zero-copy read probe over the pinned store."""
    nbytes = 1 << 30
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dev = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best_copy = 0.0
    for _ in range(5):
        s.record()
        dev.copy_(host, non_blocking=True)
        e.record()
        e.synchronize()
        best_copy = max(best_copy, nbytes / (s.elapsed_time(e) * 1e-3) / 1e9)
    del host, dev
    # zero-copy probe: read the first GiB of the request store
    rec = kv.kvoff_record_bytes(case.ctx)
    base = kv.kvoff_host_record(case.ctx, 0, case.rids[0], 0)
    n = min(nbytes, (case.reqs[0].nb * rec) // 4096 * 4096)
    sink = torch.empty(4096, dtype=torch.uint8, device="cuda")
    best_probe = 0.0
    for _ in range(5):
        s.record()
        kv.kvoff_probe_read(base, n, sink)
        e.record()
        e.synchronize()
        best_probe = max(best_probe, n / (s.elapsed_time(e) * 1e-3) / 1e9)
    return best_copy, best_probe


def hbm_read_peak():
    """Best of 5 reads of a 2 GiB device buffer with the probe kernel."""
    n = 2 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    sink = torch.empty(4096, dtype=torch.uint8, device="cuda")
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = 0.0
    for wg in (2048, 4096, 8192):
        for _ in range(3):
            s.record()
            kv.kvoff_probe_read(a, n, sink, wg)
            e.record()
            e.synchronize()
            best = max(best, n / (s.elapsed_time(e) * 1e-3) / 1e9)
    return best


def hbm_copy_peak():
    n = 2 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = 0.0
    for _ in range(5):
        s.record()
        b.copy_(a)
        e.record()
        e.synchronize()
        best = max(best, 2 * n / (s.elapsed_time(e) * 1e-3) / 1e9)
    return best


def d2h_link_peak():
    """Device -> pinned host: best of 5 one-GiB hipMemcpyAsync copies."""
    nbytes = 1 << 30
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dev = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = 0.0
    for _ in range(5):
        s.record()
        host.copy_(dev, non_blocking=True)
        e.record()
        e.synchronize()
        best = max(best, nbytes / (s.elapsed_time(e) * 1e-3) / 1e9)
    del host, dev
    return best


def offload_timing(case, sp, inputs, B):
    """Setup row, outside the step: kvoff_offload_blocks for layer 0 of every
    request again (same bytes, same digests), K and V already in HBM, timed
    with events on one stream.  It reads K and V from HBM, writes the block
    records to the pinned store over the host link and the digests to HBM."""
    kd = [H.to_dev(inputs[(0, r)].K) for r in range(B)]
    vd = [H.to_dev(inputs[(0, r)].V) for r in range(B)]
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for r in range(B):
        kv.kvoff_offload_blocks(case.ctx, 0, case.rids[r], kd[r], vd[r], case.digest[0][r],
                                stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    rec = kv.kvoff_record_bytes(case.ctx) * sum(rq.nb for rq in case.reqs)
    del kd, vd
    gbps = rec / (ms * 1e-3) / 1e9
    peak = d2h_link_peak()
    return {"what": f"kvoff_offload_blocks, one layer of {B} requests", "ms_per_layer": round(ms, 3),
            "host_write_bytes": rec, "host_write_gbps": round(gbps, 2),
            "d2h_link_peak_gbps": round(peak, 2), "frac_of_d2h_link_peak": round(gbps / peak, 4)}


def host_cpu():
    """The host the baseline ran on: CPU model string, the CPUs this process
    may run on, and the NUMA nodes those CPUs belong to."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    allowed = sorted(os.sched_getaffinity(0))
    nodes = []
    for path in sorted(glob.glob("/sys/devices/system/node/node[0-9]*/cpulist")):
        cpus = set()
        with open(path) as f:
            for part in f.read().strip().split(","):
                if part:
                    a, _, b = part.partition("-")
                    cpus.update(range(int(a), int(b or a) + 1))
        if cpus.intersection(allowed):
            nodes.append(int(os.path.basename(os.path.dirname(path))[4:]))
    return {"cpu": model, "nproc": os.cpu_count(), "cpus_allowed": len(allowed),
            "numa_nodes": nodes}


def cpu_baseline(sp, inputs, B, budget_s, keys=None, threads=None):
    """The oracle, as it is, on host cores: one request's layer-step (score,
    select, record gather of the selected blocks, fp32 attention) per call,
    over the (layer, request) slices `keys` of `inputs` (default: layer 0 of
    every request), in that order.  Timed twice for about budget_s / 2
    seconds each: on one thread, then with one worker thread per core running
    independent requests (the oracle is plain C with no shared state; ctypes
    releases the interpreter lock while it runs).  Each leg is scaled to
    layer-steps/s from its mean time per request-step: a layer-step is B
    request-steps.  When a leg ends before it has visited every slice, its
    mean is over the slices visited, which the sample string says.  The value
    is the threaded figure."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    keys = keys or [(0, r) for r in range(B)]
    threads = threads or max(1, min(16, os.cpu_count() or 1))
    digests = {}

    def digest(k):
        lr = inputs[k]
        digests[k] = oracle.digest(lr.K, sp.dtype, sp.bs)  # setup, not timed

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(digest, keys))

    def request_step(k):
        lr = inputs[k]
        S = oracle.score(lr.q, sp.dtype, digests[k])
        sel = oracle.select(S, lr.rq.k)
        for b in sel.tolist():
            t_a, t_b = b * sp.bs, min((b + 1) * sp.bs, lr.rq.ctx)
            oracle.records(lr.K[t_a:t_b], lr.V[t_a:t_b], sp.bs)
        oracle.attend_f32(lr.q, lr.K, lr.V, sp.dtype, sp.bs, sel)

    half = budget_s / 2
    n = len(keys)
    done, t0 = 0, time.perf_counter()
    while True:
        request_step(keys[done % n])
        done += 1
        el1 = time.perf_counter() - t0
        if el1 >= half:
            break
    single = 1.0 / (el1 / done * B)
    n_thr, t0 = 0, time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        while True:  # rounds of one request per thread
            list(ex.map(request_step, [keys[(n_thr + i) % n] for i in range(threads)]))
            n_thr += threads
            el2 = time.perf_counter() - t0
            if el2 >= half:
                break

    def seen(m):
        return f"all {n}" if m >= n else f"the first {m} of {n}"

    layers = sorted({k[0] for k in keys})
    where = f"layer {layers[0]}" if len(layers) == 1 else f"layers {layers}"
    return {"value": 1.0 / (el2 / n_thr * B), "unit": "layer-steps/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n_thr} request-steps of {where} on {threads} threads ({el2:.1f} s, "
                      f"{seen(n_thr)} slices), scaled to a {B}-request layer-step",
            "single_thread": {"value": single, "cores": 1,
                              "sample": f"{done} request-steps ({el1:.1f} s, {seen(done)} slices)"},
            **host_cpu()}


def fragmentation_report(args):
    """Recall of the headwise-vs-SoloHead workload: each selection mode with
    each engine; transfers, mean transfer size and recall GB/s (wall clock
    around the call, stream synchronised before and after)."""
    sp = synth.spec(5)
    reqs = synth.request_draws(sp)
    inputs = {(0, r): synth.gen_layer_request(sp, 0, r, rq) for r, rq in enumerate(reqs)}
    case = H.build_case(sp, inputs, [0], reqs, with_pool_hits=True, two_regions=False)
    inputs.clear()
    topk = [rq.k for rq in reqs]
    out = {"workload": f"{sp.name}: batch {len(reqs)}, {sp.Hq}/{sp.Hkv} heads, context "
                       f"{reqs[0].ctx}, block {sp.bs}, top-{reqs[0].k} shared or per KV head, "
                       f"{int(sp.pool_frac * 100)}% of blocks resident in the HBM pool",
           "runs": []}
    for mode, mname in ((kv.KVOFF_SOLOHEAD, "solohead"), (kv.KVOFF_HEADWISE, "headwise")):
        bufs = H.make_buffers(case, mode)
        kv.kvoff_select(case.ctx, 0, case.rids, case.q[0], case.digest[0], case.nb_max, topk,
                        mode, bufs.scores, bufs.sel_idx, bufs.sel_cnt, case.k_stride)
        for engine, ename in ((kv.KVOFF_ENGINE_ZEROCOPY, "zerocopy"), (kv.KVOFF_ENGINE_DMA, "dma"),
                              (kv.KVOFF_ENGINE_STAGED, "staged")):
            def rec(stats=False):
                return kv.kvoff_recall(case.ctx, 0, case.rids, mode, bufs.sel_idx, bufs.sel_cnt,
                                       case.k_stride, case.pool_hit[0], case.pool_slot[0],
                                       case.nb_max, case.pool, case.n_slots, case.recall_base[0],
                                       bufs.table, engine, want_stats=stats)
            st = rec(True)
            for _ in range(3):
                rec()
            torch.cuda.synchronize()
            n = 20
            t = time.perf_counter()
            for _ in range(n):
                rec()
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t) * 1e3 / n
            out["runs"].append({
                "mode": mname, "engine": ename, "ms": round(ms, 4),
                "gbps": round(st["bytes"] / (ms * 1e-3) / 1e9, 2),
                "transfers": st["transfers"], "items": st["items_recalled"],
                "pool_hits": st["pool_hits"], "bytes": st["bytes"],
                "mean_transfer_kib": round(st["bytes"] / max(1, st["transfers"]) / 1024, 2)})
            log(str(out["runs"][-1]))
    H.destroy(case)
    print(json.dumps(out), flush=True)


def admission_report(args):
    """IO-adaptive admission as a control loop on the batch-8 decode step
    shape (8 rotating layers of the 32-layer workload, HBM budget for 4 of
    them).  Each round runs a window of steps, measures the link utilisation
    (recalled bytes / (wall time x measured link peak)), asks the policy for
    the resident layers and pins or releases layers to match.  The first
    rounds issue steps back to back (the link saturates); the later ones pace
    the steps at four times the saturated step time, as a lightly loaded
    server would, so the utilisation drops and layers are handed back."""
    L = args.layers if args.layers != 4 else 8
    budget = L // 2
    sp = synth.spec(3, L=L)
    reqs = synth.request_draws(sp)
    B = len(reqs)
    layers = list(range(L))
    nb_tot = sum(rq.nb for rq in reqs)
    case = H.build_case(sp, lambda key: synth.gen_layer_request(sp, key[0], key[1], reqs[key[1]]),
                        layers, reqs, keep=lambda l, r: False, extra_slots=nb_tot * budget)
    mode, engine = kv.KVOFF_SOLOHEAD, kv.KVOFF_ENGINE_ZEROCOPY
    sets = [H.make_buffers(case, mode) for _ in range(2)]
    outs = [torch.empty_like(sets[0].out) for _ in layers]
    hit = [torch.zeros((B, case.nb_max), dtype=torch.uint8, device="cuda") for _ in layers]
    slot = [torch.full((B, case.nb_max), -1, dtype=torch.int32, device="cuda") for _ in layers]
    compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
    topk = [rq.k for rq in reqs]

    def step(want_stats=False):
        return kv.kvoff_step(
            case.ctx, layer_begin=0, layer_end=L, req_ids=case.rids, topk=topk, mode=mode,
            engine=engine, k_stride=case.k_stride, q=[case.q[l] for l in layers],
            digest=[case.digest[l] for l in layers], digest_stride=case.nb_max,
            slot_pool=case.pool, n_slots=case.n_slots, recall_base_slot=case.recall_base,
            scores=[b.scores for b in sets], sel_idx=[b.sel_idx for b in sets],
            sel_cnt=[b.sel_cnt for b in sets], block_table=[b.table for b in sets],
            scale=1.0 / math.sqrt(sp.d), out=outs, ws=sets[0].ws, pool_hit=hit,
            pool_slot=slot, pool_stride=case.nb_max, compute_stream=compute, copy_stream=copy,
            want_stats=want_stats)

    copy_peak, _ = link_peaks(case)
    policy = kv.kvoff_admission_defaults()
    policy.max_resident = budget
    resident = np.zeros(L, np.uint8)
    home = {}                          # resident layer -> its slot range index
    free = list(range(budget))

    def apply(plan):
        for l in np.flatnonzero((resident == 1) & (plan == 0)).tolist():  # release first
            for r in range(B):
                kv.kvoff_release_resident(case.ctx, l, case.rids[r], hit[l][r], stream=compute)
            free.append(home.pop(l))
        for l in np.flatnonzero((plan == 1) & (resident == 0)).tolist():
            k = free.pop(0)
            home[l] = k
            first = case.extra_base + k * nb_tot
            for r, rq in enumerate(reqs):
                kv.kvoff_make_resident(case.ctx, l, case.rids[r], case.pool, case.n_slots, first,
                                       hit[l][r], slot[l][r], stream=compute)
                first += rq.nb
        resident[:] = plan
        torch.cuda.synchronize()

    def window(n, period_s=None):
        st = step(want_stats=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            t = time.perf_counter()
            step()
            if period_s:
                torch.cuda.synchronize()
                left = period_s - (time.perf_counter() - t)
                if left > 0:
                    time.sleep(left)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return st["bytes"] * n / (wall * copy_peak * 1e9), wall / n, st["bytes"]

    step()
    torch.cuda.synchronize()
    _, sat_step_s, _ = window(4)
    rounds = []
    for rnd in range(8):
        paced = rnd >= 4
        util, step_s, recalled = window(6, 4 * sat_step_s if paced else None)
        before = np.flatnonzero(resident).tolist()
        plan = resident.copy()
        kv.kvoff_admission_plan(policy, util, plan)
        apply(plan)
        row = {"round": rnd, "load": "paced at 4x the saturated step" if paced else "back to back",
               "link_utilization": round(util, 4), "resident_before": before,
               "layer_steps_per_s": round(L / step_s, 1), "recalled_bytes_per_step": recalled,
               "resident_after": np.flatnonzero(resident).tolist()}
        log(str(row))
        rounds.append(row)
    out = {"workload": f"{sp.name}: batch {B}, {L} rotating layers, context {reqs[0].ctx}, "
                       f"top-{reqs[0].k}, overlapped kvoff_step",
           "policy": {"low": policy.low, "high": policy.high, "max_offload": policy.max_offload,
                      "step_layers": policy.step_layers, "max_resident": policy.max_resident},
           "hbm_bytes_per_resident_layer": int(nb_tot * kv.kvoff_record_bytes(case.ctx)),
           "link_peak_gbps": round(copy_peak, 2), "rounds": rounds}
    H.destroy(case)
    print(json.dumps(out), flush=True)


def groups_report(args):
    """Interruptible per-request scheduling on the variable-recall layer
    (batch 32, contexts 8K-128K, top-k 2-15%): the same kvoff_step with the
    whole batch as one group and with smaller request groups, optionally
    with a quarter of the requests pinned in HBM.  Reports the compute
    stream's wait for recalls and when requests finish."""
    sp = synth.spec(4)
    reqs = synth.request_draws(sp)
    B = len(reqs)
    n_pin = B // 4
    extra = sum(rq.nb for rq in reqs[:n_pin])
    log(f"generating '{sp.name}' ({B} requests)")
    case = H.build_case(sp, lambda key: synth.gen_layer_request(sp, key[0], key[1], reqs[key[1]]),
                        [0], reqs, keep=lambda l, r: False, extra_slots=extra)
    mode, engine = kv.KVOFF_SOLOHEAD, kv.KVOFF_ENGINE_ZEROCOPY
    sets = [H.make_buffers(case, mode) for _ in range(2)]
    out = [torch.empty_like(sets[0].out)]
    hit = [torch.zeros((B, case.nb_max), dtype=torch.uint8, device="cuda")]
    slot = [torch.full((B, case.nb_max), -1, dtype=torch.int32, device="cuda")]
    compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
    topk = [rq.k for rq in reqs]

    def step(grp, want_stats=False):
        return kv.kvoff_step(
            case.ctx, layer_begin=0, layer_end=1, req_ids=case.rids, topk=topk, mode=mode,
            engine=engine, k_stride=case.k_stride, q=[case.q[0]], digest=[case.digest[0]],
            digest_stride=case.nb_max, slot_pool=case.pool, n_slots=case.n_slots,
            recall_base_slot=case.recall_base, scores=[b.scores for b in sets],
            sel_idx=[b.sel_idx for b in sets], sel_cnt=[b.sel_cnt for b in sets],
            block_table=[b.table for b in sets], scale=1.0 / math.sqrt(sp.d), out=out,
            ws=sets[0].ws, pool_hit=hit, pool_slot=slot, pool_stride=case.nb_max,
            compute_stream=compute, copy_stream=copy, want_stats=want_stats,
            group_requests=grp, want_timing=True)

    def measure(grp, n=5):
        first = step(grp, want_stats=True)
        ts = [step(grp)["timing"] for _ in range(n)]
        res = {k: round(float(np.mean([t[k] for t in ts])), 4) for k in ts[0]}
        res["group_requests"] = grp
        res["recalled_bytes"] = first["bytes"]
        log(str(res))
        return res

    runs = [measure(g) for g in (0, 16, 8, 4, 1)]
    first = case.extra_base
    for r in range(n_pin):
        kv.kvoff_make_resident(case.ctx, 0, case.rids[r], case.pool, case.n_slots, first,
                               hit[0][r], slot[0][r])
        first += reqs[r].nb
    torch.cuda.synchronize()
    pinned = [measure(g) for g in (0, 8, 1)]
    res = {"workload": f"{sp.name}: batch {B}, {sp.Hq}/{sp.Hkv} heads, contexts "
                       f"{min(rq.ctx for rq in reqs)}-{max(rq.ctx for rq in reqs)}, top-k "
                       f"{min(topk)}-{max(topk)} blocks, one layer, zero-copy recall",
           "groups": runs, "with_first_quarter_resident": pinned}
    H.destroy(case)
    print(json.dumps(res), flush=True)


def mass_report(args):
    """Attention mass kept and recall volume of every selection mode on the
    headwise-vs-SoloHead shapes (batch 16, 32/8 heads, context 32768, top-64
    blocks per set; no pool hits): the guide's claim is that one shared set
    keeps nearly all the mass of per-head sets at a fraction of the volume."""
    sp = synth.spec(5, pool_frac=0.0)
    reqs = synth.request_draws(sp)
    B = len(reqs)
    log(f"generating '{sp.name}' ({B} requests)")
    case = H.build_case(sp, lambda key: synth.gen_layer_request(sp, key[0], key[1], reqs[key[1]]),
                        [0], reqs, keep=lambda l, r: False)
    scale = 1.0 / math.sqrt(sp.d)
    topk = [rq.k for rq in reqs]
    rec = kv.kvoff_record_bytes(case.ctx)
    runs = []
    modes = [("solohead", kv.KVOFF_SOLOHEAD, None), ("consensus", kv.KVOFF_CONSENSUS, 0.5),
             ("consensus", kv.KVOFF_CONSENSUS, 1.0), ("group_consensus", kv.KVOFF_CONSENSUS_GROUP, 0.5),
             ("group_consensus", kv.KVOFF_CONSENSUS_GROUP, 1.0), ("headwise", kv.KVOFF_HEADWISE, None)]
    for name, mode, lam in modes:
        if lam is not None:
            kv.kvoff_set_consensus_lambda(case.ctx, lam)
        bufs = H.make_buffers(case, mode)
        kv.kvoff_select(case.ctx, 0, case.rids, case.q[0], case.digest[0], case.nb_max, topk, mode,
                        bufs.scores, bufs.sel_idx, bufs.sel_cnt, case.k_stride)
        mass = torch.empty((B, sp.Hq), dtype=torch.float64, device="cuda")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        kv.kvoff_attention_mass(case.ctx, 0, case.rids, mode, case.q[0], bufs.sel_idx,
                                bufs.sel_cnt, case.k_stride, scale, mass)
        e1.record()
        st = kv.kvoff_recall(case.ctx, 0, case.rids, mode, bufs.sel_idx, bufs.sel_cnt,
                             case.k_stride, None, None, 0, case.pool, case.n_slots,
                             case.recall_base[0], bufs.table, kv.KVOFF_ENGINE_ZEROCOPY,
                             want_stats=True)
        torch.cuda.synchronize()
        sel = bufs.sel_idx.cpu().numpy()
        cnt = bufs.sel_cnt.cpu().numpy()
        distinct = sum(len(np.unique(sel[r][:, :cnt[r]])) for r in range(B))
        m = mass.cpu().numpy()
        res = {"mode": name, "lambda": lam, "mean_mass": round(float(m.mean()), 5),
               "min_head_mass": round(float(m.min()), 5), "recalled_bytes": st["bytes"],
               "transfers": st["transfers"], "distinct_blocks": int(distinct),
               "mass_kernel_ms": round(e0.elapsed_time(e1), 3)}
        log(str(res))
        runs.append(res)
    hw = runs[-1]
    for r in runs:
        r["mass_vs_headwise"] = round(r["mean_mass"] / hw["mean_mass"], 4)
        r["volume_vs_headwise"] = round(r["recalled_bytes"] / hw["recalled_bytes"], 4)
    K_bytes = sum(rq.nb for rq in reqs) * sp.Hkv * sp.bs * sp.d * sp.es
    res = {"workload": f"{sp.name} shapes: batch {B}, {sp.Hq}/{sp.Hkv} heads, context "
                       f"{reqs[0].ctx}, block {sp.bs}, top-{reqs[0].k} per set, no pool hits",
           "record_bytes": rec, "mass_kernel_reads_bytes": K_bytes, "runs": runs}
    H.destroy(case)
    print(json.dumps(res), flush=True)


def select_modes_report(args):
    """Score and top-k kernels of every selection mode on the Llama-3-8B-shaped
    layer (batch 16, 32/8 heads, context 32768, top-64 per set), kernel
    durations from start/stop events bound to each dispatch
    (kvoff_set_kernel_timing), over 4 rotating layers so that no call finds
    its digests in the MALL."""
    sp = synth.spec(2)
    reqs = synth.request_draws(sp)
    B = len(reqs)
    layers = list(range(4))
    log(f"generating {len(layers)} layers of '{sp.name}' ({B} requests)")
    case = H.build_case(sp, lambda key: synth.gen_layer_request(sp, key[0], key[1], reqs[key[1]]),
                        layers, reqs, keep=lambda l, r: False)
    topk = [rq.k for rq in reqs]
    nb_tot = sum(rq.nb for rq in reqs)
    runs = []
    modes = [("solohead", kv.KVOFF_SOLOHEAD), ("headwise", kv.KVOFF_HEADWISE),
             ("consensus", kv.KVOFF_CONSENSUS), ("group_consensus", kv.KVOFF_CONSENSUS_GROUP)]
    kv.kvoff_set_consensus_lambda(case.ctx, 0.5)
    for name, mode in modes:
        bufs = H.make_buffers(case, mode)
        sets = sp.Hkv if mode in (kv.KVOFF_HEADWISE, kv.KVOFF_CONSENSUS_GROUP) else 1

        def select(i):
            l = layers[i % len(layers)]
            kv.kvoff_select(case.ctx, l, case.rids, case.q[l], case.digest[l], case.nb_max, topk,
                            mode, bufs.scores, bufs.sel_idx, bufs.sel_cnt, case.k_stride)

        for i in range(args.warmup):
            select(i)
        kv.kvoff_set_kernel_timing(case.ctx, True)
        for i in range(args.steps):
            select(i)
        t = kv.kvoff_get_kernel_times(case.ctx)
        kv.kvoff_set_kernel_timing(case.ctx, False)
        score_bytes = nb_tot * sp.Hkv * sp.d * 4 + B * sp.Hq * sp.d * sp.es + nb_tot * sets * 8
        gbps = score_bytes / (t["score_ms"] * 1e-3) / 1e9
        res = {"mode": name, "score_us": round(t["score_ms"] * 1e3, 2),
               "topk_us": round(t["topk_ms"] * 1e3, 2), "score_bytes": score_bytes,
               "score_hbm_gbps": round(gbps, 1), "score_frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
               "calls": t["select_calls"]}
        log(str(res))
        runs.append(res)
    res = {"workload": f"{sp.name}: batch {B}, {sp.Hq}/{sp.Hkv} heads, context {reqs[0].ctx}, "
                       f"block {sp.bs}, top-{reqs[0].k} per set, {len(layers)} rotating layers",
           "how": "kernel durations from start/stop events bound to each dispatch "
                  "(kvoff_set_kernel_timing), consensus lambda 0.5", "runs": runs}
    H.destroy(case)
    print(json.dumps(res), flush=True)


def attention_cache_report(args):
    """Sparse attention on the Llama-3-8B-shaped and the variable-recall
    layers, three ways: warm (calls back to back; 128 MiB of records stay in
    the 256 MB MALL, 923 MiB do not), after a 1 GiB read (the records come
    from HBM, the caches hold clean lines), and after a 1 GiB write (the
    caches hold dirty lines that the attention's reads must evict).  Per shape
    and phase, 20 decode calls (attend_kernel + combine_kernel) in that order,
    so a kernel trace of this report splits into groups of 20 attend_kernel
    launches; the figures here are event-timed decode calls, median of the
    last 15.  Each phase's calls are queued while a spin kernel holds the
    GPU, so the events time the GPU work, not the host's launch latency."""
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    flush.fill_(1)
    out = []
    for name in ("llama3-8b-layer", "llama3-70b-variable"):
        sp = synth.spec(name)
        reqs = synth.request_draws(sp)
        log(f"generating '{sp.name}'")
        case = H.build_case(sp, lambda key: synth.gen_layer_request(sp, key[0], key[1], reqs[key[1]]),
                            [0], reqs, keep=lambda l, r: False)
        mode = kv.KVOFF_SOLOHEAD
        bufs = H.make_buffers(case, mode)
        topk = [rq.k for rq in reqs]
        kv.kvoff_select(case.ctx, 0, case.rids, case.q[0], case.digest[0], case.nb_max, topk, mode,
                        bufs.scores, bufs.sel_idx, bufs.sel_cnt, case.k_stride)
        kv.kvoff_recall(case.ctx, 0, case.rids, mode, bufs.sel_idx, bufs.sel_cnt, case.k_stride,
                        None, None, 0, case.pool, case.n_slots, case.recall_base[0], bufs.table,
                        kv.KVOFF_ENGINE_ZEROCOPY)
        scale = 1.0 / math.sqrt(sp.d)
        nbytes = sum(min(rq.k, rq.nb) for rq in reqs) * kv.kvoff_record_bytes(case.ctx)
        res = {"workload": name, "records_read_bytes": nbytes}
        for phase, before in (("warm", None), ("after_1GiB_read", lambda i: flush.view(torch.float32).sum()),
                              ("after_1GiB_write", lambda i: flush.fill_(i & 0xff))):
            evs = []
            torch.cuda.synchronize()
            torch.cuda._sleep(20_000_000)  # a few ms: every call below is queued before it ends
            for i in range(20):
                if before:
                    before(i)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                kv.kvoff_sparse_decode(case.ctx, case.rids, mode, case.q[0], case.pool, case.n_slots, bufs.table,
                                       bufs.sel_idx, bufs.sel_cnt, case.k_stride, scale, bufs.out,
                                       bufs.ws)
                e1.record()
                evs.append((e0, e1))
            torch.cuda.synchronize()
            ms = float(np.median([a.elapsed_time(b) for a, b in evs[5:]]))
            res[phase] = {"decode_us": round(ms * 1e3, 1), "tbps": round(nbytes / (ms * 1e-3) / 1e12, 2)}
        log(str(res))
        out.append(res)
        H.destroy(case)
        del case, bufs
        torch.cuda.empty_cache()
    print(json.dumps({"what": "kvoff_sparse_decode (attend_kernel + combine_kernel), event-timed, "
                              "median of 15 calls", "runs": out}), flush=True)


def attention_heads_report(args):
    """Sparse attention on the Llama-3-8B layer's records (batch 16, 8 KV
    heads, context 32768, top-64, 128 MiB) with 32, 64 and 128 query heads,
    i.e. G = 4, 8 and 16 query heads per KV head: the same bytes, G times the
    arithmetic.  Per G, 20 decode calls queued behind a spin kernel, warm;
    event-timed, median of the last 15 (a kernel trace of this report splits
    by attend_kernel's first template argument, G)."""
    out = []
    for hq in (32, 64, 128):
        sp = synth.spec("llama3-8b-layer", Hq=hq)
        reqs = synth.request_draws(sp)
        log(f"generating '{sp.name}' with {hq} query heads")
        case = H.build_case(sp, lambda key: synth.gen_layer_request(sp, key[0], key[1], reqs[key[1]]),
                            [0], reqs, keep=lambda l, r: False)
        mode = kv.KVOFF_SOLOHEAD
        bufs = H.make_buffers(case, mode)
        topk = [rq.k for rq in reqs]
        kv.kvoff_select(case.ctx, 0, case.rids, case.q[0], case.digest[0], case.nb_max, topk, mode,
                        bufs.scores, bufs.sel_idx, bufs.sel_cnt, case.k_stride)
        kv.kvoff_recall(case.ctx, 0, case.rids, mode, bufs.sel_idx, bufs.sel_cnt, case.k_stride,
                        None, None, 0, case.pool, case.n_slots, case.recall_base[0], bufs.table,
                        kv.KVOFF_ENGINE_ZEROCOPY)
        scale = 1.0 / math.sqrt(sp.d)
        nbytes = sum(min(rq.k, rq.nb) for rq in reqs) * kv.kvoff_record_bytes(case.ctx)
        evs = []
        torch.cuda.synchronize()
        torch.cuda._sleep(20_000_000)  # a few ms: every call below is queued before it ends
        for _ in range(20):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            kv.kvoff_sparse_decode(case.ctx, case.rids, mode, case.q[0], case.pool, case.n_slots, bufs.table,
                                   bufs.sel_idx, bufs.sel_cnt, case.k_stride, scale, bufs.out, bufs.ws)
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in evs[5:]]))
        res = {"q_heads": hq, "kv_heads": sp.Hkv, "G": hq // sp.Hkv, "records_read_bytes": nbytes,
               "decode_us": round(ms * 1e3, 1), "tbps": round(nbytes / (ms * 1e-3) / 1e12, 2)}
        log(str(res))
        out.append(res)
        H.destroy(case)
        del case, bufs
        torch.cuda.empty_cache()
    print(json.dumps({"what": "kvoff_sparse_decode (attend_kernel + combine_kernel), warm, "
                              "event-timed, median of 15 calls", "runs": out}), flush=True)


def decode32_report(args):
    """The 32-layer decode step (batch 8, context 32768, top-64 per layer,
    about 34 GB of pinned host KV): kvoff_step over all layers with recall of
    layer l+1 on a copy stream under select/attention of layer l, against the
    same step on one stream.  Warm: each figure is the mean of 10 steps after
    one untimed step."""
    sp = synth.spec(3)
    reqs = synth.request_draws(sp)
    B, L = len(reqs), sp.L
    layers = list(range(L))
    t0 = time.time()
    log(f"generating and offloading {L} layers x {B} requests")
    case = H.build_case(sp, lambda key: synth.gen_layer_request(sp, key[0], key[1], reqs[key[1]]),
                        layers, reqs, keep=lambda l, r: False)
    log(f"offloaded in {time.time() - t0:.1f} s")
    mode = kv.KVOFF_SOLOHEAD
    sets = [H.make_buffers(case, mode) for _ in range(2)]
    outs = [torch.empty_like(sets[0].out) for _ in layers]
    compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
    topk = [rq.k for rq in reqs]

    def step(copy_stream, want_stats=False, timing=False, grp=0):
        return kv.kvoff_step(
            case.ctx, layer_begin=0, layer_end=L, req_ids=case.rids, topk=topk, mode=mode,
            engine=kv.KVOFF_ENGINE_ZEROCOPY, k_stride=case.k_stride,
            q=[case.q[l] for l in layers], digest=[case.digest[l] for l in layers],
            digest_stride=case.nb_max, slot_pool=case.pool, n_slots=case.n_slots,
            recall_base_slot=case.recall_base, scores=[b.scores for b in sets],
            sel_idx=[b.sel_idx for b in sets], sel_cnt=[b.sel_cnt for b in sets],
            block_table=[b.table for b in sets], scale=1.0 / math.sqrt(sp.d), out=outs,
            ws=sets[0].ws, compute_stream=compute, copy_stream=copy_stream,
            want_stats=want_stats, want_timing=timing, group_requests=grp)

    def timed(copy_stream, n=10, grp=0):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        first = time.perf_counter()
        step(copy_stream, grp=grp)
        torch.cuda.synchronize()
        cold_ms = (time.perf_counter() - first) * 1e3
        e0.record(compute)
        for _ in range(n):
            step(copy_stream, grp=grp)
        e1.record(compute)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, cold_ms

    st = step(copy, want_stats=True)
    over_ms, cold_ms = timed(copy)
    serial_ms, _ = timed(compute)
    grp_ms, _ = timed(copy, grp=1)
    # the overlapped step captured into a HIP graph on the compute stream and
    # replayed (the same kernels and bytes; no host launch cost)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=compute):
        step(copy)
    torch.cuda.synchronize()
    with torch.cuda.stream(compute):
        g.replay()
    torch.cuda.synchronize()
    eg0, eg1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(compute):  # replay() launches on the current stream
        eg0.record()
        for _ in range(10):
            g.replay()
        eg1.record()
    torch.cuda.synchronize()
    graph_ms = eg0.elapsed_time(eg1) / 10
    del g
    tm = step(copy, timing=True, grp=1)["timing"]
    copy_peak, _ = link_peaks(case)
    ideal_ms = st["bytes"] / (copy_peak * 1e9) * 1e3
    res = {"workload": f"{sp.name}: batch {B}, {L} layers, {sp.Hq}/{sp.Hkv} heads, context "
                       f"{reqs[0].ctx}, block {sp.bs}, top-{reqs[0].k} per layer, zero-copy recall",
           "recalled_bytes_per_step": st["bytes"],
           "overlapped": {"ms_per_step": round(over_ms, 3),
                          "layer_steps_per_s": round(L * 1e3 / over_ms, 1)},
           "serial_one_stream": {"ms_per_step": round(serial_ms, 3),
                                 "layer_steps_per_s": round(L * 1e3 / serial_ms, 1)},
           "overlapped_request_groups_of_1": {
               "ms_per_step": round(grp_ms, 3), "layer_steps_per_s": round(L * 1e3 / grp_ms, 1),
               "mean_request_done_ms": round(tm["mean_request_done_ms"], 3)},
           "overlapped_graph_replay": {"ms_per_step": round(graph_ms, 3),
                                       "layer_steps_per_s": round(L * 1e3 / graph_ms, 1)},
           "first_step_cold_ms": round(cold_ms, 2),
           "link_bound": {"pinned_memcpy_gbps": round(copy_peak, 2), "ms_per_step": round(ideal_ms, 3),
                          "layer_steps_per_s": round(L * 1e3 / ideal_ms, 1)},
           "overlapped_frac_of_link_bound": round(ideal_ms / over_ms, 4),
           "graph_replay_frac_of_link_bound": round(ideal_ms / graph_ms, 4)}
    H.destroy(case)
    print(json.dumps(res), flush=True)


def attend_read_bytes(sp, reqs, rec_bytes):
    """Bytes the attention must read: the selected records and the queries."""
    return sum(min(rq.k, rq.nb) for rq in reqs) * rec_bytes + len(reqs) * sp.Hq * sp.d * sp.es


def score_read_bytes(sp, reqs, sets=1):
    """Bytes the score kernel must move: digests and queries read, fp64
    scores written."""
    nb_tot = sum(rq.nb for rq in reqs)
    return nb_tot * sp.Hkv * sp.d * 4 + len(reqs) * sp.Hq * sp.d * sp.es + nb_tot * sets * 8


def kernel_rate(ms, nbytes):
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"avg_us": round(ms * 1e3, 2), "algorithmic_bytes": nbytes, "hbm_gbps": round(gbps, 1),
            "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}


def recall_engines(case, layer, mode, with_pool, n=10):
    """Recall of one layer with each engine: wall clock around n calls after
    a stats call and two untimed ones (stream synchronised before and after),
    transfers and mean transfer size from the stats."""
    topk = [rq.k for rq in case.reqs]
    bufs = H.make_buffers(case, mode)
    kv.kvoff_select(case.ctx, layer, case.rids, case.q[layer], case.digest[layer], case.nb_max,
                    topk, mode, bufs.scores, bufs.sel_idx, bufs.sel_cnt, case.k_stride)
    out = {}
    for engine, ename in ((kv.KVOFF_ENGINE_ZEROCOPY, "zerocopy"), (kv.KVOFF_ENGINE_DMA, "dma"),
                          (kv.KVOFF_ENGINE_STAGED, "staged")):
        def rec(stats=False):
            return kv.kvoff_recall(case.ctx, layer, case.rids, mode, bufs.sel_idx, bufs.sel_cnt,
                                   case.k_stride, case.pool_hit.get(layer) if with_pool else None,
                                   case.pool_slot.get(layer) if with_pool else None, case.nb_max,
                                   case.pool, case.n_slots, case.recall_base[0], bufs.table, engine,
                                   want_stats=stats)
        st = rec(True)
        rec()
        rec()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(n):
            rec()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t) * 1e3 / n
        out[ename] = {"ms": round(ms, 4), "gbps": round(st["bytes"] / (ms * 1e-3) / 1e9, 2),
                      "bytes": st["bytes"], "transfers": st["transfers"],
                      "mean_transfer_kib": round(st["bytes"] / max(1, st["transfers"]) / 1024, 2)}
    return out


def co_runner(case, layer, mode):
    """What each recall engine costs a kernel running beside it: a fixed
    HBM-bound kernel (kvoff_probe_read over a 1 GiB device buffer, 2048
    workgroups) timed alone, then a batch of the same reads on a second
    stream with one recall issued right behind it on the recall stream (the
    batch lasts about three recalls, so the recall runs inside it).  Reports
    the reads' HBM rate alone and beside each engine, and each recall's own
    rate alone and with the reads beside it."""
    topk = [rq.k for rq in case.reqs]
    bufs = H.make_buffers(case, mode)
    kv.kvoff_select(case.ctx, layer, case.rids, case.q[layer], case.digest[layer], case.nb_max,
                    topk, mode, bufs.scores, bufs.sel_idx, bufs.sel_cnt, case.k_stride)
    nbytes = 1 << 30
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(4096, dtype=torch.uint8, device="cuda")
    rs, ps = torch.cuda.Stream(), torch.cuda.Stream()

    def reads(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(ps)
        for _ in range(n):
            kv.kvoff_probe_read(buf, nbytes, sink, 2048, stream=ps)
        e1.record(ps)
        return e0, e1

    def recall(engine, stats=False):
        return kv.kvoff_recall(case.ctx, layer, case.rids, mode, bufs.sel_idx, bufs.sel_cnt,
                               case.k_stride, None, None, 0, case.pool, case.n_slots,
                               case.recall_base[0], bufs.table, engine, want_stats=stats,
                               stream=rs)

    torch.cuda.synchronize()
    e0, e1 = reads(3)
    e0, e1 = reads(20)
    torch.cuda.synchronize()
    read_ms = e0.elapsed_time(e1) / 20
    res = {"kernel": "kvoff_probe_read: 1 GiB of HBM, 2048 workgroups",
           "alone_gbps": round(nbytes / (read_ms * 1e-3) / 1e9, 1), "engines": {}}
    for engine, ename in ((kv.KVOFF_ENGINE_ZEROCOPY, "zerocopy"), (kv.KVOFF_ENGINE_DMA, "dma"),
                          (kv.KVOFF_ENGINE_STAGED, "staged")):
        st = recall(engine, True)
        torch.cuda.synchronize()
        t = time.perf_counter()
        recall(engine)
        torch.cuda.synchronize()
        alone = (time.perf_counter() - t) * 1e3
        n = max(4, int(math.ceil(3 * alone / read_ms)))
        e0, e1 = reads(n)
        t = time.perf_counter()
        recall(engine)
        rs.synchronize()
        beside = (time.perf_counter() - t) * 1e3
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        res["engines"][ename] = {
            "reads_beside_gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "reads_slowdown": round(ms / read_ms, 3),
            "recall_alone_gbps": round(st["bytes"] / (alone * 1e-3) / 1e9, 2),
            "recall_beside_reads_gbps": round(st["bytes"] / (beside * 1e-3) / 1e9, 2)}
    del buf
    return res


# Layers each extra workload rotates through (tiny and headwise-vs-SoloHead:
# 4, as the headline, so no step finds its digests in the MALL; the 32-layer
# step: all 32; variable recall: one 9 GB layer, whose 272 MiB of digests
# exceed the MALL by themselves).
CONFIG_LAYERS = {1: 4, 3: 32, 4: 1, 5: 4}


def measure_config(num, args, link_peak):
    """One workload's entry of the configs object: layer-steps/s through
    kvoff_step, recall GB/s against the measured link peak, score and
    attention kernel HBM rates from events bound to each dispatch, and the
    oracle's baseline on host cores."""
    L = CONFIG_LAYERS[num]
    sp = synth.spec(num, L=L)
    reqs = synth.request_draws(sp)
    B = len(reqs)
    layers = list(range(L))
    pool = sp.pool_frac > 0
    want_cpu = not args.no_cpu_baseline
    t0 = time.time()
    log(f"[config {num}] generating and offloading {L} layers x {B} requests of '{sp.name}'")
    case = H.build_case(sp, lambda key: synth.gen_layer_request(sp, key[0], key[1], reqs[key[1]]),
                        layers, reqs, keep=lambda l, r: want_cpu and l == 0, with_pool_hits=pool)
    log(f"[config {num}] set up in {time.time() - t0:.1f} s")
    mode, engine = kv.KVOFF_SOLOHEAD, kv.KVOFF_ENGINE_ZEROCOPY
    topk = [rq.k for rq in reqs]
    scale = 1.0 / math.sqrt(sp.d)
    stream = torch.cuda.current_stream()
    sets = [H.make_buffers(case, mode) for _ in range(2)]
    bufs = sets[0]
    rec_bytes = kv.kvoff_record_bytes(case.ctx)

    def serial(l, evs=None):
        if evs:
            evs[0].record(stream)
        kv.kvoff_select(case.ctx, l, case.rids, case.q[l], case.digest[l], case.nb_max, topk, mode,
                        bufs.scores, bufs.sel_idx, bufs.sel_cnt, case.k_stride, stream=stream)
        if evs:
            evs[1].record(stream)
        kv.kvoff_recall(case.ctx, l, case.rids, mode, bufs.sel_idx, bufs.sel_cnt, case.k_stride,
                        case.pool_hit.get(l) if pool else None,
                        case.pool_slot.get(l) if pool else None, case.nb_max, case.pool,
                        case.n_slots, case.recall_base[0], bufs.table, engine, stream=stream)
        if evs:
            evs[2].record(stream)
        kv.kvoff_sparse_decode(case.ctx, case.rids, mode, case.q[l], case.pool, case.n_slots,
                               bufs.table, bufs.sel_idx, bufs.sel_cnt, case.k_stride, scale,
                               bufs.out, bufs.ws, stream=stream)
        if evs:
            evs[3].record(stream)

    n_serial = L * max(1, -(-args.steps // L))
    for i in range(min(args.warmup, n_serial)):
        serial(layers[i % L])
    torch.cuda.synchronize()
    # per-layer recalled bytes (pool hits are not moved)
    rec_by_layer = {}
    for l in layers:
        kv.kvoff_select(case.ctx, l, case.rids, case.q[l], case.digest[l], case.nb_max, topk, mode,
                        bufs.scores, bufs.sel_idx, bufs.sel_cnt, case.k_stride)
        st = kv.kvoff_recall(case.ctx, l, case.rids, mode, bufs.sel_idx, bufs.sel_cnt,
                             case.k_stride, case.pool_hit.get(l) if pool else None,
                             case.pool_slot.get(l) if pool else None, case.nb_max, case.pool,
                             case.n_slots, case.recall_base[0], bufs.table, engine, want_stats=True)
        rec_by_layer[l] = st
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_serial)]
    t = time.perf_counter()
    for i in range(n_serial):
        serial(layers[i % L], ev[i])
    torch.cuda.synchronize()
    serial_ms = (time.perf_counter() - t) * 1e3 / n_serial
    rec_ms = [e[1].elapsed_time(e[2]) for e in ev]
    rec_gbps = float(np.mean([rec_by_layer[layers[i % L]]["bytes"] / (rec_ms[i] * 1e-3) / 1e9
                              for i in range(n_serial)]))
    kv.kvoff_set_kernel_timing(case.ctx, True)
    for i in range(n_serial):
        serial(layers[i % L])
    km = kv.kvoff_get_kernel_times(case.ctx)
    kv.kvoff_set_kernel_timing(case.ctx, False)
    outs = [torch.empty_like(bufs.out) for _ in layers]
    copy = torch.cuda.Stream()

    def step(n_layers=L):
        return kv.kvoff_step(
            case.ctx, layer_begin=0, layer_end=n_layers, req_ids=case.rids, topk=topk, mode=mode,
            engine=engine, k_stride=case.k_stride, q=[case.q[l] for l in layers],
            digest=[case.digest[l] for l in layers], digest_stride=case.nb_max,
            slot_pool=case.pool, n_slots=case.n_slots, recall_base_slot=case.recall_base,
            scores=[b.scores for b in sets], sel_idx=[b.sel_idx for b in sets],
            sel_cnt=[b.sel_cnt for b in sets], block_table=[b.table for b in sets], scale=scale,
            out=outs, ws=bufs.ws, pool_hit=[case.pool_hit[l] for l in layers] if pool else None,
            pool_slot=[case.pool_slot[l] for l in layers] if pool else None,
            pool_stride=case.nb_max, compute_stream=stream, copy_stream=copy)

    n_calls = max(3, args.steps // 4) if L == 32 else max(1, -(-args.steps // L))
    step()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(n_calls):
        step()
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t) * 1e3 / (n_calls * L)
    per_step_bytes = float(np.mean([rec_by_layer[l]["bytes"] for l in layers]))
    entry = {
        "workload": f"{sp.name}: batch {B}, {sp.Hq}/{sp.Hkv} heads, head_dim {sp.d}, "
                    + (f"contexts {min(rq.ctx for rq in reqs)}-{max(rq.ctx for rq in reqs)}, "
                       f"top-k {min(topk)}-{max(topk)} blocks"
                       if sp.ctx_range else f"context {reqs[0].ctx}, top-{reqs[0].k}")
                    + f", block {sp.bs}, {'bf16' if sp.dtype == synth.BF16 else 'fp16'}"
                    + (f", {int(sp.pool_frac * 100)}% of blocks resident in the HBM pool"
                       if pool else "")
                    + (", one full decode step of 32 layers" if L == 32
                       else f", {L} rotating layers" if L > 1 else ", one layer"),
        "layer_steps_per_s": round(1e3 / step_ms, 3),
        "ms_per_layer_step": round(step_ms, 4),
        "schedule": f"kvoff_step over the {L} layers, {n_calls} calls: recall of layer l+1 on "
                    "two copy streams under select/attention of layer l" if L > 1
                    else f"kvoff_step over the one layer, {n_calls} calls",
        "serial_one_stream": {"layer_steps_per_s": round(1e3 / serial_ms, 3),
                              "ms_per_layer_step": round(serial_ms, 4)},
        "recall": {"bytes_per_layer_step": int(per_step_bytes), "gbps": round(rec_gbps, 2),
                   "frac_of_measured_link_peak": round(rec_gbps / link_peak, 4),
                   "how": f"events around each recall, {n_serial} layer-steps in serial order"},
        "kernels": {"score_kernel": kernel_rate(km["score_ms"], score_read_bytes(sp, reqs)),
                    "topk_kernel": {"avg_us": round(km["topk_ms"] * 1e3, 2)},
                    "attend_kernel": kernel_rate(km["attend_ms"],
                                                 attend_read_bytes(sp, reqs, rec_bytes)),
                    "combine_kernel": {"avg_us": round(km["combine_ms"] * 1e3, 2)},
                    "bytes": "score: digests and queries read, scores written; attention: "
                             "selected records and queries read",
                    "how": f"events bound to each dispatch, mean of {n_serial} serial layer-steps"},
    }
    if L == 32:
        entry["decode_step_ms"] = round(step_ms * L, 3)
        entry["recall"]["in_kvoff_step_gbps"] = round(per_step_bytes / (step_ms * 1e-3) / 1e9, 2)
    if pool:
        st = rec_by_layer[0]
        entry["recall"]["pool_hits"] = st["pool_hits"]
        entry["fragmentation"] = {
            "solohead": recall_engines(case, 0, kv.KVOFF_SOLOHEAD, True),
            "headwise": recall_engines(case, 0, kv.KVOFF_HEADWISE, True),
            "how": "layer 0 with its pool hits, wall clock around 10 recalls per engine"}
    if num == 4:
        entry["recall_engines"] = recall_engines(case, 0, mode, False)
    if want_cpu:
        log(f"[config {num}] timing the oracle on host cores")
        cpu = cpu_baseline(sp, case.inputs, B, args.config_cpu_seconds,
                           keys=[(0, r) for r in range(B)])
        if L == 32:
            cpu["decode_step_s"] = round(L / cpu["value"], 3)
            cpu["single_thread"]["decode_step_s"] = round(L / cpu["single_thread"]["value"], 3)
            cpu["sample"] += "; a 32-layer decode step is 32 such layer-steps"
        entry["cpu_baseline"] = cpu
    H.destroy(case)
    del case, sets, bufs, outs
    torch.cuda.empty_cache()
    log(f"[config {num}] {entry['layer_steps_per_s']} layer-steps/s in {time.time() - t0:.1f} s")
    return entry


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by request with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.report == "fragmentation":
        return fragmentation_report(args)
    if args.report == "admission":
        return admission_report(args)
    if args.report == "groups":
        return groups_report(args)
    if args.report == "mass":
        return mass_report(args)
    if args.report == "decode32":
        return decode32_report(args)
    if args.report == "attention-cache":
        return attention_cache_report(args)
    if args.report == "attention-heads":
        return attention_heads_report(args)
    if args.report == "select-modes":
        return select_modes_report(args)
    sp = synth.spec(args.config if args.config else args.workload, L=args.layers)
    reqs = synth.request_draws(sp)
    B = len(reqs)
    layers = list(range(args.layers))
    t0 = time.time()
    inputs = {}
    keep_cpu = not args.no_cpu_baseline
    log(f"generating {len(layers)} layers x {B} requests of '{sp.name}'")
    for l in layers:
        for r, rq in enumerate(reqs):
            inputs[(l, r)] = synth.gen_layer_request(sp, l, r, rq)
    log(f"generated in {time.time() - t0:.1f} s; offloading")
    engine = {"zerocopy": kv.KVOFF_ENGINE_ZEROCOPY, "dma": kv.KVOFF_ENGINE_DMA,
              "staged": kv.KVOFF_ENGINE_STAGED}[args.engine]
    host_kind = kv.KVOFF_HOST_NONCOHERENT if args.host_mem == "noncoherent" else kv.KVOFF_HOST_COHERENT
    case = H.build_case(sp, inputs, layers, reqs, host_kind=host_kind, two_regions=True)
    kv.kvoff_set_attention_qk(case.ctx, kv.KVOFF_QK_VALU if args.attn_qk == "valu" else kv.KVOFF_QK_MFMA)
    for k in [k for k in inputs if k[0] != 0]:  # layer 0: the offload timing and CPU baseline
        del inputs[k]
    log(f"setup done in {time.time() - t0:.1f} s")

    mode = kv.KVOFF_SOLOHEAD
    bufs = H.make_buffers(case, mode)
    topk = [rq.k for rq in reqs]
    scale = 1.0 / math.sqrt(sp.d)
    stream = torch.cuda.current_stream()
    n_ev = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_ev)]

    def one_step(i, evs=None):
        l = layers[i % len(layers)]
        if evs:
            evs[0].record(stream)
        kv.kvoff_select(case.ctx, l, case.rids, case.q[l], case.digest[l], case.nb_max, topk, mode,
                        bufs.scores, bufs.sel_idx, bufs.sel_cnt, case.k_stride, stream=stream)
        if evs:
            evs[1].record(stream)
        kv.kvoff_recall(case.ctx, l, case.rids, mode, bufs.sel_idx, bufs.sel_cnt, case.k_stride,
                        None, None, 0, case.pool, case.n_slots, case.recall_base[0], bufs.table,
                        engine, stream=stream)
        if evs:
            evs[2].record(stream)
        kv.kvoff_sparse_decode(case.ctx, case.rids, mode, case.q[l], case.pool, case.n_slots, bufs.table,
                               bufs.sel_idx, bufs.sel_cnt, case.k_stride, scale, bufs.out,
                               bufs.ws, stream=stream)
        if evs:
            evs[3].record(stream)

    # 1) the serial order on one stream, with events around each phase: the
    #    per-phase and per-kernel figures (not the headline)
    for i in range(args.warmup):
        one_step(i)
    torch.cuda.synchronize()
    log(f"timing {args.steps} serial layer-steps")
    t_start = time.perf_counter()
    for i in range(args.steps):
        one_step(args.warmup + i, ev[i])
    torch.cuda.synchronize()
    serial_ms = (time.perf_counter() - t_start) * 1e3 / args.steps
    sel_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    rec_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    att_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    # 1b) per-kernel durations: the serial layer-steps again, each kernel
    #     launched with start and stop events bound to its own dispatch
    #     (kvoff_set_kernel_timing; the library averages over the calls)
    kv.kvoff_set_kernel_timing(case.ctx, True)
    for i in range(args.steps):
        one_step(args.warmup + i)
    kern_ms = kv.kvoff_get_kernel_times(case.ctx)
    kv.kvoff_set_kernel_timing(case.ctx, False)
    assert kern_ms["select_calls"] == kern_ms["decode_calls"] == args.steps, kern_ms
    # 1c) the same kernels with their inputs in HBM only: a 1 GiB read of an
    #     unrelated buffer before each select and each attention evicts the
    #     256 MB MALL (the reads are not inside the kernels' events)
    flush = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.empty(4096, dtype=torch.uint8, device="cuda")

    def one_step_clean(i):
        l = layers[i % len(layers)]
        kv.kvoff_probe_read(flush, flush.numel(), sink, 2048, stream=stream)
        kv.kvoff_select(case.ctx, l, case.rids, case.q[l], case.digest[l], case.nb_max, topk, mode,
                        bufs.scores, bufs.sel_idx, bufs.sel_cnt, case.k_stride, stream=stream)
        kv.kvoff_recall(case.ctx, l, case.rids, mode, bufs.sel_idx, bufs.sel_cnt, case.k_stride,
                        None, None, 0, case.pool, case.n_slots, case.recall_base[0], bufs.table,
                        engine, stream=stream)
        kv.kvoff_probe_read(flush, flush.numel(), sink, 2048, stream=stream)
        kv.kvoff_sparse_decode(case.ctx, case.rids, mode, case.q[l], case.pool, case.n_slots,
                               bufs.table, bufs.sel_idx, bufs.sel_cnt, case.k_stride, scale,
                               bufs.out, bufs.ws, stream=stream)

    kv.kvoff_set_kernel_timing(case.ctx, True)
    for i in range(args.steps):
        one_step_clean(args.warmup + i)
    kern_clean = kv.kvoff_get_kernel_times(case.ctx)
    kv.kvoff_set_kernel_timing(case.ctx, False)
    del flush

    # 2) the headline: kvoff_step over the rotating layers, recall of layer
    #    l+1 on the copy streams under select/attention of layer l; one call
    #    is up to len(layers) layer-steps
    sets = [bufs, H.make_buffers(case, mode)]
    outs = [torch.empty_like(bufs.out) for _ in layers]
    copy = torch.cuda.Stream()

    def step_all(timing=False, n_layers=None, cs=None):
        return kv.kvoff_step(
            case.ctx, layer_begin=0, layer_end=n_layers or len(layers), req_ids=case.rids,
            topk=topk, mode=mode, engine=engine, k_stride=case.k_stride,
            q=[case.q[l] for l in layers], digest=[case.digest[l] for l in layers],
            digest_stride=case.nb_max, slot_pool=case.pool, n_slots=case.n_slots,
            recall_base_slot=case.recall_base, scores=[b.scores for b in sets],
            sel_idx=[b.sel_idx for b in sets], sel_cnt=[b.sel_cnt for b in sets],
            block_table=[b.table for b in sets], scale=scale, out=outs, ws=bufs.ws,
            compute_stream=cs or stream, copy_stream=copy, want_timing=timing)

    def run_steps(n):
        for n_layers in step_calls(n, len(layers)):
            step_all(n_layers=n_layers)

    steps_timed, warm_timed = args.steps, args.warmup
    graph_replay = None
    if args.no_overlap:
        ms_per_step = serial_ms
    else:
        n_calls = max(1, args.steps // len(layers))
        run_steps(args.warmup)
        torch.cuda.synchronize()
        log(f"timing {steps_timed} layer-steps through kvoff_step")
        t_o = time.perf_counter()
        run_steps(args.steps)
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t_o) * 1e3 / steps_timed
        # the recall's duration per launch inside this schedule: the same
        # calls again, with kvoff_step's timing events around each recall on
        # the copy streams it runs on
        rec_sum, rec_n = 0.0, 0
        for _ in range(n_calls):
            t = step_all(timing=True)["timing"]
            rec_sum += t["recall_ms"]
            rec_n += t["recalls"]
        rec_ms_step = rec_sum / rec_n
        # the same schedule replayed from a HIP graph: one kvoff_step call
        # over the layers, captured once on its compute stream (the copy
        # streams join through the step's events).  Zero-copy engine only:
        # the copy engines synchronise the host inside the call.
        if engine == kv.KVOFF_ENGINE_ZEROCOPY:
            gs = torch.cuda.Stream()
            step_all(cs=gs)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=gs):
                step_all(cs=gs)
            torch.cuda.synchronize()
            for _ in range(max(1, args.warmup // len(layers))):
                g.replay()
            torch.cuda.synchronize()
            t_g = time.perf_counter()
            for _ in range(n_calls):
                g.replay()
            torch.cuda.synchronize()
            graph_ms = (time.perf_counter() - t_g) * 1e3 / (n_calls * len(layers))
            graph_replay = {"layer_steps_per_s": round(1e3 / graph_ms, 3), "ms_per_step": round(graph_ms, 4),
                            "how": f"one kvoff_step call over the {len(layers)} layers captured into a HIP "
                                   f"graph, replayed {n_calls} times"}
            del g

    # algorithmic bytes per layer-step
    rec_bytes = kv.kvoff_record_bytes(case.ctx)
    nb_tot = sum(rq.nb for rq in reqs)
    K_tot = sum(min(rq.k, rq.nb) for rq in reqs)
    score_bytes = nb_tot * sp.Hkv * sp.d * 4 + B * sp.Hq * sp.d * sp.es + nb_tot * 8
    recall_bytes = K_tot * rec_bytes
    ws_bytes = kv.kvoff_workspace_size(case.ctx, kv.KVOFF_CALL_SPARSE_DECODE, B, case.k_stride, mode)
    attend_bytes = K_tot * rec_bytes + B * sp.Hq * sp.d * (sp.es + 4) + 2 * ws_bytes
    # the attention kernel alone: records and queries read, split partials
    # written (the whole workspace when every split has blocks, as here)
    attend_kernel_bytes = K_tot * rec_bytes + B * sp.Hq * sp.d * sp.es + ws_bytes

    def kernel_entry(name, nbytes=None):
        ms = kern_ms[name]
        e = {"avg_us": round(ms * 1e3, 2)}
        if nbytes is not None:
            gbps = nbytes / (ms * 1e-3) / 1e9
            e.update({"algorithmic_bytes": nbytes, "hbm_gbps": round(gbps, 1),
                      "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)})
        return e

    # The roofline takes the gather as it runs alone (serial order, one
    # stream).  In the kvoff_step schedule the recalls of consecutive layers
    # run two at a time on the two copy streams, so a launch lasts longer
    # while the link moves the same bytes per second; that schedule's link
    # rate is reported beside it.
    recall_gbps = recall_bytes / (rec_ms * 1e-3) / 1e9
    roof_ms, roof_gbps = rec_ms, recall_gbps
    log("measuring link and HBM copy peaks")
    copy_peak, probe_peak = link_peaks(case)
    link_peak = max(copy_peak, probe_peak)
    hbm_copy = hbm_copy_peak()
    hbm_read = hbm_read_peak()
    result = {
        "metric": METRIC,
        "value": round(1e3 / ms_per_step, 3),
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": steps_timed,
        "warmup": warm_timed,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if sp.dtype == synth.BF16 else "f16",
        "data": "synthetic",
        "config": {
            "workload": f"{sp.name}: batch {B}, {sp.Hq}/{sp.Hkv} heads, head_dim {sp.d}, "
                        f"context {reqs[0].ctx}, block {sp.bs}, top-{reqs[0].k}, "
                        f"{len(layers)} rotating layers",
            "schedule": "one stream, select -> recall -> attend per layer" if args.no_overlap
            else f"kvoff_step over the {len(layers)} layers: recall of layer l+1 on two copy "
                 "streams under select/attention of layer l",
            "engine": args.engine, "host_mem": args.host_mem, "attn_qk": args.attn_qk,
            "global_batch": B, "seq_len": reqs[0].ctx,
        },
        "roofline": {
            "kernel": {0: "gather_kernel (zero-copy recall)", 1: "hipMemcpyAsync per run",
                       2: "CPU gather + bulk hipMemcpyAsync"}[engine],
            "bound": "pcie", "achieved": round(roof_gbps, 2), "peak": PCIE_PEAK_GBPS,
            "unit": "GB/s", "frac": round(roof_gbps / PCIE_PEAK_GBPS, 4),
            "traffic": gather_traffic_bytes(sp.name, args.layers)
            if engine == kv.KVOFF_ENGINE_ZEROCOPY else None,
            "traffic_note": "counter bytes per launch: host-link fetches + HBM writes "
                            "(a copy moves each byte twice)",
            "traffic_from": "rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE passes over this command "
                            "with the current recall.hip (profiles/llama3-8b-layer_pmc_traffic.md), "
                            "stored in bench.py, not counted in this run; null when recall.hip "
                            "has changed since",
            "algorithmic_bytes": recall_bytes, "avg_ms": round(roof_ms, 4),
            "avg_ms_from": "HIP events around each recall, the layers in serial order on one stream",
            "frac_of_measured_link_peak": round(roof_gbps / link_peak, 4),
            "in_kvoff_step": None if args.no_overlap else {
                "avg_launch_ms": round(rec_ms_step, 4),
                "link_gbps": round(recall_bytes / (ms_per_step * 1e-3) / 1e9, 2),
                "note": "recalls of consecutive layers overlap on the two copy streams: "
                        "launches last longer, the link rate is recalled bytes per layer-step "
                        "over the time per layer-step"},
        },
        "phases": {
            "select": {"kernels": "score_kernel + topk_kernel", "avg_ms": round(sel_ms, 4),
                       "algorithmic_bytes": score_bytes,
                       "hbm_gbps": round(score_bytes / (sel_ms * 1e-3) / 1e9, 1),
                       "frac_of_hbm_peak": round(score_bytes / (sel_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
            "recall": {"avg_ms": round(rec_ms, 4), "bytes": recall_bytes,
                       "gbps": round(recall_gbps, 2)},
            "attend": {"kernels": "attend_kernel + combine_kernel", "avg_ms": round(att_ms, 4),
                       "algorithmic_bytes": attend_bytes,
                       "hbm_gbps": round(attend_bytes / (att_ms * 1e-3) / 1e9, 1),
                       "frac_of_hbm_peak": round(attend_bytes / (att_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        },
        "kernels": {
            "score_kernel": kernel_entry("score_ms", score_bytes),
            "topk_kernel": kernel_entry("topk_ms"),
            "attend_kernel": {**kernel_entry("attend_ms", attend_kernel_bytes),
                              "input": "warm: the records the recall wrote just before, part of "
                                       "them still in the 256 MB MALL (MALL-assisted, not an HBM "
                                       "rate; clean_hbm below is)"},
            "combine_kernel": kernel_entry("combine_ms"),
            "how": f"start/stop events bound to each kernel's dispatch (kvoff_set_kernel_timing), "
                   f"serial order on one stream, mean of {args.steps} layer-steps",
            "clean_hbm": {
                "score_kernel": kernel_rate(kern_clean["score_ms"], score_bytes),
                "attend_kernel": kernel_rate(kern_clean["attend_ms"], attend_kernel_bytes),
                "how": "the same layer-steps with a 1 GiB read of an unrelated buffer before each "
                       "select and each attention: every input byte comes from HBM"},
        },
        "serial_one_stream": {"layer_steps_per_s": round(1e3 / serial_ms, 3),
                              "ms_per_step": round(serial_ms, 4),
                              "how": "select -> recall -> attend per layer on one stream, "
                                     "events around each phase (the phase figures above)"},
        "link_peak_gbps": {"pinned_memcpy_1GiB": round(copy_peak, 2),
                           "zero_copy_probe": round(probe_peak, 2)},
        "recall_frac_of_link_peak": round(roof_gbps / link_peak, 4),
        "hbm_copy_gbps_measured": round(hbm_copy, 1),
        "hbm_read_gbps_measured": round(hbm_read, 1),
    }
    if not args.no_overlap and graph_replay is not None:
        result["graph_replay"] = graph_replay
    result["offload_setup"] = offload_timing(case, sp, inputs, B)
    log("recall engines and their cost to a co-running HBM kernel")
    result["recall_engines"] = recall_engines(case, 0, mode, False)
    result["recall_engines"]["how"] = "layer 0, wall clock around 10 recalls per engine"
    result["co_runner"] = co_runner(case, 0, mode)
    if keep_cpu:
        log("timing the oracle on host cores")
        result["cpu_baseline"] = cpu_baseline(sp, inputs, B, args.cpu_seconds)
    H.destroy(case)
    del case, bufs, sets, outs, inputs
    torch.cuda.empty_cache()
    if args.config_list:
        link_peak = max(copy_peak, probe_peak)
        cfg = {"2": {"workload": result["config"]["workload"],
                     "layer_steps_per_s": result["value"], "ms_per_layer_step": result["ms_per_step"],
                     "schedule": result["config"]["schedule"],
                     "recall": {"bytes_per_layer_step": recall_bytes,
                                "gbps": result["roofline"]["achieved"],
                                "frac_of_measured_link_peak": result["recall_frac_of_link_peak"]},
                     "kernels": {k: result["kernels"][k] for k in ("score_kernel", "attend_kernel")},
                     "cpu_baseline": result.get("cpu_baseline"),
                     "note": "the headline workload: the figures of the line above"}}
        for num in args.config_list:
            cfg[str(num)] = measure_config(num, args, link_peak)
        result["configs"] = dict(sorted(cfg.items()))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
