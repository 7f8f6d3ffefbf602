"""Benchmark of the GQA attention backward hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic inputs
already resident in HBM: attn_fwd -> attn_bwd_preprocess -> attn_bwd ->
attn_bwd_postprocess, all through the C ABI on the current HIP stream.
``value`` is the backward throughput of the step: backward FLOPs (the
convention 2.5 x the forward's 4*B*Hq*N^2*D, halved for causal; sum of L^2
for varlen; visible pairs for a sliding window) divided by the HIP-event time
of the three backward launches.  The forward runs in every step (it produces
O and lse) and is reported separately.  The deterministic backward
(attn_bwd_preprocess without the accumulator -> attn_bwd_dkdv -> attn_bwd_dq,
no atomics) is timed on the same inputs and reported under "deterministic",
with the orientation path.select_mode picks for the shape, and the backward
as path.backward(mode="auto", kv_splits="auto") runs it under "auto".

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       [--n N] [--seed S] [--no-cpu-baseline] [--no-extra] [--only-extra KEY]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import attn_inputs as ai  # noqa: E402

METRIC = "attn_bwd TFLOP/s (fp16/bf16, causal GQA) + MFMA util vs MI355X peak"
PEAK_MFMA_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBS = 8000.0
# Device-wide rate of device-scope fp32 atomic adds, measured on MI355X with a
# microbenchmark (1.1-1.25 TB/s whatever the workgroup count, bytes per wave
# instruction, return / no return and working-set size).  bench.py measures
# it again on the machine it runs on (microbench/atomic_rate.hip); this figure
# is used only if that library is missing.
ATOMIC_CEILING_GBS = 1250.0
MICROBENCH_LIB = os.path.join(ROOT, "atomics_bwd_preprocess_amd", "libattn_microbench.so")
# Pages' number for this exact workload (triton issue "atomic_add slows down
# attention backwards": fp16, batch 4, 8 heads, d64, causal, N = 32768,
# atomic_add after vectorized atomics; other hardware -- context only).
PAGES_BASELINE = {("mha_causal", 32768): 242.346481}
BWD_SOURCE = os.path.join(ROOT, "atomics_bwd_preprocess_amd", "csrc", "bwd.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bwd_traffic.json")


def bwd_flops(x: dict) -> float:
    """Backward FLOPs of the main kernel: 10 * Hq * D * (visible pairs)."""
    lengths = np.asarray(x["lengths"], dtype=np.float64)
    hq, d, w = x["hq"], x["d"], x["window"]
    if w > 0:
        pairs = sum(float(np.minimum(np.arange(L) + 1, w).sum()) for L in x["lengths"])
    elif x["causal"]:
        pairs = float((lengths ** 2).sum()) / 2.0
    else:
        pairs = float((lengths ** 2).sum())
    return 10.0 * hq * d * pairs


def bwd_atomic_bytes(x: dict) -> float:
    """Bytes of fp32 dQ atomics the main kernel issues per launch: one
    BM x D sweep per (key block of 256, query head, query block the masks let
    see the key block), with BM = 32 at D = 128 and 64 at D = 64 -- the
    kernel's own schedule (rows past a sequence end are dropped by the
    hardware and not counted)."""
    bn, d, w = 256, x["d"], x["window"]
    bm = 32 if d == 128 else 64
    g = x["hq"] // x["hkv"]
    pairs = 0
    for L in x["lengths"]:
        for kv0 in range(0, L, bn):
            kv_last = min(L, kv0 + bn) - 1
            ib0 = kv0 // bm if x["causal"] else 0
            ib1 = (L + bm - 1) // bm
            if w > 0:
                ib1 = min(ib1, (kv_last + w - 1) // bm + 1)
            # rows actually inside the sequence
            for ib in range(ib0, ib1):
                pairs += min(bm, L - ib * bm)
    return float(pairs) * g * x["hkv"] * d * 4.0


def atomic_ceiling_gbs():
    """Live device-wide rate of device-scope fp32 atomic adds (GB/s of added
    data): 32768 waves each adding to a 256-byte segment per iteration over a
    256 MiB buffer, timed with HIP events over 20 launches after 0.3 s of
    warm-up launches."""
    import ctypes

    import torch

    if not os.path.exists(MICROBENCH_LIB):
        return None
    lib = ctypes.CDLL(MICROBENCH_LIB)
    f = lib.attn_microbench_atomic_rate
    f.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int
    nseg, blocks, iters, reps = 1 << 20, 8192, 64, 20
    buf = torch.zeros(nseg * 64, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    if f(buf.data_ptr(), nseg, blocks, iters, stream.cuda_stream) != 0:
        return None
    _warm(lambda: f(buf.data_ptr(), nseg, blocks, iters, stream.cuda_stream), 0, 0.3)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        f(buf.data_ptr(), nseg, blocks, iters, stream.cuda_stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    del buf
    return reps * blocks * 256 * iters * 4 / (ms * 1e-3) / 1e9


def copy_reference_gbs(mib: int = 1024) -> float:
    """Bytes moved (read + write) per second by a plain device-to-device copy
    of `mib` MiB through PyTorch: the practical ceiling for a kernel that
    reads and writes about as much as it reads."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, device="cuda", dtype=torch.float32)
    dst = torch.empty_like(src)
    dst.copy_(src)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    del src, dst
    return 2.0 * n * 4 / (ms * 1e-3) / 1e9


def bwd_flops_nominal(x: dict) -> float:
    """The stated formula without the window: 10 * Hq * D * sum(L^2) / 2 for
    causal (reported beside the visible-pair count for windowed workloads)."""
    y = dict(x)
    y["window"] = 0
    return bwd_flops(y)


def device_info() -> dict:
    import torch

    pr = torch.cuda.get_device_properties(0)
    info = {"name": pr.name, "compute_units": pr.multi_processor_count,
            "arch": getattr(pr, "gcnArchName", "")}
    clk = getattr(pr, "clock_rate", None)
    if clk:
        info["max_clock_mhz"] = round(clk / 1000.0)
    return info


def fwd_flops(x: dict) -> float:
    return bwd_flops(x) * 4.0 / 10.0


def prepost_bytes(x: dict) -> tuple:
    """Algorithmic HBM bytes of the preprocess and postprocess launches."""
    rows = float(sum(x["lengths"])) * x["hq"]
    d, e = x["d"], 2.0
    pre = rows * d * 2 * e + rows * 4 + rows * d * 4
    if x["sink"] is not None:
        pre += rows * 8
    post = rows * d * (4 + e)
    return pre, post


def compulsory_bytes(x: dict) -> float:
    """HBM bytes any backward must move at least once: read Q, K, V, O, dO
    (storage dtype) and lse; write dQ, dK, dV (storage dtype) and Delta.
    Their time at the HBM peak is the floor of the whole backward, whatever
    the orientation (the MFMA floor is the other one)."""
    T = float(sum(x["lengths"]))
    d, e = x["d"], 2.0
    q_side = T * x["hq"] * d * e  # one of Q, O, dO, dQ
    kv_side = T * x["hkv"] * d * e  # one of K, V, dK, dV
    return 4 * q_side + 4 * kv_side + 2 * 4 * T * x["hq"]


def _code_only(text: str) -> str:
    """C++ source without comments and blank lines (string literals in these
    files hold no comment markers)."""
    import re

    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())


def _source_hash() -> str:
    """Hash of the main kernel's code (comments and blank lines ignored)."""
    h = hashlib.sha256()
    for f in (BWD_SOURCE, os.path.join(os.path.dirname(BWD_SOURCE), "common.h")):
        h.update(_code_only(open(f).read()).encode())
    return h.hexdigest()[:16]


def _traffic(workload: str):
    """HBM traffic of the main kernel from committed rocprofv3 counters, if
    they were taken on the current kernel source; else None."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != _source_hash() or t.get("workload") != workload:
        return None
    return t.get("bytes_per_launch")


def _warm(fn, count: int, warm_s: float) -> float:
    """Run fn `count` times, then keep running it until warm_s seconds have
    passed (GPU clocks ramp up over a few hundred ms of load after the idle
    host-side input generation; short workloads measured 5-12 % slow with a
    fixed handful of warm-up steps).  Returns the wall time per call of the
    time-based part (0 if none ran)."""
    import torch

    for _ in range(count):
        fn()
    torch.cuda.synchronize()
    t0, n = time.perf_counter(), 0
    while time.perf_counter() - t0 < warm_s:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / n if n else 0.0


def run_gpu(x: dict, steps: int, warmup: int, layout: str = "thd", warm_s: float = 0.0,
            min_timed_s: float = 0.0) -> dict:
    """HIP-event times of every launch of the path on x.  The first section
    (forward, then the atomic backward) runs `warmup` untimed steps and then
    `steps` timed ones; with warm_s > 0 every section also warms up for that
    long first, and with min_timed_s > 0 the step count is raised (up to
    400) until the timed steps take about that long."""
    import torch

    from atomics_bwd_preprocess_amd import (attn_bwd, attn_bwd_dkdv, attn_bwd_dq,
                                            attn_bwd_fused_cast, attn_bwd_postprocess,
                                            attn_bwd_preprocess, fused_cast_counters, path)

    inp = path.to_device(x, "cuda", layout=layout)
    ws = path.workspace(inp)
    stream = torch.cuda.current_stream()
    per_step = _warm(lambda: path.step(inp, ws), warmup, warm_s)
    if min_timed_s > 0 and per_step > 0:
        steps = int(min(400, max(steps, math.ceil(min_timed_s / per_step))))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        e = ev[i]
        e[0].record(stream)
        path.forward(inp, ws)
        e[1].record(stream)
        attn_bwd_preprocess(inp.shape, ws.o, inp.do, ws.lse, inp.cu, inp.sink, ws.delta,
                            ws.dq_accum, ws.dsink)
        e[2].record(stream)
        attn_bwd(inp.shape, inp.q, inp.k, inp.v, inp.do, ws.lse, ws.delta, inp.cu, ws.dq_accum,
                 ws.dk, ws.dv)
        e[3].record(stream)
        attn_bwd_postprocess(inp.shape, ws.dq_accum, ws.dq)
        e[4].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([[e[k].elapsed_time(e[k + 1]) for k in range(4)] for e in ev])
    mean = ms.mean(axis=0)
    out = dict(wall_ms_per_step=1e3 * wall / steps, fwd_ms=float(mean[0]), pre_ms=float(mean[1]),
               bwd_ms=float(mean[2]), post_ms=float(mean[3]),
               bwd_ms_min=float(ms[:, 2].min()), bwd_ms_median=float(np.median(ms[:, 2])))
    out["steps"] = steps
    # The same backward with the dQ cast fused into the main pass (the last
    # workgroup contributing to a query block casts it; causal problems).
    counters = torch.empty(fused_cast_counters(inp.shape), dtype=torch.int32, device="cuda")

    def fused():
        attn_bwd_preprocess(inp.shape, ws.o, inp.do, ws.lse, inp.cu, inp.sink, ws.delta,
                            ws.dq_accum, ws.dsink)
        attn_bwd_fused_cast(inp.shape, inp.q, inp.k, inp.v, inp.do, ws.lse, ws.delta, inp.cu,
                            ws.dq_accum, counters, ws.dq, ws.dk, ws.dv)

    _warm(fused, 2, warm_s)
    for i in range(steps):
        e = ev[i]
        e[0].record(stream)
        attn_bwd_preprocess(inp.shape, ws.o, inp.do, ws.lse, inp.cu, inp.sink, ws.delta,
                            ws.dq_accum, ws.dsink)
        e[1].record(stream)
        attn_bwd_fused_cast(inp.shape, inp.q, inp.k, inp.v, inp.do, ws.lse, ws.delta, inp.cu,
                            ws.dq_accum, counters, ws.dq, ws.dk, ws.dv)
        e[2].record(stream)
    torch.cuda.synchronize()
    fm = np.array([[e[k].elapsed_time(e[k + 1]) for k in range(2)] for e in ev]).mean(axis=0)
    out.update(fc_pre_ms=float(fm[0]), fc_bwd_ms=float(fm[1]))
    del counters
    # The deterministic backward on the same inputs: preprocess without the
    # accumulator, the dK/dV-only main pass, the query-stationary dQ pass.
    _warm(lambda: path.backward(inp, ws, mode="deterministic"), 2, warm_s)
    for i in range(steps):
        e = ev[i]
        e[0].record(stream)
        attn_bwd_preprocess(inp.shape, ws.o, inp.do, ws.lse, inp.cu, inp.sink, ws.delta, None,
                            ws.dsink)
        e[1].record(stream)
        attn_bwd_dkdv(inp.shape, inp.q, inp.k, inp.v, inp.do, ws.lse, ws.delta, inp.cu, ws.dk,
                      ws.dv)
        e[2].record(stream)
        attn_bwd_dq(inp.shape, inp.q, inp.k, inp.v, inp.do, ws.lse, ws.delta, inp.cu, ws.dq)
        e[3].record(stream)
    torch.cuda.synchronize()
    dm = np.array([[e[k].elapsed_time(e[k + 1]) for k in range(3)] for e in ev]).mean(axis=0)
    # ... and as path.backward runs it (path.concurrent_dq: the dQ pass
    # forming Delta first, or on a side stream beside the dK/dV pass).
    _warm(lambda: path.backward(inp, ws, mode="deterministic"), 2, warm_s)
    for i in range(steps):
        ev[i][0].record(stream)
        path.backward(inp, ws, mode="deterministic")
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    out["det_path_ms"] = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    out.update(det_pre_ms=float(dm[0]), dkdv_ms=float(dm[1]), dq_ms=float(dm[2]),
               auto_mode=path.select_mode(inp.shape, inp.lengths),
               auto_splits=path.splits_for_mode(inp.shape, inp.lengths,
                                                path.select_mode(inp.shape, inp.lengths)))
    # The whole backward as path.backward(mode="auto", kv_splits="auto") runs it.
    _warm(lambda: path.backward(inp, ws, mode="auto", kv_splits="auto"), 2, warm_s)
    for i in range(steps):
        ev[i][0].record(stream)
        path.backward(inp, ws, mode="auto", kv_splits="auto")
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    out["auto_ms"] = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    del ws, inp
    torch.cuda.empty_cache()
    return out


def deterministic_entry(x: dict, r: dict) -> dict:
    """Times and rates of the deterministic backward (query-stationary dQ):
    per pass, back to back after the preprocess (bwd_ms), and as
    path.backward runs it (bwd_ms_path: the dQ pass forming Delta first, or
    concurrent with the dK/dV pass; its ratio to the atomic path is
    vs_atomic_path).  The dK/dV pass does 8 and the dQ
    pass 6 of the 10 units of 2*BM*BN*D FLOPs per visible tile pair that the
    fused pass does."""
    f = bwd_flops(x)
    total = r["det_pre_ms"] + r["dkdv_ms"] + r["dq_ms"]
    conc = r["det_path_ms"]
    return {"bwd_ms": round(total, 4), "bwd_tflops": round(f / (total * 1e-3) / 1e12, 2),
            "bwd_ms_path": round(conc, 4),
            "bwd_tflops_path": round(f / (conc * 1e-3) / 1e12, 2),
            "attn_bwd_preprocess_ms": round(r["det_pre_ms"], 4),
            "attn_bwd_dkdv_ms": round(r["dkdv_ms"], 4),
            "attn_bwd_dq_ms": round(r["dq_ms"], 4),
            "attn_bwd_dkdv_tflops": round(0.8 * f / (r["dkdv_ms"] * 1e-3) / 1e12, 2),
            "attn_bwd_dq_tflops": round(0.6 * f / (r["dq_ms"] * 1e-3) / 1e12, 2),
            "vs_atomic_path": round((r["pre_ms"] + r["bwd_ms"] + r["post_ms"]) / conc, 4),
            "auto_mode": r["auto_mode"]}


def fused_cast_entry(x: dict, r: dict) -> dict:
    """The atomic backward with the dQ cast fused into the main pass
    (attn_bwd_fused_cast; for non-causal problems it runs the separate cast
    itself): its kernel time, the backward (preprocess + that pass), and the
    ratio of the separate-cast backward (preprocess + attn_bwd + postprocess)
    to it."""
    sep = r["pre_ms"] + r["bwd_ms"] + r["post_ms"]
    tot = r["fc_pre_ms"] + r["fc_bwd_ms"]
    return {"attn_bwd_fused_cast_ms": round(r["fc_bwd_ms"], 4), "bwd_ms": round(tot, 4),
            "bwd_tflops": round(bwd_flops(x) / (tot * 1e-3) / 1e12, 2),
            "separate_cast_bwd_ms": round(sep, 4),
            "vs_separate_cast": round(sep / tot, 4)}


def auto_entry(x: dict, r: dict) -> dict:
    """The backward as path.backward(mode="auto", kv_splits="auto") runs it."""
    return {"mode": r["auto_mode"], "kv_splits": r["auto_splits"],
            "bwd_ms": round(r["auto_ms"], 4),
            "bwd_tflops": round(bwd_flops(x) / (r["auto_ms"] * 1e-3) / 1e12, 2)}


def _oracle_unit(u: dict) -> float:
    """One (sequence, query head) problem of the CPU baseline: the fp64 oracle's
    forward + backward with one BLAS thread.  Returns its wall time."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as orc

    with threadpool_limits(1):
        t0 = time.perf_counter()
        orc.forward_backward(u)
        return time.perf_counter() - t0


def oracle_units(x: dict, n_cap: int) -> list:
    """Every (sequence, query head) of the workload as a problem of its own --
    one sequence, one query head and the kv head it reads, its sink -- with
    the sequence cut to its first n_cap rows; sequence-major, then head."""
    g = x["hq"] // x["hkv"]
    cu = x["cu_seqlens"]
    out = []
    for s in range(len(x["lengths"])):
        a = int(cu[s])
        n = min(int(cu[s + 1]) - a, n_cap)
        if n <= 0:
            continue
        for h in range(x["hq"]):
            kv = h // g
            out.append(dict(q=x["q"][a:a + n, h:h + 1], k=x["k"][a:a + n, kv:kv + 1],
                            v=x["v"][a:a + n, kv:kv + 1], do=x["do"][a:a + n, h:h + 1],
                            sink=None if x["sink"] is None else x["sink"][h:h + 1],
                            cu_seqlens=np.array([0, n], dtype=np.int32), lengths=[n], hq=1,
                            hkv=1, d=x["d"], causal=x["causal"], window=x["window"],
                            scale=x["scale"]))
    return out


def cpu_workers(cap: int = 16) -> tuple:
    """(CPUs this process may run on, workers the CPU baseline uses): one
    worker per CPU, at most `cap` (the host share of one GPU)."""
    try:
        cpus = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cpus = os.cpu_count() or 1
    return cpus, max(1, min(cap, cpus))


def cpu_baseline(x: dict, target_s: float = 12.0, workers: int | None = None) -> dict:
    """The fp64 oracle (as it stands) on a bounded sample of the workload, in
    a process pool over (sequence, query head) problems, one BLAS thread per
    worker.  A 1024-row problem timed first sets the cost model (time ~ rows
    squared); sequences are then cut to the longest prefix whose problem
    takes about target_s or less, and whole rounds of `workers` problems
    (sequence-major, then head) are taken until the pool's expected wall time
    reaches target_s (or the workload is exhausted).  The rate is the sample's
    backward FLOPs (same convention as the GPU figure) over the pool's wall
    time.  Called before the GPU is touched: the pool's workers are started
    fresh (spawn)."""
    import multiprocessing as mp

    cpus, nw = cpu_workers()
    if workers is not None:
        nw = workers
    n_max = max(x["lengths"]) if x["lengths"] else 0
    n_c = min(1024, n_max)
    t_c = max(1e-3, _oracle_unit(oracle_units(x, n_c)[0]))
    n_cap = n_max
    while n_cap > n_c and t_c * (n_cap / n_c) ** 2 > target_s:
        n_cap //= 2
    units = oracle_units(x, n_cap)
    cost = [t_c * (u["lengths"][0] / n_c) ** 2 for u in units]
    take, acc = 0, 0.0
    while take < len(units) and acc < target_s:
        rnd = cost[take:take + nw]
        acc += max(rnd)
        take += len(rnd)
    units = units[:take]
    ctx = mp.get_context("spawn")
    t0 = time.perf_counter()
    with ctx.Pool(nw) as pool:
        per = pool.map(_oracle_unit, units, chunksize=1)
    wall = time.perf_counter() - t0
    flops = sum(bwd_flops(u) for u in units)
    return {"value": flops / wall / 1e12, "unit": "TFLOP/s", "cores": int(nw),
            "workers": int(nw), "cpus_available": int(cpus), "kind": "oracle",
            "sample": (f"fp64 numpy oracle forward+backward of {len(units)} (sequence, query "
                       f"head) problems of this workload (sequences cut to their first "
                       f"{n_cap} rows; D={x['d']}, causal={x['causal']}, window={x['window']}),"
                       f" a spawn process pool of {nw} workers with 1 BLAS thread each, "
                       f"{wall:.2f} s wall ({sum(per):.1f} s of worker time); rate = backward "
                       f"FLOPs of the sample / wall time")}


def describe(name: str, x: dict) -> dict:
    return {"workload": name, "num_seqs": len(x["lengths"]), "max_seqlen": max(x["lengths"]),
            "total_tokens": int(sum(x["lengths"])), "hq": x["hq"], "hkv": x["hkv"],
            "head_dim": x["d"], "dtype": x["dtype"], "causal": bool(x["causal"]),
            "window": x["window"], "sink": x["sink"] is not None}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_gqa", choices=sorted(ai.WORKLOADS))
    ap.add_argument("--n", type=int, default=32768, help="sequence length for mha_causal")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the per-workload extras (N sweep and GQA workloads)")
    ap.add_argument("--only-extra", default=None, metavar="KEY",
                    help="run only the per-workload extra with this key (e.g. mha_causal_n4096)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (3 launches) and exit: the "
                         "reference reading for the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}); the "
              "path shards by (sequence, kv head) with no collective, so N GPUs would each run "
              "this benchmark on their own share.", file=sys.stderr)
        return 2
    w = ai.workload(args.workload, n=args.n) if args.workload == "mha_causal" else \
        ai.workload(args.workload)
    x = ai.generate(w, args.seed)
    # The CPU baseline runs before anything touches the GPU (its process pool
    # starts fresh interpreters).  Under a profiler, whose preloaded library
    # sets up the GPU before this script starts, no worker is started at all.
    profiled = any(k.startswith("ROCPROF") for k in os.environ) or \
        "rocprof" in os.environ.get("LD_PRELOAD", "")
    cpu = None if (args.no_cpu_baseline or args.copy_calibration or profiled) else \
        cpu_baseline(x)

    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, device="cuda", dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 3}))
        return 0

    # The machine's own ceilings first (they also bring the clocks up after
    # the host-side input generation); then the W warm-up and K timed steps.
    ceiling = atomic_ceiling_gbs()
    copy_gbs = copy_reference_gbs()
    r = run_gpu(x, args.steps, args.warmup)
    fl = bwd_flops(x)
    bwd_total_ms = r["pre_ms"] + r["bwd_ms"] + r["post_ms"]
    value = fl / (bwd_total_ms * 1e-3) / 1e12
    kernel_tflops = fl / (r["bwd_ms"] * 1e-3) / 1e12
    traffic = _traffic(w.name if w.name != "mha_causal" else f"mha_causal_n{args.n}")
    pre_b, post_b = prepost_bytes(x)
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["fwd_ms"] + bwd_total_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": x["dtype"],
        "data": "synthetic (seeded N(0, sigma^2) inputs of the workload's shape)",
        "config": describe(w.name, x),
        "roofline": {"bound": "mfma", "achieved": round(kernel_tflops, 3),
                     "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(kernel_tflops / PEAK_MFMA_TFLOPS, 4), "traffic": traffic,
                     "kernel": "attn_bwd main kernel", "flops_per_launch": fl,
                     "avg_launch_ms": round(r["bwd_ms"], 4)},
        "kernels_ms": {"attn_fwd": round(r["fwd_ms"], 4),
                       "attn_bwd_preprocess": round(r["pre_ms"], 4),
                       "attn_bwd": round(r["bwd_ms"], 4),
                       "attn_bwd_postprocess": round(r["post_ms"], 4)},
        "hbm_gbs": {"attn_bwd_preprocess": round(pre_b / (r["pre_ms"] * 1e-3) / 1e9, 1),
                    "attn_bwd_postprocess": round(post_b / (r["post_ms"] * 1e-3) / 1e9, 1),
                    "peak": PEAK_HBM_GBS,
                    "copy_reference": round(copy_gbs, 1)},
        "fwd_tflops": round(fwd_flops(x) / (r["fwd_ms"] * 1e-3) / 1e12, 3),
        "atomics": {"kernel": "attn_bwd main kernel",
                    "bytes_per_launch": bwd_atomic_bytes(x),
                    "achieved_gbs": round(bwd_atomic_bytes(x) / (r["bwd_ms"] * 1e-3) / 1e9, 1),
                    "ceiling_gbs": round(ceiling, 1) if ceiling else ATOMIC_CEILING_GBS,
                    "ceiling_source": ("measured in this run (microbench/atomic_rate.hip)"
                                       if ceiling else "earlier microbenchmark figure"),
                    "note": "device-scope fp32 atomic adds resolve beyond L2 on this part; "
                            "their device-wide rate, not the MFMA peak, bounds this kernel",
                    # The same kernel built without its dQ product and atomics
                    # (attn_bwd_dkdv, a library entry point) on the same inputs:
                    # the share of attn_bwd's time that the dQ product plus its
                    # atomics cost (an upper bound on the atomic overhead).
                    "without_dq_product_ms": round(r["dkdv_ms"], 4),
                    "dq_product_and_atomics_share": round(1.0 - r["dkdv_ms"] / r["bwd_ms"], 4)},
        "wall_ms_per_step": round(r["wall_ms_per_step"], 4),
        "deterministic": deterministic_entry(x, r),
        "fused_cast": fused_cast_entry(x, r),
        "auto": auto_entry(x, r),
        "device": device_info(),
    }
    base = PAGES_BASELINE.get((w.name, args.n if w.name == "mha_causal" else None))
    if base:
        line["vs_baseline"] = round(value / base, 4)
        line["baseline_note"] = ("pages' number for this workload on other hardware (triton issue "
                                 "4717, atomic_add after vectorized atomics): context only")
    if not args.no_extra:
        extra = {}
        cases = [("mha_causal", n) for n in ai.MHA_SWEEP if n != args.n or w.name != "mha_causal"]
        cases += [(nm, None) for nm in ("varlen_gqa", "sink_window", "long_gqa")
                  if nm != w.name]
        cases = [(nm, n, "thd") for nm, n in cases]
        # the MHA batch of the pages' table again as [B, H, S, D] tensors
        cases.append(("mha_causal", 32768, "bhsd"))
        for nm, n, layout in cases:
            key = (f"{nm}_n{n}" if n else nm) + ("_bhsd" if layout == "bhsd" else "")
            if args.only_extra is not None and key != args.only_extra:
                continue
            wx = ai.workload(nm, n=n) if n else ai.workload(nm)
            xx = ai.generate(wx, args.seed)
            rr = run_gpu(xx, max(3, args.steps // 4), 2, layout, warm_s=0.3, min_timed_s=0.05)
            f = bwd_flops(xx)
            extra[key] = {"bwd_tflops": round(f / ((rr["pre_ms"] + rr["bwd_ms"] + rr["post_ms"])
                                                   * 1e-3) / 1e12, 2),
                          "attn_bwd_kernel_tflops": round(f / (rr["bwd_ms"] * 1e-3) / 1e12, 2),
                          "attn_bwd_ms": round(rr["bwd_ms"], 4),
                          "frac": round(f / (rr["bwd_ms"] * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
                          "atomic_gbs": round(bwd_atomic_bytes(xx) / (rr["bwd_ms"] * 1e-3) / 1e9, 1),
                          "fwd_tflops": round(fwd_flops(xx) / (rr["fwd_ms"] * 1e-3) / 1e12, 2),
                          "attn_fwd_ms": round(rr["fwd_ms"], 4), "timed_steps": rr["steps"]}
            extra[key]["deterministic"] = deterministic_entry(xx, rr)
            extra[key]["fused_cast"] = fused_cast_entry(xx, rr)
            extra[key]["auto"] = auto_entry(xx, rr)
            cb = compulsory_bytes(xx)
            extra[key]["hbm_floor"] = {
                "compulsory_bytes": cb, "floor_ms": round(cb / (PEAK_HBM_GBS * 1e9) * 1e3, 4),
                "auto_gbs": round(cb / (rr["auto_ms"] * 1e-3) / 1e9, 1),
                "frac_of_peak": round(cb / (rr["auto_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
            if xx["window"] > 0:
                # The stated formula ignores the window: it over-counts the
                # work 16x here and is no achieved rate (the pair count is).
                extra[key]["nominal_formula_overcount"] = round(
                    bwd_flops_nominal(xx) / f, 2)
            pages = PAGES_BASELINE.get((nm, n)) if layout == "thd" else None
            if pages:
                extra[key]["vs_pages_context"] = {
                    "pages_value": pages, "ratio": round(extra[key]["bwd_tflops"] / pages, 4),
                    "note": "triton issue 4717, fp16 B4 H8 d64 causal, atomic_add after "
                            "vectorized atomics, other hardware: context only"}
            print(f"bench: {key}: {extra[key]}", file=sys.stderr, flush=True)
        line["per_workload"] = extra
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
