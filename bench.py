"""Bench: effective HBM bandwidth of the causal depthwise conv1d forward on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]

One step is one forward call (validation, dispatch, one kernel) over one batch of
synthetic input already resident in HBM.  The default workload is the
channel-first bf16 call B=4, C=2048, L=4096, K=4 with bias and SiLU.  Its
134 MB working set would fit in the 256 MB Infinity Cache, so the timed steps
rotate over enough separate input/output buffer sets (>= 1 GiB in total) that
every step reads inputs that have left the caches.

Effective bandwidth = algorithmic bytes / time, where the algorithmic bytes count
x read once, out written once, and weight, bias, seq_idx and the states once each
(halo re-reads are not counted).  Time comes from HIP events recorded on the
stream the kernels are launched on, around exactly K steps.

Printed: one JSON line with the metric, a "roofline" object for the forward
kernel (against MI355X's 8 TB/s HBM), and a "cpu_baseline" object (the CPU oracle
timed on this host over the same workload, and the element-wise parity of this
run's GPU output against it).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, decimal GB/s
ROTATION_BYTES = 1 << 30        # >= 4x the 256 MB Infinity Cache
METRIC = "causal conv1d fwd effective HBM GB/s and % of MI355X peak bandwidth"
UPDATE_METRIC = "causal conv1d update (decode) effective HBM GB/s and % of MI355X peak bandwidth"
KERNEL_SOURCES = ["causal_depthwise_conv1d_amd/csrc/ccv_cf.hip",
                  "causal_depthwise_conv1d_amd/csrc/ccv_cl.hip",
                  "causal_depthwise_conv1d_amd/csrc/ccv_device.hpp",
                  "causal_depthwise_conv1d_amd/csrc/ccv_launch.hpp",
                  "causal_depthwise_conv1d_amd/csrc/ccv_api.cpp",
                  "causal_depthwise_conv1d_amd/csrc/ccv_checks.hpp"]
BWD_SOURCES = ["causal_depthwise_conv1d_amd/csrc/ccv_bwd.hip",
               "causal_depthwise_conv1d_amd/csrc/ccv_device.hpp",
               "causal_depthwise_conv1d_amd/csrc/ccv_launch.hpp",
               "causal_depthwise_conv1d_amd/csrc/ccv_bwd_launch.hpp",
               "causal_depthwise_conv1d_amd/csrc/ccv_bwd_api.cpp",
               "causal_depthwise_conv1d_amd/csrc/ccv_checks.hpp"]
BWD_METRIC = "causal conv1d bwd effective HBM GB/s and % of MI355X peak bandwidth"
UPDATE_SOURCES = ["causal_depthwise_conv1d_amd/csrc/ccv_update.hip",
                  "causal_depthwise_conv1d_amd/csrc/ccv_device.hpp",
                  "causal_depthwise_conv1d_amd/csrc/ccv_launch.hpp",
                  "causal_depthwise_conv1d_amd/csrc/ccv_update_launch.hpp",
                  "causal_depthwise_conv1d_amd/csrc/ccv_update_api.cpp",
                  "causal_depthwise_conv1d_amd/csrc/ccv_checks.hpp"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_sources_sha256(files=None) -> str:
    h = hashlib.sha256()
    for rel in files or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def algorithmic_bytes(w) -> int:
    es = w.x.element_size()
    B, C, L, K = w.B, w.C, w.L, w.K
    n = 2 * B * C * L * es                          # x once, out once
    n += w.weight.numel() * w.weight.element_size()
    if w.bias is not None:
        n += w.bias.numel() * w.bias.element_size()
    if w.seq_idx is not None:
        n += B * L * 4
    if w.initial_states is not None:
        n += B * C * (K - 1) * es
    if w.return_final_states:
        n += B * C * (K - 1) * es
    return n


def profile_traffic(kernel_key: str, sha: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on
    the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"{kernel_key}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_sources_sha256:\s*([0-9a-f]{64})", text)
    m_tr = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not m_sha or not m_tr or m_sha.group(1) != sha:
        return None
    return int(m_tr.group(1))


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--op", default="fwd", choices=["fwd", "update", "bwd"],
                    help="fwd: the forward on --workload (default); update: the decode step; "
                         "bwd: the backward on --workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time spent timing the oracle")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the op needs no communication: batch or channel shards run independently)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import causal_depthwise_conv1d_amd as ccv
    import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ccv.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)

    if args.op == "update":
        bench_update(args, dev, props)
        return
    if args.op == "bwd":
        bench_bwd(args, dev, props)
        return

    t0 = time.time()
    w = wl.workload(args.workload)
    log(f"[bench] workload {w.name}: generated in {time.time() - t0:.1f}s")
    nbytes = algorithmic_bytes(w)
    set_bytes = 2 * w.x.numel() * w.x.element_size()
    if w.x_storage.numel() > w.x.numel():
        set_bytes = (w.x_storage.numel() + w.x.numel()) * w.x.element_size()
    nsets = max(2, math.ceil(ROTATION_BYTES / set_bytes))
    if nsets * set_bytes > 0.5 * props.total_memory:
        nsets = max(1, int(0.5 * props.total_memory // set_bytes))

    # Inputs resident in HBM: nsets copies of x (with its real strides) and out.
    weight = w.weight.to(dev)
    bias = None if w.bias is None else w.bias.to(dev)
    seq = None if w.seq_idx is None else w.seq_idx.to(dev)
    init = None
    if w.initial_states is not None:
        init = w.init_storage.to(dev).as_strided(w.initial_states.shape, w.initial_states.stride(),
                                                 w.initial_states.storage_offset())
    sets = []
    for i in range(nsets):
        xs = w.x_storage.to(dev)
        x = xs.as_strided(w.x.shape, w.x.stride(), w.x.storage_offset())
        out = ccv.empty_like_layout(x)
        fs = (torch.empty(w.B, w.K - 1, w.C, dtype=x.dtype, device=dev).transpose(1, 2)
              if w.return_final_states else None)
        a = ccv.make_args(x, weight, out, bias, seq, init, fs, w.activation)
        sets.append((xs, x, out, fs, a))
    st, plan = ccv.ccv_fwd_plan(sets[0][4])
    assert st == 0, ccv.ccv_status_str(st)
    plan = plan.as_dict()
    log(f"[bench] {nsets} buffer sets of {set_bytes / 1e6:.0f} MB; plan {plan}")

    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    fwd = ccv.lib().ccv_fwd
    import ctypes
    arg_refs = [ctypes.byref(s[4]) for s in sets]
    sp = ctypes.c_void_p(sptr)

    def step(i):
        rc = fwd(arg_refs[i % nsets], sp)
        if rc != 0:
            raise RuntimeError(ccv.ccv_status_str(rc))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    ms_per_step = total_ms / args.steps
    gbps = nbytes / (ms_per_step * 1e-3) / 1e9
    log(f"[bench] timed {args.steps} steps: {ms_per_step * 1e3:.2f} us/step, {gbps:.0f} GB/s")

    copy_gbps, empty_us = context_measurements(nbytes, dev, stream, args.steps)
    flushed = flushed_timing(step, dev, stream, nbytes)
    graph = graph_timing(fwd, arg_refs, nsets, nbytes)

    kernel_key = ("cf_fwd" if plan["path"] == ccv.CCV_PATH_CHANNEL_FIRST else "cl_fwd") + \
        f"_{w.x_dtype}_B{w.B}_C{w.C}_L{w.L}_K{w.K}"
    sha = kernel_sources_sha256()
    traffic = profile_traffic(kernel_key, sha)

    result = {
        "metric": METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "description": w.notes.get("description"),
            "B": w.B, "C": w.C, "L": w.L, "K": w.K,
            "x_strides": list(w.x.stride()),
            "activation": w.activation,
            "storage_dtype": w.x_dtype,
            "algorithmic_bytes": nbytes,
            "buffer_sets": nsets,
            "kernel": kernel_key,
            "plan": plan,
        },
        "pct_of_peak": round(100.0 * gbps / PEAK_HBM_GBPS, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbps, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(gbps / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "kernel": kernel_key,
            "avg_launch_us": round(ms_per_step * 1e3, 3),
            "algorithmic_bytes_per_launch": nbytes,
        },
        "context": {
            "copy_same_bytes_GBps": round(copy_gbps, 1),
            "copy_frac_of_peak": round(copy_gbps / PEAK_HBM_GBPS, 4),
            "empty_kernel_us": round(empty_us, 3),
            "flushed_calls": flushed,
            "graph_replay": graph,
            "device": props.name,
            "cu_count": props.multi_processor_count,
            "device_properties": device_properties(props),
            "kernel_sources_sha256": sha,
            "env_overrides": env_overrides(),
        },
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, sets[0][2], nbytes, args.cpu_seconds)

    print(json.dumps(result), flush=True)


def context_measurements(nbytes, dev, stream, steps):
    """Context on the same GPU: a plain copy kernel moving the same bytes (half read,
    half written, rotated over >= 1 GiB), and the launch floor of an empty kernel."""
    import ctypes

    import torch

    import causal_depthwise_conv1d_amd as ccv
    sp = ctypes.c_void_p(stream.cuda_stream)
    calib = ctypes.CDLL(ccv.CALIB_LIB_PATH)
    calib.ccv_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    calib.ccv_calib_empty.argtypes = [ctypes.c_void_p]
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    half = (nbytes // 2) // 16 * 16
    csets = max(2, math.ceil(ROTATION_BYTES / (2 * half)))
    bufs = [(torch.empty(half, dtype=torch.uint8, device=dev), torch.zeros(half, dtype=torch.uint8, device=dev))
            for _ in range(csets)]
    for i in range(20):
        d, s_ = bufs[i % csets]
        calib.ccv_calib_copy(d.data_ptr(), s_.data_ptr(), half, sp)
    ev0.record(stream)
    for i in range(steps):
        d, s_ = bufs[i % csets]
        calib.ccv_calib_copy(d.data_ptr(), s_.data_ptr(), half, sp)
    ev1.record(stream)
    torch.cuda.synchronize()
    copy_ms = ev0.elapsed_time(ev1) / steps
    copy_gbps = 2 * half / (copy_ms * 1e-3) / 1e9
    del bufs
    for _ in range(50):
        calib.ccv_calib_empty(sp)
    ev0.record(stream)
    for _ in range(1000):
        calib.ccv_calib_empty(sp)
    ev1.record(stream)
    torch.cuda.synchronize()
    empty_us = ev0.elapsed_time(ev1)  # ms for 1000 launches = us per launch
    log(f"[bench] copy of the same bytes: {copy_gbps:.0f} GB/s; empty kernel {empty_us:.2f} us")
    return copy_gbps, empty_us


def graph_timing(fwd, arg_refs, nsets, nbytes, calls=100, reps=5):
    """The same calls (rotating over the buffer sets) captured in one HIP graph of
    `calls` launches and replayed `reps` times: time per call with the host's launch
    cost taken out, which is what a launch-bound caller gets from a graph."""
    import ctypes

    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for i in range(calls):
            rc = fwd(arg_refs[i % nsets], s)
            if rc != 0:
                raise RuntimeError(f"ccv_fwd returned {rc} while capturing")
    g.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / (calls * reps)
    del g
    log(f"[bench] graph replay: {us:.2f} us per call ({calls} calls per graph)")
    return {"calls_per_graph": calls, "replays": reps, "us_per_call": round(us, 3),
            "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}


def env_overrides() -> dict:
    """The library's tuning / ablation environment variables set for this run (none
    in a default run; any set here change the launch the numbers come from)."""
    names = ("CCV_CF_WAVES_PER_CU", "CCV_CL_WAVES_PER_CU", "CCV_CL_TILE_T", "CCV_CU_COUNT", "CCV_FORCE_SCALAR")
    return {n: os.environ[n] for n in names if n in os.environ}


def flushed_timing(step, dev, stream, nbytes, iters=20):
    """Single calls with the caches flushed before each (a 1 GiB copy, more than the
    256 MB Infinity Cache and the L2s), each between its own pair of HIP events:
    median, min and max over `iters` calls.  Context beside the back-to-back figure."""
    import ctypes

    import torch

    import causal_depthwise_conv1d_amd as ccv
    sp = ctypes.c_void_p(stream.cuda_stream)
    calib = ctypes.CDLL(ccv.CALIB_LIB_PATH)
    calib.ccv_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    half = 512 << 20
    src = torch.zeros(half, dtype=torch.uint8, device=dev)
    dst = torch.empty(half, dtype=torch.uint8, device=dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    us = []
    for i in range(iters):
        calib.ccv_calib_copy(dst.data_ptr(), src.data_ptr(), half, sp)
        ev0.record(stream)
        step(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        us.append(ev0.elapsed_time(ev1) * 1e3)
    del src, dst
    us.sort()
    med = us[len(us) // 2] if len(us) % 2 else 0.5 * (us[len(us) // 2 - 1] + us[len(us) // 2])
    log(f"[bench] flushed single calls: median {med:.2f} us (min {us[0]:.2f}, max {us[-1]:.2f})")
    return {"iters": iters, "median_us": round(med, 3), "min_us": round(us[0], 3), "max_us": round(us[-1], 3),
            "median_GBps": round(nbytes / (med * 1e-6) / 1e9, 1)}


def device_properties(props) -> dict:
    """What the runtime reports about the GPU (names vary across torch builds)."""
    out = {}
    for name in ("gcnArchName", "total_memory", "multi_processor_count", "L2_cache_size",
                 "max_threads_per_multi_processor", "warp_size", "regs_per_multiprocessor",
                 "shared_memory_per_multiprocessor", "clock_rate", "memory_clock_rate", "memory_bus_width"):
        v = getattr(props, name, None)
        if isinstance(v, (int, float, str)):
            out[name] = v
    return out


def update_bytes(w) -> int:
    """Algorithmic bytes of one update call: x and out once, the state read and
    written once, weight and bias once."""
    es = w.x.element_size()
    B, C, L, K = w.B, w.C, w.L, w.K
    n = 2 * B * C * L * es + 2 * B * C * (K - 1) * es
    n += w.weight.numel() * w.weight.element_size()
    if w.bias is not None:
        n += w.bias.numel() * w.bias.element_size()
    return n


def bench_update(args, dev, props):
    """The update (decode) call on the decode workload: a first call whose output
    and new state the cpu_baseline leg checks against the oracle, then W warm-up
    and K timed calls rotating over >= 1 GiB of (x, state, out) sets, so every call
    reads its inputs from HBM."""
    import ctypes

    import torch

    import causal_depthwise_conv1d_amd as ccv
    import workloads as wl

    w = wl.decode_workload()
    B, C, L, K = w.B, w.C, w.L, w.K
    es = w.x.element_size()
    nbytes = update_bytes(w)
    set_bytes = (2 * B * C * L + B * C * (K - 1)) * es
    nsets = max(2, math.ceil(ROTATION_BYTES / set_bytes))
    weight = w.weight.to(dev)
    bias = None if w.bias is None else w.bias.to(dev)
    sets = []
    for _ in range(nsets):
        x = w.x.to(dev).contiguous()
        state = w.initial_states.to(dev).contiguous()
        out = torch.empty(B, C, L, dtype=x.dtype, device=dev)
        sets.append((x, state, out, ccv.make_update_args(x, weight, state, out, bias, w.activation)))
    st, plan = ccv.ccv_update_plan(sets[0][3])
    assert st == 0, ccv.ccv_status_str(st)
    plan = plan.as_dict()
    log(f"[bench] update: {nsets} buffer sets of {set_bytes / 1e6:.1f} MB; plan {plan}")

    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    upd = ccv.lib().ccv_update
    refs = [ctypes.byref(s[3]) for s in sets]

    # The first call's output and new state, kept for the check against the oracle
    # in the cpu_baseline leg (before the states start to move).
    rc = upd(refs[0], sp)
    if rc != 0:
        raise RuntimeError(ccv.ccv_status_str(rc))
    torch.cuda.synchronize()
    first_out, first_state = sets[0][2].cpu(), sets[0][1].cpu()

    def step(i):
        rc = upd(refs[i % nsets], sp)
        if rc != 0:
            raise RuntimeError(ccv.ccv_status_str(rc))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    gbps = nbytes / (ms_per_step * 1e-3) / 1e9
    log(f"[bench] update: {ms_per_step * 1e3:.2f} us/call, {gbps:.0f} GB/s")
    copy_gbps, empty_us = context_measurements(nbytes, dev, stream, args.steps)

    kernel_key = f"update_{w.x_dtype}_B{B}_C{C}_L{L}_K{K}"
    sha = kernel_sources_sha256(UPDATE_SOURCES)
    result = {
        "metric": UPDATE_METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "description": w.notes.get("description"),
            "B": B, "C": C, "L": L, "K": K,
            "activation": w.activation,
            "storage_dtype": w.x_dtype,
            "algorithmic_bytes": nbytes,
            "buffer_sets": nsets,
            "kernel": kernel_key,
            "plan": plan,
        },
        "pct_of_peak": round(100.0 * gbps / PEAK_HBM_GBPS, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbps, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(gbps / PEAK_HBM_GBPS, 4),
            "traffic": profile_traffic(kernel_key, sha),
            "kernel": kernel_key,
            "avg_launch_us": round(ms_per_step * 1e3, 3),
            "algorithmic_bytes_per_launch": nbytes,
        },
        "context": {
            "copy_same_bytes_GBps": round(copy_gbps, 1),
            "copy_frac_of_peak": round(copy_gbps / PEAK_HBM_GBPS, 4),
            "empty_kernel_us": round(empty_us, 3),
            "device": props.name,
            "cu_count": props.multi_processor_count,
            "kernel_sources_sha256": sha,
            "env_overrides": env_overrides(),
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = update_cpu_baseline(w, nbytes, args.cpu_seconds, first_out, first_state)
    print(json.dumps(result), flush=True)


def bwd_bytes(w) -> int:
    """Algorithmic bytes of one backward call: x and dout read once, dx written
    once, the parameters read and their gradients written once, the states and
    their gradients once.  The partial-sum workspace is overhead."""
    es = w.x.element_size()
    B, C, L, K = w.B, w.C, w.L, w.K
    pb = w.weight.element_size()
    n = 3 * B * C * L * es + 2 * C * K * pb
    if w.bias is not None:
        n += 2 * C * pb
    if w.initial_states is not None:
        n += 2 * B * C * (K - 1) * es
    return n


def bench_bwd(args, dev, props):
    """The backward on the chosen workload's shape: a first call whose gradients
    the cpu_baseline leg checks against the oracle, then W warm-up and K timed
    calls rotating over >= 1 GiB of (x, dout, dx) sets."""
    import ctypes

    import torch

    import causal_depthwise_conv1d_amd as ccv
    import workloads as wl

    w = wl.workload(args.workload)
    B, C, L, K = w.B, w.C, w.L, w.K
    es = w.x.element_size()
    nbytes = bwd_bytes(w)
    dout_cpu = wl.to_storage(wl.draw(B * C * L, w.seed, 5, "normal", 1.0), w.x_dtype).reshape(B, C, L)
    set_bytes = 3 * B * C * L * es
    nsets = max(2, math.ceil(ROTATION_BYTES / set_bytes))
    if nsets * set_bytes > 0.5 * props.total_memory:
        nsets = max(1, int(0.5 * props.total_memory // set_bytes))
    weight = w.weight.to(dev)
    bias = None if w.bias is None else w.bias.to(dev)
    seq = None if w.seq_idx is None else w.seq_idx.to(dev)
    init = None if w.initial_states is None else w.initial_states.to(dev)
    dweight = torch.empty(C, K, dtype=weight.dtype, device=dev)
    dbias = None if bias is None else torch.empty(C, dtype=weight.dtype, device=dev)
    sets = []
    workspace = None
    for _ in range(nsets):
        xs = w.x_storage.to(dev)
        x = xs.as_strided(w.x.shape, w.x.stride(), w.x.storage_offset())
        dout = ccv.empty_like_layout(x).copy_(dout_cpu.to(dev))      # the layout of out
        dx = ccv.empty_like_layout(x)
        a = ccv.make_bwd_args(x, weight, bias, dout, dx, dweight, dbias, seq, init, None, None, w.activation)
        if workspace is None:
            workspace = torch.empty(max(16, ccv.ccv_bwd_workspace_size(a)), dtype=torch.uint8, device=dev)
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
        sets.append((xs, dout, dx, a))
    st, plan = ccv.ccv_bwd_plan(sets[0][3])
    assert st == 0, ccv.ccv_status_str(st)
    plan = plan.as_dict()
    log(f"[bench] bwd: {nsets} buffer sets of {set_bytes / 1e6:.0f} MB; workspace "
        f"{workspace.numel() / 1e6:.1f} MB; plan {plan}")

    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    fn = ccv.lib().ccv_bwd
    refs = [ctypes.byref(s[3]) for s in sets]

    def step(i):
        rc = fn(refs[i % nsets], sp)
        if rc != 0:
            raise RuntimeError(ccv.ccv_status_str(rc))

    # The first call's gradients, kept for the check against the oracle in the
    # cpu_baseline leg.
    step(0)
    torch.cuda.synchronize()
    first = (sets[0][2].cpu(), dweight.cpu(), None if dbias is None else dbias.cpu())
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    gbps = nbytes / (ms_per_step * 1e-3) / 1e9
    log(f"[bench] bwd: {ms_per_step * 1e3:.2f} us/call, {gbps:.0f} GB/s")
    copy_gbps, empty_us = context_measurements(nbytes, dev, stream, min(args.steps, 200))

    kernel_key = f"bwd_{w.x_dtype}_B{B}_C{C}_L{L}_K{K}"
    sha = kernel_sources_sha256(BWD_SOURCES)
    result = {
        "metric": BWD_METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "description": w.notes.get("description"),
            "B": B, "C": C, "L": L, "K": K,
            "activation": w.activation,
            "storage_dtype": w.x_dtype,
            "algorithmic_bytes": nbytes,
            "buffer_sets": nsets,
            "kernel": kernel_key,
            "plan": plan,
        },
        "pct_of_peak": round(100.0 * gbps / PEAK_HBM_GBPS, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbps, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(gbps / PEAK_HBM_GBPS, 4),
            "traffic": profile_traffic(kernel_key, sha),
            "kernel": kernel_key,
            "avg_launch_us": round(ms_per_step * 1e3, 3),
            "algorithmic_bytes_per_launch": nbytes,
        },
        "context": {
            "copy_same_bytes_GBps": round(copy_gbps, 1),
            "copy_frac_of_peak": round(copy_gbps / PEAK_HBM_GBPS, 4),
            "empty_kernel_us": round(empty_us, 3),
            "device": props.name,
            "cu_count": props.multi_processor_count,
            "kernel_sources_sha256": sha,
            "env_overrides": env_overrides(),
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = bwd_cpu_baseline(w, dout_cpu, nbytes, args.cpu_seconds, first, plan)
    print(json.dumps(result), flush=True)


def bwd_parity(w, r, first, plan):
    """The first backward call's gradients against the oracle's fp64 result r (every
    dx, dweight and dbias element), with the tolerances of the GPU tests: for the
    parameter gradients (n + 32 * levels + K + 8) / 4 roundings, n the terms of a
    lane's in-order sum (the register-only channel-first path: span / 64 plus the 7
    additions of the 64-lane sum; the others: tiles per partial row times the tile
    length)."""
    from oracle import compare as ocmp
    from oracle.from_torch import dtype_name, raw

    span, tpi = plan["span"], plan["unroll"]
    if plan["vector"] == 3:
        n, parts = span // 64 + 7, w.B * max(1, math.ceil(w.L / span))
    else:
        n, parts = tpi * span, w.B * max(1, math.ceil(math.ceil(w.L / span) / tpi))
    levels = 1
    while parts > 32:                                  # levels of the fan-in-32 reduction tree
        parts, levels = -(-parts // 32), levels + 1
    pk = math.ceil((n + 32 * levels + w.K + 8) / 4)
    dx, dweight, dbias = first
    out = {}
    for name, got, ref, scale, kk in (("dx", dx, r["dx"], r["ex"], w.K + 2),
                                      ("dweight", dweight, r["dw"], r["ew"], pk),
                                      ("dbias", dbias, r["db"], r["eb"], pk)):
        if got is None:
            continue
        g = got.contiguous()
        res = ocmp.compare(dtype_name(g), kk, raw(g), ref, scale)
        out[name] = {"n": res["n"], "out_of_tolerance": res["n_bad"], "max_ulp": res["max_ulp"],
                     "max_rel": res["max_rel"]}
    return out


def bwd_cpu_baseline(w, dout_cpu, nbytes, min_seconds, first, plan):
    """The oracle's backward as written (single-threaded fp64 loops: dx, dweight,
    dbias and their error scales) on this host's CPU over the whole workload,
    repeated until at least `min_seconds` have passed; then the first GPU call's
    gradients checked against it."""
    from oracle.from_torch import bwd, case

    c = case(w.x, w.weight, w.bias, w.seq_idx, w.initial_states, w.activation)
    passes, t_total, r = 0, 0.0, None
    while passes == 0 or t_total < min_seconds:
        t0 = time.perf_counter()
        r = bwd(c, dout_cpu, None)
        t_total += time.perf_counter() - t0
        passes += 1
    sec = t_total / passes
    log(f"[bench] cpu oracle bwd: {passes} passes, {sec:.2f} s per pass")
    parity = bwd_parity(w, r, first, plan)
    log(f"[bench] bwd parity: {parity}")
    return {"value": round(nbytes / sec / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the whole workload ({w.B * w.C * w.L} elements), {passes} pass(es) of the "
                      "single-threaded fp64 oracle backward (dx, dweight, dbias and their error scales)",
            "seconds_per_pass": round(sec, 3), "parity": parity}


def update_parity(w, out_gpu, state_gpu):
    """One update call against the oracle: out within tolerance of the forward with
    the old state as initial states, the new state bit-exact to its final states."""
    import numpy as np

    from oracle import compare as ocmp
    from oracle.from_torch import case, dtype_name, raw

    c = case(w.x, w.weight, w.bias, None, w.initial_states, w.activation)
    y, s = c.fwd()
    g = raw(out_gpu.cpu().contiguous())
    res = ocmp.compare(dtype_name(out_gpu), w.K, g, y, s)
    got = raw(state_gpu.cpu().contiguous())
    want = c.final_states()
    bits = np.uint32 if got.dtype == np.float32 else np.uint16
    return {"outputs": res["n"], "out_of_tolerance": res["n_bad"], "max_ulp": res["max_ulp"],
            "bit_equal": res["bit_equal"],
            "state_bit_exact": bool(np.array_equal(got.view(bits), want.view(bits)))}


def update_cpu_baseline(w, nbytes, min_seconds, first_out, first_state):
    """The oracle as written for one update call (its forward with the state as
    initial states, plus the final states), repeated for at least `min_seconds`;
    then the first GPU call's output and new state checked against it."""
    from oracle import round_out
    from oracle.from_torch import case

    c = case(w.x, w.weight, w.bias, None, w.initial_states, w.activation)
    passes, t_total = 0, 0.0
    while passes == 0 or t_total < min_seconds:
        t0 = time.perf_counter()
        y, _ = c.fwd(want_sabs=False)
        round_out(w.x_dtype, y)
        c.final_states()
        t_total += time.perf_counter() - t0
        passes += 1
    sec = t_total / passes
    parity = update_parity(w, first_out, first_state)
    log(f"[bench] update parity: {parity}")
    return {"value": round(nbytes / sec / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the whole decode call ({w.B * w.C} rows), {passes} passes of the single-threaded "
                      "fp64 oracle incl. rounding and the new state",
            "seconds_per_pass": round(sec, 4), "parity": parity}


def cpu_baseline(w, out_gpu, nbytes, min_seconds):
    """The oracle as written (single-threaded fp64 loop) on this host's CPU, over
    the whole workload, repeated until at least `min_seconds` have passed; then the
    GPU output of this run compared with it at every output."""
    import numpy as np
    import torch

    from oracle import compare as ocmp
    from oracle import round_out
    from oracle.from_torch import case, dtype_name, raw

    c = case(w.x, w.weight, w.bias, w.seq_idx, w.initial_states, w.activation)
    passes, t_total = 0, 0.0
    y = s = None
    while passes == 0 or t_total < min_seconds:
        t0 = time.perf_counter()
        y, s = c.fwd()
        round_out(w.x_dtype, y)
        t_total += time.perf_counter() - t0
        passes += 1
    sec = t_total / passes
    log(f"[bench] cpu oracle: {passes} passes, {sec:.2f} s per pass")
    # The same loop on all of this host's cores (context, not the baseline): rows of
    # (b, c) split between threads, results bit-identical to the single thread.
    from oracle import GCC_CMD
    nthr = max(1, min(16, len(os.sched_getaffinity(0))))
    mt_passes, mt_total, ymt = 0, 0.0, None
    while mt_passes == 0 or mt_total < min(min_seconds, 3.0):
        t0 = time.perf_counter()
        ymt, _ = c.fwd_threads(nthr)
        round_out(w.x_dtype, ymt)
        mt_total += time.perf_counter() - t0
        mt_passes += 1
    mt_sec = mt_total / mt_passes
    log(f"[bench] cpu oracle on {nthr} threads: {mt_passes} passes, {mt_sec:.3f} s per pass")
    g = raw(out_gpu.cpu().contiguous())
    res = ocmp.compare(dtype_name(out_gpu), w.K, g, y, s)
    cpu_name = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(nbytes / sec / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"the whole workload ({w.B * w.C * w.L} outputs), {passes} pass(es) of the "
                  "single-threaded fp64 oracle incl. rounding to the output dtype",
        "seconds_per_pass": round(sec, 3),
        "host_cpu": cpu_name,
        "host_threads_available": os.cpu_count(),
        "compile_flags": " ".join(f for f in GCC_CMD[1:] if f.startswith("-") and f not in ("-o", "-shared")),
        "all_cores": {"value": round(nbytes / mt_sec / 1e9, 4), "unit": "GB/s", "threads": nthr,
                      "seconds_per_pass": round(mt_sec, 4), "passes": mt_passes,
                      "bit_identical_to_one_thread": bool(np.array_equal(ymt.view(np.uint64), y.view(np.uint64)))},
        "parity": {"outputs": res["n"], "out_of_tolerance": res["n_bad"], "max_ulp": res["max_ulp"],
                   "max_rel": res["max_rel"], "floor_only": res["n_floor_only"],
                   "bit_equal": res["bit_equal"]},
    }


if __name__ == "__main__":
    main()
