"""Bench: effective HBM bandwidth of the causal depthwise conv1d forward on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload N]

One step is one forward call (validation, dispatch, one kernel) over one batch of
synthetic input already resident in HBM.  By default every one of the five
named workloads is measured, and the printed line's headline is the largest one
(workload 5: fp32, B=2, C=128, L=1048576, K=3, carried states, 2.15 GB per call);
--workload N measures one workload and makes it the headline.

Timing, per workload: W warm-up and then exactly K timed calls, each preceded by
an untimed cache flush (a 1 GiB copy, then a 1 GiB read-only sweep, so the 256 MB
Infinity Cache and the L2s hold clean lines of other data) and bracketed by its
own pair of HIP events on the stream the kernel is launched on.  The headline
value is the median; the roofline object uses the mean (the average launch
duration).  Beside it, as context: K back-to-back calls rotating over >= 1 GiB of
buffer sets, the same calls replayed from a HIP graph, a streaming copy kernel
moving the same number of bytes, the empty-kernel launch floor, and the
rocprofv3 kernel-trace average of the flushed calls from the committed profile
(`kernel_trace`, when that profile was taken on the current kernel sources).

Effective bandwidth = algorithmic bytes / time, where the algorithmic bytes count
x read once, out written once, and weight, bias, seq_idx and the states once each
(halo re-reads are not counted).

Printed: one JSON line with the metric, a "roofline" object for the headline
kernel (against MI355X's 8 TB/s HBM), a "cpu_baseline" object (the CPU oracle
timed on this host, on one thread over a bounded sample and on all cores over the
whole workload, and the element-wise parity of this run's GPU output against it
at every output), and under context.per_workload the same figures for every
other measured workload.
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
FWD_SHARED = ["causal_depthwise_conv1d_amd/csrc/ccv_device.hpp",
              "causal_depthwise_conv1d_amd/csrc/ccv_launch.hpp",
              "causal_depthwise_conv1d_amd/csrc/ccv_api.cpp",
              "causal_depthwise_conv1d_amd/csrc/ccv_checks.hpp"]
CF_SOURCES = ["causal_depthwise_conv1d_amd/csrc/ccv_cf.hip"] + FWD_SHARED
CL_SOURCES = ["causal_depthwise_conv1d_amd/csrc/ccv_cl.hip"] + FWD_SHARED
KERNEL_SOURCES = CF_SOURCES[:1] + CL_SOURCES
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


def profile_kernel_time(kernel_key: str, sha: str, nbytes: int):
    """The rocprofv3 kernel-trace average of the forward kernel over the flushed
    calls, from the committed trace summary, if it was taken on the current kernel
    sources; otherwise None.  Shown beside the HIP-event figures, which also hold
    the dispatch of each single call."""
    path = os.path.join(ROOT, "profiles", f"{kernel_key}_trace.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_sources_sha256:\s*([0-9a-f]{64})", text)
    m_us = re.search(r"kernel_avg_us:\s*([0-9.]+)", text)
    if not m_sha or not m_us or m_sha.group(1) != sha:
        return None
    us = float(m_us.group(1))
    return {"us": us, "GBps": round(gbps(nbytes, us), 1), "frac": round(gbps(nbytes, us) / PEAK_HBM_GBPS, 4),
            "source": f"profiles/{kernel_key}_trace.md: rocprofv3 --kernel-trace average over the flushed calls "
                      "of a traced run of this bench"}


HEADLINE_WORKLOAD = 5           # the largest single-GPU workload (2,147,489,280 bytes per call)
FLUSH_BYTES = 1 << 30


class Calib:
    """The measurement helpers of libccv_calib.so (copy, read-only sweep, empty
    kernel) and the buffers of the cache flush."""

    def __init__(self, dev):
        import ctypes

        import torch

        import causal_depthwise_conv1d_amd as ccv
        c = ctypes.CDLL(ccv.CALIB_LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        c.ccv_calib_copy_ex.argtypes = [vp, vp, i64, i32, i32, vp]
        c.ccv_calib_copy.argtypes = [vp, vp, i64, vp]
        c.ccv_calib_read.argtypes = [vp, i64, ctypes.c_uint32, vp, vp]
        c.ccv_calib_empty.argtypes = [vp]
        self.lib = c
        self.dev = dev
        half = FLUSH_BYTES // 2
        self.fsrc = torch.zeros(half, dtype=torch.uint8, device=dev)
        self.fdst = torch.empty(half, dtype=torch.uint8, device=dev)
        self.fread = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        self.sink = torch.zeros(64, dtype=torch.int32, device=dev)

    def flush(self, sp):
        """Write 512 MB, then read 1 GiB of other data: what the caches hold after
        this is clean and unrelated to the next call."""
        rc = self.lib.ccv_calib_copy(self.fdst.data_ptr(), self.fsrc.data_ptr(), self.fsrc.numel(), sp)
        rc = rc or self.lib.ccv_calib_read(self.fread.data_ptr(), self.fread.numel(), 0x9E3779B9,
                                           self.sink.data_ptr(), sp)
        if rc != 0:
            raise RuntimeError(f"cache flush failed ({rc})")


def timed_calls(step, warmup, steps, calib, stream):
    """W flushed warm-up calls, then exactly K flushed calls, each between its own
    HIP events on `stream`; returns the K per-call times in microseconds."""
    import ctypes

    import torch
    sp = ctypes.c_void_p(stream.cuda_stream)
    for i in range(warmup):
        calib.flush(sp)
        step(i)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        calib.flush(sp)
        a.record(stream)
        step(warmup + i)
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in evs]


def back_to_back(step, steps, stream):
    """K calls in a row (the caller rotates buffer sets): microseconds per call."""
    import torch
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(5):
        step(i)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) * 1e3 / steps


def sustained_warmup(step, warmup, stream, min_ms=100.0, max_calls=5000):
    """W warm-up calls, and more until about `min_ms` of back-to-back work has run:
    back-to-back calls of the backward on the large shapes run about 10% slower
    for their first few tens of milliseconds of continuous load than afterwards
    (30 timed calls after 5 warm-up calls against after 100 or more), so a short
    warm-up would time the ramp.  Returns the number of warm-up calls made."""
    import torch
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(3):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    est_ms = max(ev0.elapsed_time(ev1) / 3, 1e-3)
    n = max(warmup, min(max_calls, math.ceil(min_ms / est_ms)))
    for i in range(n):
        step(i)
    torch.cuda.synchronize()
    return n


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def gbps(nbytes, us):
    return nbytes / (us * 1e-6) / 1e9


def copy_ceiling(nbytes, dev, stream, calib, steps):
    """A streaming copy that reads and writes nbytes / 2 each (rotated over >= 1 GiB
    of buffers), in three forms: non-temporal with 16 waves per CU walking 4 KB
    chunks, non-temporal with one wave per chunk, and ordinary accesses with one
    wave per chunk.  Returns the fastest, with all three."""
    import ctypes

    import torch
    sp = ctypes.c_void_p(stream.cuda_stream)
    half = max(16, (nbytes // 2) // 16 * 16)
    csets = max(2, math.ceil(ROTATION_BYTES / (2 * half)))
    bufs = [(torch.empty(half, dtype=torch.uint8, device=dev), torch.zeros(half, dtype=torch.uint8, device=dev))
            for _ in range(csets)]
    forms = {"nt_16_waves_per_cu": (16, 1), "nt_wave_per_chunk": (0, 1), "plain_wave_per_chunk": (0, 0)}
    res = {}
    for name, (wpc, nt) in forms.items():
        def step(i, wpc=wpc, nt=nt):
            d, s_ = bufs[i % csets]
            if calib.lib.ccv_calib_copy_ex(d.data_ptr(), s_.data_ptr(), half, wpc, nt, sp) != 0:
                raise RuntimeError("copy failed")
        us = back_to_back(step, steps, stream)
        res[name] = round(gbps(2 * half, us), 1)
    del bufs
    best = max(res, key=res.get)
    return {"GBps": res[best], "frac": round(res[best] / PEAK_HBM_GBPS, 4), "form": best, "forms": res}


def empty_floor(stream, calib):
    """Device time per launch of an empty kernel over 1000 back-to-back launches."""
    import ctypes

    import torch
    sp = ctypes.c_void_p(stream.cuda_stream)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(50):
        calib.lib.ccv_calib_empty(sp)
    ev0.record(stream)
    for _ in range(1000):
        calib.lib.ccv_calib_empty(sp)
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1)           # ms for 1000 launches = us per launch


def kernel_key_of(w, plan):
    """The profile name of this call's forward kernel (the channel-last LDS forms,
    chosen with CCV_CL_LDS, have their own: the plan shows which one runs)."""
    import causal_depthwise_conv1d_amd as ccv
    cl = plan["path"] == ccv.CCV_PATH_CHANNEL_LAST
    form = ""
    if cl and plan["channels_per_item"] == 256:
        form = "_tr"
    elif cl and plan["vector"] == 1 and plan["span"] == 16 and plan["unroll"] == 16:
        form = "_lds"
    return ("cl_fwd" if cl else "cf_fwd") + f"_{w.x_dtype}_B{w.B}_C{w.C}_L{w.L}_K{w.K}" + \
        ("" if w.w_dtype == w.x_dtype else f"_w{w.w_dtype}") + form


def measure_forward(n, args, dev, props, calib):
    """GPU half of one workload's record: flushed timed calls, back-to-back calls,
    graph replay and the copy ceiling; returns (record, workload, host copy of out,
    host copy of final_states or None)."""
    import ctypes

    import torch

    import causal_depthwise_conv1d_amd as ccv
    import workloads as wl

    t0 = time.time()
    w = wl.workload(n)
    if args.w_dtype and args.w_dtype != w.w_dtype:
        # the same weight values stored in another dtype (exact when widening)
        w.weight = w.weight.to(wl.TORCH_DTYPES[args.w_dtype])
        w.bias = None if w.bias is None else w.bias.to(wl.TORCH_DTYPES[args.w_dtype])
        w.w_dtype = args.w_dtype
        w.name += f"_w{args.w_dtype}"
    log(f"[bench] workload {n} {w.name}: generated in {time.time() - t0:.1f}s")
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
    for _ in range(nsets):
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
    fwd = ccv.lib().ccv_fwd
    arg_refs = [ctypes.byref(s[4]) for s in sets]
    sp = ctypes.c_void_p(stream.cuda_stream)

    def step(i):
        rc = fwd(arg_refs[i % nsets], sp)
        if rc != 0:
            raise RuntimeError(ccv.ccv_status_str(rc))

    # The timed region: every call reads x from HBM with clean, unrelated caches.
    us = timed_calls(lambda i: step(0), args.warmup, args.steps, calib, stream)
    med, mean = median(us), sum(us) / len(us)
    rec = {
        "workload": w.name,
        "description": w.notes.get("description"),
        "B": w.B, "C": w.C, "L": w.L, "K": w.K,
        "x_strides": list(w.x.stride()),
        "activation": w.activation,
        "storage_dtype": w.x_dtype,
        "weight_dtype": w.w_dtype,
        "algorithmic_bytes": nbytes,
        "kernel": kernel_key_of(w, plan),
        "plan": plan,
        "flushed_calls": {"calls": len(us), "median_us": round(med, 3), "mean_us": round(mean, 3),
                          "min_us": round(min(us), 3), "max_us": round(max(us), 3),
                          "median_GBps": round(gbps(nbytes, med), 1),
                          "median_frac": round(gbps(nbytes, med) / PEAK_HBM_GBPS, 4),
                          "mean_GBps": round(gbps(nbytes, mean), 1)},
    }
    log(f"[bench] flushed calls: median {med:.2f} us ({gbps(nbytes, med):.0f} GB/s), mean {mean:.2f} us, "
        f"min {min(us):.2f}, max {max(us):.2f}")
    out_host = sets[0][2].cpu()
    fs_host = None if sets[0][3] is None else sets[0][3].cpu()

    if not args.timed_only:
        b2b = back_to_back(step, args.steps, stream)
        rec["back_to_back"] = {"calls": args.steps, "buffer_sets": nsets, "us_per_call": round(b2b, 3),
                               "GBps": round(gbps(nbytes, b2b), 1),
                               "frac": round(gbps(nbytes, b2b) / PEAK_HBM_GBPS, 4)}
        log(f"[bench] back-to-back: {b2b:.2f} us per call, {gbps(nbytes, b2b):.0f} GB/s")
        rec["graph_replay"] = graph_timing(fwd, arg_refs, nsets, nbytes)
        rec["copy_same_bytes"] = copy_ceiling(nbytes, dev, stream, calib, args.steps)
        log(f"[bench] copy of the same bytes: {rec['copy_same_bytes']}")
    # the sources of this record's kernel: a profile stays valid while they are unchanged
    sha = kernel_sources_sha256(CF_SOURCES if plan["path"] == ccv.CCV_PATH_CHANNEL_FIRST else CL_SOURCES)
    rec["kernel_sources_sha256"] = sha
    traffic = profile_traffic(rec["kernel"], sha)
    rec["traffic_bytes"] = traffic
    rec["traffic_ratio"] = None if traffic is None else round(traffic / nbytes, 4)
    rec["kernel_trace"] = profile_kernel_time(rec["kernel"], sha, nbytes)
    del sets, arg_refs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec, w, out_host, fs_host


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=0, choices=[0, 1, 2, 3, 4, 5],
                    help="0 (default): all five, headline on workload 5; N: only workload N")
    ap.add_argument("--op", default="fwd", choices=["fwd", "update", "bwd"],
                    help="fwd: the forward (default); update: the decode step; "
                         "bwd: the backward on --workload (default 2)")
    ap.add_argument("--w-dtype", default=None, choices=["f32", "bf16", "f16"],
                    help="store the workload's weights and bias in this dtype instead (same values "
                         "when widening): a mixed x / weight dtype call")
    ap.add_argument("--seqs", type=int, default=0,
                    help="--op bwd: pack each row with this many sequences (seq_idx)")
    ap.add_argument("--timed-only", action="store_true",
                    help="only the warm-up and timed calls (for profiling): no back-to-back, graph or copy runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=2.0,
                    help="minimum time spent timing the one-thread oracle, per workload")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the op needs no communication: batch or channel shards run independently)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import causal_depthwise_conv1d_amd as ccv

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ccv.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)

    if args.op == "update":
        args.workload = 0
        bench_update(args, dev, props)
        return
    if args.op == "bwd":
        args.workload = args.workload or 2
        bench_bwd(args, dev, props)
        return

    calib = Calib(dev)
    stream = torch.cuda.current_stream()
    floor_us = empty_floor(stream, calib)
    log(f"[bench] empty kernel: {floor_us:.2f} us per launch")
    flushed_floor = None
    if not args.timed_only:
        # The same single-call timing around an empty kernel: what a flushed call
        # costs beyond its kernel's own duration (dispatch from an idle queue).
        import ctypes
        sp = ctypes.c_void_p(stream.cuda_stream)
        t = timed_calls(lambda i: calib.lib.ccv_calib_empty(sp), args.warmup, args.steps, calib, stream)
        flushed_floor = {"median_us": round(median(t), 3), "min_us": round(min(t), 3), "max_us": round(max(t), 3)}
        log(f"[bench] empty kernel as a flushed single call: {flushed_floor['median_us']:.2f} us (median)")
    ns = [args.workload] if args.workload else [1, 2, 3, 4, 5]
    head = args.workload or HEADLINE_WORKLOAD
    records = {}
    for n in ns:
        rec, w, out_host, fs_host = measure_forward(n, args, dev, props, calib)
        if not args.no_cpu_baseline:
            rec["oracle"] = oracle_leg(w, out_host, fs_host, rec["algorithmic_bytes"], args.cpu_seconds)
        records[n] = rec
        del w, out_host, fs_host

    r = records[head]
    fl = r["flushed_calls"]
    med_us, mean_us = fl["median_us"], fl["mean_us"]
    value = gbps(r["algorithmic_bytes"], med_us)
    achieved = gbps(r["algorithmic_bytes"], mean_us)
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(med_us * 1e-3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {k: r[k] for k in ("workload", "description", "B", "C", "L", "K", "x_strides", "activation",
                                     "storage_dtype", "weight_dtype", "algorithmic_bytes", "kernel", "plan")},
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBPS, 2),
        "timing": "value: algorithmic bytes / median of the K flushed single calls (HIP events on the "
                  "launch stream); roofline.achieved: the same bytes / their mean",
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": r["traffic_bytes"],
            "kernel": r["kernel"],
            "avg_launch_us": mean_us,
            "algorithmic_bytes_per_launch": r["algorithmic_bytes"],
        },
        "context": {
            "headline_record": {k: v for k, v in r.items() if k != "oracle"},
            "per_workload": {str(n): v for n, v in records.items() if n != head},
            "empty_kernel_us": round(floor_us, 3),
            "empty_kernel_flushed_call": flushed_floor,
            "device": props.name,
            "cu_count": props.multi_processor_count,
            "device_properties": device_properties(props),
            "kernel_sources_sha256": kernel_sources_sha256(),
            "env_overrides": env_overrides(),
        },
    }
    if "oracle" in r:
        o = r["oracle"]
        result["cpu_baseline"] = dict(o["one_thread"], all_cores=o["all_cores"], parity=o["parity"],
                                      host_cpu=o["host_cpu"], compile_flags=o["compile_flags"])
    print(json.dumps(result), flush=True)


def context_measurements(nbytes, dev, stream, steps):
    """The copy ceiling and the empty-kernel floor, for the update and backward
    lines: (best copy GB/s, empty kernel us)."""
    calib = Calib(dev)
    c = copy_ceiling(nbytes, dev, stream, calib, steps)
    floor_us = empty_floor(stream, calib)
    log(f"[bench] copy of the same bytes: {c['GBps']:.0f} GB/s ({c['form']}); empty kernel {floor_us:.2f} us")
    return c["GBps"], floor_us


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
    names = ("CCV_CF_WAVES_PER_CU", "CCV_CL_WAVES_PER_CU", "CCV_CL_TILE_T", "CCV_CL_LDS", "CCV_CU_COUNT",
             "CCV_FORCE_SCALAR")
    return {n: os.environ[n] for n in names if n in os.environ}


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

    warm_calls = sustained_warmup(step, args.warmup, stream)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    gbps = nbytes / (ms_per_step * 1e-3) / 1e9
    log(f"[bench] update: {warm_calls} warm-up calls, then {ms_per_step * 1e3:.2f} us/call, {gbps:.0f} GB/s")
    copy_gbps, empty_us = context_measurements(nbytes, dev, stream, args.steps)

    kernel_key = f"update_{w.x_dtype}_B{B}_C{C}_L{L}_K{K}"
    sha = kernel_sources_sha256(UPDATE_SOURCES)
    result = {
        "metric": UPDATE_METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warm_calls,
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
        "timing": (f"K calls back to back (HIP events on the launch stream), after {warm_calls} warm-up "
                   f"calls: at least W={args.warmup} and about 100 ms of continuous calls"),
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
    once, the parameters read and their gradients written once, seq_idx read once,
    the states and their gradients once.  The partial-sum workspace is overhead."""
    es = w.x.element_size()
    B, C, L, K = w.B, w.C, w.L, w.K
    pb = w.weight.element_size()
    n = 3 * B * C * L * es + 2 * C * K * pb
    if w.seq_idx is not None:
        n += B * L * 4
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
    if args.seqs:
        # the same rows packed with that many sequences (uniform lengths, at least 64 steps)
        w.seq_idx = wl.seq_idx_from_lengths(wl.packed_lengths(w.L, args.seqs, 64, w.seed), w.B)
        w.name += f"_seq{args.seqs}"
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
    warm_calls = sustained_warmup(step, args.warmup, stream)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    gbps = nbytes / (ms_per_step * 1e-3) / 1e9
    log(f"[bench] bwd: {warm_calls} warm-up calls, then {ms_per_step * 1e3:.2f} us/call, {gbps:.0f} GB/s")
    copy_gbps, empty_us = context_measurements(nbytes, dev, stream, min(args.steps, 200))

    kernel_key = f"bwd_{w.x_dtype}_B{B}_C{C}_L{L}_K{K}" + (f"_seq{args.seqs}" if args.seqs else "")
    sha = kernel_sources_sha256(BWD_SOURCES)
    result = {
        "metric": BWD_METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warm_calls,
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
        "timing": (f"K calls back to back (HIP events on the launch stream), after {warm_calls} warm-up "
                   f"calls: at least W={args.warmup} and about 100 ms of continuous calls"),
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


def host_cpu_name() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def oracle_pieces(w, max_outputs):
    """(b, c0, c1) pieces of at most max_outputs outputs (at least one channel)
    that together cover the workload once; channels are independent, so each
    piece is an exact sub-problem."""
    ch = max(1, min(w.C, max_outputs // max(1, w.L)))
    return [(b, c0, min(w.C, c0 + ch)) for b in range(w.B) for c0 in range(0, w.C, ch)]


def sub_case(w, b, c0, c1):
    from oracle.from_torch import case
    return case(w.x[b:b + 1, c0:c1], w.weight[c0:c1], None if w.bias is None else w.bias[c0:c1],
                None if w.seq_idx is None else w.seq_idx[b:b + 1],
                None if w.initial_states is None else w.initial_states[b:b + 1, c0:c1], w.activation)


def oracle_leg(w, out_host, fs_host, nbytes, min_seconds):
    """The oracle as written on this host's CPU.

    One thread (the baseline): the plain fp64 loop, rounding included, over a
    bounded sample -- the whole workload when it has at most 2^25 outputs,
    otherwise its first (b, channel range) piece of at most 2^25 outputs --
    repeated until at least `min_seconds` have passed; GB/s = the sample's share
    of the algorithmic bytes / time.

    All cores (context): the same per-output function on up to 16 threads over
    the whole workload, piece by piece; every output of this run's GPU result is
    compared with it at the stated tolerances, and the final states bit for bit."""
    import numpy as np

    from oracle import GCC_CMD, round_out
    from oracle import compare as ocmp
    from oracle.from_torch import dtype_name, raw

    total = w.B * w.C * w.L
    pieces = oracle_pieces(w, 1 << 25)
    b, c0, c1 = pieces[0]
    sample = sub_case(w, b, c0, c1)
    n_sample = (c1 - c0) * w.L
    passes, t_total, y1 = 0, 0.0, None
    while passes == 0 or t_total < min_seconds:
        t0 = time.perf_counter()
        y1, _ = sample.fwd()
        round_out(w.x_dtype, y1)
        t_total += time.perf_counter() - t0
        passes += 1
    sec = t_total / passes
    share = n_sample / total
    log(f"[bench] cpu oracle, one thread: {n_sample} outputs, {passes} passes, {sec:.3f} s per pass")
    one = {"value": round(nbytes * share / sec / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": (f"batch {b}, channels [{c0},{c1}) x {w.L} steps = {n_sample} of {total} outputs "
                      f"({100 * share:.1f}%), {passes} pass(es) of the single-threaded fp64 oracle incl. "
                      "rounding to the output dtype; GB/s scaled by that share of the algorithmic bytes"),
           "seconds_per_pass": round(sec, 4),
           "seconds_whole_workload_est": round(sec / share, 3)}

    nthr = max(1, min(16, len(os.sched_getaffinity(0))))
    out_c = out_host.contiguous()
    t_oracle, t_check = 0.0, 0.0
    tot = {"outputs": 0, "out_of_tolerance": 0, "max_ulp": 0, "max_rel": 0.0, "floor_only": 0, "bit_equal": 0}
    same_as_one_thread = None
    for (b, c0, c1) in pieces:
        c = sub_case(w, b, c0, c1)
        t0 = time.perf_counter()
        y, s = c.fwd_threads(nthr)
        round_out(w.x_dtype, y)
        t_oracle += time.perf_counter() - t0
        if same_as_one_thread is None:
            same_as_one_thread = bool(np.array_equal(y.view(np.uint64), y1.view(np.uint64)))
        t0 = time.perf_counter()
        g = out_c[b:b + 1, c0:c1].contiguous()
        res = ocmp.compare(dtype_name(g), w.K, raw(g), y, s)
        t_check += time.perf_counter() - t0
        tot["outputs"] += res["n"]
        tot["out_of_tolerance"] += res["n_bad"]
        tot["floor_only"] += res["n_floor_only"]
        tot["bit_equal"] += res["bit_equal"]
        tot["max_ulp"] = max(tot["max_ulp"], res["max_ulp"] or 0)
        tot["max_rel"] = max(tot["max_rel"], res["max_rel"])
    if w.x_dtype == "f32":
        tot["max_ulp"] = None
    if fs_host is not None:
        from oracle.from_torch import case
        want = case(w.x, w.weight, w.bias, w.seq_idx, w.initial_states, w.activation).final_states()
        got = raw(fs_host.contiguous())
        bits = np.uint32 if got.dtype == np.float32 else np.uint16
        tot["final_states_bit_exact"] = bool(np.array_equal(got.view(bits), want.view(bits)))
    log(f"[bench] cpu oracle on {nthr} threads: whole workload in {t_oracle:.2f} s; parity {tot} "
        f"(checked in {t_check:.1f} s)")
    allc = {"value": round(nbytes / t_oracle / 1e9, 4), "unit": "GB/s", "threads": nthr,
            "seconds_whole_workload": round(t_oracle, 3), "pieces": len(pieces),
            "first_piece_bit_identical_to_one_thread": same_as_one_thread}
    return {"one_thread": one, "all_cores": allc, "parity": tot, "host_cpu": host_cpu_name(),
            "host_threads_available": os.cpu_count(),
            "compile_flags": " ".join(f for f in GCC_CMD[1:] if f.startswith("-") and f not in ("-o", "-shared"))}


if __name__ == "__main__":
    main()
