"""The five named workloads at their full sizes, in the launch configuration the
bench times (default plan, torch's current stream).

The small channel-first workload and the channel-first bf16 workload are compared
with the oracle at every output.  The three large ones are compared at sampled
outputs the oracle computes one by one (uniform random positions plus every
wave-segment / time-tile boundary, sequence boundary and sequence start/end),
over the whole time axis of a slice of channels (channels are independent, so a
channel slice is an exact sub-problem), and by properties that hold at any size
(every output finite; final states bit-exact in full)."""
import time

import numpy as np
import pytest
import torch

import causal_depthwise_conv1d_amd as ccv
import workloads as wl
from gpu_support import assert_close, assert_final_states, gpu_args, log, oracle_case
from oracle import compare as ocmp
from oracle.from_torch import case, dtype_name, raw

pytestmark = pytest.mark.gpu


def run(w):
    kw = gpu_args(w)
    plan = ccv.plan_for(x=kw["x"], weight=kw["weight"], bias=kw["bias"], seq_idx=kw["seq_idx"],
                        initial_states=kw["initial_states"], activation=kw["activation"])
    res = ccv.causal_conv1d_fwd(**kw)
    torch.cuda.synchronize()
    out, fs = res if w.return_final_states else (res, None)
    return kw, plan, out, fs


def boundary_times(L, step, K):
    ts = set(range(min(L, K + 3))) | set(range(max(0, L - K - 3), L))
    for m in range(step, L, step):
        ts |= set(range(max(0, m - K - 1), min(L, m + K + 1)))
    return np.array(sorted(ts), dtype=np.int64)


def sampled_check(w, out_gpu, extra_t=None, n_random=200_000, seed=0):
    B, C, L = w.B, w.C, w.L
    g = np.random.default_rng(seed)
    idx = np.stack([g.integers(0, B, n_random), g.integers(0, C, n_random), g.integers(0, L, n_random)], 1)
    if extra_t is not None:
        nb = min(C, 64)
        bb, cc, tt = np.meshgrid(np.arange(B), g.choice(C, nb, replace=False), extra_t, indexing="ij")
        idx = np.concatenate([idx, np.stack([bb.ravel(), cc.ravel(), tt.ravel()], 1)])
    c = oracle_case(w)
    t0 = time.time()
    y, s = c.points(idx)
    log(f"  oracle: {len(idx)} sampled outputs in {time.time() - t0:.1f}s")
    ti = torch.from_numpy(idx).cuda()
    gv = out_gpu[ti[:, 0], ti[:, 1], ti[:, 2]].cpu()
    res = ocmp.compare(dtype_name(gv), w.K, raw(gv), y, s)
    if res["n_bad"]:
        raise AssertionError(ocmp.describe_failures(res, y, s, raw(gv), dtype_name(gv)))
    return res


def channel_slice_check(w, kw, out_gpu, c0, c1, b=0):
    """Every output of channels [c0, c1) of batch b against the oracle run on the
    same sub-problem."""
    x = w.x[b:b + 1, c0:c1]
    init = None if w.initial_states is None else w.initial_states[b:b + 1, c0:c1]
    seq = None if w.seq_idx is None else w.seq_idx[b:b + 1]
    sub = case(x, w.weight[c0:c1], None if w.bias is None else w.bias[c0:c1], seq, init, w.activation)
    t0 = time.time()
    y, s = sub.fwd()
    log(f"  oracle: channel slice [{c0},{c1}) x {w.L} steps in {time.time() - t0:.1f}s")
    g = out_gpu[b:b + 1, c0:c1].cpu().contiguous()
    res = ocmp.compare(dtype_name(g), w.K, raw(g), y, s)
    if res["n_bad"]:
        raise AssertionError(ocmp.describe_failures(res, y, s, raw(g), dtype_name(g), shape=tuple(g.shape)))
    return res


def fma_chain_check(w, out_gpu, extra_t, c0, c1, n_random=200_000, seed=1):
    """Without an activation the kernel sums exactly as the oracle's binary32 mode
    does (bias first, one fused multiply-add per kept term, k ascending): sampled
    outputs and one whole channel slice must be bit-identical to it."""
    assert w.activation is None and w.x_dtype == "f32"
    B, C, L = w.B, w.C, w.L
    g = np.random.default_rng(seed)
    idx = np.stack([g.integers(0, B, n_random), g.integers(0, C, n_random), g.integers(0, L, n_random)], 1)
    bb, cc, tt = np.meshgrid(np.arange(B), g.choice(C, min(C, 32), replace=False), extra_t, indexing="ij")
    idx = np.concatenate([idx, np.stack([bb.ravel(), cc.ravel(), tt.ravel()], 1)])
    want = oracle_case(w).points_f32(idx)
    ti = torch.from_numpy(idx).cuda()
    got = out_gpu[ti[:, 0], ti[:, 1], ti[:, 2]].cpu().numpy()
    diff = got.view(np.uint32) != want.view(np.uint32)
    assert not diff.any(), f"{int(diff.sum())} sampled outputs differ, first at {idx[diff][:4].tolist()}"
    init = None if w.initial_states is None else w.initial_states[:1, c0:c1]
    sub = case(w.x[:1, c0:c1], w.weight[c0:c1], None if w.bias is None else w.bias[c0:c1], None, init, None)
    want = sub.fwd_f32()
    got = out_gpu[:1, c0:c1].cpu().contiguous().numpy()
    diff = got.view(np.uint32) != want.view(np.uint32)
    assert not diff.any(), f"{int(diff.sum())} outputs of channels [{c0},{c1}) differ"
    log(f"  binary32 chain: {len(idx)} samples and channels [{c0},{c1}) bit-identical")


def test_workload_1_small_channel_first_all_outputs():
    w = wl.workload(1)
    kw, plan, out, _ = run(w)
    assert plan["path"] == ccv.CCV_PATH_CHANNEL_FIRST and plan["vector"] == 1
    y, s = oracle_case(w).fwd()
    res = assert_close(w, out.cpu().contiguous(), y, s)
    log(f"  workload 1: {res['n']} outputs, max rel {res['max_rel']:.2e}, floor-only {res['n_floor_only']}")


def test_workload_2_channel_first_bf16_all_outputs():
    w = wl.workload(2)
    kw, plan, out, _ = run(w)
    assert plan["path"] == ccv.CCV_PATH_CHANNEL_FIRST and plan["vector"] == 1
    t0 = time.time()
    y, s = oracle_case(w).fwd()
    log(f"  oracle: all {y.size} outputs in {time.time() - t0:.1f}s")
    res = assert_close(w, out.cpu().contiguous(), y, s)
    log(f"  workload 2: max ulp {res['max_ulp']}, floor-only {res['n_floor_only']}, "
        f"bit-equal {res['bit_equal']}/{res['n']}")


def test_workload_3_channel_last_view_with_states():
    t0 = time.time()
    w = wl.workload(3, poison_unused=True)      # channels >= 4096 of the buffer are NaN
    log(f"  generated in {time.time() - t0:.1f}s")
    kw, plan, out, fs = run(w)
    assert plan["path"] == ccv.CCV_PATH_CHANNEL_LAST and plan["vector"] == 1
    assert kw["x"].stride() == (8192 * 10240, 1, 10240)
    assert bool(torch.isfinite(out).all()), "an output read outside the view"
    assert_final_states(w, fs.cpu().contiguous())
    sampled_check(w, out, boundary_times(w.L, plan["span"], w.K))
    channel_slice_check(w, kw, out, 0, 64, b=0)
    channel_slice_check(w, kw, out, 4096 - 40, 4096, b=7)


def test_workload_4_packed_varlen_fp16():
    w = wl.workload(4)
    kw, plan, out, _ = run(w)
    assert plan["path"] == ccv.CCV_PATH_CHANNEL_LAST
    ids = w.seq_idx[0].numpy()
    starts = np.flatnonzero(np.diff(ids)) + 1
    assert len(starts) == 63 and np.diff(np.concatenate([[0], starts, [w.L]])).min() >= 64
    extra = set(boundary_times(w.L, plan["span"], w.K).tolist())
    for s0 in starts:
        extra |= set(range(max(0, s0 - 4), min(w.L, s0 + 4)))
    assert bool(torch.isfinite(out).all())
    sampled_check(w, out, np.array(sorted(extra)))
    channel_slice_check(w, kw, out, 0, 16)
    channel_slice_check(w, kw, out, 2560 - 16, 2560)


def test_workload_5_long_sequence_channel_first():
    t0 = time.time()
    w = wl.workload(5)
    log(f"  generated in {time.time() - t0:.1f}s")
    kw, plan, out, fs = run(w)
    assert plan["path"] == ccv.CCV_PATH_CHANNEL_FIRST and plan["vector"] == 1
    # 256 rows of 1M steps: each row must be split over many waves (runs of segments)
    assert plan["work_items"] >= 16 * 256, "long rows must be split across many waves"
    assert plan["span"] < w.L
    assert bool(torch.isfinite(out).all())
    assert_final_states(w, fs.cpu().contiguous())
    sampled_check(w, out, boundary_times(w.L, plan["span"], w.K))
    channel_slice_check(w, kw, out, 0, 2, b=0)
    channel_slice_check(w, kw, out, 126, 128, b=1)
    fma_chain_check(w, out, boundary_times(w.L, plan["span"], w.K), 40, 41)
