"""ccv_bwd_static (the backward with its partial sums in the library's fixed device
array) against ccv_bwd (the same backward with a caller-provided workspace),
through the C ABI: every gradient bit for bit, on two calls in a row, the second
with a smaller input, so the second call runs over the first call's leftovers in
the shared array.  The workspace path itself is checked against the oracle by the
backward parity tests; here the oracle check is repeated for the static path.
Also the use it exists for: the call captured in a HIP graph and replayed."""
import ctypes

import numpy as np
import pytest
import torch

import causal_depthwise_conv1d_amd as ccv
import workloads as wl
from gpu_support import to_gpu_view
from oracle import compare as ocmp
from oracle.from_torch import bwd as oracle_bwd
from oracle.from_torch import case, dtype_name, raw

pytestmark = pytest.mark.gpu

DOUT_ID, DFS_ID = 5, 6


def problem(B, C, L, K, dtype, layout, seed, seq=False):
    w = wl.make_case(B=B, C=C, L=L, K=K, x_dtype=dtype, layout=layout, seed=seed, bias=True, init=True,
                     activation="silu", seq_lengths=[L // 3, L - L // 3] if seq else None)
    g = wl.to_storage(wl.draw(B * C * L, seed, DOUT_ID, "normal", 1.0), dtype)
    dout = g.reshape(B, C, L) if layout == "cf" else g.reshape(B, L, C).transpose(1, 2)
    dfs = wl.to_storage(wl.draw(B * C * (K - 1), seed, DFS_ID, "normal", 1.0), dtype).reshape(B, C, K - 1)
    return w, g, dout, dfs


def outputs(w):
    """Fresh gradient buffers, filled with NaN so a missed write shows."""
    B, C, L, K = w.B, w.C, w.L, w.K
    xd = w.x.dtype
    dx = (torch.full((B, C, L), float("nan"), dtype=xd, device="cuda") if w.layout == "cf"
          else torch.full((B, L, C), float("nan"), dtype=xd, device="cuda").transpose(1, 2))
    dw = torch.full((C, K), float("nan"), dtype=w.weight.dtype, device="cuda")
    db = torch.full((C,), float("nan"), dtype=w.weight.dtype, device="cuda")
    dinit = torch.full((B, K - 1, C), float("nan"), dtype=xd, device="cuda").transpose(1, 2)
    return dx, dw, db, dinit


def run(w, g, dout, dfs, static):
    x = to_gpu_view(w.x_storage, w.x)
    dout_g = to_gpu_view(g, dout)
    weight, bias = w.weight.cuda(), w.bias.cuda()
    seq = None if w.seq_idx is None else w.seq_idx.cuda()
    init, dfs_g = to_gpu_view(w.init_storage, w.initial_states), dfs.cuda()
    dx, dw, db, dinit = outputs(w)
    a = ccv.make_bwd_args(x, weight, bias, dout_g, dx, dw, db, seq, init, dfs_g, dinit, w.activation)
    stream = torch.cuda.current_stream().cuda_stream
    if static:
        st = ccv.ccv_bwd_static(a, stream)
    else:
        ws = ccv.ccv_bwd_workspace_size(a)
        assert 0 < ws <= ccv.CCV_BWD_STATIC_SCRATCH_BYTES, ws
        workspace = torch.empty(ws, dtype=torch.uint8, device="cuda")
        a.workspace, a.workspace_bytes = workspace.data_ptr(), ws
        st = ccv.ccv_bwd(a, stream)
    assert st == 0, ccv.ccv_status_str(st)
    torch.cuda.synchronize()
    return [t.cpu().contiguous() for t in (dx, dw, db, dinit)]


def same_bits(a, b):
    va = a.view(torch.int32 if a.dtype == torch.float32 else torch.int16)
    vb = b.view(torch.int32 if b.dtype == torch.float32 else torch.int16)
    return torch.equal(va, vb)


def test_static_scratch_equals_workspace_on_two_calls():
    cases = [problem(2, 1024, 8192, 4, "bf16", "cl", 71, seq=True),   # 2.6 MB of partial sums
             problem(1, 96, 1000, 3, "f32", "cf", 72)]                 # the second call: smaller
    for i, (w, g, dout, dfs) in enumerate(cases):
        ref = run(w, g, dout, dfs, static=False)
        got = run(w, g, dout, dfs, static=True)
        for name, r, t in zip(("dx", "dweight", "dbias", "dinitial_states"), ref, got):
            assert not torch.isnan(t).any(), (i, name)
            assert same_bits(r, t), (i, name)
        # and the static path against the oracle at the backward's tolerances (the
        # parameter sums at the backward tests' cap of 64 roundings' worth)
        c = case(w.x, w.weight, w.bias, w.seq_idx, w.initial_states, w.activation)
        r = oracle_bwd(c, dout, dfs)
        for name, t, want, scale, kk in (("dx", got[0], r["dx"], r["ex"], w.K + 2),
                                         ("dinit", got[3], r["dinit"], r["einit"], w.K + 2),
                                         ("dweight", got[1], r["dw"], r["ew"], 64),
                                         ("dbias", got[2], r["db"], r["eb"], 64)):
            res = ocmp.compare(dtype_name(t), kk, raw(t), want, scale)
            assert res["n_bad"] == 0, (i, name, ocmp.describe_failures(res, want, scale, raw(t), dtype_name(t)))


def test_static_scratch_refuses_calls_beyond_its_size():
    """A call needing more than the fixed array returns CCV_E_SCRATCH before any
    launch (checked with never-dereferenced addresses)."""
    a = ccv.ccv_bwd_args_t()
    a.B, a.C, a.L, a.K = 16, 8192, 8192, 4
    a.x_dtype = a.w_dtype = ccv.CCV_BF16
    a.x, a.dout, a.dx, a.weight, a.dweight = (0x100000 * (i + 1) for i in range(5))
    st = (8192 * 8192, 1, 8192)
    for f in ("x_stride", "dout_stride", "dx_stride"):
        setattr(a, f, type(getattr(a, f))(*st))
    assert ccv.ccv_bwd_workspace_size(a) > ccv.CCV_BWD_STATIC_SCRATCH_BYTES
    assert ccv.STATUS[ccv.lib().ccv_bwd_static(ctypes.byref(a), None)] == "CCV_E_SCRATCH"
    assert np.int64(ccv.CCV_BWD_STATIC_SCRATCH_BYTES) == 64 << 20


@pytest.mark.parametrize("layout", ["cf", "cl"])
def test_static_backward_in_a_graph(layout):
    """The callers ccv_bwd_static is for: captured in a HIP graph (torch.cuda.graph)
    with no workspace to allocate, and replayed with new inputs written eagerly in
    between; every replay equals an eager ccv_bwd (workspace path) on the same
    inputs bit for bit."""
    B, C, L, K = 2, 136, 2100, 4
    gw = torch.Generator().manual_seed(7900)
    weight = (torch.randn(C, K, generator=gw) * 0.5).to(torch.bfloat16).cuda()
    bias = (torch.randn(C, generator=gw) * 0.3).to(torch.bfloat16).cuda()

    def fresh(seed):
        g = torch.Generator().manual_seed(seed)
        shape = (B, C, L) if layout == "cf" else (B, L, C)
        x = torch.randn(*shape, generator=g).to(torch.bfloat16).cuda()
        dout = torch.randn(*shape, generator=g).to(torch.bfloat16).cuda()
        return (x, dout) if layout == "cf" else (x.transpose(1, 2), dout.transpose(1, 2))

    x, dout = fresh(7901)
    dx = ccv.empty_like_layout(x)
    dw = torch.empty(C, K, dtype=torch.bfloat16, device="cuda")
    db = torch.empty(C, dtype=torch.bfloat16, device="cuda")
    a = ccv.make_bwd_args(x, weight, bias, dout, dx, dw, db, activation="silu")

    def call():
        st = ccv.ccv_bwd_static(a, torch.cuda.current_stream().cuda_stream)
        assert st == 0, ccv.ccv_status_str(st)

    side = torch.cuda.Stream()                      # warm-up call off the capture
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for r in range(4):
        nx, ndout = fresh(7910 + r)
        x.copy_(nx)
        dout.copy_(ndout)
        ref = ccv.causal_conv1d_bwd(nx, weight, bias, ndout, activation="silu")
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("dx", "dweight", "dbias"), (dx, dw, db), ref):
            assert same_bits(got.cpu().contiguous(), want.cpu().contiguous()), (layout, r, name)
