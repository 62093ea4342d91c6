"""GPU parity of the backward through the C ABI, and of the autograd function.

dx, dweight, dbias and d(initial_states) are compared with the oracle's fp64
backward (the chain rule of the forward, pinned against torch autograd and
finite differences) element by element.  The tolerance is the forward's, with
the oracle's per-element error scale in place of S: for dx the sum of the
magnitudes of its terms, each dz also carrying |dout| * S_z; for the parameter
gradients, sums over B * L such terms in fp32, whose rounding grows with the
tile length and the number of partial sums.  Invariants checked bit for bit:
repeated runs, layout independence, packed = separate sequences for dx."""
import math

import numpy as np
import pytest
import torch

import causal_depthwise_conv1d_amd as ccv
import workloads as wl
from gpu_support import log, to_gpu_view
from oracle import compare as ocmp
from oracle.from_torch import bwd as oracle_bwd
from oracle.from_torch import case, dtype_name, raw

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    ccv.lib()

DTYPES = ["f32", "bf16", "f16"]
KS = [2, 3, 4]
DOUT_ID, DFS_ID = 5, 6


def tile_steps(dtype):
    """Time steps per tile of the backward."""
    return 32


def grad_inputs(w, layout, with_dfs, seed):
    """dout [B, C, L] (channel-first or channel-last storage) and dfinal_states."""
    B, C, L, K = w.B, w.C, w.L, w.K
    g = wl.to_storage(wl.draw(B * C * L, seed, DOUT_ID, "normal", 1.0), w.x_dtype)
    dout = g.reshape(B, C, L) if layout.startswith("cf") else g.reshape(B, L, C).transpose(1, 2)
    dfs = None
    if with_dfs:
        dfs = wl.to_storage(wl.draw(B * C * (K - 1), seed, DFS_ID, "normal", 1.0), w.x_dtype).reshape(B, C, K - 1)
    return dout, dfs


def gpu_ids(w, seq_gpu=None):
    return seq_gpu if seq_gpu is not None else (None if w.seq_idx is None else w.seq_idx.cuda())


def unaligned_ids(w):
    """w's seq_idx on the GPU, contiguous but 4 bytes off 16-byte alignment."""
    buf = torch.zeros(w.B * w.L + 1, dtype=torch.int32, device="cuda")
    buf[1:] = w.seq_idx.reshape(-1).cuda()
    ids = buf[1:].view(w.B, w.L)
    assert ids.data_ptr() % 16 != 0 and ids.is_contiguous()
    return ids


def run_bwd(w, dout, dfs, want_dinit, seq_gpu=None):
    x = to_gpu_view(w.x_storage, w.x)
    init = None if w.initial_states is None else to_gpu_view(w.init_storage, w.initial_states)
    res = ccv.causal_conv1d_bwd(
        x, w.weight.cuda(), None if w.bias is None else w.bias.cuda(), dout.cuda(),
        gpu_ids(w, seq_gpu), init, None if dfs is None else dfs.cuda(),
        w.activation, return_dinitial_states=want_dinit)
    torch.cuda.synchronize()
    return [None if t is None else t.cpu().contiguous() for t in res]


def reduction_levels(parts):
    levels, n = 1, parts
    while n > 32:
        n, levels = -(-n // 32), levels + 1
    return levels


def bwd_plan(x, weight, dout, seq=None):
    """The launch ccv_bwd makes for these tensors (dx in x's layout)."""
    C, K = weight.shape
    args = ccv.make_bwd_args(x, weight, None, dout, ccv.empty_like_layout(x),
                             torch.empty(C, K, dtype=weight.dtype, device="cuda"), seq_idx=seq)
    st, plan = ccv.ccv_bwd_plan(args)
    assert st == 0, st
    return plan


# The most roundings' worth the parameter-gradient tolerance may grant, fixed by
# the tests rather than by the kernels' plans: a kernel change that lengthens a
# lane's in-order sum (longer tiles, more tiles per partial row, a deeper tree)
# past it fails here instead of silently widening the tolerance.  The current
# plans need at most 59 (channel-last: 4 tiles of 32 steps per partial row, three
# tree levels).
PARAM_TERMS_CAP = 64


def param_terms_for(plan, B, L, K):
    """compare()'s K for the parameter gradients: (n + 32 * levels + K + 8) / 4
    roundings of 2^-22 cover a lane's in-order sum of n terms, the levels of the
    fan-in-32 reduction tree over the partial rows, and the error of dz.  The
    register-only channel-first path: n = its span / 64 elements plus the 7 additions of
    the 64-lane sum, a partial row per segment; the other paths: n = the tiles
    per partial row times the tile length.  Never more than PARAM_TERMS_CAP."""
    if plan.vector == 3:
        n, parts = plan.span // 64 + 7, B * max(1, math.ceil(L / plan.span))
    else:
        n, parts = plan.unroll * plan.span, B * max(1, math.ceil(math.ceil(L / plan.span) / plan.unroll))
    k = math.ceil((n + 32 * reduction_levels(parts) + K + 8) / 4)
    assert k <= PARAM_TERMS_CAP, f"the plan's parameter sums need {k} > {PARAM_TERMS_CAP} roundings' worth"
    return k


def param_terms(w, plan):
    return param_terms_for(plan, w.B, w.L, w.K)


def check_bwd(w, dout, dfs, want_dinit, where, seq_gpu=None, want_path=None):
    dx, dw, db, dinit = run_bwd(w, dout, dfs, want_dinit, seq_gpu)
    plan = bwd_plan(to_gpu_view(w.x_storage, w.x), w.weight.cuda(), dout.cuda(), gpu_ids(w, seq_gpu))
    assert want_path is None or plan.vector == want_path, plan.as_dict()
    c = case(w.x, w.weight, w.bias, w.seq_idx, w.initial_states, w.activation)
    r = oracle_bwd(c, dout, dfs)
    K = w.K
    checks = [("dx", dx, r["dx"], r["ex"], K + 2)]
    if want_dinit:
        checks.append(("dinit", dinit, r["dinit"], r["einit"], K + 2))
    pk = param_terms(w, plan)
    checks.append(("dweight", dw, r["dw"], r["ew"], pk))
    if w.bias is not None:
        checks.append(("dbias", db, r["db"], r["eb"], pk))
    for name, got, ref, scale, kk in checks:
        res = ocmp.compare(dtype_name(got), kk, raw(got), ref, scale)
        if res["n_bad"]:
            raise AssertionError(f"{where} {name}: " + ocmp.describe_failures(
                res, ref, scale, raw(got), dtype_name(got), shape=tuple(got.shape)))
    return dx, dw, db, dinit


def build(B, C, L, K, dtype, layout, seed, w_dtype=None, seq=None, init=False, bias=True, act="silu"):
    kw = {}
    if layout == "cf_view":
        kw = dict(layout="cf", c_pad=3, c_off=1, t_pad=13, t_off=5)
    elif layout == "cl_view":
        kw = dict(layout="cl", c_pad=8)
    else:
        kw = dict(layout=layout)
    lengths = wl.packed_lengths(L, min(seq, L), 1, seed).tolist() if (seq and L > 0) else None
    return wl.make_case(B=B, C=C, L=L, K=K, x_dtype=dtype, w_dtype=w_dtype, bias=bias, init=init,
                        seq_lengths=lengths, activation=act, seed=seed, **kw)


@pytest.mark.parametrize("layout", ["cf", "cl", "cf_view", "cl_view"])
@pytest.mark.parametrize("K", KS)
@pytest.mark.parametrize("dtype", DTYPES)
def test_bwd_matches_oracle(dtype, K, layout):
    cases = [  # L, C, B, features
        (1, 7, 2, dict(bias=True, act="silu")),
        (K - 1, 8, 1, dict(init=True, dfs=True, dinit=True)),
        (63, 70, 2, dict(bias=True, act="silu", init=True, dfs=True, dinit=True)),
        (64, 64, 1, dict(bias=False, act=None)),
        (65, 130, 3, dict(bias=True, act="silu", seq=5)),
        (300, 33, 2, dict(bias=True, act=None, init=True, dinit=True)),
        (1000, 9, 1, dict(bias=True, act="silu", seq=17, w_dtype="f32")),
        # seq_idx together with history, dfinal_states and d(initial_states)
        (520, 64, 2, dict(bias=True, act="silu", seq=6, init=True, dfs=True, dinit=True)),
        (K - 1, 8, 2, dict(seq=2, init=True, dfs=True, dinit=True)),
    ]
    for i, (L, C, B, f) in enumerate(cases):
        seed = 3000 + 100 * K + i
        w = build(B, C, L, K, dtype, layout, seed, w_dtype=f.get("w_dtype"), seq=f.get("seq"),
                  init=f.get("init", False), bias=f.get("bias", True), act=f.get("act", "silu"))
        dout, dfs = grad_inputs(w, layout, f.get("dfs", False), seed)
        log(f"  bwd {dtype}/{w.w_dtype} K={K} {layout} L={L} C={C} B={B} {f}")
        check_bwd(w, dout, dfs, f.get("dinit", False), f"[{dtype} K={K} {layout} L={L}]")


@pytest.mark.parametrize("layout", ["cf", "cl"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_bwd_fast_paths_equal_element_path(dtype, layout, monkeypatch):
    """The kernels chosen for unit-stride layouts against the element kernel, with a
    ragged last tile, a partial group of 64 channels, history, dfinal_states and
    seq_idx (short sequences, and long ones whose tiles mostly hold one id), and
    (register path) rows that end inside a segment or exactly at a segment's end,
    and rows whose length is not a multiple of the vector, with and without seq_idx:
    dx and d(initial_states) have the same bits on every path.  The channel-last LDS kernel also gives the same dweight and
    dbias bits; the register-only channel-first kernel sums the parameter gradients
    in another order, so there they meet the oracle's bound."""
    T = tile_steps(dtype)
    span = 64 * 4 * (4 if dtype == "f32" else 8)        # the register path's segment
    for K in KS:
        # seq=2: long sequences, so most LDS tiles hold one id and take the unmasked walk
        for f in (dict(init=True, dfs=True), dict(seq=7), dict(seq=2)):
            # the register path: one partial segment; one segment ending at L; an inner
            # segment then one ending at L; an inner segment then a partial one; rows
            # that are not 16-byte aligned (L not a multiple of the vector), one of them
            # shorter than a vector for bf16 / f16
            Ls = [4 * T + 8] + ([span, 2 * span, span + 40, span + 41, 2 * span + 3, 5]
                                if layout == "cf" else [])
            for L in Ls:
                B, C = 2, 136
                log(f"  bwd fast vs element {dtype} {layout} K={K} L={L} {f}")
                w = build(B, C, L, K, dtype, layout, 5100 + K, seq=f.get("seq"), init=f.get("init", False))
                dout, dfs = grad_inputs(w, layout, f.get("dfs", False), 5100 + K)
                if f.get("seq") == 2 and L > T:        # some tile right of t = 0 holds a single id
                    ids, H = w.seq_idx[0].tolist(), K - 1
                    assert any(len(set(ids[t0 - H:min(t0 + T + H, L)])) == 1 for t0 in range(T, L, T))
                res = []
                fast = 3 if layout == "cf" else 2
                for force, want in (("0", fast), ("1", 0)):
                    monkeypatch.setenv("CCV_FORCE_SCALAR", force)
                    x = to_gpu_view(w.x_storage, w.x)
                    args = ccv.make_bwd_args(x, w.weight.cuda(), w.bias.cuda(), dout.cuda(), ccv.empty_like_layout(x),
                                             torch.empty(C, K, dtype=w.weight.dtype, device="cuda"),
                                             seq_idx=None if w.seq_idx is None else w.seq_idx.cuda())
                    st, plan = ccv.ccv_bwd_plan(args)
                    assert st == 0 and plan.vector == want, (force, plan.as_dict())
                    res.append(run_bwd(w, dout, dfs, bool(f.get("init"))))
                bits = torch.int32 if dtype == "f32" else torch.int16
                for name, t0, t1 in zip(("dx", "dweight", "dbias", "dinit"), *res):
                    if t0 is not None and (fast != 3 or name in ("dx", "dinit")):
                        assert torch.equal(t0.view(bits), t1.view(bits)), (K, L, f, name)
                if fast == 3:
                    monkeypatch.setenv("CCV_FORCE_SCALAR", "0")
                    check_bwd(w, dout, dfs, bool(f.get("init")), f"[register path K={K} L={L}]")


@pytest.mark.parametrize("dtype", DTYPES)
def test_bwd_channel_last_unaligned_rows(dtype, monkeypatch):
    """Channel-last step rows that are not 16-byte aligned (C not a multiple of 16 /
    element size, or a view at an odd channel offset) run the LDS-staged channel-last
    kernel's own variant: unaligned 16-byte loads and stores, the channel vector
    that straddles C element by element.  Every gradient has the element path's
    bits (the two share the walk and the tile grouping) and meets the oracle."""
    T = tile_steps(dtype)
    for i, (B, C, L, layout, f) in enumerate([(2, 139, 4 * T + 9, "cl", dict(init=True, dfs=True)),
                                              (1, 70, 3 * T + 1, "cl", dict(seq=5)),
                                              (2, 75, 2 * T + 5, "cl_odd", dict(seq=3, init=True, dfs=True))]):
        K = 4
        kw = dict(layout="cl", c_pad=5, c_off=3) if layout == "cl_odd" else dict(layout="cl")
        lengths = wl.packed_lengths(L, f["seq"], 1, 5400 + i).tolist() if f.get("seq") else None
        w = wl.make_case(B=B, C=C, L=L, K=K, x_dtype=dtype, bias=True, init=f.get("init", False),
                         seq_lengths=lengths, activation="silu", seed=5400 + i, **kw)
        dout, dfs = grad_inputs(w, "cl", f.get("dfs", False), 5400 + i)
        res = []
        for force, want in (("0", 2), ("1", 0)):
            monkeypatch.setenv("CCV_FORCE_SCALAR", force)
            x = to_gpu_view(w.x_storage, w.x)
            args = ccv.make_bwd_args(x, w.weight.cuda(), w.bias.cuda(), dout.cuda(), ccv.empty_like_layout(x),
                                     torch.empty(C, K, dtype=w.weight.dtype, device="cuda"),
                                     seq_idx=None if w.seq_idx is None else w.seq_idx.cuda())
            st, plan = ccv.ccv_bwd_plan(args)
            assert st == 0 and plan.vector == want, (force, plan.as_dict())
            res.append(run_bwd(w, dout, dfs, bool(f.get("init"))))
        monkeypatch.setenv("CCV_FORCE_SCALAR", "0")
        log(f"  bwd channel-last unaligned rows {dtype} {layout} B={B} C={C} L={L} {f}")
        bits = torch.int32 if dtype == "f32" else torch.int16
        for name, t0, t1 in zip(("dx", "dweight", "dbias", "dinit"), *res):
            if t0 is not None:
                assert torch.equal(t0.view(bits), t1.view(bits)), (i, name)
        check_bwd(w, dout, dfs, bool(f.get("init")), f"[channel-last unaligned rows {dtype} case {i}]")


@pytest.mark.parametrize("dtype", DTYPES)
def test_bwd_unaligned_seq_idx_takes_the_lds_path(dtype):
    """Channel-first with a seq_idx that is not 16-byte aligned (a view one element
    into its buffer) runs the LDS-staged kernel; its dx and d(initial_states) have the
    register path's bits, and every gradient meets the oracle."""
    K, B, C, L = 4, 2, 70, 4 * 32 * 8
    w = build(B, C, L, K, dtype, "cf", 5300, seq=9, init=True)
    dout, dfs = grad_inputs(w, "cf", True, 5300)
    x = to_gpu_view(w.x_storage, w.x)
    seq_off = unaligned_ids(w)
    res = {}
    for name, seq in (("aligned", w.seq_idx.cuda()), ("unaligned", seq_off)):
        plan = bwd_plan(x, w.weight.cuda(), dout.cuda(), seq)
        assert plan.vector == (3 if name == "aligned" else 1), (name, plan.as_dict())
        res[name] = ccv.causal_conv1d_bwd(x, w.weight.cuda(), w.bias.cuda(), dout.cuda(), seq,
                                          to_gpu_view(w.init_storage, w.initial_states), dfs.cuda(), "silu",
                                          return_dinitial_states=True)
        torch.cuda.synchronize()
    bits = torch.int32 if dtype == "f32" else torch.int16
    for i, name in ((0, "dx"), (3, "dinit")):
        assert torch.equal(res["aligned"][i].cpu().contiguous().view(bits),
                           res["unaligned"][i].cpu().contiguous().view(bits)), name
    c = case(w.x, w.weight, w.bias, w.seq_idx, w.initial_states, w.activation)
    r = oracle_bwd(c, dout, dfs)
    dx, dw, db, dinit = (t.cpu().contiguous() for t in res["unaligned"])
    for name, got, ref, scale, kk in (("dx", dx, r["dx"], r["ex"], K + 2), ("dinit", dinit, r["dinit"], r["einit"], K + 2),
                                      ("dw", dw, r["dw"], r["ew"], PARAM_TERMS_CAP),
                                      ("db", db, r["db"], r["eb"], PARAM_TERMS_CAP)):
        res_c = ocmp.compare(dtype_name(got), kk, raw(got), ref, scale)
        assert res_c["n_bad"] == 0, (name, ocmp.describe_failures(res_c, ref, scale, raw(got), dtype_name(got)))


def test_bwd_random_shapes():
    g = np.random.default_rng(77)
    for i in range(40):
        K = int(g.integers(2, 5))
        dtype = DTYPES[g.integers(0, 3)]
        w_dtype = DTYPES[g.integers(0, 3)]
        layout = ["cf", "cl", "cf_view", "cl_view"][g.integers(0, 4)]
        B, C, L = int(g.integers(1, 4)), int(g.integers(1, 200)), int(g.integers(0, 700))
        seq = int(g.integers(1, 9)) if (g.random() < 0.3 and L > 0) else None
        init = g.random() < 0.5
        w = build(B, C, L, K, dtype, layout, 4000 + i, w_dtype=w_dtype, seq=seq, init=init,
                  bias=bool(g.random() < 0.6), act=["silu", None][g.integers(0, 2)])
        dout, dfs = grad_inputs(w, layout, g.random() < 0.5, 4000 + i)
        log(f"  random bwd {i}: {dtype}/{w_dtype} K={K} {layout} B={B} C={C} L={L} seq={seq} init={init}")
        check_bwd(w, dout, dfs, init, f"[random {i}]")


def test_bwd_random_long_rows():
    """Rows long enough for several segments of the register-only channel-first
    kernel (2048 steps for 16-bit data, 1024 for fp32) and several tile groups of
    the channel-last kernels: lengths that end inside a segment, exactly at a
    segment's end, or just past one, in every layout, with and without seq_idx."""
    g = np.random.default_rng(78)
    for i in range(16):
        K = int(g.integers(2, 5))
        dtype = DTYPES[g.integers(0, 3)]
        span = 64 * 4 * (4 if dtype == "f32" else 8)
        V = 4 if dtype == "f32" else 8
        L = [span * int(g.integers(1, 3)), span * int(g.integers(1, 3)) + V * int(g.integers(1, 4)),
             int(g.integers(1, 5000))][i % 3]
        layout = ["cf", "cl", "cf_view", "cl_view"][g.integers(0, 4)]
        B, C = int(g.integers(1, 4)), int(g.integers(1, 100))
        seq = int(g.integers(1, 9)) if g.random() < 0.3 else None
        init = g.random() < 0.5
        w = build(B, C, L, K, dtype, layout, 4100 + i, seq=seq, init=init, bias=bool(g.random() < 0.6),
                  act=["silu", None][g.integers(0, 2)])
        dout, dfs = grad_inputs(w, layout, g.random() < 0.5, 4100 + i)
        log(f"  random long bwd {i}: {dtype} K={K} {layout} B={B} C={C} L={L} seq={seq} init={init}")
        check_bwd(w, dout, dfs, init, f"[random long {i}]")


def test_bwd_reduction_with_level_kernels():
    """More than 512 partial rows: level kernels of the reduction tree run before the
    final kernel (2500 rows -> 79 -> the final kernel's 3 waves), with a partial
    group of 64 channels, on the LDS channel-first path (a seq_idx one element off
    16-byte alignment sends it there); and the register-only path with 2048 partial
    rows."""
    for dtype, act in (("f32", None), ("bf16", "silu")):
        w = build(2, 72, 40000, 3, dtype, "cf", 4700, init=True, act=act, seq=3)
        assert w.B * -(-w.L // tile_steps(dtype)) == 2500
        dout, dfs = grad_inputs(w, "cf", True, 4700)
        log(f"  bwd level kernels {dtype}: B=2 C=72 L=40000 K=3")
        check_bwd(w, dout, dfs, True, f"[levels {dtype}]", seq_gpu=unaligned_ids(w), want_path=1)
    w = build(2, 72, 1024 * 1024, 3, "f32", "cf", 4710, init=True, act=None)   # 2 x 1024 segments
    dout, dfs = grad_inputs(w, "cf", True, 4710)
    log("  bwd register path, 2048 partial rows: B=2 C=72 L=1M K=3")
    check_bwd(w, dout, dfs, True, "[levels register path]")


def test_bwd_zero_length_sequence():
    """L = 0: dx is empty, d(initial_states) is dfinal_states passed through, and
    dweight / dbias are zero."""
    w = build(2, 12, 0, 4, "f32", "cf", 4500, init=True)
    dout, dfs = grad_inputs(w, "cf", True, 4500)
    dx, dw, db, dinit = check_bwd(w, dout, dfs, True, "[L=0]")
    assert dx.shape == (2, 12, 0)
    assert torch.equal(dinit, dfs) and not dw.any() and not db.any()


def test_bwd_repeat_runs_bit_identical():
    w = build(3, 256, 777, 4, "bf16", "cf", 4600, init=True)
    dout, dfs = grad_inputs(w, "cf", True, 4600)
    a = run_bwd(w, dout, dfs, True)
    for _ in range(3):
        b = run_bwd(w, dout, dfs, True)
        for t0, t1 in zip(a, b):
            assert torch.equal(t0.view(torch.int16), t1.view(torch.int16))


@pytest.mark.parametrize("dtype", DTYPES)
def test_bwd_layout_independent(dtype):
    """The same logical problem stored channel-first and channel-last (x, dout and
    dx): dx and d(initial_states) have the same bits (the per-element arithmetic
    does not depend on the strides); dweight and dbias, summed in a different order
    per layout, each meet the oracle's bound."""
    w = build(2, 72, 300, 4, dtype, "cf", 4700, init=True)
    dout, dfs = grad_inputs(w, "cf", True, 4700)
    x = w.x.cuda()
    args = (w.weight.cuda(), w.bias.cuda())
    init, dfs = w.initial_states.cuda(), dfs.cuda()

    def cl(t):
        return t.transpose(1, 2).contiguous().transpose(1, 2)

    res, plans = [], []
    for xv, gv in ((x, dout.cuda()), (cl(x), cl(dout.cuda()))):
        plans.append(bwd_plan(xv, args[0], gv))
        out = ccv.causal_conv1d_bwd(xv, *args, gv, None, init, dfs, "silu", return_dinitial_states=True)
        torch.cuda.synchronize()
        assert out[0].stride() == xv.stride()                 # dx follows x's layout
        res.append([t.cpu().contiguous() for t in out])
    bits = torch.int32 if dtype == "f32" else torch.int16
    # dx and d(initial_states): the same bits.  dweight and dbias are summed over
    # differently grouped tiles per layout, so each must meet the oracle's bound.
    r = oracle_bwd(case(w.x, w.weight, w.bias, None, w.initial_states, "silu"), dout, dfs.cpu())
    for name, t0, t1 in zip(("dx", "dweight", "dbias", "dinit"), *res):
        if name in ("dx", "dinit"):
            assert torch.equal(t0.view(bits), t1.view(bits)), name
            continue
        ref, scale = (r["dw"], r["ew"]) if name == "dweight" else (r["db"], r["eb"])
        for t, plan in zip((t0, t1), plans):
            res_c = ocmp.compare(dtype_name(t), param_terms(w, plan), raw(t), ref, scale)
            assert res_c["n_bad"] == 0, (name, ocmp.describe_failures(res_c, ref, scale, raw(t), dtype_name(t)))


def test_bwd_packed_dx_equals_separate_runs():
    """dx of a packed run with seq_idx equals dx of each sequence run alone, bit for
    bit; dweight and dbias agree within the parameter tolerance of their sum."""
    K, C = 4, 40
    lengths = [3, 70, 1, 64, 129, 5]
    L = sum(lengths)
    w = wl.make_case(B=1, C=C, L=L, K=K, x_dtype="bf16", layout="cl", bias=True, activation="silu",
                     seq_lengths=lengths, seed=4800)
    dout, _ = grad_inputs(w, "cl", False, 4800)
    dx, dw, db, _ = run_bwd(w, dout, None, False)
    pos = 0
    for n in lengths:
        xp = torch.empty(1, C, n, dtype=w.x.dtype).copy_(w.x[:, :, pos:pos + n])   # fresh storage
        part = wl.Workload(name="part", B=1, C=C, L=n, K=K, x_dtype="bf16", w_dtype="bf16",
                           x_storage=xp, x=xp, weight=w.weight, bias=w.bias,
                           seq_idx=None, init_storage=None, initial_states=None,
                           return_final_states=False, activation="silu", layout="cf", seed=0)
        dp = torch.empty(1, C, n, dtype=dout.dtype).copy_(dout[:, :, pos:pos + n])
        pdx, _, _, _ = run_bwd(part, dp, None, False)
        assert torch.equal(dx[:, :, pos:pos + n].view(torch.int16), pdx.view(torch.int16)), n
        pos += n


def test_bwd_workload_size_channel_first_bf16():
    """The bench's channel-first bf16 shape (B=4, C=2048, L=4096, K=4, bias, SiLU):
    every gradient element against the oracle."""
    w = wl.workload(2)
    dout, _ = grad_inputs(w, "cf", False, 1002)
    check_bwd(w, dout, None, False, "[workload 2 shape]")


def test_autograd_function_matches_oracle():
    """causal_conv1d_fn: torch.autograd through the forward and backward kernels
    gives the oracle's gradients for x, weight, bias and initial_states, and the
    forward value of causal_conv1d_fwd."""
    for dtype in ("f32", "bf16"):
        w = build(2, 48, 150, 4, dtype, "cl", 4900, init=True)
        dout, dfs = grad_inputs(w, "cl", True, 4900)
        x = to_gpu_view(w.x_storage, w.x).detach().requires_grad_()
        weight = w.weight.cuda().requires_grad_()
        bias = w.bias.cuda().requires_grad_()
        init = to_gpu_view(w.init_storage, w.initial_states).detach().requires_grad_()
        out, fs = ccv.causal_conv1d_fn(x, weight, bias, None, init, True, None, "silu")
        ref_out = ccv.causal_conv1d_fwd(x.detach(), weight.detach(), bias.detach(), initial_states=init.detach(),
                                        activation="silu")
        assert torch.equal(out.detach(), ref_out)
        torch.autograd.backward([out, fs], [dout.cuda(), dfs.cuda()])
        torch.cuda.synchronize()
        c = case(w.x, w.weight, w.bias, None, w.initial_states, "silu")
        r = oracle_bwd(c, dout, dfs)
        pk = param_terms(w, bwd_plan(x.detach(), weight.detach(), dout.cuda()))
        for name, got, ref, scale, kk in (("dx", x.grad, r["dx"], r["ex"], 6), ("dw", weight.grad, r["dw"], r["ew"], pk),
                                          ("db", bias.grad, r["db"], r["eb"], pk),
                                          ("dinit", init.grad, r["dinit"], r["einit"], 6)):
            g = got.cpu().contiguous()
            res = ocmp.compare(dtype_name(g), kk, raw(g), ref, scale)
            assert res["n_bad"] == 0, (dtype, name, ocmp.describe_failures(res, ref, scale, raw(g), dtype_name(g)))


def test_bwd_argument_errors_raise():
    x = torch.zeros(2, 8, 16, device="cuda")
    w = torch.zeros(8, 4, device="cuda")
    with pytest.raises(ValueError):
        ccv.causal_conv1d_bwd(x, w, None, x.half())                    # dout dtype
    with pytest.raises(ValueError):
        ccv.causal_conv1d_bwd(x, w, None, x, return_dinitial_states=True)   # no initial_states
    with pytest.raises(ValueError):
        ccv.causal_conv1d_bwd(x, w, None, x, dx=x)                     # dx is dout: alias


def _bwd_big(x, dout, dx, weight, bias, want_path):
    """ccv_bwd through the C ABI on prepared device views; returns (plan, dweight, dbias)."""
    C, K = weight.shape
    dw = torch.empty(C, K, dtype=weight.dtype, device="cuda")
    db = torch.empty(C, dtype=weight.dtype, device="cuda")
    args = ccv.make_bwd_args(x, weight.cuda(), bias.cuda(), dout, dx, dw, db, activation="silu")
    st, plan = ccv.ccv_bwd_plan(args)
    assert st == 0 and plan.vector == want_path, plan.as_dict()
    ws = torch.empty(max(16, ccv.ccv_bwd_workspace_size(args)), dtype=torch.uint8, device="cuda")
    args.workspace, args.workspace_bytes = ws.data_ptr(), ws.numel()
    assert ccv.ccv_bwd(args) == 0
    torch.cuda.synchronize()
    return plan, dw, db


def _check_all(x, dout, dx, dw, db, weight, bias, plan, where):
    B, C, L = x.shape
    c = case(x.cpu(), weight, bias, None, None, "silu")
    r = oracle_bwd(c, dout.cpu())
    pk = param_terms_for(plan, B, L, weight.shape[1])
    for name, got, ref, scale, kk in (("dx", dx, r["dx"], r["ex"], weight.shape[1] + 2),
                                      ("dweight", dw, r["dw"], r["ew"], pk), ("dbias", db, r["db"], r["eb"], pk)):
        g = got.cpu().contiguous()
        res = ocmp.compare(dtype_name(g), kk, raw(g), ref, scale)
        assert res["n_bad"] == 0, f"{where} {name}: " + ocmp.describe_failures(res, ref, scale, raw(g), dtype_name(g))


def test_bwd_offsets_beyond_4_gib():
    """The backward on views more than 4 GiB past the buffer start: x and dx
    channel-last views of 512 channels in rows of 8192 (two batches of 150,000
    rows, 4.9 GB per buffer) on the channel-last LDS kernel, and x and dx
    channel-first views of 2 channels with a channel stride of 2^31 + 4096
    elements on the register kernel.  Every dx, dweight and dbias element matches
    the oracle; the dx buffers keep their NaN outside the views."""
    K, C, W, B, L = 4, 512, 8192, 2, 150_000
    gc = torch.Generator().manual_seed(4601)
    weight = (torch.randn(C, K, generator=gc) * 0.5).to(torch.bfloat16)
    bias = (torch.randn(C, generator=gc) * 0.3).to(torch.bfloat16)
    g = torch.Generator(device="cuda").manual_seed(4600)

    xbuf = torch.full((B, L, W), float("nan"), dtype=torch.bfloat16, device="cuda")
    xbuf[:, :, :C] = torch.randn(B, L, C, dtype=torch.bfloat16, device="cuda", generator=g)
    gbuf = torch.full_like(xbuf, float("nan"))
    x, dx = xbuf[:, :, :C].transpose(1, 2), gbuf[:, :, :C].transpose(1, 2)
    dout = torch.randn(B, L, C, dtype=torch.bfloat16, device="cuda", generator=g).transpose(1, 2)
    plan, dw, db = _bwd_big(x, dout, dx, weight, bias, 2)
    assert bool(torch.isnan(gbuf[:, :, C:]).all()), "a dx store landed outside the channel-last view"
    _check_all(x, dout, dx, dw, db, weight, bias, plan, "channel-last")
    log(f"  channel-last backward: rows up to {xbuf.numel() * 2 / 2 ** 30:.2f} GiB from the buffer start")
    del xbuf, gbuf, x, dx, dout
    torch.cuda.empty_cache()

    C2, L2, S = 2, 5000, 2 ** 31 + 4096
    xbuf = torch.full((C2 * S,), float("nan"), dtype=torch.bfloat16, device="cuda")
    x = xbuf.as_strided((1, C2, L2), (C2 * S, S, 1))
    x.copy_(torch.randn(1, C2, L2, dtype=torch.bfloat16, device="cuda", generator=g))
    gbuf = torch.full_like(xbuf, float("nan"))
    dx = gbuf.as_strided((1, C2, L2), (C2 * S, S, 1))
    dout = torch.randn(1, C2, L2, dtype=torch.bfloat16, device="cuda", generator=g)
    plan, dw, db = _bwd_big(x, dout, dx, weight[:C2], bias[:C2], 3)
    assert int(torch.isnan(gbuf).sum()) == gbuf.numel() - C2 * L2, "a dx store landed outside the channel-first view"
    _check_all(x, dout, dx, dw, db, weight[:C2], bias[:C2], plan, "channel-first")
    log(f"  channel-first backward: channel 1 at {S * 2 / 2 ** 30:.2f} GiB from the buffer start")
    del xbuf, gbuf, x, dx, dout
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_register_path_single_sequence_segments(dtype):
    """The register kernel runs a segment that holds one sequence (its steps, the
    K-1 before it and the V past it) without masks.  Sequence starts placed at and
    around segment edges, so that segments on either side of each start take one
    form or the other: dx and d(initial_states) have the bits of the LDS path (an
    unaligned seq_idx sends the call there), and every gradient meets the oracle."""
    K, B, C = 4, 1, 66
    span = 64 * 4 * (4 if dtype == "f32" else 8)
    L = 3 * span
    starts_cases = [[span], [span + 2], [2 * span - 3], [2 * span + 7], [2 * span + 8], [span - 1, 2 * span + 1]]
    for i, starts in enumerate(starts_cases):
        for with_init in (False, True):
            lengths = np.diff(np.concatenate([[0], starts, [L]])).tolist()
            w = wl.make_case(B=B, C=C, L=L, K=K, x_dtype=dtype, layout="cf", bias=True, init=with_init,
                             seq_lengths=lengths, activation="silu", seed=5600 + i)
            dout, dfs = grad_inputs(w, "cf", True, 5600 + i)
            x = to_gpu_view(w.x_storage, w.x)
            init = to_gpu_view(w.init_storage, w.initial_states) if with_init else None
            res = {}
            for name, seq, path in (("register", w.seq_idx.cuda(), 3), ("lds", unaligned_ids(w), 1)):
                assert bwd_plan(x, w.weight.cuda(), dout.cuda(), seq).vector == path
                res[name] = ccv.causal_conv1d_bwd(x, w.weight.cuda(), w.bias.cuda(), dout.cuda(), seq, init,
                                                  dfs.cuda(), "silu", return_dinitial_states=with_init)
                torch.cuda.synchronize()
            bits = torch.int32 if dtype == "f32" else torch.int16
            for j, name in ((0, "dx"), (3, "dinit")):
                if res["register"][j] is not None:
                    assert torch.equal(res["register"][j].cpu().contiguous().view(bits),
                                       res["lds"][j].cpu().contiguous().view(bits)), (starts, with_init, name)
            log(f"  register path {dtype}, sequence starts {starts}, history {with_init}")
            check_bwd(w, dout, dfs, with_init, f"[single-sequence segments {starts}]", want_path=3)
