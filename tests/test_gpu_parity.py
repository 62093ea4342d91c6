"""GPU parity: the HIP path through the C ABI against the oracle, element by element.

Small shapes that span several wave segments / time tiles and ragged tails, every
dtype, K and layout (channel-first, channel-last, strided views of wider buffers,
unaligned views that take the element-wise path), with and without bias, SiLU,
seq_idx, initial and final states; seeded random shapes; edge cases; invariants
that must hold bit for bit on the GPU."""
import os

import numpy as np
import pytest
import torch

import causal_depthwise_conv1d_amd as ccv
import oracle
import workloads as wl
from gpu_support import (assert_close, assert_final_states, bits_equal, check_full, gpu_args, log,
                         oracle_case, run_gpu, to_gpu_view)
from oracle.from_torch import raw

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    ccv.lib()

DTYPES = ["f32", "bf16", "f16"]
KS = [2, 3, 4]
LAYOUTS = ["cf", "cf_pitch", "cf_view", "cl", "cl_view", "cl_misaligned"]
ES = {"f32": 4, "bf16": 2, "f16": 2}


def layout_kw(layout, dtype, C, L):
    V = 16 // ES[dtype]
    if layout == "cf":
        return dict(layout="cf")
    if layout == "cf_pitch":          # rows 16-byte aligned but longer than L
        return dict(layout="cf", t_pad=(-L) % V + V)
    if layout == "cf_view":           # unaligned window of a bigger buffer
        return dict(layout="cf", c_pad=3, c_off=1, t_pad=13, t_off=5)
    if layout == "cl":
        return dict(layout="cl")
    if layout == "cl_view":           # channels [0, C) of a wider [B, L, C + pad] buffer
        return dict(layout="cl", c_pad=(-C) % V + 2 * V)
    if layout == "cl_misaligned":     # channel offset 3: not 16-byte aligned
        return dict(layout="cl", c_pad=5, c_off=3, t_pad=2, t_off=1)
    raise ValueError(layout)


def seq_lengths(L, n, seed):
    n = max(1, min(n, L))
    return wl.packed_lengths(L, n, 1, seed).tolist()


# (L, C, B, features) -- L spans 1, K-1, K, several wave segments / time tiles, ragged tails
def matrix_cases(K):
    return [
        (1, 7, 2, dict(bias=True, activation="silu")),
        (K - 1, 8, 1, dict(init=True, final=True)),
        (K, 64, 2, dict(bias=True, init=True, final=True, activation="silu")),
        (255, 130, 2, dict(bias=True, seq=9, activation="silu")),
        (257, 8, 3, dict(bias=False, activation=None)),
        (513, 64, 1, dict(init=True, final=True, activation="silu")),
        (2049, 7, 2, dict(bias=True, activation="silu")),
        (4099, 72, 1, dict(bias=True, seq=40, activation=None)),
        # seq_idx together with history and final states
        (777, 72, 2, dict(bias=True, seq=6, init=True, final=True, activation="silu")),
        (K - 1, 16, 2, dict(seq=2, init=True, final=True)),
    ]


def build(L, C, B, K, dtype, layout, feats, seed, w_dtype=None):
    f = dict(feats)
    nseq = f.pop("seq", None)
    return wl.make_case(B=B, C=C, L=L, K=K, x_dtype=dtype, w_dtype=w_dtype, seed=seed,
                        seq_lengths=seq_lengths(L, nseq, seed) if nseq else None,
                        **layout_kw(layout, dtype, C, L), **f)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("K", KS)
@pytest.mark.parametrize("dtype", DTYPES)
def test_matrix(dtype, K, layout):
    for i, (L, C, B, feats) in enumerate(matrix_cases(K)):
        w = build(L, C, B, K, dtype, layout, feats, seed=100 * K + i)
        log(f"  case L={L} C={C} B={B} {feats}")
        check_full(w, where=f"[{dtype} K={K} {layout} L={L} C={C}]")


def _raw_bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint32 if a.dtype == np.float32 else np.uint16)


def _fma_chain_reference(w):
    """The oracle's binary32 mode (bias first, one fused multiply-add per kept term,
    k ascending), rounded to the output dtype: raw storage [B, C, L]."""
    z = oracle_case(w).fwd_f32()
    if w.x_dtype == "f32":
        return z
    return oracle.f32_to_bf16(z) if w.x_dtype == "bf16" else oracle.f32_to_f16(z)


_INF_BITS = {"bf16": 0x7f80, "f16": 0x7c00}


def assert_same_bits(got: np.ndarray, want: np.ndarray, dtype: str, where=""):
    """Bit-identical raw storage (the sign of zero included); NaN equals any NaN."""
    g, r = _raw_bits(got), _raw_bits(want)
    assert g.shape == r.shape, where
    if dtype == "f32":
        nan = np.isnan(got) & np.isnan(want)
    else:
        nan = ((g & 0x7fff) > _INF_BITS[dtype]) & ((r & 0x7fff) > _INF_BITS[dtype])
    diff = (g != r) & ~nan
    if diff.any():
        bad = np.argwhere(diff)[:6]
        raise AssertionError(f"{where}: {int(diff.sum())} of {diff.size} differ; first at " + ", ".join(
            f"{tuple(i)}: {g[tuple(i)]:#x} vs {r[tuple(i)]:#x}" for i in bad.tolist()))


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("dtype", DTYPES)
def test_no_activation_is_the_fp32_fma_chain(dtype, layout, monkeypatch):
    """Without an activation every kernel path sums exactly as the oracle's binary32
    mode does, so its output is bit-identical to that sum rounded to the output
    dtype: vector and element paths, with bias, history, seq_idx and weights of
    every dtype."""
    for force_scalar in ("0", "1"):
        monkeypatch.setenv("CCV_FORCE_SCALAR", force_scalar)
        for K in KS:
            cases = [
                (1, 7, 2, dict(bias=True), None),
                (K - 1, 8, 1, dict(init=True, final=True), None),
                (257, 8, 3, dict(bias=False), None),
                (513, 64, 1, dict(bias=True, init=True, final=True), "f32"),
                (1537, 72, 2, dict(bias=True, seq=13), None),
                (4099, 9, 1, dict(bias=True, seq=40), "bf16"),
                (2050, 130, 1, dict(bias=True), "f16"),
            ]
            for i, (L, C, B, feats, w_dtype) in enumerate(cases):
                w = build(L, C, B, K, dtype, layout, dict(feats, activation=None), seed=7000 + 10 * K + i,
                          w_dtype=w_dtype)
                log(f"  fma chain: scalar={force_scalar} K={K} L={L} C={C} B={B} w={w.w_dtype} {feats}")
                out, _ = run_gpu(w)
                assert_same_bits(raw(out), _fma_chain_reference(w), dtype,
                                 where=f"[{dtype}/{w.w_dtype} K={K} {layout} L={L} scalar={force_scalar}]")


def test_random_shapes():
    g = np.random.default_rng(2024)
    for i in range(150):
        K = int(g.integers(2, 5))
        dtype = DTYPES[g.integers(0, 3)]
        w_dtype = DTYPES[g.integers(0, 3)]
        layout = LAYOUTS[g.integers(0, len(LAYOUTS))]
        B = int(g.integers(1, 4))
        C = int(g.integers(1, 300))
        L = int(g.integers(0, 3000)) if g.random() < 0.9 else int(g.integers(0, 8))
        use_seq = g.random() < 0.25 and L > 0
        feats = dict(bias=bool(g.random() < 0.5), activation=["silu", "swish", None][g.integers(0, 3)])
        if use_seq:
            feats["seq"] = int(g.integers(1, 20))
        feats["init"] = bool(g.random() < 0.5)
        feats["final"] = bool(g.random() < 0.5)
        w = build(L, C, B, K, dtype, layout, feats, seed=5000 + i, w_dtype=w_dtype)
        log(f"  random {i}: {dtype}/{w_dtype} K={K} {layout} B={B} C={C} L={L} {feats}")
        check_full(w, where=f"[random {i}]")


def test_empty_extents():
    for B, C, L in ((0, 8, 16), (2, 0, 16), (2, 8, 0)):
        w = wl.make_case(B=B, C=C, L=L, K=4, x_dtype="bf16", layout="cf", seed=1)
        out, _ = run_gpu(w)
        assert tuple(out.shape) == (B, C, L)


@pytest.mark.parametrize("layout", ["cf", "cl"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_zero_length_final_states_are_the_history(dtype, layout):
    for init in (True, False):
        w = wl.make_case(B=2, C=5, L=0, K=4, x_dtype=dtype, layout=layout, init=init, final=True, seed=3)
        out, fs = run_gpu(w)
        assert out.numel() == 0
        assert_final_states(w, fs)


@pytest.mark.parametrize("dtype", DTYPES)
def test_mixed_weight_dtypes(dtype):
    for wd in DTYPES:
        for layout in ("cf", "cl"):
            w = wl.make_case(B=2, C=40, L=700, K=4, x_dtype=dtype, w_dtype=wd, layout=layout,
                             bias=True, init=True, final=True, activation="silu", seed=77)
            check_full(w, where=f"[x {dtype} w {wd} {layout}]")


@pytest.mark.parametrize("K", [3, 4])
@pytest.mark.parametrize("dtype", DTYPES)
def test_mixed_weight_dtypes_take_the_straight_line_tiles(dtype, K):
    """Channel-last whole tiles of whole channel groups run the straight-line path for
    every pair of x and weight dtypes (the plan reports two row batches in flight),
    including fp32 x with 16-bit weights, whose per-lane weight and bias blocks are
    8 or 24 bytes, and agree with the oracle."""
    for wd in DTYPES:
        w = wl.make_case(B=2, C=1024, L=300, K=K, x_dtype=dtype, w_dtype=wd, layout="cl",
                         bias=True, init=True, final=True, activation="silu", seed=78 + K)
        kw = gpu_args(w)
        plan = ccv.plan_for(x=kw["x"], weight=kw["weight"], bias=kw["bias"],
                            initial_states=kw["initial_states"], activation="silu")
        assert plan["path"] == ccv.CCV_PATH_CHANNEL_LAST and plan["vector"] == 1 and plan["unroll"] == 8, plan
        log(f"  x {dtype} w {wd} K={K}: straight-line tiles")
        check_full(w, where=f"[x {dtype} w {wd} K={K} cl]")


@pytest.mark.parametrize("dtype", DTYPES)
def test_lds_staged_tiles_equal_register_tiles(dtype, monkeypatch):
    """Channel-last tiles staged through LDS (CCV_CL_LDS=1: 16-row tiles whose rows
    go straight from global memory into LDS) give the register path's bits, with
    bias, SiLU, seq_idx, history and final states, ragged time tails and a partial
    channel group, and agree with the oracle."""
    cases = [(2, 1024, 300, 4, dict(bias=True, init=True, final=True, activation="silu")),
             (1, 600, 777, 3, dict(bias=True, seq=9, activation="silu")),
             (2, 520, 96, 2, dict(bias=False, seq=3, init=True, final=True, activation=None))]
    for i, (B, C, L, K, feats) in enumerate(cases):
        w = build(L, C, B, K, dtype, "cl", feats, seed=4300 + i)
        res = []
        for lds in ("0", "1"):
            monkeypatch.setenv("CCV_CL_LDS", lds)
            kw = gpu_args(w)
            plan = ccv.plan_for(x=kw["x"], weight=kw["weight"], bias=kw["bias"], seq_idx=kw["seq_idx"],
                                initial_states=kw["initial_states"], activation=kw["activation"])
            assert plan["span"] == (16 if lds == "1" else 32), plan
            assert plan["unroll"] == (16 if lds == "1" else 8), plan
            res.append(run_gpu(w))
        log(f"  LDS tiles {dtype} B={B} C={C} L={L} K={K} {feats}")
        assert bits_equal(res[0][0], res[1][0]), (i, "out")
        if w.return_final_states:
            assert bits_equal(res[0][1], res[1][1]), (i, "final states")
        check_full(w, where=f"[LDS tiles {dtype} case {i}]")


def test_grid_is_sized_for_the_device_cu_count(monkeypatch):
    """A launch reads the GPU's compute-unit count from the runtime; plans made
    after it size the grid for that GPU (16 waves per CU for bf16 with SiLU, for
    the whole segments; L = 4099 adds a workgroup per 4 rows for the rows' last,
    shorter segments).  A smaller count from CCV_CU_COUNT (an odd one, so the
    waves' segment walks end unevenly) changes the grid, not the bits."""
    B, C, L = 2, 96, 4099
    w = build(L, C, B, 4, "bf16", "cf", dict(bias=True, activation="silu"), seed=4400)
    base = run_gpu(w)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    kw = gpu_args(w)
    plan = ccv.plan_for(x=kw["x"], weight=kw["weight"], bias=kw["bias"], activation="silu")
    whole = B * C * (L // plan["span"])
    tail_groups = -(-B * C // plan["waves_per_group"])
    assert L % plan["span"] and whole > 7 * 16
    assert plan["grid"] == -(-min(whole, cus * 16) // plan["waves_per_group"]) + tail_groups, (cus, plan)
    monkeypatch.setenv("CCV_CU_COUNT", "7")
    plan7 = ccv.plan_for(x=kw["x"], weight=kw["weight"], bias=kw["bias"], activation="silu")
    assert plan7["grid"] == 7 * 16 // plan7["waves_per_group"] + tail_groups, plan7
    assert bits_equal(base[0], run_gpu(w)[0])
    log(f"  {cus} CUs: grid {plan['grid']}; CCV_CU_COUNT=7: grid {plan7['grid']}, same bits")
    check_full(w, where="[CU count]")


@pytest.mark.parametrize("dtype", DTYPES)
def test_transposing_tiles_equal_register_tiles(dtype, monkeypatch):
    """The pages' channel-last tile (CCV_CL_LDS=2: 256 channels x 64 rows, 32 for
    fp32, staged along channels, computed one channel per thread along time, stored
    along channels) gives the register path's bits: partial channel blocks, ragged
    time tails, rows shorter than a tile, bias, SiLU, seq_idx, history and final
    states; and agrees with the oracle."""
    V = 16 // ES[dtype]
    cases = [(2, 1024, 300, 4, dict(bias=True, init=True, final=True, activation="silu")),
             (1, 600 - 600 % V, 777, 3, dict(bias=True, seq=9, activation="silu")),
             (2, 520, 96, 2, dict(bias=False, seq=3, init=True, final=True, activation=None)),
             (3, 256, 2, 4, dict(bias=True, init=True, final=True, activation="silu"))]
    for i, (B, C, L, K, feats) in enumerate(cases):
        w = build(L, C, B, K, dtype, "cl", feats, seed=4800 + i)
        res = []
        for mode in ("0", "2"):
            monkeypatch.setenv("CCV_CL_LDS", mode)
            kw = gpu_args(w)
            plan = ccv.plan_for(x=kw["x"], weight=kw["weight"], bias=kw["bias"], seq_idx=kw["seq_idx"],
                                initial_states=kw["initial_states"], activation=kw["activation"])
            if mode == "2":
                assert plan["channels_per_item"] == 256 and plan["span"] == (32 if dtype == "f32" else 64), plan
            res.append(run_gpu(w))
        log(f"  transposing tiles {dtype} B={B} C={C} L={L} K={K} {feats}")
        assert bits_equal(res[0][0], res[1][0]), (i, "out")
        if w.return_final_states:
            assert bits_equal(res[0][1], res[1][1]), (i, "final states")
        check_full(w, where=f"[transposing tiles {dtype} case {i}]")


@pytest.mark.parametrize("layout", ["cf", "cl"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_down_convert_rounds_to_nearest_even(dtype, layout):
    """With one nonzero tap, no bias and no activation, z = w*x is exact in fp32, so
    the only rounding is the store: the GPU must return RNE(z) bit for bit."""
    g = torch.Generator().manual_seed(9)
    B, C, L = 2, 520, 1100
    w = wl.make_case(B=B, C=C, L=L, K=2, x_dtype=dtype, layout=layout, bias=False, activation=None, seed=9)
    wt = torch.zeros(C, 2)
    wt[:, 1] = torch.rand(C, generator=g) * 3 + 0.1
    w.weight = wt.to(wl.TORCH_DTYPES[dtype])
    out, _ = run_gpu(w)
    y, _ = oracle_case(w).fwd(want_sabs=False)
    import oracle
    ref = oracle.round_out(dtype, y)
    assert np.array_equal(raw(out), ref), "down-convert is not round-to-nearest-even"


@pytest.mark.parametrize("force_scalar", [False, True])
@pytest.mark.parametrize("layout", ["cf", "cl"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_one_hot_weight_copies_input_bits(dtype, layout, force_scalar, monkeypatch):
    """w = e_k, no bias, no activation: out[t] = x~[t-K+1+k] exactly, so every path
    (16-byte and element-wise) must reproduce the input bits, subnormals included."""
    if force_scalar:
        monkeypatch.setenv("CCV_FORCE_SCALAR", "1")
    K, B, C, L = 4, 2, 256, 2100
    w = wl.make_case(B=B, C=C, L=L, K=K, x_dtype=dtype, layout=layout, bias=False, activation=None,
                     init=True, final=True, seed=16)
    tdt = wl.TORCH_DTYPES[dtype]
    # every subnormal pattern of the format, both signs, tiled over the input
    nbits = 16 if dtype != "f32" else 32
    if nbits == 16:
        mant = 1023 if dtype == "f16" else 127
        pats = torch.arange(1, mant + 1, dtype=torch.int32)
        pats = torch.cat([pats, pats | 0x8000]).to(torch.int16)
        sub = pats.view(tdt)
    else:
        pats = torch.randint(1, 1 << 23, (4096,), generator=torch.Generator().manual_seed(1), dtype=torch.int32)
        sub = torch.cat([pats, pats | (-(1 << 31))]).view(torch.float32)
    n = B * C * L
    vals = sub.repeat(n // sub.numel() + 1)[:n].reshape(B, C, L)
    mix = torch.rand(B, C, L, generator=torch.Generator().manual_seed(2)) < 0.5
    w.x.copy_(torch.where(mix, vals, w.x))
    ext = torch.cat([w.initial_states, w.x], dim=2)
    for k in range(K):
        wt = torch.zeros(C, K)
        wt[:, k] = 1
        w.weight = wt.to(tdt)
        out, fs = run_gpu(w)
        ref = ext[:, :, k:k + L].contiguous()
        iv = torch.int16 if nbits == 16 else torch.int32
        diff = (out.view(iv) != ref.view(iv)).nonzero()[:5].tolist()
        assert not diff, (k, [(i, out[tuple(i)].item(), ref[tuple(i)].item()) for i in diff])


def test_nonfinite_values_propagate():
    for layout in ("cf", "cl"):
        w = wl.make_case(B=1, C=16, L=300, K=4, x_dtype="f32", layout=layout, bias=True,
                         activation="silu", seed=4)
        xv = w.x
        xv[0, 0, 10] = float("nan")
        xv[0, 1, 20] = float("inf")
        xv[0, 2, 30] = float("-inf")
        xv[0, 3, 40] = 3e38
        check_full(w, where=f"[nonfinite {layout}]")


def test_masked_nan_does_not_leak():
    for layout in ("cf", "cl"):
        lengths = [50, 3, 97, 150]
        w = wl.make_case(B=1, C=20, L=300, K=4, x_dtype="bf16", layout=layout, bias=True,
                         activation="silu", seq_lengths=lengths, seed=5)
        w.x[0, :, 49] = float("nan")       # last step of sequence 0
        w.x[0, :, 52] = float("nan")       # last step of sequence 1
        out, _ = run_gpu(w)
        o = out.float()
        assert torch.isnan(o[0, :, 49]).all() and torch.isnan(o[0, :, 52]).all()
        assert not torch.isnan(o[0, :, 53:]).any(), "NaN crossed a sequence boundary"
        assert not torch.isnan(o[0, :, 50:52]).any()
        check_full(w, where=f"[masked nan {layout}]")


def _guarded(shape_alloc, view_fn, dtype, n_guard=4096):
    numel = int(np.prod(shape_alloc))
    buf = torch.full((n_guard + numel + n_guard,), float("nan"), dtype=dtype, device="cuda")
    inner = buf[n_guard:n_guard + numel].view(*shape_alloc)
    return buf, view_fn(inner)


@pytest.mark.parametrize("layout", ["cf", "cl"])
@pytest.mark.parametrize("L", [1037, 1040, 3])
def test_guard_bands_untouched(layout, L):
    """out and final_states live inside NaN-filled buffers: everything outside the
    views must be untouched (elements are written exactly once, in place).  The
    channel-first rows take the 16-byte path, whose one segment per row ends at L:
    the lanes past it must store nothing, and with L = 1037 and 3 (rows not 16-byte
    aligned) the vector that straddles L must store only its elements before L."""
    B, C, K = 2, 72, 4
    w = wl.make_case(B=B, C=C, L=L, K=K, x_dtype="bf16", layout=layout, bias=True, init=True,
                     final=True, activation="silu", seed=6)
    kw = gpu_args(w)
    dt = kw["x"].dtype
    if layout == "cf":
        obuf, out = _guarded((B, C + 2, L + 8), lambda t: t[:, 1:1 + C, :L], dt)
        assert ccv.plan_for(x=kw["x"], weight=kw["weight"], out=out)["vector"] == 1
    else:
        obuf, out = _guarded((B, L, C + 8), lambda t: t[:, :, :C].transpose(1, 2), dt)
    fbuf, fs = _guarded((B, K - 1, C + 4), lambda t: t[:, :, 2:2 + C].transpose(1, 2), dt)
    snap_o, snap_f = obuf.clone(), fbuf.clone()
    out_r, fs_r = ccv.causal_conv1d_fwd(out=out, final_states_out=fs, **kw)
    torch.cuda.synchronize()
    assert out_r.data_ptr() == out.data_ptr() and fs_r.data_ptr() == fs.data_ptr()
    mask_o = torch.ones_like(obuf, dtype=torch.bool)
    mask_o[out.storage_offset() + torch.as_strided(torch.arange(obuf.numel(), device="cuda"),
                                                   out.shape, out.stride(), 0).reshape(-1)] = False
    assert bits_equal(obuf[mask_o].cpu(), snap_o[mask_o].cpu()), "write outside out"
    mask_f = torch.ones_like(fbuf, dtype=torch.bool)
    mask_f[fs.storage_offset() + torch.as_strided(torch.arange(fbuf.numel(), device="cuda"),
                                                  fs.shape, fs.stride(), 0).reshape(-1)] = False
    assert bits_equal(fbuf[mask_f].cpu(), snap_f[mask_f].cpu()), "write outside final_states"
    y, s = oracle_case(w).fwd()
    assert_close(w, out.cpu().contiguous(), y, s)
    assert_final_states(w, fs.cpu().contiguous())


@pytest.mark.parametrize("layout", ["cf", "cl"])
def test_unused_channels_poisoned(layout):
    """Every storage element outside the view is NaN; a read outside the view would
    poison an output."""
    w = wl.make_case(B=2, C=100, L=900, K=4, x_dtype="bf16", layout=layout, bias=True,
                     c_pad=28, c_off=0 if layout == "cl" else 5, t_pad=16, t_off=8,
                     init=True, final=True, activation="silu", seed=7, poison_unused=True)
    res = check_full(w, where="[poisoned]")
    assert res["n_bad"] == 0


def test_repeat_runs_bit_identical():
    for layout in ("cf", "cl"):
        w = wl.make_case(B=2, C=300, L=3000, K=4, x_dtype="bf16", layout=layout, bias=True,
                         activation="silu", seed=8)
        a, _ = run_gpu(w)
        for _ in range(3):
            b, _ = run_gpu(w)
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("layout", ["cf", "cl"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_chunking_bit_exact(dtype, layout):
    """run([x1 | x2]) == run(x1) -> final_states -> run(x2, initial_states=...),
    bit for bit, for split points at and around the history length and the
    kernels' segment / tile sizes."""
    K = 4
    B, C, L = 2, 136, 3000
    w = wl.make_case(B=B, C=C, L=L, K=K, x_dtype=dtype, layout=layout, bias=True, init=True,
                     final=True, activation="silu", seed=10)
    kw = gpu_args(w)
    full, fs_full = ccv.causal_conv1d_fwd(**kw)
    for L1 in (0, 1, K - 2, K - 1, K, 63, 64, 65, 511, 513, 1024, 2047, 2049, L):
        k1 = dict(kw, x=kw["x"][:, :, :L1])
        o1, f1 = ccv.causal_conv1d_fwd(**k1)
        k2 = dict(kw, x=kw["x"][:, :, L1:], initial_states=f1)
        o2, f2 = ccv.causal_conv1d_fwd(**k2)
        torch.cuda.synchronize()
        eq = bits_equal(torch.cat([o1, o2], dim=2).cpu(), full.cpu())
        assert eq, (L1, eq)
        assert torch.equal(f2.cpu().view(torch.int16 if dtype != "f32" else torch.int32),
                           fs_full.cpu().view(torch.int16 if dtype != "f32" else torch.int32)), L1


@pytest.mark.parametrize("layout", ["cf", "cl"])
def test_packed_equals_separate(layout):
    lengths = [1, 2, 3, 4, 5, 64, 65, 300, 511, 2, 1000]
    L = sum(lengths)
    w = wl.make_case(B=1, C=96, L=L, K=4, x_dtype="bf16", layout=layout, bias=True,
                     activation="silu", seq_lengths=lengths, seed=11)
    kw = gpu_args(w)
    packed = ccv.causal_conv1d_fwd(**kw)
    pos = 0
    for n in lengths:
        part = ccv.causal_conv1d_fwd(**dict(kw, x=kw["x"][:, :, pos:pos + n], seq_idx=None))
        torch.cuda.synchronize()
        assert bits_equal(packed[:, :, pos:pos + n].cpu(), part.cpu()), (pos, n)
        pos += n


@pytest.mark.parametrize("dtype", DTYPES)
def test_channel_first_equals_channel_last(dtype):
    """Both kernels take the terms in the same order, so they agree bit for bit."""
    w = wl.make_case(B=2, C=200, L=2500, K=4, x_dtype=dtype, layout="cf", bias=True, init=True,
                     final=True, activation="silu", seed=12)
    kw = gpu_args(w)
    a, fa = ccv.causal_conv1d_fwd(**kw)
    x_cl = kw["x"].transpose(1, 2).contiguous().transpose(1, 2)
    b, fb = ccv.causal_conv1d_fwd(**dict(kw, x=x_cl))
    assert ccv.plan_for(x=x_cl, weight=kw["weight"])["path"] == ccv.CCV_PATH_CHANNEL_LAST
    torch.cuda.synchronize()
    assert bits_equal(a.cpu(), b.cpu())
    assert bits_equal(fa.cpu(), fb.cpu())


@pytest.mark.parametrize("layout", ["cf", "cl"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_element_path_equals_vector_path(dtype, layout, monkeypatch):
    """The 16-byte and the element-wise code paths round identically."""
    w = wl.make_case(B=2, C=136, L=1504, K=3, x_dtype=dtype, layout=layout, bias=True,
                     init=True, final=True, activation="silu", seed=13)
    kw = gpu_args(w)
    assert ccv.plan_for(x=kw["x"], weight=kw["weight"])["vector"] == 1
    a, fa = ccv.causal_conv1d_fwd(**kw)
    monkeypatch.setenv("CCV_FORCE_SCALAR", "1")
    assert ccv.plan_for(x=kw["x"], weight=kw["weight"])["vector"] == 0
    b, fb = ccv.causal_conv1d_fwd(**kw)
    torch.cuda.synchronize()
    eq = bits_equal(a.cpu(), b.cpu())
    assert eq, eq
    assert bits_equal(fa.cpu(), fb.cpu())


@pytest.mark.parametrize("dtype", DTYPES)
def test_channel_first_ragged_last_segment(dtype, monkeypatch):
    """L not a multiple of a segment: the row's last segment runs on the 16-byte
    path with its lanes past L storing nothing; when L is not a multiple of 16 /
    element size either, the rows are not 16-byte aligned and the one vector that
    straddles L moves element by element.  Same bits as the element path and every
    output against the oracle, for contiguous rows, rows with a padded pitch and an
    unaligned window of a bigger buffer (the guard-band test checks that nothing is
    written past L)."""
    V = 16 // ES[dtype]
    span = 64 * 4 * V
    cases = [(2, 6, 2 * span + V, 4, dict(bias=True, init=True, final=True, activation="silu")),
             (3, 5, span - V, 3, dict(bias=True, seq=7, activation="silu")),
             (1, 4, 3 * V, 2, dict(bias=False, init=True, final=True, activation=None)),
             (2, 3, span + 17 * V, 4, dict(bias=True, seq=5, init=True, final=True, activation="silu")),
             # rows of a length that is not a multiple of the vector
             (2, 6, 2 * span + V + 3, 4, dict(bias=True, init=True, final=True, activation="silu")),
             (3, 5, span - 1, 3, dict(bias=True, seq=7, activation="silu")),
             (2, 7, span + 1, 2, dict(bias=False, seq=3, init=True, final=True, activation=None)),
             (3, 9, V - 1, 4, dict(bias=True, init=True, final=True, activation="silu")),
             (2, 5, 2, 3, dict(bias=True, seq=1, init=True, final=True, activation="silu")),
             (1, 3, 5 * span, 4, dict(bias=True, seq=11, init=True, final=True, activation="silu"))]
    for i, (B, C, L, K, feats) in enumerate(cases):
        for layout in ("cf", "cf_pitch", "cf_view"):
            w = build(L, C, B, K, dtype, layout, feats, seed=4900 + i)
            kw = gpu_args(w)
            assert ccv.plan_for(x=kw["x"], weight=kw["weight"])["vector"] == 1
            a = run_gpu(w)
            monkeypatch.setenv("CCV_FORCE_SCALAR", "1")
            b = run_gpu(w)
            monkeypatch.delenv("CCV_FORCE_SCALAR")
            log(f"  ragged last segment {dtype} {layout} B={B} C={C} L={L} K={K} {feats}")
            assert bits_equal(a[0], b[0]), (i, layout)
            if w.return_final_states:
                assert bits_equal(a[1], b[1]), (i, layout)
            check_full(w, where=f"[ragged last segment {dtype} {layout} case {i}]")


@pytest.mark.parametrize("dtype", DTYPES)
def test_channel_last_unaligned_rows(dtype, monkeypatch):
    """Channel-last time rows that are not 16-byte aligned (C not a multiple of
    16 / element size, or a view at channel offset 3): whole channel vectors take
    unaligned 16-byte accesses on the register tiles, a lane's partial vector moves
    element by element, and a last group of a few channels runs with lanes over time
    rows.  Same bits as the element path, every output against the oracle, several
    whole channel groups plus a partial one."""
    cases = [(2, 1100, 300, 4, "cl_misaligned", dict(bias=True, init=True, final=True, activation="silu")),
             (1, 1027, 257, 3, "cl", dict(bias=True, seq=9, activation="silu")),
             (2, 600, 130, 2, "cl", dict(bias=False, init=True, final=True, seq=4, activation=None)),
             # a last channel group of 6 channels: lanes walk time rows there
             (2, 1030, 200, 4, "cl", dict(bias=True, init=True, final=True, seq=5, activation="silu")),
             (1, 1030, 70, 3, "cl_misaligned", dict(bias=True, init=True, activation=None))]
    for i, (B, C, L, K, layout, feats) in enumerate(cases):
        w = build(L, C, B, K, dtype, layout, feats, seed=5200 + i)
        kw = gpu_args(w)
        assert ccv.plan_for(x=kw["x"], weight=kw["weight"])["vector"] == 1
        a = run_gpu(w)
        monkeypatch.setenv("CCV_FORCE_SCALAR", "1")
        b = run_gpu(w)
        monkeypatch.delenv("CCV_FORCE_SCALAR")
        log(f"  unaligned channel-last rows {dtype} {layout} B={B} C={C} L={L} K={K} {feats}")
        assert bits_equal(a[0], b[0]), (i, layout)
        if w.return_final_states:
            assert bits_equal(a[1], b[1]), (i, layout)
        check_full(w, where=f"[unaligned channel-last rows {dtype} case {i}]")


@pytest.mark.parametrize("packed", [False, True])
def test_channel_last_tile_sweep_bit_identical(packed, monkeypatch):
    """Every tile length gives the same bits; with packed sequences (short ones, so
    that many 4-row batches straddle a start) both the masked and the unmasked
    batch code run at every tile length, single-batch tiles included."""
    w = wl.make_case(B=2, C=520, L=2000, K=4, x_dtype="f16", layout="cl", bias=True, init=True,
                     final=True, activation="silu", seed=14,
                     seq_lengths=seq_lengths(2000, 60, 14) if packed else None)
    kw = gpu_args(w)
    ref, fref = ccv.causal_conv1d_fwd(**kw)
    for tile in (4, 8, 13, 32, 100, 256, 4096):
        monkeypatch.setenv("CCV_CL_TILE_T", str(tile))
        o, f = ccv.causal_conv1d_fwd(**kw)
        torch.cuda.synchronize()
        assert bits_equal(o.cpu(), ref.cpu()) and bits_equal(f.cpu(), fref.cpu()), tile
    check_full(w, where=f"[tile sweep, packed={packed}]")


def test_noncontiguous_input_is_copied_and_reported():
    w = wl.make_case(B=2, C=16, L=100, K=4, x_dtype="f32", layout="cf", seed=15)
    x = w.x.cuda()
    y = torch.empty(2, 16, 200, device="cuda")[:, :, ::2]
    y.copy_(x)
    info = {}
    out = ccv.causal_conv1d_fwd(y, w.weight.cuda(), info=info)
    assert info["x_copied"] is True
    ref = ccv.causal_conv1d_fwd(x, w.weight.cuda())
    torch.cuda.synchronize()
    assert bits_equal(out.cpu(), ref.cpu())


@pytest.mark.parametrize("layout", ["cf", "cl"])
def test_packed_rows_split_anywhere(layout):
    """seq_idx with states: a packed row run in two calls, the second taking the
    first's final states as history where its first sequence continues and zeros
    where one starts, gives the one-call result bit for bit (outputs and final
    states), for splits inside sequences and on their boundaries."""
    K, C, B = 4, 72, 2
    lengths = [130, 1, 70, 2, 97, 300, 24]
    L = sum(lengths)
    w = wl.make_case(B=B, C=C, L=L, K=K, x_dtype="bf16", layout=layout, bias=True, init=True, final=True,
                     activation="silu", seq_lengths=lengths, seed=6100)
    kw = gpu_args(w)
    full, fs_full = ccv.causal_conv1d_fwd(**kw)
    seq = kw["seq_idx"]
    starts = np.cumsum(lengths)[:-1]
    for L1 in sorted({1, 64, 129, 130, 131, 200, 201, 202, int(starts[3]) + 1, 600, L - 1}):
        x1, x2 = kw["x"][:, :, :L1], kw["x"][:, :, L1:]
        o1, f1 = ccv.causal_conv1d_fwd(x1, kw["weight"], kw["bias"], seq[:, :L1].contiguous(),
                                       kw["initial_states"], True, activation="silu")
        cont = (seq[:, L1] == seq[:, L1 - 1]).reshape(B, 1, 1)
        h2 = torch.where(cont, f1, torch.zeros_like(f1))
        o2, f2 = ccv.causal_conv1d_fwd(x2, kw["weight"], kw["bias"], seq[:, L1:].contiguous(), h2, True,
                                       activation="silu")
        torch.cuda.synchronize()
        assert bits_equal(torch.cat([o1, o2], 2).cpu(), full.cpu()), L1
        assert bits_equal(f2.cpu(), fs_full.cpu()), L1
    check_full(w, where=f"[packed with states {layout}]")


def test_argument_errors_raise():
    x = torch.zeros(1, 4, 8, device="cuda")
    with pytest.raises(ValueError):
        ccv.causal_conv1d_fwd(x, torch.zeros(4, 5, device="cuda"))
    with pytest.raises(ValueError):
        ccv.causal_conv1d_fwd(x, torch.zeros(4, 4, device="cuda"), activation="relu")
    with pytest.raises(ValueError):
        ccv.causal_conv1d_fwd(x, torch.zeros(4, 4, device="cuda"),
                              final_states_out=torch.zeros(1, 4, 3, device="cuda"))



def _compare_all(out_gpu, x_gpu, weight, bias, activation, where):
    """Every output of out_gpu [B, C, L] against the oracle on all host cores."""
    from oracle import compare as ocmp
    from oracle.from_torch import case, dtype_name
    y, s = case(x_gpu.cpu(), weight, bias, None, None, activation).fwd_threads(min(16, len(os.sched_getaffinity(0))))
    g = out_gpu.cpu().contiguous()
    res = ocmp.compare(dtype_name(g), weight.shape[1], raw(g), y, s)
    assert res["n_bad"] == 0, where + ": " + ocmp.describe_failures(res, y, s, raw(g), dtype_name(g),
                                                                     shape=tuple(g.shape))
    return res


def test_offsets_beyond_4_gib():
    """Views whose elements lie more than 4 GiB past the buffer start, read and
    written, on both kernels: a channel-last view of 512 channels in rows of 8192
    (two batches of 150,000 rows: 4.9 GB per buffer, so batch 1 crosses the 4 GiB
    line, with a ragged last tile), and a channel-first view of 2 channels whose
    channel stride is 2^31 + 4096 elements (4.3 GB; whole segments and a ragged
    tail).  Every output matches the oracle, and every element of the output
    buffers outside the view keeps its NaN."""
    K, C, W, B, L = 4, 512, 8192, 2, 150_000
    gc = torch.Generator().manual_seed(4501)
    weight = (torch.randn(C, K, generator=gc) * 0.5).to(torch.bfloat16)
    bias = (torch.randn(C, generator=gc) * 0.3).to(torch.bfloat16)
    wd, bd = weight.cuda(), bias.cuda()
    g = torch.Generator(device="cuda").manual_seed(4500)
    stream = torch.cuda.current_stream()

    # channel-last
    xbuf = torch.full((B, L, W), float("nan"), dtype=torch.bfloat16, device="cuda")
    xbuf[:, :, :C] = torch.randn(B, L, C, dtype=torch.bfloat16, device="cuda", generator=g)
    obuf = torch.full_like(xbuf, float("nan"))
    x, out = xbuf[:, :, :C].transpose(1, 2), obuf[:, :, :C].transpose(1, 2)
    assert xbuf.numel() * 2 > 2 ** 32
    args = ccv.make_args(x, wd, out, bd, None, None, None, "silu")
    st, plan = ccv.ccv_fwd_plan(args)
    assert st == 0 and plan.path == ccv.CCV_PATH_CHANNEL_LAST and plan.vector == 1 and plan.unroll == 8
    assert ccv.ccv_fwd(args, stream) == 0
    torch.cuda.synchronize()
    assert bool(torch.isnan(obuf[:, :, C:]).all()), "a store landed outside the channel-last view"
    res = _compare_all(out, x, weight, bias, "silu", "channel-last")
    log(f"  channel-last: rows up to {xbuf.numel() * 2 / 2 ** 30:.2f} GiB from the buffer start; "
        f"{res['n']} outputs, max ulp {res['max_ulp']}")
    del xbuf, obuf, x, out
    torch.cuda.empty_cache()

    # channel-first
    C2, L2, S = 2, 5000, 2 ** 31 + 4096
    xbuf = torch.full((C2 * S,), float("nan"), dtype=torch.bfloat16, device="cuda")
    x = xbuf.as_strided((1, C2, L2), (C2 * S, S, 1))
    x.copy_(torch.randn(1, C2, L2, dtype=torch.bfloat16, device="cuda", generator=g))
    obuf = torch.full_like(xbuf, float("nan"))
    out = obuf.as_strided((1, C2, L2), (C2 * S, S, 1))
    args = ccv.make_args(x, wd[:C2], out, bd[:C2], None, None, None, "silu")
    st, plan = ccv.ccv_fwd_plan(args)
    assert st == 0 and plan.path == ccv.CCV_PATH_CHANNEL_FIRST and plan.vector == 1
    assert ccv.ccv_fwd(args, stream) == 0
    torch.cuda.synchronize()
    assert int(torch.isnan(obuf).sum()) == obuf.numel() - C2 * L2, "a store landed outside the channel-first view"
    _compare_all(out, x, weight[:C2], bias[:C2], "silu", "channel-first")
    log(f"  channel-first: channel 1 at {S * 2 / 2 ** 30:.2f} GiB from the buffer start")
    del xbuf, obuf, x, out
    torch.cuda.empty_cache()
