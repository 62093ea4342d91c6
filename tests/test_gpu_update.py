"""GPU parity of the update (decode) call through the C ABI.

The update convolves a few new steps against the K-1 step history in a state
buffer and advances the state in place.  Its reference is the oracle's forward
with initial_states = the state before the call (for out) and that forward's
final states (for the new state, bit for bit).  Besides the oracle, decoding one
step (or a few) at a time must reproduce the GPU forward over the whole sequence
bit for bit, since both sum the same terms in the same order."""
import numpy as np
import pytest
import torch

import causal_depthwise_conv1d_amd as ccv
import oracle
import workloads as wl
from gpu_support import log
from oracle import compare as ocmp
from oracle.from_torch import case, dtype_name, raw

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    ccv.lib()

DTYPES = ["f32", "bf16", "f16"]
KS = [2, 3, 4]
TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def rand(shape, dtype, seed, tid, scale=1.0):
    n = int(np.prod(shape))
    return wl.to_storage(wl.draw(n, seed, tid, "normal", scale), dtype).reshape(shape)


def x_view(B, C, L, dtype, layout, seed):
    """New steps on the GPU: [B, C] ("2d", one step), [B, C, L] channel-first ("cf")
    or a transposed [B, L, C] ("cl")."""
    if layout == "2d":
        assert L == 1
        return rand((B, C), dtype, seed, 0).cuda()
    if layout == "cf":
        return rand((B, C, L), dtype, seed, 0).cuda()
    return rand((B, L, C), dtype, seed, 0).cuda().transpose(1, 2)


def state_view(B, C, H, dtype, layout, seed):
    """[B, C, H] state on the GPU: time fastest ("bci"), channels fastest ("bic"), or
    a window of a longer per-row buffer ("slice")."""
    if layout == "bci":
        return rand((B, C, H), dtype, seed, 1).cuda()
    if layout == "bic":
        return rand((B, H, C), dtype, seed, 1).cuda().transpose(1, 2)
    buf = rand((B, C, H + 5), dtype, seed, 1).cuda()
    return buf[:, :, 2:2 + H]


def params(C, K, w_dtype, bias, seed):
    w = rand((C, K), w_dtype, seed, 2, scale=0.5).cuda()
    b = rand((C,), w_dtype, seed, 3, scale=0.3).cuda() if bias else None
    return w, b


def reference(x, state_before, w, b, act):
    """Oracle out (fp64 values and Σ|terms|) and new state for one update call."""
    x3 = x.unsqueeze(2) if x.dim() == 2 else x
    c = case(x3.cpu(), w.cpu(), None if b is None else b.cpu(), None, state_before, act)
    y, s = c.fwd()
    return c, y, s, c.final_states()


def check_update(x, state, w, b, act, where):
    before = state.cpu()                        # the state is overwritten in place
    c, y, s, fs = reference(x, before, w, b, act)
    out = ccv.causal_conv1d_update(x, state, w, b, act)
    torch.cuda.synchronize()
    assert out.shape == x.shape and out.dtype == x.dtype
    o3 = (out.unsqueeze(2) if out.dim() == 2 else out).cpu().contiguous()
    res = ocmp.compare(dtype_name(o3), w.shape[1], raw(o3), y, s)
    if res["n_bad"]:
        raise AssertionError(f"{where}: " + ocmp.describe_failures(res, y, s, raw(o3), dtype_name(o3),
                                                                   shape=tuple(o3.shape)))
    got = raw(state.cpu().contiguous())
    bits = np.uint32 if got.dtype == np.float32 else np.uint16
    assert np.array_equal(got.view(bits), fs.view(bits)), f"{where}: new state differs"
    return c, out


@pytest.mark.parametrize("K", KS)
@pytest.mark.parametrize("dtype", DTYPES)
def test_update_matches_oracle(dtype, K):
    H = K - 1
    cases = [  # B, C, L, x layout, state layout, bias, activation, weight dtype
        (3, 77, 1, "2d", "bci", True, "silu", None),
        (2, 300, 1, "cf", "bic", False, None, "f32"),
        (4, 64, 3, "cl", "slice", True, "silu", None),
        (1, 1, 7, "cf", "bci", True, None, None),
        (5, 513, 2, "cl", "bic", True, "swish", "bf16"),
        (1, 2000, 1, "2d", "slice", False, "silu", "f16"),
        # the 16-byte path: C a multiple of 8, [B, C, K-1] state, weights in x's dtype
        (4, 256, 1, "2d", "bci", True, "silu", None),
        (2, 512, 3, "cl", "bci", False, None, None),
        (3, 1024, 1, "cf", "bci", True, None, None),
    ]
    for i, (B, C, L, xl, sl, bias, act, w_dtype) in enumerate(cases):
        seed = 900 + 10 * K + i
        x = x_view(B, C, L, dtype, xl, seed)
        st = state_view(B, C, H, dtype, sl, seed)
        w, b = params(C, K, w_dtype or dtype, bias, seed)
        plan = ccv.update_plan_for(x, st, w, b, act)
        assert plan["vector"] == (1 if i >= 6 else 0), (i, plan)
        log(f"  update {dtype}/{w.dtype} K={K} B={B} C={C} L={L} x={xl} state={sl} bias={bias} act={act} "
            f"vector={plan['vector']}")
        check_update(x, st, w, b, act, f"[{dtype} K={K} case {i}]")


@pytest.mark.parametrize("dtype", DTYPES)
def test_update_vector_path_takes_any_weight_dtype(dtype):
    """The 16-byte path with weights and bias of each other dtype (16- or 8-byte
    parameter blocks per lane) against the oracle."""
    for K in KS:
        for wd in DTYPES:
            for i, (B, C, L, xl, bias, act) in enumerate(((4, 256, 1, "2d", True, "silu"),
                                                          (2, 512, 3, "cl", False, None))):
                seed = 940 + 10 * K + i
                x = x_view(B, C, L, dtype, xl, seed)
                st = state_view(B, C, K - 1, dtype, "bci", seed)
                w, b = params(C, K, wd, bias, seed)
                assert ccv.update_plan_for(x, st, w, b, act)["vector"] == 1, (K, wd, i)
                log(f"  update {dtype}/{wd} K={K} B={B} C={C} L={L}: 16-byte path")
                check_update(x, st, w, b, act, f"[{dtype} w {wd} K={K} case {i}]")


@pytest.mark.parametrize("dtype", DTYPES)
def test_update_vector_path_equals_element_path(dtype, monkeypatch):
    """The 16-byte path and the element path give the same bits (out and new state)."""
    for K in KS:
        for L, xl, wd in ((1, "2d", dtype), (4, "cl", dtype), (2, "cl", "f32" if dtype != "f32" else "bf16")):
            B, C = 3, 1024
            seed = 960 + K + L
            x = x_view(B, C, L, dtype, xl, seed)
            st0 = state_view(B, C, K - 1, dtype, "bci", seed)
            w, b = params(C, K, wd, True, seed)
            res = []
            for force in ("0", "1"):
                monkeypatch.setenv("CCV_FORCE_SCALAR", force)
                assert ccv.update_plan_for(x, st0, w, b, "silu")["vector"] == (force == "0")
                st = st0.clone()
                out = ccv.causal_conv1d_update(x, st, w, b, "silu")
                torch.cuda.synchronize()
                res.append((raw(out.cpu().contiguous()), raw(st.cpu())))
            bits = np.uint32 if dtype == "f32" else np.uint16
            assert np.array_equal(res[0][0].view(bits), res[1][0].view(bits)), (K, L, "out")
            assert np.array_equal(res[0][1].view(bits), res[1][1].view(bits)), (K, L, "state")


@pytest.mark.parametrize("C", [130, 256])
@pytest.mark.parametrize("act", [None, "silu"])
@pytest.mark.parametrize("K", KS)
@pytest.mark.parametrize("dtype", DTYPES)
def test_decode_equals_forward(dtype, K, act, C):
    """The forward over 41 steps from a history h0, and the same steps fed to the
    update in chunks of 1, 2, 3 and 5 from the same h0: identical bits for every
    output and for the final state.  C = 130 takes the element path of the update,
    C = 256 its 16-byte path (the steps are then given channel-last)."""
    B, L, H = 2, 41, K - 1
    seed = 950 + K
    if C % 8:
        x = rand((B, C, L), dtype, seed, 0).cuda()
    else:
        x = rand((B, L, C), dtype, seed, 0).cuda().transpose(1, 2)
    h0 = rand((B, C, H), dtype, seed, 1).cuda()
    w, b = params(C, K, dtype, True, seed)
    ref, fs = ccv.causal_conv1d_fwd(x, w, b, initial_states=h0, return_final_states=True,
                                    activation=act)
    for chunks in ([1] * L, [2] * 20 + [1], [3, 5, 1, 5, 3, 5, 5, 5, 5, 4]):
        assert sum(chunks) == L
        state = h0.clone()
        assert ccv.update_plan_for(x[:, :, :1], state, w, b, act)["vector"] == (C % 8 == 0)
        outs, t = [], 0
        for n in chunks:
            xs = x[:, :, t:t + n]
            outs.append(ccv.causal_conv1d_update(xs[:, :, 0] if n == 1 else xs, state, w, b, act)
                        .reshape(B, C, n))
            t += n
        got = torch.cat(outs, 2)
        torch.cuda.synchronize()
        same = (got.cpu().view(torch.int16 if dtype != "f32" else torch.int32)
                == ref.cpu().view(torch.int16 if dtype != "f32" else torch.int32))
        assert bool(same.all()), f"{chunks[:3]}...: {int((~same).sum())} outputs differ from the forward"
        assert torch.equal(state.cpu().view(torch.int16 if dtype != "f32" else torch.int32),
                           fs.cpu().contiguous().view(torch.int16 if dtype != "f32" else torch.int32))


@pytest.mark.parametrize("dtype", DTYPES)
def test_update_no_activation_is_the_fp32_fma_chain(dtype):
    """Without an activation the update sums exactly as the oracle's binary32 mode."""
    for K in KS:
        B, C, L = 3, 200, 4
        seed = 980 + K
        x = rand((B, C, L), dtype, seed, 0).cuda()
        st = state_view(B, C, K - 1, dtype, "bic", seed)
        w, b = params(C, K, dtype, True, seed)
        z = case(x.cpu(), w.cpu(), b.cpu(), None, st.cpu(), None).fwd_f32()
        want = z if dtype == "f32" else (oracle.f32_to_bf16(z) if dtype == "bf16" else oracle.f32_to_f16(z))
        out = ccv.causal_conv1d_update(x, st, w, b, None)
        got = raw(out.cpu())
        bits = np.uint32 if dtype == "f32" else np.uint16
        assert np.array_equal(got.view(bits), want.view(bits)), (dtype, K)


@pytest.mark.parametrize("C", [4100, 4096])
def test_update_many_rows(C):
    """About 262,000 rows over many workgroups: C = 4100 on the element path (a
    ragged last workgroup), C = 4096 on the 16-byte path."""
    B, K = 64, 4
    x = rand((B, C), "bf16", 990, 0).cuda()
    st = state_view(B, C, K - 1, "bf16", "bci", 990)
    w, b = params(C, K, "bf16", True, 990)
    assert ccv.update_plan_for(x, st, w, b, "silu")["vector"] == (C % 8 == 0)
    check_update(x, st, w, b, "silu", f"[many rows C={C}]")


def test_update_writes_only_its_elements():
    """x, out and the state sit inside NaN-filled buffers: everything outside the
    views stays untouched, and the state is updated in place."""
    B, C, L, K = 3, 70, 2, 4
    H = K - 1
    g = 4096
    sbuf = torch.full((g + B * C * (H + 2) + g,), float("nan"), dtype=torch.bfloat16, device="cuda")
    st = sbuf[g:g + B * C * (H + 2)].view(B, C, H + 2)[:, :, 1:1 + H]
    st.copy_(rand((B, C, H), "bf16", 995, 1).cuda())
    obuf = torch.full((g + B * C * L + g,), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = obuf[g:g + B * C * L].view(B, C, L)
    x = rand((B, C, L), "bf16", 995, 0).cuda()
    w, b = params(C, K, "bf16", True, 995)
    snap_s, snap_o = sbuf.clone(), obuf.clone()
    before = st.cpu()
    _, y, s, fs = reference(x, before, w, b, "silu")
    res = ccv.causal_conv1d_update(x, st, w, b, "silu", out=out)
    torch.cuda.synchronize()
    assert res.data_ptr() == out.data_ptr()
    mask_s = torch.ones_like(sbuf, dtype=torch.bool)
    mask_s[g:g + B * C * (H + 2)].view(B, C, H + 2)[:, :, 1:1 + H] = False
    mask_o = torch.ones_like(obuf, dtype=torch.bool)
    mask_o[g:g + B * C * L] = False
    assert torch.equal(sbuf[mask_s].isnan(), snap_s[mask_s].isnan()), "write outside the state"
    assert bool(obuf[mask_o].isnan().all()), "write outside out"
    assert np.array_equal(raw(st.cpu().contiguous()).view(np.uint16), fs.view(np.uint16))
    res = ocmp.compare("bf16", K, raw(out.cpu().contiguous()), y, s)
    assert res["n_bad"] == 0


def test_update_zero_steps_leaves_state():
    B, C, K = 2, 9, 3
    st = state_view(B, C, K - 1, "f32", "bci", 997)
    before = st.clone()
    x = torch.empty(B, C, 0, device="cuda")
    w, b = params(C, K, "f32", True, 997)
    out = ccv.causal_conv1d_update(x, st, w, b, "silu")
    torch.cuda.synchronize()
    assert out.shape == (B, C, 0)
    assert torch.equal(st.view(torch.int32), before.view(torch.int32))


def test_update_twice_advances_twice():
    """Two calls with the same step: the state moves by two steps."""
    B, C, K = 2, 33, 4
    x = rand((B, C), "f16", 998, 0).cuda()
    st = state_view(B, C, K - 1, "f16", "bci", 998)
    h0 = st.clone()
    w, b = params(C, K, "f16", False, 998)
    ccv.causal_conv1d_update(x, st, w, b, None)
    ccv.causal_conv1d_update(x, st, w, b, None)
    torch.cuda.synchronize()
    want = torch.cat([h0, x.unsqueeze(2), x.unsqueeze(2)], 2)[:, :, -(K - 1):]
    assert torch.equal(st.view(torch.int16), want.contiguous().view(torch.int16))


def test_update_argument_errors_raise():
    B, C, K = 2, 8, 4
    x = torch.zeros(B, C, 1, device="cuda")
    w = torch.zeros(C, K, device="cuda")
    st = torch.zeros(B, C, K - 1, device="cuda")
    with pytest.raises(ValueError):                       # state is x
        xs = torch.zeros(B, C, K - 1, device="cuda")
        ccv.causal_conv1d_update(xs, xs, w)
    with pytest.raises(ValueError):                       # state rows on top of each other
        ccv.causal_conv1d_update(x, torch.zeros(C, K - 1, device="cuda").expand(B, C, K - 1), w)
    with pytest.raises(ValueError):                       # state dtype
        ccv.causal_conv1d_update(x, st.half(), w)
    with pytest.raises(ValueError):                       # state shape
        ccv.causal_conv1d_update(x, st[:, :, :2], w)
    with pytest.raises(ValueError):
        ccv.causal_conv1d_update(x, st, w, activation="relu")
