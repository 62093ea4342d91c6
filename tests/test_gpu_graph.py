"""The three calls captured in a HIP graph (torch.cuda.graph) and replayed, and
issued on concurrent streams.

None of them clears memory with a memset or allocates inside the library: the
forward and the update are one kernel each, the backward its gradient kernel and
the reduction kernels over a workspace that the binding allocates (from the
graph's pool while capturing).  Each graph is replayed several times with new
inputs written eagerly in between, and every replay must equal an eager call on
the same inputs bit for bit."""
import numpy as np
import pytest
import torch

import causal_depthwise_conv1d_amd as ccv
import workloads as wl
from gpu_support import log

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    ccv.lib()

REPLAYS = 4


def rand(shape, dtype, seed, tid, scale=1.0):
    n = int(np.prod(shape))
    return wl.to_storage(wl.draw(n, seed, tid, "normal", scale), dtype).reshape(shape).cuda()


def bits(t):
    t = t.contiguous()
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def capture(fn):
    """fn() captured in a graph after a warm-up call on a side stream; returns the
    graph and the tensors fn returned while being captured (its static outputs)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()
    torch.cuda.synchronize()
    return g, outs


@pytest.mark.parametrize("layout", ["cf", "cl"])
def test_forward_graph_replays_equal_eager(layout):
    B, C, L, K = 2, 96, 300, 4
    w = rand((C, K), "bf16", 7000, 2, 0.5)
    b = rand((C,), "bf16", 7000, 3, 0.3)

    def fresh(seed):
        x = rand((B, C, L), "bf16", seed, 0) if layout == "cf" else rand((B, L, C), "bf16", seed, 0).transpose(1, 2)
        return x, rand((B, C, K - 1), "bf16", seed, 1)

    x, init = fresh(7001)
    out = ccv.empty_like_layout(x)
    fs = torch.empty(B, K - 1, C, dtype=x.dtype, device="cuda").transpose(1, 2)
    g, _ = capture(lambda: ccv.causal_conv1d_fwd(x, w, b, initial_states=init, return_final_states=True,
                                                 final_states_out=fs, activation="silu", out=out))
    for r in range(REPLAYS):
        nx, ninit = fresh(7100 + r)
        x.copy_(nx)
        init.copy_(ninit)
        ref_out, ref_fs = ccv.causal_conv1d_fwd(nx, w, b, initial_states=ninit, return_final_states=True,
                                                activation="silu")
        g.replay()
        torch.cuda.synchronize()
        log(f"  forward graph {layout} replay {r}")
        assert torch.equal(bits(out), bits(ref_out)), r
        assert torch.equal(bits(fs), bits(ref_fs)), r


def test_update_graph_replays_advance_the_state():
    """A captured one-step update, replayed: each replay reads the state the previous
    one left and must match eager updates step by step."""
    B, C, K = 8, 512, 4
    w = rand((C, K), "bf16", 7200, 2, 0.5)
    b = rand((C,), "bf16", 7200, 3, 0.3)
    x = rand((B, C), "bf16", 7201, 0)
    state = rand((B, C, K - 1), "bf16", 7201, 1)
    ref_state = state.clone()
    out = torch.empty_like(x)
    # capture() runs the call once before capturing it, which advances the state:
    # mirror that step eagerly
    g, _ = capture(lambda: ccv.causal_conv1d_update(x, state, w, b, activation="silu", out=out))
    ccv.causal_conv1d_update(x, ref_state, w, b, activation="silu")
    assert torch.equal(bits(state), bits(ref_state))
    for r in range(REPLAYS):
        nx = rand((B, C), "bf16", 7300 + r, 0)
        x.copy_(nx)
        ref_out = ccv.causal_conv1d_update(nx, ref_state, w, b, activation="silu")
        g.replay()
        torch.cuda.synchronize()
        log(f"  update graph replay {r}")
        assert torch.equal(bits(out), bits(ref_out)), r
        assert torch.equal(bits(state), bits(ref_state)), r


@pytest.mark.parametrize("layout", ["cf", "cl"])
def test_backward_graph_replays_equal_eager(layout):
    B, C, L, K = 2, 136, 700, 3
    w = rand((C, K), "bf16", 7400, 2, 0.5)
    b = rand((C,), "bf16", 7400, 3, 0.3)

    def fresh(seed):
        if layout == "cf":
            x, dout = rand((B, C, L), "bf16", seed, 0), rand((B, C, L), "bf16", seed, 4)
        else:
            x = rand((B, L, C), "bf16", seed, 0).transpose(1, 2)
            dout = rand((B, L, C), "bf16", seed, 4).transpose(1, 2)
        return x, dout, rand((B, C, K - 1), "bf16", seed, 1), rand((B, C, K - 1), "bf16", seed, 5)

    x, dout, init, dfs = fresh(7401)
    g, outs = capture(lambda: ccv.causal_conv1d_bwd(x, w, b, dout, initial_states=init, dfinal_states=dfs,
                                                    activation="silu", return_dinitial_states=True))
    for r in range(REPLAYS):
        nx, ndout, ninit, ndfs = fresh(7500 + r)
        x.copy_(nx)
        dout.copy_(ndout)
        init.copy_(ninit)
        dfs.copy_(ndfs)
        ref = ccv.causal_conv1d_bwd(nx, w, b, ndout, initial_states=ninit, dfinal_states=ndfs,
                                    activation="silu", return_dinitial_states=True)
        g.replay()
        torch.cuda.synchronize()
        log(f"  backward graph {layout} replay {r}")
        for name, got, want in zip(("dx", "dweight", "dbias", "dinit"), outs, ref):
            assert torch.equal(bits(got), bits(want)), (r, name)


@pytest.mark.parametrize("layout", ["cf", "cl"])
def test_backward_graph_with_packed_sequences(layout):
    """seq_idx on the LDS kernels (ids staged with each tile; long sequences, so many
    tiles take the unmasked walk): replays equal eager calls bit for bit."""
    B, C, L, K = 2, 200, 4096, 4
    w = rand((C, K), "bf16", 7700, 2, 0.5)
    b = rand((C,), "bf16", 7700, 3, 0.3)
    seq = wl.seq_idx_from_lengths(wl.packed_lengths(L, 5, 64, 7701), B).cuda()

    def fresh(seed):
        if layout == "cf":
            return rand((B, C, L), "bf16", seed, 0), rand((B, C, L), "bf16", seed, 4)
        return (rand((B, L, C), "bf16", seed, 0).transpose(1, 2), rand((B, L, C), "bf16", seed, 4).transpose(1, 2))

    x, dout = fresh(7702)
    g, outs = capture(lambda: ccv.causal_conv1d_bwd(x, w, b, dout, seq_idx=seq, activation="silu"))
    for r in range(REPLAYS):
        nx, ndout = fresh(7800 + r)
        x.copy_(nx)
        dout.copy_(ndout)
        ref = ccv.causal_conv1d_bwd(nx, w, b, ndout, seq_idx=seq, activation="silu")
        g.replay()
        torch.cuda.synchronize()
        log(f"  backward graph with seq_idx {layout} replay {r}")
        for name, got, want in zip(("dx", "dweight", "dbias"), outs, ref):
            assert torch.equal(bits(got), bits(want)), (r, name)


def test_calls_on_concurrent_streams_equal_sequential():
    """The library keeps no state between calls: forwards and backwards issued on two
    streams at once give the bits they give one at a time."""
    B, C, L, K = 2, 256, 2048, 4
    w = rand((C, K), "bf16", 7600, 2, 0.5)
    b = rand((C,), "bf16", 7600, 3, 0.3)
    xs = [rand((B, C, L), "bf16", 7601 + i, 0) for i in range(4)]
    douts = [rand((B, C, L), "bf16", 7611 + i, 4) for i in range(4)]
    ref_f = [ccv.causal_conv1d_fwd(x, w, b, activation="silu") for x in xs]
    ref_b = [ccv.causal_conv1d_bwd(x, w, b, d, activation="silu") for x, d in zip(xs, douts)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    got_f, got_b = [None] * 4, [None] * 4
    for i in range(4):
        with torch.cuda.stream(streams[i % 2]):
            got_f[i] = ccv.causal_conv1d_fwd(xs[i], w, b, activation="silu")
            got_b[i] = ccv.causal_conv1d_bwd(xs[i], w, b, douts[i], activation="silu")
    torch.cuda.synchronize()
    for i in range(4):
        assert torch.equal(bits(got_f[i]), bits(ref_f[i])), i
        for name, g_, r_ in zip(("dx", "dweight", "dbias"), got_b[i][:3], ref_b[i][:3]):
            assert torch.equal(bits(g_), bits(r_)), (i, name)
