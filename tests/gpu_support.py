"""Helpers for the GPU parity tests: move a synthetic workload to the GPU with its
real strides, run the HIP path through the C ABI, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import causal_depthwise_conv1d_amd as ccv
import oracle
from oracle import compare as ocmp
from oracle.from_torch import case, dtype_name, raw


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_gpu_view(storage: torch.Tensor, view: torch.Tensor) -> torch.Tensor:
    """The same view (shape, strides, offset) over a GPU copy of its storage."""
    dev = storage.cuda()
    return dev.as_strided(view.shape, view.stride(), view.storage_offset())


def gpu_args(w):
    x = to_gpu_view(w.x_storage, w.x)
    init = None if w.initial_states is None else to_gpu_view(w.init_storage, w.initial_states)
    return dict(x=x, weight=w.weight.cuda(), bias=None if w.bias is None else w.bias.cuda(),
                seq_idx=None if w.seq_idx is None else w.seq_idx.cuda(), initial_states=init,
                return_final_states=w.return_final_states, activation=w.activation)


def run_gpu(w, **over):
    """(out [B,C,L] contiguous CPU tensor, final_states CPU tensor or None)."""
    kw = gpu_args(w)
    kw.update(over)
    res = ccv.causal_conv1d_fwd(**kw)
    torch.cuda.synchronize()
    if w.return_final_states:
        out, fs = res
        return out.cpu().contiguous(), fs.cpu().contiguous()
    return res.cpu().contiguous(), None


def oracle_case(w):
    return case(w.x, w.weight, w.bias, w.seq_idx, w.initial_states, w.activation)


def assert_close(w, out_cpu: torch.Tensor, y, sabs, where=""):
    """Every output within tolerance of the oracle."""
    g = raw(out_cpu)
    res = ocmp.compare(dtype_name(out_cpu), w.K, g, y, sabs)
    if res["n_bad"]:
        raise AssertionError(f"{where} {w.name}: " + ocmp.describe_failures(
            res, y, sabs, g, dtype_name(out_cpu), shape=tuple(out_cpu.shape)))
    return res


def assert_final_states(w, fs_cpu: torch.Tensor, c=None):
    c = c or oracle_case(w)
    ref = c.final_states()
    got = raw(fs_cpu)
    assert got.shape == ref.shape
    if not np.array_equal(got.view(np.uint32 if got.dtype == np.float32 else np.uint16),
                          ref.view(np.uint32 if ref.dtype == np.float32 else np.uint16)):
        bad = np.argwhere(got.view(np.uint16 if got.dtype != np.float32 else np.uint32)
                          != ref.view(np.uint16 if ref.dtype != np.float32 else np.uint32))
        raise AssertionError(f"{w.name}: final_states differ at {bad[:8].tolist()}")


def check_full(w, where=""):
    """Run on the GPU and compare every output (and final states) with the oracle."""
    out, fs = run_gpu(w)
    c = oracle_case(w)
    y, s = c.fwd()
    res = assert_close(w, out, y, s, where)
    if w.return_final_states:
        assert_final_states(w, fs, c)
    return res


class _Equal:
    """Truthy when two tensors hold the same values (+0 == -0, NaN == NaN); its repr
    names the first differing elements."""

    def __init__(self, a: torch.Tensor, b: torch.Tensor):
        a64, b64 = a.double(), b.double()
        same = (a64 == b64) | (torch.isnan(a64) & torch.isnan(b64))
        self.ok = bool(same.all())
        self.detail = ""
        if not self.ok:
            bad = (~same).nonzero()[:6].tolist()
            self.detail = f"{int((~same).sum())} differ; first at " + ", ".join(
                f"{tuple(i)}: {a64[tuple(i)].item()!r} vs {b64[tuple(i)].item()!r}" for i in bad)

    def __bool__(self):
        return self.ok

    def __repr__(self):
        return self.detail or "equal"


def bits_equal(a: torch.Tensor, b: torch.Tensor) -> "_Equal":
    """Same values, where +0 == -0 and NaN == NaN."""
    return _Equal(a, b)
