"""Marshal torch CPU tensors (storage + strided views) into an oracle ``Case``.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  No arithmetic here.
"""
from __future__ import annotations

import numpy as np
import torch

from . import Case

_DT = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}


def dtype_name(t: torch.Tensor) -> str:
    return _DT[t.dtype]


def raw(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a contiguous CPU tensor: float32, or uint16 bit patterns."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def _base_and_offset(view: torch.Tensor):
    """The flat storage under `view` and the element offset of view[0,0,0]."""
    n = view.untyped_storage().nbytes() // view.element_size()
    base = torch.empty(0, dtype=view.dtype).set_(view.untyped_storage(), 0, (n,), (1,))
    return raw(base), view.storage_offset()


def case(x, weight, bias=None, seq_idx=None, initial_states=None, activation=None) -> Case:
    """An oracle Case for x [B,C,L] (any strides) and the other contract arguments."""
    B, C, L = x.shape
    K = weight.shape[1]
    xb, xo = _base_and_offset(x)
    kw = {}
    if initial_states is not None:
        ib, io = _base_and_offset(initial_states)
        kw.update(init=ib, init_off=io, init_strides=tuple(initial_states.stride()))
    return Case(B=B, C=C, L=L, K=K, x=xb, x_off=xo, x_dtype=dtype_name(x), x_strides=tuple(x.stride()),
                w=raw(weight), w_dtype=dtype_name(weight), bias=None if bias is None else raw(bias),
                seq=None if seq_idx is None else np.asarray(seq_idx.cpu().numpy(), dtype=np.int32),
                silu=activation in ("silu", "swish"), **kw)


def bwd(c: Case, dout: torch.Tensor, dfinal_states=None) -> dict:
    """Oracle gradients of case `c` for dout [B,C,L] and dfinal_states [B,C,K-1] (any
    strides, x's dtype)."""
    db_, do = _base_and_offset(dout)
    kw = {}
    if dfinal_states is not None:
        fb, fo = _base_and_offset(dfinal_states)
        kw = dict(dfs=fb, dfs_off=fo, dfs_strides=tuple(dfinal_states.stride()))
    return c.bwd(db_, tuple(dout.stride()), do, **kw)


def case_from_workload(w) -> Case:
    return case(w.x, w.weight, w.bias, w.seq_idx, w.initial_states, w.activation)
