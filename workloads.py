"""Seeded synthetic inputs for the causal depthwise conv1d forward.

This module is shared by the tests, the bench and the smoke check.  It draws
random numbers and lays them out in memory (shapes, dtypes, strides, packed
sequence ids); it holds none of the method's arithmetic.

Recipe (the same everywhere):
  * every tensor has its own random stream; a tensor of n elements is cut into
    blocks of ``BLOCK`` elements in C order, and block i is filled by
    ``numpy.random.Generator(PCG64(SeedSequence(seed, spawn_key=(tensor_id, i))))``
    drawing float32 values (blocks are filled concurrently; the result does not
    depend on the thread count);
  * "N(0, v)" names the variance v (standard deviation sqrt(v)); "U(a, b)" is
    uniform on [a, b);
  * values are drawn in float32 and rounded to the storage dtype by torch's
    round-to-nearest-even conversion;
  * tensor ids: 0 x, 1 weight, 2 bias, 3 initial_states, 4 sequence lengths.

The five named workloads mirror the shapes the method is described with: a small
channel-first call, a plain channel-first bf16 call, a channel-last view sliced
out of a wider projection buffer (s_L != C) with carried states, packed
variable-length sequences with seq_idx, and one very long sequence with few
channels and carried states (Ch.4 "Dao interface and source map", sections
"Contract of the full-sequence interface" and "Why one shape still has two
layouts"; Ch.5 "Dao forward CUDA implementation", sections "Task split of the
time-contiguous path" and "Three kinds of boundary handled separately").
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

BLOCK = 1 << 22
TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
_THREADS = 16

X_ID, W_ID, BIAS_ID, INIT_ID, SEQ_ID = 0, 1, 2, 3, 4


def _rng(seed: int, tensor_id: int, block: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tensor_id, block))))


def draw(n: int, seed: int, tensor_id: int, dist: str, scale: float) -> np.ndarray:
    """n float32 draws: dist "normal" -> N(0, scale**2), "uniform" -> U(-scale, scale)."""
    out = np.empty(n, dtype=np.float32)
    nblocks = max(1, math.ceil(n / BLOCK))

    def fill(i):
        lo, hi = i * BLOCK, min(n, (i + 1) * BLOCK)
        g = _rng(seed, tensor_id, i)
        if dist == "normal":
            g.standard_normal(out=out[lo:hi], dtype=np.float32)
            out[lo:hi] *= np.float32(scale)
        elif dist == "uniform":
            g.random(out=out[lo:hi], dtype=np.float32)
            out[lo:hi] *= np.float32(2.0 * scale)
            out[lo:hi] -= np.float32(scale)
        else:
            raise ValueError(dist)

    if nblocks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(min(_THREADS, nblocks)) as ex:
            list(ex.map(fill, range(nblocks)))
    return out


def to_storage(a: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 numpy -> torch CPU tensor of the storage dtype (RNE)."""
    t = torch.from_numpy(a)
    return t if dtype == "f32" else t.to(TORCH_DTYPES[dtype])


def packed_lengths(total: int, nseq: int, min_len: int, seed: int) -> np.ndarray:
    """A uniform draw over compositions of `total` into `nseq` parts, each >= min_len.

    Stars and bars: choose nseq-1 distinct bar positions among
    (total - nseq*min_len) + nseq - 1 slots; the gaps are the spare lengths."""
    spare = total - nseq * min_len
    if spare < 0:
        raise ValueError("total too small for nseq * min_len")
    slots = spare + nseq - 1
    g = _rng(seed, SEQ_ID)
    bars = np.sort(g.choice(slots, size=nseq - 1, replace=False)) if nseq > 1 else np.zeros(0, np.int64)
    edges = np.concatenate([[-1], bars, [slots]])
    parts = np.diff(edges) - 1
    return (parts + min_len).astype(np.int64)


def seq_idx_from_lengths(lengths, B: int = 1) -> torch.Tensor:
    ids = np.repeat(np.arange(len(lengths), dtype=np.int32), np.asarray(lengths))
    # a C-order copy: a plain copy of the broadcast view would keep the batch axis fastest
    return torch.from_numpy(np.array(np.broadcast_to(ids, (B, ids.size)), order="C"))


@dataclass
class Workload:
    """One synthetic problem.  All tensors are torch CPU tensors.

    ``x`` is the logical [B, C, L] view (with its real strides) of ``x_storage``;
    ``initial_states`` is the logical [B, C, K-1] view of ``init_storage``.
    """
    name: str
    B: int
    C: int
    L: int
    K: int
    x_dtype: str
    w_dtype: str
    x_storage: torch.Tensor
    x: torch.Tensor
    weight: torch.Tensor
    bias: Optional[torch.Tensor]
    seq_idx: Optional[torch.Tensor]
    init_storage: Optional[torch.Tensor]
    initial_states: Optional[torch.Tensor]
    return_final_states: bool
    activation: Optional[str]
    layout: str
    seed: int
    notes: dict = field(default_factory=dict)

    @property
    def silu(self) -> bool:
        return self.activation in ("silu", "swish")


def _x_view(storage: torch.Tensor, layout: str, B, C, L, c_off=0, t_off=0):
    """Logical [B, C, L] view of a storage tensor.

    layout "cf": storage [B, Cp, Lp]  -> x = storage[:, c_off:c_off+C, t_off:t_off+L]
    layout "cl": storage [B, Lp, Cp]  -> x = storage[:, t_off:t_off+L, c_off:c_off+C].transpose(1, 2)
    """
    if layout == "cf":
        return storage[:, c_off:c_off + C, t_off:t_off + L]
    if layout == "cl":
        return storage[:, t_off:t_off + L, c_off:c_off + C].transpose(1, 2)
    raise ValueError(layout)


def make_case(*, B, C, L, K, x_dtype="f32", w_dtype=None, layout="cf", bias=True,
              seq_lengths=None, init=False, final=False, activation="silu", seed=0,
              c_pad=0, c_off=0, t_pad=0, t_off=0, x_dist="normal", x_scale=1.0,
              w_var=None, bias_var=0.1, init_var=1.0, init_layout="channel_fast",
              poison_unused=False) -> Workload:
    """A general synthetic case.

    The storage of x is [B, C + c_pad, L + t_pad] ("cf") or [B, L + t_pad, C + c_pad]
    ("cl"), and x is the [B, C, L] window at channel offset c_off and time offset t_off
    (so the real strides differ from the compact ones whenever a pad is nonzero).
    With ``poison_unused`` every storage element outside the window is NaN.
    ``seq_lengths`` (list of ints summing to L) gives packed ids shared by every batch.
    ``init_layout`` "channel_fast" stores initial_states as [B, K-1, C] (channel stride 1);
    "time_fast" stores it as [B, C, K-1].
    """
    w_dtype = w_dtype or x_dtype
    w_var = (1.0 / K) if w_var is None else w_var
    Cp, Lp = C + c_pad, L + t_pad
    if c_off + C > Cp or t_off + L > Lp:
        raise ValueError("window exceeds storage")
    shape = (B, Cp, Lp) if layout == "cf" else (B, Lp, Cp)
    n = int(np.prod(shape))
    xs = draw(n, seed, X_ID, x_dist, x_scale).reshape(shape)
    if poison_unused and n:
        # every storage element outside the [B, C, L] window becomes NaN
        if layout == "cf":
            xs[:, :c_off] = np.nan
            xs[:, c_off + C:] = np.nan
            xs[:, c_off:c_off + C, :t_off] = np.nan
            xs[:, c_off:c_off + C, t_off + L:] = np.nan
        else:
            xs[:, :t_off] = np.nan
            xs[:, t_off + L:] = np.nan
            xs[:, t_off:t_off + L, :c_off] = np.nan
            xs[:, t_off:t_off + L, c_off + C:] = np.nan
    x_storage = to_storage(xs, x_dtype)
    x = _x_view(x_storage, layout, B, C, L, c_off, t_off)
    weight = to_storage(draw(C * K, seed, W_ID, "normal", math.sqrt(w_var)).reshape(C, K), w_dtype)
    b = to_storage(draw(C, seed, BIAS_ID, "normal", math.sqrt(bias_var)), w_dtype) if bias else None
    init_storage = initial_states = None
    if init:
        if init_layout == "channel_fast":
            init_storage = to_storage(draw(B * (K - 1) * C, seed, INIT_ID, "normal", math.sqrt(init_var))
                                      .reshape(B, K - 1, C), x_dtype)
            initial_states = init_storage.transpose(1, 2)
        else:
            init_storage = to_storage(draw(B * C * (K - 1), seed, INIT_ID, "normal", math.sqrt(init_var))
                                      .reshape(B, C, K - 1), x_dtype)
            initial_states = init_storage
    seq = None
    if seq_lengths is not None:
        if int(np.sum(seq_lengths)) != L:
            raise ValueError("sequence lengths must sum to L")
        seq = seq_idx_from_lengths(seq_lengths, B)
    return Workload(name=f"case_B{B}_C{C}_L{L}_K{K}_{x_dtype}_{layout}", B=B, C=C, L=L, K=K,
                    x_dtype=x_dtype, w_dtype=w_dtype, x_storage=x_storage, x=x, weight=weight,
                    bias=b, seq_idx=seq, init_storage=init_storage, initial_states=initial_states,
                    return_final_states=bool(final), activation=activation, layout=layout, seed=seed)


# ---- the five named workloads -------------------------------------------------

WORKLOADS = {
    1: "small channel-first: B=1 C=64 L=2048 K=4 fp32 [B,C,L], bias, SiLU",
    2: "channel-first bf16: B=4 C=2048 L=4096 K=4 [B,C,L], bias, SiLU, zero left halo",
    3: "channel-last strided bf16 view: B=8 C=4096 L=8192 K=4, channels [0,4096) of a "
       "[B,L,10240] buffer (strides (L*10240, 1, 10240)), initial+final states, SiLU, no bias",
    4: "packed varlen fp16 channel-last: B=1 C=2560 L=65536 K=4, [B,L,C] transposed, "
       "64 packed sequences (min length 64), bias, SiLU",
    5: "long sequence fp32 channel-first: B=2 C=128 L=1048576 K=3, x~U(-1,1), no bias, "
       "no activation, initial+final states",
}
WORKLOAD_KEYS = {
    1: "cf_f32_B1_C64_L2048_K4_silu",
    2: "cf_bf16_B4_C2048_L4096_K4_silu",
    3: "cl_bf16_view_B8_C4096_L8192_K4_states_silu",
    4: "cl_f16_varlen64_B1_C2560_L65536_K4_silu",
    5: "cf_f32_B2_C128_L1048576_K3_states",
}


def workload(i: int, poison_unused: bool = False, L_override: Optional[int] = None) -> Workload:
    """The i-th named workload (1..5), seed 1000 + i.

    ``L_override`` shortens the time axis (same recipe, same strides rule) for
    cheaper variants of a workload; it is never used for the measured line."""
    seed = 1000 + i
    if i == 1:
        w = make_case(B=1, C=64, L=L_override or 2048, K=4, x_dtype="f32", layout="cf",
                      bias=True, activation="silu", seed=seed, w_var=0.25)
    elif i == 2:
        w = make_case(B=4, C=2048, L=L_override or 4096, K=4, x_dtype="bf16", layout="cf",
                      bias=True, activation="silu", seed=seed, w_var=0.25)
    elif i == 3:
        w = make_case(B=8, C=4096, L=L_override or 8192, K=4, x_dtype="bf16", layout="cl",
                      c_pad=10240 - 4096, c_off=0, bias=False, init=True, final=True,
                      activation="silu", seed=seed, w_var=0.25, poison_unused=poison_unused)
    elif i == 4:
        L = L_override or 65536
        lengths = packed_lengths(L, 64, 64, seed) if L >= 64 * 64 else None
        w = make_case(B=1, C=2560, L=L, K=4, x_dtype="f16", layout="cl", bias=True,
                      seq_lengths=lengths, activation="silu", seed=seed, w_var=0.25)
    elif i == 5:
        w = make_case(B=2, C=128, L=L_override or 1048576, K=3, x_dtype="f32", layout="cf",
                      bias=False, init=True, final=True, activation=None, seed=seed,
                      x_dist="uniform", x_scale=1.0, w_var=1.0 / 3.0)
    else:
        raise KeyError(i)
    w.name = WORKLOAD_KEYS[i]
    w.notes["description"] = WORKLOADS[i]
    return w


# ---- the update (decode) bench case ---------------------------------------------

DECODE_DESCRIPTION = ("decode step bf16: B=256 sequences, C=4096 channels, one new step each, K=4, "
                      "state [B,C,3] time-fastest, SiLU, no bias")


def decode_workload() -> Workload:
    """The update (decode) bench case, seed 1006: x [B, C, 1] ~ N(0,1), weight
    ~ N(0, 1/4), the state (carried as initial_states, stored [B, C, K-1]) ~ N(0,1);
    the channel count and dtype of the strided channel-last workload."""
    w = make_case(B=256, C=4096, L=1, K=4, x_dtype="bf16", layout="cf", bias=False, init=True,
                  init_layout="time_fast", activation="silu", seed=1006, w_var=0.25)
    w.name = "update_bf16_B256_C4096_L1_K4_silu"
    w.notes["description"] = DECODE_DESCRIPTION
    return w
