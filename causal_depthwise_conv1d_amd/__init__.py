"""causal_depthwise_conv1d_amd -- Python binding of libccv (the causal depthwise
conv1d forward for AMD gfx950).

Argument marshalling only: every step of the computation runs in the HIP kernels
behind the C ABI of ``include/ccv.h``; PyTorch provides device memory and
streams.  There is no CPU fallback: without the built library, or with tensors
that are not on a GPU, calls raise.

Low level (same names as the C ABI):
    ccv_fwd(args, stream=None), ccv_fwd_check(args), ccv_fwd_plan(args),
    ccv_update(args, stream=None), ccv_update_check(args), ccv_update_plan(args),
    ccv_bwd(args, stream=None), ccv_bwd_check(args), ccv_bwd_plan(args),
    ccv_bwd_workspace_size(args),
    ccv_status_str(code), ccv_abi_version()
High level (the full-sequence contract of Ch.4 "Dao interface and source map",
section "Contract of the full-sequence interface"; and the update kernel of the
same page's section "Reading the source along the call chain"):
    causal_conv1d_fwd(x, weight, bias=None, seq_idx=None, initial_states=None,
                      return_final_states=False, final_states_out=None,
                      activation=None)
    causal_conv1d_update(x, conv_state, weight, bias=None, activation=None)
    causal_conv1d_bwd(x, weight, bias, dout, seq_idx=None, initial_states=None,
                      dfinal_states=None, activation=None, ...)
    causal_conv1d_fn(x, weight, bias=None, seq_idx=None, initial_states=None,
                     return_final_states=False, final_states_out=None, activation=None)
        (differentiable: a torch.autograd.Function over the forward and backward)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libccv.so")
CALIB_LIB_PATH = os.path.join(_HERE, "libccv_calib.so")

CCV_ABI_VERSION = 1
CCV_F32, CCV_F16, CCV_BF16 = 0, 1, 2
CCV_ACT_NONE, CCV_ACT_SILU = 0, 1
CCV_PATH_NONE, CCV_PATH_CHANNEL_FIRST, CCV_PATH_CHANNEL_LAST, CCV_PATH_UPDATE, CCV_PATH_BACKWARD = 0, 1, 2, 3, 4
STATUS = {
    0: "CCV_OK", -1: "CCV_E_NULL", -2: "CCV_E_SHAPE", -3: "CCV_E_KSIZE", -4: "CCV_E_DTYPE",
    -5: "CCV_E_LAYOUT", -6: "CCV_E_UNSUPPORTED", -7: "CCV_E_ALIAS", -8: "CCV_E_HIP",
    -9: "CCV_E_INTERNAL", -10: "CCV_E_ABI", -11: "CCV_E_SCRATCH",
}
CCV_BWD_STATIC_SCRATCH_BYTES = 64 << 20
DTYPE_CODE = {torch.float32: CCV_F32, torch.float16: CCV_F16, torch.bfloat16: CCV_BF16}

_I64x3 = ctypes.c_int64 * 3


class ccv_fwd_args_t(ctypes.Structure):
    """Mirror of ``ccv_fwd_args_t`` in include/ccv.h (field order and types)."""
    _fields_ = [
        ("struct_size", ctypes.c_int64),
        ("B", ctypes.c_int64), ("C", ctypes.c_int64), ("L", ctypes.c_int64),
        ("K", ctypes.c_int32), ("activation", ctypes.c_int32),
        ("x_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("x_stride", _I64x3),
        ("weight", ctypes.c_void_p),
        ("bias", ctypes.c_void_p),
        ("seq_idx", ctypes.c_void_p),
        ("initial_states", ctypes.c_void_p), ("init_stride", _I64x3),
        ("final_states_out", ctypes.c_void_p), ("final_stride", _I64x3),
        ("out", ctypes.c_void_p), ("out_stride", _I64x3),
    ]

    def __init__(self, **kw):
        super().__init__(**kw)
        self.struct_size = ctypes.sizeof(ccv_fwd_args_t)


class ccv_update_args_t(ctypes.Structure):
    """Mirror of ``ccv_update_args_t`` in include/ccv.h (field order and types)."""
    _fields_ = [
        ("struct_size", ctypes.c_int64),
        ("B", ctypes.c_int64), ("C", ctypes.c_int64), ("L", ctypes.c_int64),
        ("K", ctypes.c_int32), ("activation", ctypes.c_int32),
        ("x_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("x_stride", _I64x3),
        ("weight", ctypes.c_void_p),
        ("bias", ctypes.c_void_p),
        ("state", ctypes.c_void_p), ("state_stride", _I64x3),
        ("out", ctypes.c_void_p), ("out_stride", _I64x3),
    ]

    def __init__(self, **kw):
        super().__init__(**kw)
        self.struct_size = ctypes.sizeof(ccv_update_args_t)


class ccv_bwd_args_t(ctypes.Structure):
    """Mirror of ``ccv_bwd_args_t`` in include/ccv.h (field order and types)."""
    _fields_ = [
        ("struct_size", ctypes.c_int64),
        ("B", ctypes.c_int64), ("C", ctypes.c_int64), ("L", ctypes.c_int64),
        ("K", ctypes.c_int32), ("activation", ctypes.c_int32),
        ("x_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("x_stride", _I64x3),
        ("weight", ctypes.c_void_p),
        ("bias", ctypes.c_void_p),
        ("seq_idx", ctypes.c_void_p),
        ("initial_states", ctypes.c_void_p), ("init_stride", _I64x3),
        ("dout", ctypes.c_void_p), ("dout_stride", _I64x3),
        ("dfinal_states", ctypes.c_void_p), ("dfinal_stride", _I64x3),
        ("dx", ctypes.c_void_p), ("dx_stride", _I64x3),
        ("dweight", ctypes.c_void_p),
        ("dbias", ctypes.c_void_p),
        ("dinitial_states", ctypes.c_void_p), ("dinit_stride", _I64x3),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
    ]

    def __init__(self, **kw):
        super().__init__(**kw)
        self.struct_size = ctypes.sizeof(ccv_bwd_args_t)


class ccv_plan_t(ctypes.Structure):
    """Mirror of ``ccv_plan_t`` in include/ccv.h."""
    _fields_ = [
        ("path", ctypes.c_int32), ("vector", ctypes.c_int32),
        ("elems_per_lane", ctypes.c_int32), ("unroll", ctypes.c_int32),
        ("grid", ctypes.c_int64), ("block", ctypes.c_int32), ("waves_per_group", ctypes.c_int32),
        ("work_items", ctypes.c_int64), ("span", ctypes.c_int64), ("channels_per_item", ctypes.c_int64),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class CcvError(RuntimeError):
    def __init__(self, status: int, where: str = "ccv_fwd"):
        self.status = status
        super().__init__(f"{where} failed: {STATUS.get(status, status)}")


class CcvArgumentError(CcvError, ValueError):
    pass


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libccv.so.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m causal_depthwise_conv1d_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(ccv_fwd_args_t)
        L.ccv_fwd.argtypes = [P, ctypes.c_void_p]
        L.ccv_fwd.restype = ctypes.c_int
        L.ccv_fwd_check.argtypes = [P]
        L.ccv_fwd_check.restype = ctypes.c_int
        L.ccv_fwd_plan.argtypes = [P, ctypes.POINTER(ccv_plan_t)]
        L.ccv_fwd_plan.restype = ctypes.c_int
        U = ctypes.POINTER(ccv_update_args_t)
        L.ccv_update.argtypes = [U, ctypes.c_void_p]
        L.ccv_update.restype = ctypes.c_int
        L.ccv_update_check.argtypes = [U]
        L.ccv_update_check.restype = ctypes.c_int
        L.ccv_update_plan.argtypes = [U, ctypes.POINTER(ccv_plan_t)]
        L.ccv_update_plan.restype = ctypes.c_int
        G = ctypes.POINTER(ccv_bwd_args_t)
        L.ccv_bwd.argtypes = [G, ctypes.c_void_p]
        L.ccv_bwd.restype = ctypes.c_int
        L.ccv_bwd_check.argtypes = [G]
        L.ccv_bwd_check.restype = ctypes.c_int
        L.ccv_bwd_plan.argtypes = [G, ctypes.POINTER(ccv_plan_t)]
        L.ccv_bwd_plan.restype = ctypes.c_int
        L.ccv_bwd_static.argtypes = [G, ctypes.c_void_p]
        L.ccv_bwd_static.restype = ctypes.c_int
        L.ccv_bwd_workspace_size.argtypes = [G]
        L.ccv_bwd_workspace_size.restype = ctypes.c_int64
        L.ccv_status_str.argtypes = [ctypes.c_int]
        L.ccv_status_str.restype = ctypes.c_char_p
        L.ccv_abi_version.argtypes = []
        L.ccv_abi_version.restype = ctypes.c_int
        if L.ccv_abi_version() != CCV_ABI_VERSION:
            raise RuntimeError("libccv ABI version mismatch")
        _lib = L
    return _lib


# ---- the C ABI, one to one ----------------------------------------------------------

def _stream_handle(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return stream


def ccv_fwd(args: ccv_fwd_args_t, stream=None) -> int:
    """Enqueue the forward on `stream` (a torch stream, a raw hipStream_t int, or None
    for torch's current stream).  Returns the status code."""
    return lib().ccv_fwd(ctypes.byref(args), ctypes.c_void_p(_stream_handle(stream)))


def ccv_fwd_check(args: ccv_fwd_args_t) -> int:
    return lib().ccv_fwd_check(ctypes.byref(args))


def ccv_fwd_plan(args: ccv_fwd_args_t):
    """(status, ccv_plan_t) without touching the device."""
    p = ccv_plan_t()
    st = lib().ccv_fwd_plan(ctypes.byref(args), ctypes.byref(p))
    return st, p


def ccv_update(args: ccv_update_args_t, stream=None) -> int:
    """Enqueue one update (decode) call on `stream`; returns the status code."""
    return lib().ccv_update(ctypes.byref(args), ctypes.c_void_p(_stream_handle(stream)))


def ccv_update_check(args: ccv_update_args_t) -> int:
    return lib().ccv_update_check(ctypes.byref(args))


def ccv_update_plan(args: ccv_update_args_t):
    """(status, ccv_plan_t) of an update call, without touching the device."""
    p = ccv_plan_t()
    st = lib().ccv_update_plan(ctypes.byref(args), ctypes.byref(p))
    return st, p


def ccv_bwd(args: ccv_bwd_args_t, stream=None) -> int:
    """Enqueue the backward (two kernels) on `stream`; returns the status code."""
    return lib().ccv_bwd(ctypes.byref(args), ctypes.c_void_p(_stream_handle(stream)))


def ccv_bwd_static(args: ccv_bwd_args_t, stream=None) -> int:
    """ccv_bwd with the partial sums in the library's fixed device array (no
    workspace, nothing allocated)."""
    return lib().ccv_bwd_static(ctypes.byref(args), ctypes.c_void_p(_stream_handle(stream)))


def ccv_bwd_check(args: ccv_bwd_args_t) -> int:
    return lib().ccv_bwd_check(ctypes.byref(args))


def ccv_bwd_plan(args: ccv_bwd_args_t):
    """(status, ccv_plan_t) of a backward call, without touching the device."""
    p = ccv_plan_t()
    st = lib().ccv_bwd_plan(ctypes.byref(args), ctypes.byref(p))
    return st, p


def ccv_bwd_workspace_size(args: ccv_bwd_args_t) -> int:
    """Workspace bytes the backward needs (>= 0), or a negative status."""
    return lib().ccv_bwd_workspace_size(ctypes.byref(args))


def ccv_status_str(status: int) -> str:
    return lib().ccv_status_str(int(status)).decode()


def ccv_abi_version() -> int:
    return lib().ccv_abi_version()


# ---- tensors -> args -------------------------------------------------------------------

def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _strides3(t: Optional[torch.Tensor]):
    return _I64x3(*(t.stride() if t is not None else (0, 0, 0)))


def _contiguous_ids(seq_idx):
    """The C ABI reads seq_idx as a contiguous [B, L] array: refuse any other layout
    (a view with other strides would be read as different ids)."""
    if seq_idx is not None and not seq_idx.is_contiguous():
        raise ValueError("seq_idx must be contiguous [B, L] for the C ABI; call .contiguous() first")
    return seq_idx


def make_args(x, weight, out, bias=None, seq_idx=None, initial_states=None,
              final_states_out=None, activation=None) -> ccv_fwd_args_t:
    """Fill a ccv_fwd_args_t from tensors (no checks beyond dtype codes and a
    contiguous seq_idx)."""
    _contiguous_ids(seq_idx)
    B, C, L = x.shape
    a = ccv_fwd_args_t()
    a.B, a.C, a.L = B, C, L
    a.K = weight.shape[1]
    a.activation = CCV_ACT_SILU if activation in ("silu", "swish") else CCV_ACT_NONE
    a.x_dtype = DTYPE_CODE[x.dtype]
    a.w_dtype = DTYPE_CODE[weight.dtype]
    a.x, a.x_stride = _ptr(x), _strides3(x)
    a.weight = _ptr(weight)
    a.bias = _ptr(bias)
    a.seq_idx = _ptr(seq_idx)
    a.initial_states, a.init_stride = _ptr(initial_states), _strides3(initial_states)
    a.final_states_out, a.final_stride = _ptr(final_states_out), _strides3(final_states_out)
    a.out, a.out_stride = _ptr(out), _strides3(out)
    return a


def make_update_args(x, weight, state, out, bias=None, activation=None) -> ccv_update_args_t:
    """Fill a ccv_update_args_t from tensors: x and out [B, C, L], state [B, C, K-1]."""
    B, C, L = x.shape
    a = ccv_update_args_t()
    a.B, a.C, a.L = B, C, L
    a.K = weight.shape[1]
    a.activation = CCV_ACT_SILU if activation in ("silu", "swish") else CCV_ACT_NONE
    a.x_dtype = DTYPE_CODE[x.dtype]
    a.w_dtype = DTYPE_CODE[weight.dtype]
    a.x, a.x_stride = _ptr(x), _strides3(x)
    a.weight = _ptr(weight)
    a.bias = _ptr(bias)
    a.state, a.state_stride = _ptr(state), _strides3(state)
    a.out, a.out_stride = _ptr(out), _strides3(out)
    return a


def _raise(status: int, where: str = "ccv_fwd"):
    if status == 0:
        return
    if status == -8:
        raise CcvError(status, where)
    raise CcvArgumentError(status, where)


def empty_like_layout(x: torch.Tensor) -> torch.Tensor:
    """A new [B, C, L] tensor with x's dtype, device and unit-stride dimension."""
    B, C, L = x.shape
    if x.stride(2) == 1 or L <= 1 and x.stride(1) != 1:
        return torch.empty(B, C, L, dtype=x.dtype, device=x.device)
    return torch.empty(B, L, C, dtype=x.dtype, device=x.device).transpose(1, 2)


def causal_conv1d_fwd(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
                      seq_idx: Optional[torch.Tensor] = None,
                      initial_states: Optional[torch.Tensor] = None,
                      return_final_states: bool = False,
                      final_states_out: Optional[torch.Tensor] = None,
                      activation: Optional[str] = None, out: Optional[torch.Tensor] = None,
                      info: Optional[dict] = None):
    """Causal depthwise conv1d forward on the GPU.

    x [B, C, L] (unit stride in time or in channels; any other strides are copied to
    contiguous first and ``info["x_copied"]`` says so), weight [C, K] (oldest ->
    current), bias [C] (weight dtype), seq_idx int32 [B, L], initial_states
    [B, C, K-1] (x dtype).  Returns out [B, C, L] in x's dtype and layout, or
    (out, final_states) when return_final_states.  final_states is [B, C, K-1] with
    channel stride 1 unless ``final_states_out`` provides the storage.
    """
    if activation not in (None, "silu", "swish"):
        raise ValueError(f"activation must be None, 'silu' or 'swish', not {activation!r}")
    if final_states_out is not None and not return_final_states:
        raise ValueError("final_states_out given but return_final_states is False")
    if x.dim() != 3 or weight.dim() != 2 or weight.shape[0] != x.shape[1]:
        raise ValueError("expected x [B, C, L] and weight [C, K]")
    if not x.is_cuda:
        raise ValueError("x must be a GPU tensor (there is no CPU path)")
    for name, t in (("weight", weight), ("bias", bias), ("seq_idx", seq_idx),
                    ("initial_states", initial_states), ("final_states_out", final_states_out),
                    ("out", out)):
        if t is not None and t.device != x.device:
            raise ValueError(f"{name} must be on {x.device}")
    B, C, L = x.shape
    K = weight.shape[1]
    copied = False
    if not (x.stride(2) == 1 or x.stride(1) == 1 or L <= 1 or C <= 1):
        x = x.contiguous()          # neither time nor channels unit-stride
        copied = True
    weight = weight.contiguous()
    if bias is not None:
        if bias.dtype != weight.dtype:
            raise ValueError("bias must have the weight's dtype")
        bias = bias.contiguous()
    if seq_idx is not None:
        if seq_idx.dtype != torch.int32 or tuple(seq_idx.shape) != (B, L):
            raise ValueError("seq_idx must be int32 [B, L]")
        seq_idx = seq_idx.contiguous()
    if initial_states is not None:
        if initial_states.dtype != x.dtype or tuple(initial_states.shape) != (B, C, K - 1):
            raise ValueError("initial_states must be [B, C, K-1] in x's dtype")
    fs = None
    if return_final_states:
        if final_states_out is not None:
            if final_states_out.dtype != x.dtype or tuple(final_states_out.shape) != (B, C, K - 1):
                raise ValueError("final_states_out must be [B, C, K-1] in x's dtype")
            fs = final_states_out
        else:
            fs = torch.empty(B, K - 1, C, dtype=x.dtype, device=x.device).transpose(1, 2)
    if out is None:
        out = empty_like_layout(x)
    elif out.dtype != x.dtype or tuple(out.shape) != (B, C, L):
        raise ValueError("out must be [B, C, L] in x's dtype")
    args = make_args(x, weight, out, bias, seq_idx, initial_states, fs, activation)
    with torch.cuda.device(x.device):
        st = ccv_fwd(args)
    _raise(st)
    if info is not None:
        info["x_copied"] = copied
    return (out, fs) if return_final_states else out


def plan_for(x, weight, out=None, **kw) -> dict:
    """The launch causal_conv1d_fwd would make for these tensors (no device work)."""
    if out is None:
        out = empty_like_layout(x)
    st, p = ccv_fwd_plan(make_args(x, weight, out, **kw))
    _raise(st)
    return p.as_dict()


def causal_conv1d_update(x: torch.Tensor, conv_state: torch.Tensor, weight: torch.Tensor,
                         bias: Optional[torch.Tensor] = None, activation: Optional[str] = None,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One update (decode) call on the GPU: convolve the new steps x against the
    history in ``conv_state`` and advance ``conv_state`` in place.

    x [B, C] (one step) or [B, C, L]; conv_state [B, C, K-1] in x's dtype, time
    ascending (the last K-1 inputs seen so far); weight [C, K] (oldest -> current);
    bias [C] in the weight's dtype.  Any strides are used as they are.  Returns out
    with x's shape and dtype, allocated with x's unit-stride dimension.  Afterwards conv_state holds the last K-1 inputs of
    (old state followed by x), exactly as ``causal_conv1d_fwd`` would return them as
    final states.
    """
    if activation not in (None, "silu", "swish"):
        raise ValueError(f"activation must be None, 'silu' or 'swish', not {activation!r}")
    one_step = x.dim() == 2
    x3 = x.unsqueeze(2) if one_step else x
    if x3.dim() != 3 or weight.dim() != 2 or weight.shape[0] != x3.shape[1]:
        raise ValueError("expected x [B, C] or [B, C, L] and weight [C, K]")
    if not x3.is_cuda:
        raise ValueError("x must be a GPU tensor (there is no CPU path)")
    for name, t in (("conv_state", conv_state), ("weight", weight), ("bias", bias), ("out", out)):
        if t is not None and t.device != x3.device:
            raise ValueError(f"{name} must be on {x3.device}")
    B, C, L = x3.shape
    K = weight.shape[1]
    if conv_state.dtype != x3.dtype or tuple(conv_state.shape) != (B, C, K - 1):
        raise ValueError("conv_state must be [B, C, K-1] in x's dtype")
    weight = weight.contiguous()
    if bias is not None:
        if bias.dtype != weight.dtype:
            raise ValueError("bias must have the weight's dtype")
        bias = bias.contiguous()
    if out is None:
        out3 = empty_like_layout(x3)
    else:
        if out.dtype != x3.dtype or tuple(out.shape) != tuple(x.shape):
            raise ValueError("out must have x's shape and dtype")
        out3 = out.unsqueeze(2) if one_step else out
    args = make_update_args(x3, weight, conv_state, out3, bias, activation)
    with torch.cuda.device(x3.device):
        st = ccv_update(args)
    _raise(st, "ccv_update")
    return out3.squeeze(2) if one_step else out3


def update_plan_for(x, conv_state, weight, bias=None, activation=None) -> dict:
    """The launch causal_conv1d_update would make for these tensors (no device work)."""
    x3 = x.unsqueeze(2) if x.dim() == 2 else x
    out = empty_like_layout(x3)
    st, p = ccv_update_plan(make_update_args(x3, weight.contiguous(), conv_state, out, bias, activation))
    _raise(st, "ccv_update")
    return p.as_dict()


def make_bwd_args(x, weight, bias, dout, dx, dweight, dbias=None, seq_idx=None, initial_states=None,
                  dfinal_states=None, dinitial_states=None, activation=None,
                  workspace=None) -> ccv_bwd_args_t:
    """Fill a ccv_bwd_args_t from tensors (no checks beyond dtype codes and a
    contiguous seq_idx)."""
    _contiguous_ids(seq_idx)
    B, C, L = x.shape
    a = ccv_bwd_args_t()
    a.B, a.C, a.L = B, C, L
    a.K = weight.shape[1]
    a.activation = CCV_ACT_SILU if activation in ("silu", "swish") else CCV_ACT_NONE
    a.x_dtype = DTYPE_CODE[x.dtype]
    a.w_dtype = DTYPE_CODE[weight.dtype]
    a.x, a.x_stride = _ptr(x), _strides3(x)
    a.weight, a.bias, a.seq_idx = _ptr(weight), _ptr(bias), _ptr(seq_idx)
    a.initial_states, a.init_stride = _ptr(initial_states), _strides3(initial_states)
    a.dout, a.dout_stride = _ptr(dout), _strides3(dout)
    a.dfinal_states, a.dfinal_stride = _ptr(dfinal_states), _strides3(dfinal_states)
    a.dx, a.dx_stride = _ptr(dx), _strides3(dx)
    a.dweight, a.dbias = _ptr(dweight), _ptr(dbias)
    a.dinitial_states, a.dinit_stride = _ptr(dinitial_states), _strides3(dinitial_states)
    if workspace is not None:
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    return a


def causal_conv1d_bwd(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor],
                      dout: torch.Tensor, seq_idx: Optional[torch.Tensor] = None,
                      initial_states: Optional[torch.Tensor] = None,
                      dfinal_states: Optional[torch.Tensor] = None,
                      activation: Optional[str] = None, dx: Optional[torch.Tensor] = None,
                      return_dinitial_states: bool = False, want_dbias: Optional[bool] = None):
    """Gradients of causal_conv1d_fwd on the GPU: (dx, dweight, dbias, dinitial_states).

    dout [B, C, L] and dfinal_states [B, C, K-1] are in x's dtype; dx is allocated
    in x's layout unless given (any strides); dweight [C, K] and dbias [C] come back
    in the weight's dtype (accumulated in fp32); dbias is None unless a bias was
    given (or want_dbias); dinitial_states [B, C, K-1] only with
    return_dinitial_states (it needs initial_states).  The fp32 workspace for the
    parameter sums is allocated here, through torch.
    """
    if activation not in (None, "silu", "swish"):
        raise ValueError(f"activation must be None, 'silu' or 'swish', not {activation!r}")
    if x.dim() != 3 or weight.dim() != 2 or weight.shape[0] != x.shape[1]:
        raise ValueError("expected x [B, C, L] and weight [C, K]")
    if not x.is_cuda:
        raise ValueError("x must be a GPU tensor (there is no CPU path)")
    B, C, L = x.shape
    K = weight.shape[1]
    for name, t in (("weight", weight), ("bias", bias), ("dout", dout), ("seq_idx", seq_idx),
                    ("initial_states", initial_states), ("dfinal_states", dfinal_states), ("dx", dx)):
        if t is not None and t.device != x.device:
            raise ValueError(f"{name} must be on {x.device}")
    if dout.dtype != x.dtype or tuple(dout.shape) != (B, C, L):
        raise ValueError("dout must be [B, C, L] in x's dtype")
    if dfinal_states is not None and (dfinal_states.dtype != x.dtype or tuple(dfinal_states.shape) != (B, C, K - 1)):
        raise ValueError("dfinal_states must be [B, C, K-1] in x's dtype")
    if initial_states is not None and (initial_states.dtype != x.dtype
                                       or tuple(initial_states.shape) != (B, C, K - 1)):
        raise ValueError("initial_states must be [B, C, K-1] in x's dtype")
    if return_dinitial_states and initial_states is None:
        raise ValueError("dinitial_states needs initial_states")
    if seq_idx is not None:
        if seq_idx.dtype != torch.int32 or tuple(seq_idx.shape) != (B, L):
            raise ValueError("seq_idx must be int32 [B, L]")
        seq_idx = seq_idx.contiguous()
    weight = weight.contiguous()
    if bias is not None:
        if bias.dtype != weight.dtype:
            raise ValueError("bias must have the weight's dtype")
        bias = bias.contiguous()
    if dx is None:
        dx = empty_like_layout(x)
    elif dx.dtype != x.dtype or tuple(dx.shape) != (B, C, L):
        raise ValueError("dx must be [B, C, L] in x's dtype")
    dweight = torch.empty(C, K, dtype=weight.dtype, device=x.device)
    want_db = (bias is not None) if want_dbias is None else want_dbias
    dbias = torch.empty(C, dtype=weight.dtype, device=x.device) if want_db else None
    dinit = (torch.empty(B, K - 1, C, dtype=x.dtype, device=x.device).transpose(1, 2)
             if return_dinitial_states else None)
    args = make_bwd_args(x, weight, bias, dout, dx, dweight, dbias, seq_idx, initial_states,
                         dfinal_states, dinit, activation)
    ws = ccv_bwd_workspace_size(args)
    _raise(int(ws) if ws < 0 else 0, "ccv_bwd")
    workspace = torch.empty(max(int(ws), 16), dtype=torch.uint8, device=x.device)
    args.workspace, args.workspace_bytes = workspace.data_ptr(), workspace.numel()
    with torch.cuda.device(x.device):
        st = ccv_bwd(args)
    _raise(st, "ccv_bwd")
    return dx, dweight, dbias, dinit


class _CausalConv1dFn(torch.autograd.Function):
    """Forward and backward through the C ABI.  Saves x, weight, bias,
    initial_states and seq_idx (Ch.4 "Dao interface and source map", section "How
    autograd links forward and backward"); z is recomputed in the backward."""

    @staticmethod
    def forward(ctx, x, weight, bias, seq_idx, initial_states, return_final_states, final_states_out,
                activation):
        res = causal_conv1d_fwd(x, weight, bias, seq_idx, initial_states, return_final_states,
                                final_states_out, activation)
        ctx.save_for_backward(x, weight, bias, seq_idx, initial_states)
        ctx.activation = activation
        ctx.return_final_states = return_final_states
        return res

    @staticmethod
    def backward(ctx, dout, *rest):
        x, weight, bias, seq_idx, initial_states = ctx.saved_tensors
        dfs = rest[0] if ctx.return_final_states and rest else None
        if dout is None:
            dout = torch.zeros_like(x)
        dout = dout.to(x.dtype)
        if dfs is not None:
            dfs = dfs.to(x.dtype)
        want_dinit = initial_states is not None and ctx.needs_input_grad[4]
        dx, dw, db, dinit = causal_conv1d_bwd(
            x, weight, bias, dout, seq_idx, initial_states, dfs, ctx.activation,
            return_dinitial_states=want_dinit, want_dbias=bias is not None and ctx.needs_input_grad[2])
        return dx, dw, db, None, dinit, None, None, None


def causal_conv1d_fn(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
                     seq_idx: Optional[torch.Tensor] = None,
                     initial_states: Optional[torch.Tensor] = None, return_final_states: bool = False,
                     final_states_out: Optional[torch.Tensor] = None, activation: Optional[str] = None):
    """Differentiable causal depthwise conv1d (the full-sequence contract of
    causal_conv1d_fwd, with gradients for x, weight, bias and initial_states through
    causal_conv1d_bwd)."""
    return _CausalConv1dFn.apply(x, weight, bias, seq_idx, initial_states, return_final_states,
                                 final_states_out, activation)
