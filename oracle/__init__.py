"""Plain CPU oracle for the causal depthwise conv1d forward (ctypes binding).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the bench's
``cpu_baseline`` leg may import this module; the product package never does, and
the two share no code.

The arithmetic lives in ``ccv_oracle.c`` (fp64, one output at a time, straight
from the stencil equation of Ch.5 "Dao forward CUDA implementation", section
"How adjacent threads and chunks exchange history", with the argument meanings
of Ch.4 "Dao interface and source map", section "Contract of the full-sequence
interface").  This module only marshals numpy buffers.

Buffers are numpy arrays of raw storage: float32 for ``"f32"`` and uint16 bit
patterns for ``"f16"`` / ``"bf16"``.  A strided view is given as a flat buffer,
an element offset and (s_B, s_C, s_L) element strides.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libccv_oracle.so")
_SRC = os.path.join(_HERE, "ccv_oracle.c")

DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
_NP_STORAGE = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16}

GCC_CMD = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-pthread", "-o", _SO, _SRC, "-lm"]


class _Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64), ("C", ctypes.c_int64), ("L", ctypes.c_int64),
        ("K", ctypes.c_int32), ("silu", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("x_dtype", ctypes.c_int32), ("xs", ctypes.c_int64 * 3),
        ("w", ctypes.c_void_p), ("w_dtype", ctypes.c_int32),
        ("bias", ctypes.c_void_p),
        ("seq", ctypes.c_void_p),
        ("init", ctypes.c_void_p), ("is_", ctypes.c_int64 * 3),
    ]


class _Grad(ctypes.Structure):
    _fields_ = [("dout", ctypes.c_void_p), ("ds", ctypes.c_int64 * 3),
                ("dfs", ctypes.c_void_p), ("fs", ctypes.c_int64 * 3)]


_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no FMA contraction, no fast-math)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < max(
            os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "ccv_oracle.h"))):
        subprocess.run(GCC_CMD, check=True)
    return _SO


def _load(path):
    L = ctypes.CDLL(path)
    P = ctypes.POINTER(_Problem)
    i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)
    L.ora_point.argtypes = [P, i64, i64, i64, dp, dp, dp]
    L.ora_fwd.argtypes = [P, vp, vp]
    L.ora_fwd_threads.argtypes = [P, vp, vp, ctypes.c_int]
    L.ora_points.argtypes = [P, i64, vp, vp, vp]
    L.ora_final_states.argtypes = [P, vp]
    L.ora_bwd.argtypes = [P, ctypes.POINTER(_Grad)] + [vp] * 8
    L.ora_point_f32.argtypes = [P, i64, i64, i64, ctypes.POINTER(ctypes.c_float)]
    L.ora_fwd_f32.argtypes = [P, vp]
    L.ora_points_f32.argtypes = [P, i64, vp, vp]
    L.ora_round_out.argtypes = [ctypes.c_int32, vp, i64, vp]
    L.ora_f64_to_f32.argtypes = [ctypes.c_double]
    L.ora_f64_to_f32.restype = ctypes.c_float
    for name in ("ora_f32_to_bf16_array", "ora_f32_to_f16_array"):
        getattr(L, name).argtypes = [vp, vp, i64]
    for name in ("ora_f16_to_f64_array", "ora_bf16_to_f64_array"):
        getattr(L, name).argtypes = [vp, vp, i64]
    return L


def lib():
    global _lib
    if _lib is None:
        build()
        _lib = _load(_SO)
    return _lib


@contextlib.contextmanager
def using_library(path):
    """Temporarily route every call to another build of the oracle (the tests use
    this to check that deliberately broken copies fail the pins)."""
    global _lib
    saved = _lib
    _lib = _load(path)
    try:
        yield
    finally:
        _lib = saved


def _ptr(a):
    return None if a is None else a.ctypes.data


class Case:
    """One problem instance: storage buffers plus shapes, strides and flags.

    x:      flat storage buffer; x[b,c,t] = x_buf[x_off + b*s_B + c*s_C + t*s_L]
    w:      [C, K] storage (oldest -> current), contiguous
    bias:   None or [C] storage in w's dtype
    seq:    None or int32 [B, L], contiguous
    init:   None or flat storage in x's dtype; init[b,c,i] at
            init_off + b*is_B + c*is_C + i*is_I (i = 0..K-2, time ascending)
    """

    def __init__(self, *, B, C, L, K, x, x_dtype, x_strides, w, w_dtype, bias=None,
                 seq=None, init=None, init_strides=None, silu=False, x_off=0, init_off=0):
        self.B, self.C, self.L, self.K = int(B), int(C), int(L), int(K)
        self.x_dtype, self.w_dtype = x_dtype, w_dtype
        st = _NP_STORAGE[x_dtype]
        self._x = np.ascontiguousarray(np.asarray(x).reshape(-1)).view(st)
        self._w = np.ascontiguousarray(np.asarray(w).reshape(-1)).view(_NP_STORAGE[w_dtype])
        if self._w.size != self.C * self.K:
            raise ValueError("weight must hold C*K elements")
        self._bias = None if bias is None else np.ascontiguousarray(
            np.asarray(bias).reshape(-1)).view(_NP_STORAGE[w_dtype])
        self._seq = None if seq is None else np.ascontiguousarray(
            np.asarray(seq, dtype=np.int32).reshape(-1))
        self._init = None if init is None else np.ascontiguousarray(
            np.asarray(init).reshape(-1)).view(st)
        es = self._x.itemsize
        p = _Problem()
        p.B, p.C, p.L, p.K, p.silu = self.B, self.C, self.L, self.K, int(bool(silu))
        p.x = self._x.ctypes.data + int(x_off) * es
        p.x_dtype = DTYPES[x_dtype]
        p.xs = (ctypes.c_int64 * 3)(*[int(s) for s in x_strides])
        p.w = self._w.ctypes.data
        p.w_dtype = DTYPES[w_dtype]
        p.bias = _ptr(self._bias)
        p.seq = _ptr(self._seq)
        if self._init is not None:
            if init_strides is None:
                raise ValueError("init_strides required with init")
            p.init = self._init.ctypes.data + int(init_off) * es
            p.is_ = (ctypes.c_int64 * 3)(*[int(s) for s in init_strides])
        else:
            p.init = None
            p.is_ = (ctypes.c_int64 * 3)(0, 0, 0)
        self._p = p

    # ---- calls ---------------------------------------------------------------
    def fwd(self, want_sabs: bool = True):
        """y (fp64, after the activation) and sabs for every output, [B, C, L]."""
        n = self.B * self.C * self.L
        y = np.empty(n, dtype=np.float64)
        s = np.empty(n, dtype=np.float64) if want_sabs else None
        if lib().ora_fwd(ctypes.byref(self._p), y.ctypes.data, _ptr(s)) != 0:
            raise RuntimeError("ora_fwd failed")
        shape = (self.B, self.C, self.L)
        return y.reshape(shape), (None if s is None else s.reshape(shape))

    def fwd_threads(self, nthreads: int, want_sabs: bool = True):
        """fwd() on up to `nthreads` host threads (rows split between them); the
        same outputs bit for bit."""
        n = self.B * self.C * self.L
        y = np.empty(n, dtype=np.float64)
        s = np.empty(n, dtype=np.float64) if want_sabs else None
        if lib().ora_fwd_threads(ctypes.byref(self._p), y.ctypes.data, _ptr(s), int(nthreads)) != 0:
            raise RuntimeError("ora_fwd_threads failed")
        shape = (self.B, self.C, self.L)
        return y.reshape(shape), (None if s is None else s.reshape(shape))

    def point(self, b, c, t):
        y, z, s = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
        if lib().ora_point(ctypes.byref(self._p), b, c, t, ctypes.byref(y), ctypes.byref(z),
                           ctypes.byref(s)) != 0:
            raise IndexError((b, c, t))
        return y.value, z.value, s.value

    def points(self, idx):
        idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int64).reshape(-1, 3))
        n = idx.shape[0]
        y = np.empty(n, dtype=np.float64)
        s = np.empty(n, dtype=np.float64)
        if lib().ora_points(ctypes.byref(self._p), n, idx.ctypes.data, y.ctypes.data,
                            s.ctypes.data) != 0:
            raise IndexError("sample index out of range")
        return y, s

    def fwd_f32(self):
        """Diagnostic binary32 mode for every output, [B, C, L] float32: the stencil
        summed with one fused multiply-add per kept term, bias first, k ascending;
        no activation."""
        z = np.empty(self.B * self.C * self.L, dtype=np.float32)
        if lib().ora_fwd_f32(ctypes.byref(self._p), z.ctypes.data) != 0:
            raise RuntimeError("ora_fwd_f32 failed")
        return z.reshape(self.B, self.C, self.L)

    def points_f32(self, idx):
        """Diagnostic binary32 mode at n sampled (b, c, t) triples."""
        idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int64).reshape(-1, 3))
        z = np.empty(idx.shape[0], dtype=np.float32)
        if lib().ora_points_f32(ctypes.byref(self._p), idx.shape[0], idx.ctypes.data,
                                z.ctypes.data) != 0:
            raise IndexError("sample index out of range")
        return z

    def bwd(self, dout, dout_strides, dout_off=0, dfs=None, dfs_strides=None, dfs_off=0):
        """Gradients in fp64 (the chain rule of the forward) and their error scales.

        dout: flat storage in x's dtype, dout[b,c,t] at dout_off + b*s0 + c*s1 + t*s2;
        dfs: None or flat storage of dfinal_states [B, C, K-1] in x's dtype.
        Returns dict(dx, dinit, dw, db, ex, einit, ew, eb) of float64 arrays
        ([B,C,L], [B,C,K-1] or None, [C,K], [C] and the same for the scales)."""
        st = _NP_STORAGE[self.x_dtype]
        dout = np.ascontiguousarray(np.asarray(dout).reshape(-1)).view(st)
        es = dout.itemsize
        g = _Grad()
        g.dout = dout.ctypes.data + int(dout_off) * es
        g.ds = (ctypes.c_int64 * 3)(*[int(v) for v in dout_strides])
        if dfs is not None:
            dfs = np.ascontiguousarray(np.asarray(dfs).reshape(-1)).view(st)
            g.dfs = dfs.ctypes.data + int(dfs_off) * es
            g.fs = (ctypes.c_int64 * 3)(*[int(v) for v in dfs_strides])
        else:
            g.dfs = None
            g.fs = (ctypes.c_int64 * 3)(0, 0, 0)
        B, C, L, K = self.B, self.C, self.L, self.K
        has_init = self._init is not None
        out = {
            "dx": np.zeros((B, C, L)), "ex": np.zeros((B, C, L)),
            "dinit": np.zeros((B, C, K - 1)) if has_init else None,
            "einit": np.zeros((B, C, K - 1)) if has_init else None,
            "dw": np.zeros((C, K)), "ew": np.zeros((C, K)), "db": np.zeros(C), "eb": np.zeros(C),
        }
        ptrs = [_ptr(out[k]) for k in ("dx", "dinit", "dw", "db", "ex", "einit", "ew", "eb")]
        if lib().ora_bwd(ctypes.byref(self._p), ctypes.byref(g), *ptrs) != 0:
            raise RuntimeError("ora_bwd failed")
        _keep = (dout, dfs)   # noqa: F841  (buffers stay alive through the call)
        return out

    def final_states(self):
        """Raw storage [B, C, K-1] of the last K-1 extended inputs."""
        fs = np.zeros(self.B * self.C * (self.K - 1), dtype=_NP_STORAGE[self.x_dtype])
        lib().ora_final_states(ctypes.byref(self._p), fs.ctypes.data)
        return fs.reshape(self.B, self.C, self.K - 1)


def round_out(dtype: str, y):
    """o32 = RNE_f32(y); for 16-bit storage, RNE of o32 to that format (raw)."""
    y = np.ascontiguousarray(np.asarray(y, dtype=np.float64))
    out = np.empty(y.shape, dtype=_NP_STORAGE[dtype])
    lib().ora_round_out(DTYPES[dtype], y.ctypes.data, y.size, out.ctypes.data)
    return out


def f32_to_bf16(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    out = np.empty(a.shape, dtype=np.uint16)
    lib().ora_f32_to_bf16_array(a.ctypes.data, out.ctypes.data, a.size)
    return out


def f32_to_f16(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    out = np.empty(a.shape, dtype=np.uint16)
    lib().ora_f32_to_f16_array(a.ctypes.data, out.ctypes.data, a.size)
    return out


def decode(dtype: str, a):
    """Exact fp64 values of raw storage."""
    a = np.ascontiguousarray(np.asarray(a))
    if dtype == "f32":
        return a.view(np.float32).astype(np.float64)
    a = a.view(np.uint16)
    out = np.empty(a.shape, dtype=np.float64)
    fn = lib().ora_f16_to_f64_array if dtype == "f16" else lib().ora_bf16_to_f64_array
    fn(a.ctypes.data, out.ctypes.data, a.size)
    return out
