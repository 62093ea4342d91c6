"""Element-wise comparison of GPU outputs with the oracle, at the stated tolerances.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Let y be the oracle's fp64 result, S = |bias| + sum over kept terms of |w * x~|
(the oracle's ``sabs``), K the tap count and g the GPU value.

  fp32 output:    pass iff g == o32 or |g - o32| <= 1e-5 * |y| + K * 2^-22 * S,
                  with o32 = RNE_fp32(y);
  16-bit output:  pass iff g is within 2 ulps of o16 = RNE_16(o32), or
                  |g - y| <= K * 2^-22 * S + ulp(g).

The S term is the first-order bound of fp32 recursive summation of K+1 terms
(each rounding <= 2^-24 of a partial sum bounded by S), with a 4x margin that
also covers the SiLU slope (<= 1.1).  Without it a correct fp32 kernel fails
wherever z cancels to much less than S.  NaN must match NaN; infinities must
match exactly.  Every output is checked; nothing is reduced to a norm.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import decode, lib, round_out

_MBITS = {"bf16": 7, "f16": 10}
_BIAS = {"bf16": 127, "f16": 15}


def _ord16(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def _ulp_table(dtype: str) -> np.ndarray:
    """ulp of the 16-bit format for each value of its exponent field (subnormals and
    zero share the smallest normal exponent's spacing)."""
    m = _MBITS[dtype]
    e = np.maximum(np.arange(1 << (15 - m), dtype=np.int64), 1)
    return np.ldexp(1.0, e - _BIAS[dtype] - m)


_ULP_TABLES = {d: _ulp_table(d) for d in _MBITS}


def ulp16(dtype: str, bits: np.ndarray) -> np.ndarray:
    """Spacing of the 16-bit format at each value (its exponent's ulp)."""
    m = _MBITS[dtype]
    e = (np.asarray(bits, dtype=np.uint16) >> m) & ((1 << (15 - m)) - 1)
    return _ULP_TABLES[dtype][e]


_CHUNK = 1 << 20
_THREADS = min(16, len(os.sched_getaffinity(0)))


def compare(dtype: str, K: int, g_raw: np.ndarray, y: np.ndarray, sabs: np.ndarray) -> dict:
    """g_raw: GPU output storage (float32 or uint16 bits), same shape as y and sabs.

    Returns a dict with ``bad`` (boolean mask of failures), ``n``, ``n_bad``,
    ``max_rel`` (max |g - o| / |o| over finite nonzero o), ``max_ulp`` (16-bit),
    ``n_floor_only`` (passed only through the S term) and ``bit_equal`` (count of
    outputs equal to the rounded oracle value).  Large inputs are checked in
    chunks on several host threads; every element gets the same test either way."""
    y = np.asarray(y, dtype=np.float64).reshape(-1)
    s = np.asarray(sabs, dtype=np.float64).reshape(-1)
    g_raw = np.ascontiguousarray(g_raw).reshape(-1)
    n = y.size
    bad = np.zeros(n, dtype=bool)
    bounds = [(lo, min(n, lo + _CHUNK)) for lo in range(0, n, _CHUNK)]
    lib()                                          # load (or build) before any thread uses it

    def one(lo_hi):
        lo, hi = lo_hi
        return _compare_chunk(dtype, K, g_raw[lo:hi], y[lo:hi], s[lo:hi], bad[lo:hi])

    if len(bounds) > 1 and _THREADS > 1:
        with ThreadPoolExecutor(_THREADS) as ex:
            parts = list(ex.map(one, bounds))
    else:
        parts = [one(b) for b in bounds]
    ulps = [p["max_ulp"] for p in parts if p["max_ulp"] is not None]
    return {
        "bad": bad,
        "n": int(n),
        "n_bad": sum(p["n_bad"] for p in parts),
        "max_rel": max([p["max_rel"] for p in parts], default=0.0),
        "max_ulp": None if dtype == "f32" else max(ulps, default=0),
        "n_floor_only": sum(p["n_floor_only"] for p in parts),
        "bit_equal": sum(p["bit_equal"] for p in parts),
    }


def _compare_chunk(dtype: str, K: int, g_raw, y, s, bad) -> dict:
    """compare() on one slice; writes the slice's failures into `bad` (a view)."""
    floor = K * 2.0 ** -22 * s
    o_raw = round_out(dtype, y)
    g = decode(dtype, g_raw)
    o = decode(dtype, o_raw)
    nan_g, nan_y = np.isnan(g), np.isnan(y)
    bad[:] = nan_g != nan_y
    both = ~nan_g & ~nan_y
    with np.errstate(invalid="ignore", over="ignore"):
        exact = g == o
        if dtype == "f32":
            primary = exact | (np.abs(g - o) <= 1e-5 * np.abs(y))
            lenient = np.abs(g - o) <= 1e-5 * np.abs(y) + floor
            max_ulp = None
        else:
            dist = np.abs(_ord16(g_raw.view(np.uint16)) - _ord16(o_raw.view(np.uint16)))
            primary = exact | (dist <= 2)
            lenient = np.abs(g - y) <= floor + ulp16(dtype, g_raw.view(np.uint16))
            finite = both & np.isfinite(g) & np.isfinite(o)
            max_ulp = int(dist[finite].max()) if finite.any() else 0
        inf_mismatch = both & (np.isinf(g) | np.isinf(o)) & ~exact
        ok = (primary | lenient) & ~inf_mismatch
        bad |= both & ~ok
        fin = both & np.isfinite(o) & (o != 0) & np.isfinite(g)
        rel = np.abs(g[fin] - o[fin]) / np.abs(o[fin])
    return {
        "n_bad": int(bad.sum()),
        "max_rel": float(rel.max()) if rel.size else 0.0,
        "max_ulp": max_ulp,
        "n_floor_only": int((both & ~primary & lenient & ~inf_mismatch).sum()),
        "bit_equal": int((exact | (nan_g & nan_y)).sum()),
    }


def describe_failures(res: dict, y, sabs, g_raw, dtype: str, shape=None, limit: int = 8) -> str:
    idx = np.flatnonzero(res["bad"])[:limit]
    g = decode(dtype, np.ascontiguousarray(g_raw).reshape(-1))
    yy = np.asarray(y).reshape(-1)
    ss = np.asarray(sabs).reshape(-1)
    lines = [f"{res['n_bad']} of {res['n']} outputs out of tolerance"]
    for i in idx:
        pos = np.unravel_index(i, shape) if shape is not None else i
        lines.append(f"  at {pos}: gpu {g[i]!r} oracle {yy[i]!r} sabs {ss[i]!r}")
    return "\n".join(lines)
