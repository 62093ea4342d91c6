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

import numpy as np

from . import decode, round_out

_MBITS = {"bf16": 7, "f16": 10}
_BIAS = {"bf16": 127, "f16": 15}


def _ord16(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp16(dtype: str, bits: np.ndarray) -> np.ndarray:
    """Spacing of the 16-bit format at each value (its exponent's ulp)."""
    m = _MBITS[dtype]
    e = (bits.astype(np.int64) >> m) & ((1 << (15 - m)) - 1)
    e = np.maximum(e, 1)
    return np.ldexp(1.0, (e - _BIAS[dtype] - m).astype(np.int64))


def compare(dtype: str, K: int, g_raw: np.ndarray, y: np.ndarray, sabs: np.ndarray) -> dict:
    """g_raw: GPU output storage (float32 or uint16 bits), same shape as y and sabs.

    Returns a dict with ``bad`` (boolean mask of failures), ``n``, ``n_bad``,
    ``max_rel`` (max |g - o| / |o| over finite nonzero o), ``max_ulp`` (16-bit),
    ``n_floor_only`` (passed only through the S term) and ``bit_equal`` (count of
    outputs equal to the rounded oracle value)."""
    y = np.asarray(y, dtype=np.float64).reshape(-1)
    s = np.asarray(sabs, dtype=np.float64).reshape(-1)
    g_raw = np.ascontiguousarray(g_raw).reshape(-1)
    floor = K * 2.0 ** -22 * s
    o_raw = round_out(dtype, y)
    g = decode(dtype, g_raw)
    o = decode(dtype, o_raw)
    nan_g, nan_y = np.isnan(g), np.isnan(y)
    bad = nan_g != nan_y
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
        "bad": bad,
        "n": int(y.size),
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
