"""The parity comparison itself (CPU): exact oracle values pass, values a few ulps
away fail unless the cancellation floor covers them, NaN and infinities must match."""
import numpy as np

import oracle
from oracle import compare as ocmp


def test_exact_values_pass_and_far_values_fail():
    g = np.random.default_rng(0)
    y = g.standard_normal(10000) * 10
    s = np.abs(y) + 0.0            # tiny floor: S == |y|
    for dt in ("f32", "bf16", "f16"):
        o = oracle.round_out(dt, y)
        res = ocmp.compare(dt, 4, o, y, s)
        assert res["n_bad"] == 0 and res["bit_equal"] == y.size
        if dt == "f32":
            bumped = (o.view(np.uint32) + 200).view(np.float32)      # ~1.2e-5 relative
        else:
            bumped = (o.view(np.uint16) + 3).astype(np.uint16)        # 3 ulps
        res = ocmp.compare(dt, 4, bumped, y, s)
        assert res["n_bad"] > 0.9 * y.size, dt


def test_two_ulps_pass_for_16_bit():
    y = np.linspace(0.5, 3.0, 1000)
    for dt in ("bf16", "f16"):
        o = oracle.round_out(dt, y)
        res = ocmp.compare(dt, 4, (o.view(np.uint16) + 2).astype(np.uint16), y, np.abs(y))
        assert res["n_bad"] == 0 and res["max_ulp"] == 2


def test_cancellation_floor():
    # z cancels to 1e-6 while the terms are O(10): fp32 rounding of partial sums may
    # move the result by ~K * 2^-24 * 10, far beyond 1e-5 relative of 1e-6.
    y = np.full(10, 1e-6)
    s = np.full(10, 40.0)
    g = (y + 4 * 2.0 ** -24 * 40).astype(np.float32)
    assert ocmp.compare("f32", 4, g, y, s)["n_bad"] == 0
    g = (y + 8 * 2.0 ** -22 * 40).astype(np.float32)
    assert ocmp.compare("f32", 4, g, y, s)["n_bad"] == 10


def test_nan_and_inf_must_match():
    y = np.array([np.nan, np.inf, -np.inf, 1.0])
    s = np.array([np.nan, np.inf, np.inf, 1.0])
    ok = np.array([np.nan, np.inf, -np.inf, 1.0], dtype=np.float32)
    assert ocmp.compare("f32", 4, ok, y, s)["n_bad"] == 0
    bad = np.array([1.0, np.inf, np.inf, np.nan], dtype=np.float32)
    assert ocmp.compare("f32", 4, bad, y, s)["n_bad"] == 3
