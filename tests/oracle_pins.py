"""Pins that tie the oracle to facts other than its own code.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with:
  * hand-worked examples of the stencil equation (tests/golden/),
  * closed forms (decimal digit read-out, one-hot weights, a delta input, a
    constant input),
  * a library routine that implements the same cross-correlation
    (torch.nn.functional.conv1d in fp64 on the CPU, grouped by channel),
  * invariants the definition implies (chunking with carried states, packed
    sequences equal separate runs, layout independence, masked NaN not leaking),
  * torch's own dtype conversions and SiLU,
  * for the diagnostic binary32 mode: an exact-rational emulation of its
    fused multiply-add chain, exactness on integer data, and the K-rounding bound,
  * for the backward: torch autograd in fp64, central finite differences of the
    forward oracle, and the packing and chunking invariants of the gradients.

The functions take the ``oracle`` module so that ``test_oracle_mutants`` can run
them against deliberately broken builds of the oracle.
"""
from __future__ import annotations

import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _raw(t: torch.Tensor) -> np.ndarray:
    t = t.contiguous()
    return t.numpy() if t.dtype == torch.float32 else t.view(torch.int16).numpy().view(np.uint16)


def _cf_case(ora, x, w, bias=None, seq=None, init=None, silu=False):
    """Oracle case for a contiguous [B,C,L] torch tensor x (any of the 3 dtypes)."""
    B, C, L = x.shape
    K = w.shape[1]
    kw = {}
    if init is not None:
        kw.update(init=_raw(init), init_strides=init.stride())
    return ora.Case(B=B, C=C, L=L, K=K, x=_raw(x), x_dtype=_name(x), x_strides=x.stride(),
                    w=_raw(w), w_dtype=_name(w), bias=None if bias is None else _raw(bias),
                    seq=None if seq is None else seq.numpy(), silu=silu, **kw)


def _name(t):
    return {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[t.dtype]


def _gen(seed):
    return torch.Generator().manual_seed(seed)


# ---- golden fixtures ------------------------------------------------------------

def load_golden():
    cases = []
    for fn in sorted(os.listdir(GOLDEN)):
        if not fn.endswith(".txt"):
            continue
        d = {}
        with open(os.path.join(GOLDEN, fn)) as f:
            for line in f:
                line = line.split("#", 1)[0].strip()
                if not line:
                    continue
                key, *vals = line.split()
                d[key] = [float(v) for v in vals]
        d["name"] = fn
        cases.append(d)
    return cases


def pin_golden(ora):
    cases = load_golden()
    assert len(cases) >= 7
    for d in cases:
        K = int(d["K"][0])
        for dt in ("f32", "f16", "bf16"):
            x = torch.tensor(d["x"], dtype=torch.float64).to(DT[dt]).reshape(1, 1, -1)
            w = torch.tensor(d["w"], dtype=torch.float64).to(DT[dt]).reshape(1, K)
            bias = torch.tensor(d["bias"], dtype=torch.float64).to(DT[dt]) if "bias" in d else None
            init = (torch.tensor(d["init"], dtype=torch.float64).to(DT[dt]).reshape(1, 1, K - 1)
                    if "init" in d else None)
            seq = torch.tensor([int(v) for v in d["seq"]], dtype=torch.int32).reshape(1, -1) if "seq" in d else None
            c = _cf_case(ora, x, w, bias, seq, init)
            y, _ = c.fwd()
            assert np.array_equal(y.reshape(-1), np.array(d["z"])), (d["name"], dt, y.reshape(-1), d["z"])
            if "final" in d:
                fs = ora.decode(dt, c.final_states()).reshape(-1)
                assert np.array_equal(fs, np.array(d["final"])), (d["name"], dt, fs, d["final"])


# ---- closed forms ---------------------------------------------------------------

def pin_digits(ora):
    """w = (1, 10, ..., 10^(K-1)) and inputs in 0..9: z[t] is an integer whose
    decimal digits are x[t], x[t-1], ..., x[t-K+1] (newest first)."""
    g = np.random.default_rng(7)
    for K in (2, 3, 4):
        for dt in ("f32", "bf16", "f16"):
            L = 37
            xd = g.integers(0, 10, size=L)
            hd = g.integers(0, 10, size=K - 1)
            x = torch.tensor(xd, dtype=torch.float64).to(DT[dt]).reshape(1, 1, L)
            w = torch.tensor([10.0 ** k for k in range(K)], dtype=torch.float64).to(DT[dt]).reshape(1, K)
            init = torch.tensor(hd, dtype=torch.float64).to(DT[dt]).reshape(1, 1, K - 1)
            y, _ = _cf_case(ora, x, w, init=init).fwd()
            ext = np.concatenate([hd, xd])
            for t in range(L):
                window = ext[t:t + K]            # x~[t-K+1 .. t], oldest first
                z = int(y[0, 0, t])
                assert z == y[0, 0, t]
                digits = [int(ch) for ch in str(z).zfill(K)]
                assert digits == list(window[::-1]), (K, dt, t, z, window)


def pin_one_hot(ora):
    """w = e_k (no bias, no activation) shifts the extended input: z[t] = x~[t-K+1+k]."""
    g = _gen(11)
    for K in (2, 3, 4):
        for dt in ("f32", "bf16", "f16"):
            B, C, L = 2, 3, 29
            x = torch.randn(B, C, L, generator=g).to(DT[dt])
            init = torch.randn(B, C, K - 1, generator=g).to(DT[dt])
            ext = torch.cat([init, x], dim=2).double()
            for k in range(K):
                w = torch.zeros(C, K, dtype=DT[dt])
                w[:, k] = 1
                y, _ = _cf_case(ora, x, w, init=init).fwd()
                expect = ext[:, :, k:k + L].numpy()
                assert np.array_equal(y, expect), (K, dt, k)


def pin_delta(ora):
    """x = delta(t - t0) with zero history returns the weights reversed after t0:
    z[t0 + j] = bias + w[K-1-j] for 0 <= j < K, and bias elsewhere."""
    g = _gen(12)
    for K in (2, 3, 4):
        C, L, t0 = 4, 16, 5
        x = torch.zeros(1, C, L)
        x[:, :, t0] = 1
        w = torch.randn(C, K, generator=g)
        bias = torch.randn(C, generator=g)
        y, _ = _cf_case(ora, x, w, bias).fwd()
        expect = np.repeat(bias.double().numpy()[:, None], L, axis=1)
        for j in range(K):
            expect[:, t0 + j] = (bias.double() + w[:, K - 1 - j].double()).numpy()
        assert np.array_equal(y[0], expect), K


def pin_constant(ora):
    """x = a with zero history: z[t] = bias + a * sum_{k >= K-1-t} w[k] (t < K-1),
    then bias + a * sum(w)."""
    for K in (2, 3, 4):
        a = 0.75
        w = torch.tensor([[1.0, 2.0, 4.0, 8.0][:K]])
        bias = torch.tensor([0.5])
        L = 9
        x = torch.full((1, 1, L), a)
        y, _ = _cf_case(ora, x, w, bias).fwd()
        for t in range(L):
            expect = 0.5 + a * sum(float(w[0, k]) for k in range(K) if k >= K - 1 - t)
            assert y[0, 0, t] == expect, (K, t, y[0, 0, t], expect)


# ---- library routine --------------------------------------------------------------

def _torch_ref(x, w, bias, init, silu):
    """torch.nn.functional.conv1d in fp64 (grouped per channel) over the input
    extended on the left by the history: the cross-correlation Conv1d computes."""
    B, C, L = x.shape
    K = w.shape[1]
    hist = init.double() if init is not None else torch.zeros(B, C, K - 1, dtype=torch.float64)
    ext = torch.cat([hist, x.double()], dim=2)
    z = torch.nn.functional.conv1d(ext, w.double().reshape(C, 1, K),
                                   None if bias is None else bias.double(), groups=C)
    sabs = torch.nn.functional.conv1d(ext.abs(), w.double().abs().reshape(C, 1, K),
                                      None if bias is None else bias.double().abs(), groups=C)
    y = torch.nn.functional.silu(z) if silu else z
    return y.numpy(), sabs.numpy()


def pin_conv1d(ora):
    g = _gen(13)
    combos = [("f32", "f32"), ("bf16", "bf16"), ("f16", "f16"), ("bf16", "f32"), ("f32", "f16"),
              ("f16", "bf16")]
    for K in (2, 3, 4):
        for xd, wd in combos:
            for use_bias, use_init, silu in ((True, False, True), (False, True, False), (True, True, True)):
                B, C, L = 2, 5, 67
                x = (torch.randn(B, C, L, generator=g) * 2).to(DT[xd])
                w = torch.randn(C, K, generator=g).to(DT[wd])
                bias = torch.randn(C, generator=g).to(DT[wd]) if use_bias else None
                init = torch.randn(B, C, K - 1, generator=g).to(DT[xd]) if use_init else None
                y, s = _cf_case(ora, x, w, bias, init=init, silu=silu).fwd()
                ry, rs = _torch_ref(x, w, bias, init, silu)
                tol = 1e-14 * rs + 1e-300
                assert np.all(np.abs(y - ry) <= tol), (K, xd, wd, np.max(np.abs(y - ry) / tol))
                assert np.all(np.abs(s - rs) <= 1e-14 * rs + 1e-300), (K, xd, wd)


# ---- invariants -------------------------------------------------------------------

def pin_chunking(ora):
    """Running [x1 | x2] equals running x1, then x2 with x1's final states as its
    initial states: every output bit-identical, and the same final states."""
    g = _gen(14)
    for K in (2, 3, 4):
        for dt in ("f32", "bf16", "f16"):
            B, C, L = 2, 3, 40
            x = torch.randn(B, C, L, generator=g).to(DT[dt])
            w = torch.randn(C, K, generator=g).to(DT[dt])
            bias = torch.randn(C, generator=g).to(DT[dt])
            init = torch.randn(B, C, K - 1, generator=g).to(DT[dt])
            full = _cf_case(ora, x, w, bias, init=init, silu=True)
            y_full, _ = full.fwd()
            fs_full = full.final_states()
            for L1 in sorted({0, 1, K - 2, K - 1, K, 17, L}):
                x1, x2 = x[:, :, :L1].contiguous(), x[:, :, L1:].contiguous()
                c1 = _cf_case(ora, x1, w, bias, init=init, silu=True)
                y1, _ = c1.fwd()
                f1 = c1.final_states()
                f1_t = (torch.from_numpy(f1.copy()) if dt == "f32"
                        else torch.from_numpy(f1.view(np.int16).copy()).view(DT[dt]))
                c2 = _cf_case(ora, x2, w, bias, init=f1_t, silu=True)
                y2, _ = c2.fwd()
                assert np.array_equal(np.concatenate([y1, y2], axis=2).view(np.uint64),
                                      y_full.view(np.uint64)), (K, dt, L1)
                assert np.array_equal(c2.final_states(), fs_full), (K, dt, L1)


def pin_packing(ora):
    """A packed run with seq_idx equals separate runs of each sequence (zero history)."""
    g = _gen(15)
    for K in (2, 3, 4):
        for dt in ("f32", "bf16"):
            lengths = [1, 5, K - 1, 9, 2, 13, K]
            L = sum(lengths)
            C = 3
            x = torch.randn(1, C, L, generator=g).to(DT[dt])
            w = torch.randn(C, K, generator=g).to(DT[dt])
            bias = torch.randn(C, generator=g).to(DT[dt])
            seq = torch.tensor(np.repeat(np.arange(len(lengths)), lengths), dtype=torch.int32).reshape(1, L)
            y, _ = _cf_case(ora, x, w, bias, seq=seq, silu=True).fwd()
            pos = 0
            for n in lengths:
                part = x[:, :, pos:pos + n].contiguous()
                yp, _ = _cf_case(ora, part, w, bias, silu=True).fwd()
                assert np.array_equal(y[:, :, pos:pos + n].view(np.uint64), yp.view(np.uint64)), (K, dt, n)
                pos += n


def _fs_tensor(raw_fs, dt):
    return (torch.from_numpy(raw_fs.copy()) if dt == "f32"
            else torch.from_numpy(raw_fs.view(np.int16).copy()).view(DT[dt]))


def pin_packed_chunking(ora):
    """seq_idx together with states: a packed row split anywhere equals the whole
    row when chunk 2's history is chunk 1's final states if its first sequence
    continues chunk 1's last one, and zeros if it starts there.  That holds only
    if the history counts for the row's first sequence and final states keep the
    row's last sequence only.  Every output and final state, bit for bit."""
    g = _gen(26)
    for K in (2, 3, 4):
        for dt in ("f32", "bf16"):
            lengths = [3, 1, 6, 2, 9]
            L, C, B = sum(lengths), 3, 2
            x = torch.randn(B, C, L, generator=g).to(DT[dt])
            w = torch.randn(C, K, generator=g).to(DT[dt])
            bias = torch.randn(C, generator=g).to(DT[dt])
            h = torch.randn(B, C, K - 1, generator=g).to(DT[dt])
            ids = np.repeat(np.arange(len(lengths)), lengths)
            seq = torch.tensor(np.stack([ids, ids[::-1] + 10]), dtype=torch.int32)
            full = _cf_case(ora, x, w, bias, seq=seq, init=h, silu=True)
            y_full, _ = full.fwd()
            fs_full = full.final_states()
            for L1 in range(1, L):
                c1 = _cf_case(ora, x[:, :, :L1].contiguous(), w, bias, seq=seq[:, :L1].contiguous(), init=h,
                              silu=True)
                y1, _ = c1.fwd()
                f1 = _fs_tensor(c1.final_states(), dt)
                cont = (seq[:, L1] == seq[:, L1 - 1]).reshape(B, 1, 1)
                h2 = torch.where(cont, f1, torch.zeros_like(f1))
                c2 = _cf_case(ora, x[:, :, L1:].contiguous(), w, bias, seq=seq[:, L1:].contiguous(), init=h2,
                              silu=True)
                y2, _ = c2.fwd()
                assert np.array_equal(np.concatenate([y1, y2], 2).view(np.uint64), y_full.view(np.uint64)), (K, dt, L1)
                assert np.array_equal(c2.final_states(), fs_full), (K, dt, L1)


def pin_mask_nan(ora):
    """A masked term is dropped, not multiplied by zero: a NaN in another sequence
    does not reach this one, while a NaN inside the window does."""
    K, L = 4, 8
    x = torch.arange(1, L + 1, dtype=torch.float32).reshape(1, 1, L)
    x[0, 0, 2] = float("nan")
    w = torch.ones(1, K)
    seq = torch.tensor([[0, 0, 0, 1, 1, 1, 1, 1]], dtype=torch.int32)
    y, _ = _cf_case(ora, x, w, seq=seq).fwd()
    assert np.isnan(y[0, 0, 2]) and np.isnan(y[0, 0, 1] + y[0, 0, 2])
    assert not np.isnan(y[0, 0, 3:]).any(), y
    assert list(y[0, 0, 3:]) == [4.0, 9.0, 15.0, 22.0, 26.0]
    y2, _ = _cf_case(ora, x, w).fwd()
    assert np.isnan(y2[0, 0, 2:6]).all() and not np.isnan(y2[0, 0, 6:]).any()


def pin_layout(ora):
    """The same logical x stored channel-first, channel-last, or as a strided view of a
    wider buffer gives bit-identical results (offsets follow s_B, s_C, s_L)."""
    g = _gen(16)
    B, C, L, K = 2, 6, 23, 4
    x = torch.randn(B, C, L, generator=g).to(torch.bfloat16)
    w = torch.randn(C, K, generator=g).to(torch.bfloat16)
    bias = torch.randn(C, generator=g).to(torch.bfloat16)
    ref, _ = _cf_case(ora, x, w, bias, silu=True).fwd()
    cl = x.transpose(1, 2).contiguous()              # [B, L, C]
    c = ora.Case(B=B, C=C, L=L, K=K, x=_raw(cl), x_dtype="bf16", x_strides=(L * C, 1, C),
                 w=_raw(w), w_dtype="bf16", bias=_raw(bias), silu=True)
    assert np.array_equal(c.fwd()[0].view(np.uint64), ref.view(np.uint64))
    wide = torch.full((B, L, C + 5), float("nan")).to(torch.bfloat16)
    wide[:, :, 3:3 + C] = cl
    c = ora.Case(B=B, C=C, L=L, K=K, x=_raw(wide), x_off=3, x_dtype="bf16",
                 x_strides=(L * (C + 5), 1, C + 5), w=_raw(w), w_dtype="bf16", bias=_raw(bias), silu=True)
    assert np.array_equal(c.fwd()[0].view(np.uint64), ref.view(np.uint64))


# ---- activation and conversions ------------------------------------------------------

def pin_silu(ora):
    """SiLU against torch's fp64 silu, plus silu(0) = 0, the odd-part identity
    silu(z) - silu(-z) = z, and the limits silu(z) -> z (z >> 0), -> 0 (z << 0)."""
    zs = np.concatenate([np.linspace(-30, 30, 601), [0.0, 1e-30, -1e-30, 80.0, -80.0, 700.0, -700.0]])
    L = zs.size
    x = torch.tensor(zs, dtype=torch.float64).to(torch.float32).reshape(1, 1, L)
    w = torch.tensor([[0.0, 0.0, 1.0]])             # one-hot on the current step: z = x
    y, _ = _cf_case(ora, x, w, silu=True).fwd()
    z = x.double().reshape(-1)
    ref = torch.nn.functional.silu(z).numpy()
    assert np.all(np.abs(y.reshape(-1) - ref) <= 1e-15 * np.abs(ref) + 1e-300)
    y = y.reshape(-1)
    zz = z.numpy()
    i0 = int(np.where(zz == 0.0)[0][0])
    assert y[i0] == 0.0
    neg = {v: i for i, v in enumerate(zz)}
    for i, v in enumerate(zz):
        if -v in neg and abs(v) < 40:
            assert abs((y[i] - y[neg[-v]]) - v) <= 1e-14 * max(1.0, abs(v)), v
    assert y[list(zz).index(80.0)] == 80.0            # 80 - 80*e^-80 rounds to 80 in fp64
    assert 0 < -y[list(zz).index(-80.0)] < 1e-30      # about -80*e^-80


def pin_converters(ora):
    """Decoding of every 16-bit pattern and RNE encoding of fp32 against torch."""
    pats = np.arange(65536, dtype=np.uint16)
    for dt, tdt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        ref = torch.from_numpy(pats.view(np.int16)).view(tdt).double().numpy()
        got = ora.decode(dt, pats)
        both_nan = np.isnan(ref) & np.isnan(got)
        assert np.array_equal(np.isnan(ref), np.isnan(got)), dt
        assert np.array_equal(got[~both_nan], ref[~both_nan]), dt
    g = np.random.default_rng(17)
    vals = np.concatenate([
        g.standard_normal(200_000).astype(np.float32) * np.float32(1000),
        (g.standard_normal(100_000) * 1e-5).astype(np.float32),
        g.integers(0, 2**32, 200_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
        np.array([0.0, -0.0, 65504, 65519.99, 65520, 65536, -65520, 6e-8, 2.98e-8, 5.96e-8,
                  6.1035e-5, 6.1e-5, 3.4e38, -3.4e38, np.inf, -np.inf, np.nan], dtype=np.float32),
    ])
    # exact ties for both formats
    base = g.integers(0, 2**16, 50_000, dtype=np.uint32)
    vals = np.concatenate([vals, ((base << 16) | 0x8000).view(np.float32),
                           (np.float32(1.0) + np.float32(2.0 ** -11) * np.arange(1, 64, 2, dtype=np.float32))])
    for dt, tdt, fn in (("bf16", torch.bfloat16, ora.f32_to_bf16), ("f16", torch.float16, ora.f32_to_f16)):
        ref = torch.from_numpy(vals).to(tdt).view(torch.int16).numpy().view(np.uint16)
        got = fn(vals)
        rnan = np.isnan(torch.from_numpy(vals).to(tdt).float().numpy())
        gnan = np.isnan(ora.decode(dt, got))
        assert np.array_equal(rnan, gnan), dt
        assert np.array_equal(got[~rnan], ref[~rnan]), (dt, vals[~rnan][got[~rnan] != ref[~rnan]][:5])


def pin_round_out(ora):
    """Output rounding: fp64 -> fp32 (RNE), then fp32 -> 16-bit (RNE), as torch does."""
    g = np.random.default_rng(18)
    y = np.concatenate([g.standard_normal(50_000) * 300, g.standard_normal(1000) * 1e-6, [0.0, -0.0]])
    for dt, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16), ("f16", torch.float16)):
        got = ora.round_out(dt, y)
        ref = torch.from_numpy(y).to(torch.float32).to(tdt)
        ref = ref.numpy() if dt == "f32" else ref.view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got.view(np.uint32 if dt == "f32" else np.uint16),
                              ref.view(np.uint32 if dt == "f32" else np.uint16)), dt


# ---- diagnostic binary32 mode -------------------------------------------------------

def _rne_f32(q):
    """Round an exact rational to the nearest binary32 (ties to even), with gradual
    underflow and overflow to infinity, written from the IEEE-754 definition.  An
    exact zero gives +0 (the sums below never cancel to zero)."""
    from fractions import Fraction
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()   # 2^e <= a < 2^(e+2)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                     # below 2^-126 the spacing stays 2^-149
    ulp = Fraction(2) ** (e - 23)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * ulp
    if v >= Fraction(2) ** 128:
        return sign * float("inf")
    return sign * float(v)


def _f32_cases(g, K, dt_x, dt_w, *, bias, seq, init, integer=False, B=2, C=3, L=11):
    def draw(*shape, dt):
        v = torch.randint(-8, 9, shape, generator=g).float() if integer else torch.randn(*shape, generator=g)
        return v.to(DT[dt])
    x = draw(B, C, L, dt=dt_x)
    w = draw(C, K, dt=dt_w)
    b = draw(C, dt=dt_w) if bias else None
    h = draw(B, C, K - 1, dt=dt_x) if init else None
    s = None
    if seq:
        ids = np.repeat(np.arange(4), [2, 1, 5, L - 8])
        s = torch.tensor(np.stack([ids, ids[::-1].copy()]), dtype=torch.int32)[:B]
    return x, w, b, s, h


def pin_f32_mode_exact_rational(ora):
    """The binary32 mode against an exact-rational emulation of its definition: each
    step is w*x + acc computed exactly and rounded once to binary32, bias first,
    k ascending, dropped terms skipped."""
    from fractions import Fraction
    g = _gen(19)
    for K in (2, 3, 4):
        for dt_x, dt_w in (("f32", "f32"), ("bf16", "bf16"), ("f16", "f32")):
            for bias, seq, init in ((True, False, True), (False, True, False), (True, True, False)):
                x, w, b, s, h = _f32_cases(g, K, dt_x, dt_w, bias=bias, seq=seq, init=init)
                got = _cf_case(ora, x, w, b, seq=s, init=h).fwd_f32()
                B, C, L = x.shape
                xe = torch.cat([h if h is not None else torch.zeros(B, C, K - 1, dtype=x.dtype), x], 2)
                xe = xe.double().numpy()
                wd = w.double().numpy()
                for bb in range(B):
                    for c in range(C):
                        for t in range(L):
                            acc = Fraction(float(b[c])) if b is not None else Fraction(0)
                            for k in range(K):
                                src = t - K + 1 + k
                                if s is not None and (src < 0 or int(s[bb, src]) != int(s[bb, t])):
                                    continue
                                acc = Fraction(_rne_f32(Fraction(float(wd[c, k])) * Fraction(float(xe[bb, c, src + K - 1])) + acc))
                            want = np.float32(float(acc))
                            assert got[bb, c, t].view(np.uint32) == want.view(np.uint32), (
                                K, dt_x, dt_w, bias, seq, init, bb, c, t, got[bb, c, t], want)


def pin_f32_mode_integers_are_exact(ora):
    """With small integer inputs every partial sum is an integer below 2^24, so the
    binary32 mode must equal the fp64 oracle exactly, in every layout, with and
    without history, mask and bias."""
    g = _gen(20)
    for K in (2, 3, 4):
        for dt in ("f32", "bf16", "f16"):
            for bias, seq, init in ((True, False, True), (False, True, False), (False, False, False)):
                x, w, b, s, h = _f32_cases(g, K, dt, dt, bias=bias, seq=seq, init=init, integer=True,
                                           C=5, L=37)
                case = _cf_case(ora, x, w, b, seq=s, init=h)
                z64, _ = case.fwd()
                z32 = case.fwd_f32()
                assert np.array_equal(z32.astype(np.float64), z64), (K, dt, bias, seq, init)
                # the same problem stored channel-last
                xl = x.transpose(1, 2).contiguous().transpose(1, 2)
                kw = {} if h is None else dict(init=_raw(h), init_strides=h.stride())
                cl = ora.Case(B=x.shape[0], C=x.shape[1], L=x.shape[2], K=K, x=_raw(xl.transpose(1, 2)),
                              x_dtype=dt, x_strides=xl.stride(), w=_raw(w), w_dtype=dt,
                              bias=None if b is None else _raw(b), seq=None if s is None else s.numpy(), **kw)
                assert np.array_equal(cl.fwd_f32(), z32), (K, dt, bias, seq, init)


def pin_f32_mode_error_bound(ora):
    """On random data the binary32 mode stays within K roundings of the fp64 result:
    |z32 - z64| <= K * 2^-24 * S, S = |bias| + sum of |kept terms|; and sampled
    points agree with the whole-array call."""
    g = _gen(21)
    for K in (2, 3, 4):
        for dt in ("f32", "bf16"):
            x, w, b, s, h = _f32_cases(g, K, dt, dt, bias=True, seq=False, init=True, C=8, L=300)
            case = _cf_case(ora, x, w, b, init=h)
            z64, sabs = case.fwd()
            z32 = case.fwd_f32().astype(np.float64)
            assert np.all(np.abs(z32 - z64) <= K * 2.0 ** -24 * sabs * (1 + 1e-6)), (K, dt)
            assert np.any(z32 != z64), "binary32 mode rounds nothing"
            idx = np.array([[1, 7, 299], [0, 0, 0], [1, 3, 150]])
            assert np.array_equal(case.points_f32(idx), case.fwd_f32()[idx[:, 0], idx[:, 1], idx[:, 2]])


def pin_points(ora):
    """The sampled entry (the fp64 values at a list of (b, c, t) triples, used for the
    large workloads) returns exactly what the whole-array call returns at those
    triples: y and sabs bit for bit, with seq_idx and a history, on a strided
    channel-last view of a wider buffer, for all three storage dtypes.  The triples
    are random plus every boundary (first and last step, batch, channel), and no
    dimension sizes agree, so a permuted index reads another output."""
    g = _gen(23)
    B, C, L, K = 3, 5, 37, 4
    for dt, wdt in (("f32", "f32"), ("bf16", "bf16"), ("f16", "f32")):
        x = torch.randn(B, L, C + 4, generator=g).to(DT[dt])          # [B, L, C + 4] parent
        w = (torch.randn(C, K, generator=g) * 0.5).to(DT[wdt])
        bias = torch.randn(C, generator=g).to(DT[wdt])
        init = torch.randn(B, C, K - 1, generator=g).to(DT[dt])
        seq = torch.tensor([[0] * 9 + [4] * 20 + [2] * 8, [1] * 37, [3] * 2 + [5] * 35],
                           dtype=torch.int32)
        case = ora.Case(B=B, C=C, L=L, K=K, x=_raw(x), x_off=2, x_dtype=dt,
                        x_strides=(L * (C + 4), 1, C + 4), w=_raw(w), w_dtype=wdt,
                        bias=_raw(bias), seq=seq.numpy(), init=_raw(init),
                        init_strides=init.stride(), silu=True)
        y, s = case.fwd()
        rng = np.random.default_rng(24)
        rand = np.stack([rng.integers(0, B, 200), rng.integers(0, C, 200),
                         rng.integers(0, L, 200)], 1)
        edge = np.array([[b, c, t] for b in (0, B - 1) for c in (0, C - 1)
                         for t in (0, 1, K - 2, K - 1, 8, 9, 28, 29, L - 1)])
        idx = np.concatenate([rand, edge])
        try:
            py, ps = case.points(idx)
        except IndexError:
            raise AssertionError(f"{dt}: an in-range index was refused")
        want_y = y[idx[:, 0], idx[:, 1], idx[:, 2]]
        want_s = s[idx[:, 0], idx[:, 1], idx[:, 2]]
        assert np.array_equal(py.view(np.uint64), want_y.view(np.uint64)), dt
        assert np.array_equal(ps.view(np.uint64), want_s.view(np.uint64)), dt
        for bad in ([B, 0, 0], [0, C, 0], [0, 0, L], [-1, 0, 0], [0, 0, -1]):
            try:
                case.points(np.array([bad]))
            except IndexError:
                continue
            raise AssertionError(f"index {bad} out of range was accepted")


# ---- backward -------------------------------------------------------------------------

def _bwd(ora, x, w, b=None, seq=None, init=None, silu=False, dout=None, dfs=None):
    from oracle.from_torch import bwd
    c = _cf_case(ora, x, w, b, seq=seq, init=init, silu=silu)
    return bwd(c, dout, dfs)


def _autograd(x, w, b, init, silu, dout, dfs):
    """torch autograd in fp64 through grouped conv1d on the history-extended input."""
    K = w.shape[1]
    xd = x.double().requires_grad_()
    wd = w.double().requires_grad_()
    bd = None if b is None else b.double().requires_grad_()
    hd = (init.double() if init is not None else torch.zeros(x.shape[0], x.shape[1], K - 1,
                                                             dtype=torch.float64)).requires_grad_()
    xt = torch.cat([hd, xd], 2)
    z = torch.nn.functional.conv1d(xt, wd[:, None, :], bd, groups=x.shape[1])
    y = torch.nn.functional.silu(z) if silu else z
    loss = (y * dout.double()).sum()
    if dfs is not None:
        loss = loss + (xt[:, :, xt.shape[2] - (K - 1):] * dfs.double()).sum()
    loss.backward()
    return dict(dx=xd.grad, dw=wd.grad, db=None if b is None else bd.grad,
                dinit=hd.grad if init is not None else None)


def pin_bwd_autograd(ora):
    """Every gradient against torch autograd (fp64, CPU), all K, storage dtypes, with
    and without bias, history, dfinal_states and SiLU, including L < K-1."""
    g = _gen(22)
    for K in (2, 3, 4):
        for dt, wdt in (("f32", "f32"), ("bf16", "bf16"), ("f16", "f32")):
            for L, bias, init, dfs_on, silu in ((13, True, True, True, True), (9, False, False, False, False),
                                                (max(1, K - 2), True, True, True, True), (1, True, False, True, True)):
                B, C = 2, 3
                x = torch.randn(B, C, L, generator=g).to(DT[dt])
                w = (torch.randn(C, K, generator=g) * 0.5).to(DT[wdt])
                b = torch.randn(C, generator=g).to(DT[wdt]) if bias else None
                h = torch.randn(B, C, K - 1, generator=g).to(DT[dt]) if init else None
                dout = torch.randn(B, C, L, generator=g).to(DT[dt])
                dfs = torch.randn(B, C, K - 1, generator=g).to(DT[dt]) if dfs_on else None
                r = _bwd(ora, x, w, b, init=h, silu=silu, dout=dout, dfs=dfs)
                ref = _autograd(x, w, b, h, silu, dout, dfs)
                for name in ("dx", "dw", "db", "dinit"):
                    if ref[name] is None:
                        continue
                    want = ref[name].numpy()
                    scale = np.maximum(np.abs(want), 1.0)
                    assert np.all(np.abs(r[name] - want) <= 1e-12 * scale), (K, dt, L, name)


def _loss(ora, x, w, b, seq, init, silu, dout, dfs):
    c = _cf_case(ora, x, w, b, seq=seq, init=init, silu=silu)
    y, _ = c.fwd(want_sabs=False)
    loss = float(np.sum(y * dout.double().numpy()))
    if dfs is not None:                       # the oracle's final states (fp32 storage)
        loss += float(np.sum(c.final_states().astype(np.float64) * dfs.double().numpy()))
    return loss


def pin_bwd_finite_differences(ora):
    """Central differences of the forward oracle's loss sum(dout * y) + sum(dfs * fs)
    on dyadic data (so x +- h is exact in fp32): every gradient entry, with a
    seq_idx mask and with history."""
    g = _gen(23)
    h = 2.0 ** -10

    def dyadic(*shape):
        return torch.randint(-256, 257, shape, generator=g).float() / 128.0

    for K, L, seq, init in ((3, 9, [0, 0, 0, 1, 1, 2, 2, 2, 2], False), (4, 7, None, True),
                            (4, 8, [5, 5, 6, 6, 6, 6, 6, 7], True), (3, 5, [1, 1, 1, 1, 1], True)):
        B, C = 1, 2
        x, w, b = dyadic(B, C, L), dyadic(C, K) / 2, dyadic(C)
        hist = dyadic(B, C, K - 1) if init else None
        s = None if seq is None else torch.tensor([seq], dtype=torch.int32)
        dout = dyadic(B, C, L)
        dfs = dyadic(B, C, K - 1) if init else None
        r = _bwd(ora, x, w, b, seq=s, init=hist, silu=True, dout=dout, dfs=dfs)
        params = {"dx": x, "dw": w, "db": b}
        if init:
            params["dinit"] = hist
        for name, t in params.items():
            flat = t.view(-1)
            for i in range(flat.numel()):
                v = float(flat[i])
                flat[i] = v + h
                up = _loss(ora, x, w, b, s, hist, True, dout, dfs)
                flat[i] = v - h
                dn = _loss(ora, x, w, b, s, hist, True, dout, dfs)
                flat[i] = v
                fd = (up - dn) / (2 * h)
                got = r[name].reshape(-1)[i]
                assert abs(got - fd) <= 1e-4 * max(1.0, abs(fd)), (name, i, got, fd)


def pin_bwd_packing(ora):
    """A packed backward with seq_idx equals separate backward runs of each sequence:
    dx bit for bit (the same terms in the same order), dw and db as the sums."""
    g = _gen(24)
    for K in (2, 3, 4):
        lengths = [1, 5, K - 1, 9, 2, 13, K]
        L, C = sum(lengths), 3
        x = torch.randn(1, C, L, generator=g)
        w = torch.randn(C, K, generator=g) * 0.5
        b = torch.randn(C, generator=g)
        dout = torch.randn(1, C, L, generator=g)
        seq = torch.tensor(np.repeat(np.arange(len(lengths)), lengths), dtype=torch.int32).reshape(1, L)
        r = _bwd(ora, x, w, b, seq=seq, silu=True, dout=dout)
        pos, dw, db = 0, 0.0, 0.0
        for n in lengths:
            part = _bwd(ora, x[:, :, pos:pos + n].contiguous(), w, b, silu=True,
                        dout=dout[:, :, pos:pos + n].contiguous())
            assert np.array_equal(r["dx"][:, :, pos:pos + n], part["dx"]), (K, n)
            dw, db = dw + part["dw"], db + part["db"]
            pos += n
        assert np.allclose(r["dw"], dw, rtol=1e-13, atol=1e-13), K
        assert np.allclose(r["db"], db, rtol=1e-13, atol=1e-13), K


def pin_bwd_chunking(ora):
    """The backward of [x1 | x2] equals chunk 2's backward (history = chunk 1's final
    states) followed by chunk 1's backward with dfinal_states = chunk 2's
    d(initial_states): dx, d(initial_states) and the summed dw, db.  Dyadic data and
    no activation keep every sum exact, so the comparison is exact too (the
    d(initial_states) handed between chunks is stored in fp32)."""
    g = _gen(25)

    def dyadic(*shape):
        return torch.randint(-64, 65, shape, generator=g).float() / 32.0

    for K in (2, 3, 4):
        B, C, L = 2, 3, 30
        x, w, b = dyadic(B, C, L), dyadic(C, K), dyadic(C)
        h, dout, dfs = dyadic(B, C, K - 1), dyadic(B, C, L), dyadic(B, C, K - 1)
        ids = np.repeat(np.arange(4), [5, 9, 1, 15])
        for seq in (None, torch.tensor(np.stack([ids, ids[::-1] + 7]), dtype=torch.int32)):
            full = _bwd(ora, x, w, b, seq=seq, init=h, dout=dout, dfs=dfs)
            for L1 in sorted({1, K - 2, K - 1, K, 5, 14, 15, 17} - {0}):
                x1, x2 = x[:, :, :L1].contiguous(), x[:, :, L1:].contiguous()
                s1 = None if seq is None else seq[:, :L1].contiguous()
                s2 = None if seq is None else seq[:, L1:].contiguous()
                # chunk 2's history: chunk 1's final states, or zeros where a sequence starts at L1
                cont = torch.ones(B, 1, 1, dtype=torch.bool) if seq is None else \
                    (seq[:, L1] == seq[:, L1 - 1]).reshape(B, 1, 1)
                f1 = torch.from_numpy(_cf_case(ora, x1, w, b, seq=s1, init=h).final_states().copy())
                f1 = torch.where(cont, f1, torch.zeros_like(f1))
                r2 = _bwd(ora, x2, w, b, seq=s2, init=f1, dout=dout[:, :, L1:].contiguous(), dfs=dfs)
                d2 = torch.from_numpy(r2["dinit"]).float()
                assert np.array_equal(d2.double().numpy(), r2["dinit"])       # exact in fp32
                d2 = torch.where(cont, d2, torch.zeros_like(d2))
                r1 = _bwd(ora, x1, w, b, seq=s1, init=h, dout=dout[:, :, :L1].contiguous(), dfs=d2)
                where = (K, L1, seq is not None)
                assert np.array_equal(np.concatenate([r1["dx"], r2["dx"]], 2), full["dx"]), where
                assert np.array_equal(r1["dinit"], full["dinit"]), where
                assert np.array_equal(r1["dw"] + r2["dw"], full["dw"]), where
                assert np.array_equal(r1["db"] + r2["db"], full["db"]), where


ALL_PINS = [pin_golden, pin_digits, pin_one_hot, pin_delta, pin_constant, pin_conv1d,
            pin_chunking, pin_packing, pin_mask_nan, pin_layout, pin_silu, pin_converters,
            pin_round_out, pin_f32_mode_exact_rational, pin_f32_mode_integers_are_exact,
            pin_f32_mode_error_bound, pin_bwd_autograd, pin_bwd_finite_differences, pin_bwd_packing,
            pin_bwd_chunking, pin_packed_chunking, pin_points]
