"""The oracle against its pins (CPU only): hand-worked examples, closed forms,
torch's fp64 conv1d, invariants, SiLU and dtype conversions."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(ora, pin):
    pin(ora)


def test_converters_1e8_random_patterns(ora):
    """RNE encoding of fp32 to bf16 and fp16 against torch on 10^8 random fp32 bit
    patterns per format (every exponent, subnormals, infinities, NaNs), in chunks."""
    import numpy as np
    import torch

    g = np.random.default_rng(19)
    n_chunk, chunks = 10_000_000, 10
    for _ in range(chunks):
        vals = g.integers(0, 2**32, n_chunk, dtype=np.uint64).astype(np.uint32).view(np.float32)
        tv = torch.from_numpy(vals)
        for dt, tdt, fn in (("bf16", torch.bfloat16, ora.f32_to_bf16), ("f16", torch.float16, ora.f32_to_f16)):
            ref_t = tv.to(tdt)
            ref = ref_t.view(torch.int16).numpy().view(np.uint16)
            got = fn(vals)
            rnan = torch.isnan(ref_t).numpy()
            gnan = np.isnan(ora.decode(dt, got))
            assert np.array_equal(rnan, gnan), dt
            assert np.array_equal(got[~rnan], ref[~rnan]), dt


def test_threaded_oracle_is_bit_identical(ora):
    """ora_fwd_threads (the same per-output loop on several host threads, used to time
    the oracle on all cores) returns the single-threaded outputs bit for bit."""
    import numpy as np
    import torch

    from oracle_pins import _cf_case

    g = torch.Generator().manual_seed(20)
    B, C, L, K = 3, 11, 97, 4
    x = torch.randn(B, C, L, generator=g).to(torch.bfloat16)
    w = torch.randn(C, K, generator=g).to(torch.float32)
    bias = torch.randn(C, generator=g)
    init = torch.randn(B, C, K - 1, generator=g).to(torch.bfloat16)
    seq = torch.tensor([[0] * 40 + [1] * 30 + [2] * 27] * B, dtype=torch.int32)
    c = _cf_case(ora, x, w, bias, seq=seq, init=init, silu=True)
    y1, s1 = c.fwd()
    for n in (1, 2, 3, 7, 33, 64):
        yn, sn = c.fwd_threads(n)
        assert np.array_equal(yn.view(np.uint64), y1.view(np.uint64)), n
        assert np.array_equal(sn.view(np.uint64), s1.view(np.uint64)), n
