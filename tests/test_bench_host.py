"""The bench's accounting on the CPU: algorithmic bytes per call, the profile
lookup that feeds roofline.traffic, and the one-GPU refusal.

The byte totals of the five forward workloads are fixed by their definitions
(x read once, out written once, weight, bias, seq_idx and the states once):

    [1,64,2048] fp32, bias                                   1,049,856
    [4,2048,4096] bf16, bias                               134,238,208
    [8,4096,8192] bf16 view, no bias, initial + final      1,074,167,808
    [1,2560,65536] fp16, bias, seq_idx                       671,376,384
    [2,128,1048576] fp32 K=3, no bias, initial + final   2,147,489,280

Building a workload at full length is too slow for the CPU suite, so each is
built at two short lengths; the accounting is affine in L, and the line through
the two points is extended to the full length and compared with the total."""
import subprocess
import sys

import pytest

import bench
import workloads as wl

TOTALS = {1: (2048, 1_049_856), 2: (4096, 134_238_208), 3: (8192, 1_074_167_808),
          4: (65536, 671_376_384), 5: (1_048_576, 2_147_489_280)}


@pytest.mark.parametrize("i", sorted(TOTALS))
def test_forward_bytes_match_the_workload_totals(i):
    L_full, total = TOTALS[i]
    # workload 4 draws its 64 packed sequences only from 4096 steps on
    L1, L2 = (4096, 8192) if i == 4 else (64, 128)
    b1 = bench.algorithmic_bytes(wl.workload(i, L_override=L1))
    b2 = bench.algorithmic_bytes(wl.workload(i, L_override=L2))
    per_step = (b2 - b1) // (L2 - L1)
    assert per_step * (L2 - L1) == b2 - b1
    assert b1 + per_step * (L_full - L1) == total


def test_backward_bytes_of_the_bf16_shape():
    # x and dout read once, dx written once (3 x 2 B per element), weight and bias
    # read once and their gradients written once (2 x 2 B per parameter)
    w = wl.workload(2, L_override=64)
    assert bench.bwd_bytes(w) == 3 * 4 * 2048 * 64 * 2 + 2 * 2048 * 4 * 2 + 2 * 2048 * 2


def test_update_bytes_of_the_decode_case():
    # x, out (one step each) and the state read and written: (2 + 2 x 3) x 2 B per row,
    # plus the weights
    w = wl.decode_workload()
    assert bench.update_bytes(w) == 256 * 4096 * (2 + 2 * 3) * 2 + 4096 * 4 * 2 == 16_809_984


def test_profile_traffic_needs_the_current_sources(tmp_path, monkeypatch):
    """roofline.traffic comes from a committed counters summary only while the
    kernel sources hash to the value the summary records."""
    sha, other = "ab" * 32, "cd" * 32
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "k_counters.md").write_text(f"```\ntraffic_bytes_per_launch: 1234\nkernel_sources_sha256: {sha}\n```\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profile_traffic("k", sha) == 1234
    assert bench.profile_traffic("k", other) is None
    assert bench.profile_traffic("missing", sha) is None


def test_profile_kernel_time_needs_the_current_sources(tmp_path, monkeypatch):
    """The kernel-trace figure beside the HIP-event ones comes from a committed
    trace summary only while the kernel sources hash to the value it records."""
    sha, other = "ab" * 32, "cd" * 32
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "k_trace.md").write_text(f"```\nkernel_avg_us: 25.0\nkernel_sources_sha256: {sha}\n```\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    got = bench.profile_kernel_time("k", sha, 200_000_000)
    assert got["us"] == 25.0 and got["GBps"] == 8000.0 and got["frac"] == 1.0
    assert bench.profile_kernel_time("k", other, 1) is None
    assert bench.profile_kernel_time("missing", sha, 1) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0 and "one GPU" in r.stdout + r.stderr


@pytest.mark.parametrize("i", [1, 3, 5])
def test_oracle_pieces_cover_every_row_once(i):
    import numpy as np
    w = wl.workload(i, L_override=4096 if i != 1 else None)
    seen = np.zeros((w.B, w.C), dtype=int)
    for b, c0, c1 in bench.oracle_pieces(w, 1 << 16):
        assert c1 > c0 and (c1 - c0) * w.L <= max(1 << 16, w.L)
        seen[b, c0:c1] += 1
    assert (seen == 1).all()


def test_oracle_leg_accounting_on_the_small_workload():
    """The oracle leg on a result that is the oracle's own rounded output: every
    output counted once, none out of tolerance, all bit-equal, and the one-thread
    sample scaled to the whole workload's bytes."""
    import torch

    from oracle import round_out
    from oracle.from_torch import case
    w = wl.workload(1)
    y, _ = case(w.x, w.weight, w.bias, w.seq_idx, w.initial_states, w.activation).fwd()
    out = torch.from_numpy(round_out("f32", y))
    r = bench.oracle_leg(w, out, None, bench.algorithmic_bytes(w), 0.01)
    p = r["parity"]
    assert p["outputs"] == p["bit_equal"] == 64 * 2048 and p["out_of_tolerance"] == 0
    assert r["one_thread"]["cores"] == 1 and "2048" in r["one_thread"]["sample"]
    assert r["all_cores"]["first_piece_bit_identical_to_one_thread"]
