"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that the
pins catch every one of them.  Each mutant is the oracle's C source with one
textual change, compiled with the same gcc line into a temporary directory.

A mutant runs the pins in an interpreter of its own: some mistakes (a swapped
stride) read outside the input arrays, which may read garbage (a pin fails) or
may leave the process's memory altogether; a mutant whose run dies that way is
caught too, and cannot take the test session down with it."""
import os
import subprocess
import sys

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "ccv_oracle.c")

# (name, original text, mutated text)
MUTANTS = [
    ("taps_reversed", "double term = ora_decode(p->w, p->w_dtype, c * K + k)",
     "double term = ora_decode(p->w, p->w_dtype, c * K + (K - 1 - k))"),
    ("source_off_by_one", "int64_t src = t - K + 1 + k;              /*", "int64_t src = t - K + k;              /*"),
    ("oldest_tap_dropped", "for (int k = 0; k < K; ++k) {\n    int64_t src = t - K + 1 + k;              /*",
     "for (int k = 1; k < K; ++k) {\n    int64_t src = t - K + 1 + k;              /*"),
    ("silu_sign", "acc / (1.0 + exp(-acc))", "acc / (1.0 + exp(acc))"),
    ("silu_missing_z", "out = acc / (1.0 + exp(-acc));", "out = 1.0 / (1.0 + exp(-acc));"),
    ("bias_dropped", "acc = beta;", "acc = 0.0;"),
    ("history_reversed", "int64_t i = j + p->K - 1;\n  return", "int64_t i = -j - 1;\n  return"),
    ("mask_never", "return id == p->seq[b * p->L + t];", "return id == id;"),
    ("mask_multiplies",
     "if (!ora_keep(p, b, t, k)) continue;      /* dropped */",
     "if (!ora_keep(p, b, t, k)) { acc += 0.0 * ora_xt(p, b, c, src); continue; }"),
    ("final_off_by_one", "int64_t j = p->L - K + 1 + i;", "int64_t j = p->L - K + i;"),
    ("f16_exponent_bias", "ldexp((double)(1024 + m), e - 25)", "ldexp((double)(1024 + m), e - 24)"),
    ("bf16_ties_away", "(lower == 0x8000u && (upper & 1u))", "(lower == 0x8000u)"),
    ("rne_ties_down", "return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl;"),
    ("sabs_signed", "s += fabs(term);", "s += term;"),
    ("x_stride_swapped", "b * p->xs[0] + c * p->xs[1] + j * p->xs[2]);\n  if (p->init", "b * p->xs[0] + c * p->xs[2] + j * p->xs[1]);\n  if (p->init"),
    ("init_zero", "if (p->init == NULL) return 0.0;", "return 0.0;"),
    # the diagnostic binary32 mode
    ("f32_two_roundings", "acc = fmaf(wv, xv, acc);", "acc = acc + wv * xv;"),
    ("f32_k_descending", "for (int k = 0; k < K; ++k) {\n    int64_t src = t - K + 1 + k;\n",
     "for (int kk = 0; kk < K; ++kk) {\n    int k = K - 1 - kk;\n    int64_t src = t - K + 1 + k;\n"),
    ("f32_bias_dropped", "if (p->bias != NULL) acc = (float)ora_decode(p->bias, p->w_dtype, c);", ""),
    ("f32_taps_reversed", "float wv = (float)ora_decode(p->w, p->w_dtype, c * K + k);",
     "float wv = (float)ora_decode(p->w, p->w_dtype, c * K + (K - 1 - k));"),
    # seq_idx together with states
    ("history_id_of_last_sequence", "*id = p->seq[b * p->L];", "*id = p->seq[b * p->L + p->L - 1];"),
    ("history_never_counts_with_seq", "if (p->init == NULL || p->L == 0) return 0;", "return 0;"),
    ("final_states_not_masked", "if (p->seq == NULL || p->L == 0) return 1;", "return 1;"),
    # the sampled entry
    ("points_index_order", "ora_point(p, idx[3 * i], idx[3 * i + 1], idx[3 * i + 2], &yy, NULL, &ss)",
     "ora_point(p, idx[3 * i + 1], idx[3 * i], idx[3 * i + 2], &yy, NULL, &ss)"),
    ("points_time_channel_swapped", "ora_point(p, idx[3 * i], idx[3 * i + 1], idx[3 * i + 2], &yy, NULL, &ss)",
     "ora_point(p, idx[3 * i], idx[3 * i + 2], idx[3 * i + 1], &yy, NULL, &ss)"),
    ("points_sabs_as_y", "if (y) y[i] = yy;", "if (y) y[i] = ss;"),
    # the backward
    ("bwd_no_activation_slope", "dz[t] = go * slope;", "dz[t] = go;"),
    ("bwd_slope_sign", "slope = s * (1.0 + z * (1.0 - s));", "slope = s * (1.0 - z * (1.0 - s));"),
    ("bwd_dx_taps_reversed", "int64_t t = j + K - 1 - k;", "int64_t t = j + k;"),
    ("bwd_dx_mask_ignored", "if (t < 0 || t >= L || !ora_keep(p, b, t, k)) continue;",
     "if (t < 0 || t >= L) continue;"),
    ("bwd_dfinal_ignored", "acc += v;", "acc += 0.0 * v;"),
    ("bwd_dfinal_reversed", "int64_t i = j - (L - H);", "int64_t i = (H - 1) - (j - (L - H));"),
    ("bwd_dinit_reversed", "int64_t o = (b * C + c) * H + (j + H);",
     "int64_t o = (b * C + c) * H + (H - 1 - (j + H));"),
    ("bwd_dw_mask_ignored", "if (!ora_keep(p, b, t, k)) continue;\n          double xv",
     "double xv"),
    ("bwd_db_halved", "if (db) db[c] += dz[t];", "if (db) db[c] += 0.5 * dz[t];"),
]


def _build(tmp_path, name, src_text):
    c = tmp_path / f"{name}.c"
    c.write_text(src_text)
    so = tmp_path / f"lib{name}.so"
    hdr_dir = os.path.dirname(SRC)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-std=c11", "-fPIC", "-shared", "-w",
                    "-I", hdr_dir, "-o", str(so), str(c), "-lm"], check=True)
    return str(so)


def test_unmutated_copy_passes(tmp_path):
    so = _build(tmp_path, "clean", open(SRC).read())
    with oracle.using_library(so):
        for pin in ALL_PINS:
            pin(oracle)


_TESTS = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_TESTS)
_RUN_PINS = """
import sys
sys.path[:0] = [{tests!r}, {root!r}]
import oracle
from oracle_pins import ALL_PINS
caught = []
with oracle.using_library({so!r}):
    for pin in ALL_PINS:
        try:
            pin(oracle)
        except AssertionError:
            caught.append(pin.__name__)
            break                                  # one catch is enough
print("CAUGHT:" + ",".join(caught))
"""


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not unique"
    so = _build(tmp_path, name, text.replace(old, new))
    r = subprocess.run([sys.executable, "-c", _RUN_PINS.format(tests=_TESTS, root=_ROOT, so=so)],
                       capture_output=True, text=True, timeout=900)
    if r.returncode < 0:
        return                                     # the mutant's run died on a signal: caught
    assert r.returncode == 0, r.stderr[-2000:]     # any other error is the harness's, not a catch
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("CAUGHT:")]
    assert lines and lines[-1] != "CAUGHT:", f"no pin caught mutant {name}"
