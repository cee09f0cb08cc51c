"""The oracle's pins catch plausible mistakes.  CPU only.

Each case plants one mistake in a copy of the oracle's C source (a dropped
term, a wrong sign or index, a wrong order, a wrong rounding), builds that copy
into a temporary library and runs the pin tests against it in a subprocess:
the pins must fail.  Nothing here touches the real oracle library.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "lq_oracle.c")
PINS = ["tests/test_oracle_recurrence.py", "tests/test_oracle_quantizer.py",
        "tests/test_oracle_window.py", "tests/test_oracle_fp8.py", "tests/test_oracle_fp16_buffer.py"]

MUTANTS = {
    "delta_sign": ("S[(size_t)i * dk + j] - (double)beta * Mk[i]", "S[(size_t)i * dk + j] + (double)beta * Mk[i]"),
    "injection_without_beta": ("(double)beta * (double)v[i] * (double)k[j]", "(double)v[i] * (double)k[j]"),
    "gate_dropped": ("S[(size_t)i * dk + j] *= gj;", "S[(size_t)i * dk + j] *= 1.0;"),
    "output_uses_key": ("acc += S[(size_t)i * dk + j] * (double)q[j];", "acc += S[(size_t)i * dk + j] * (double)k[j];"),
    "score_l1": ("a += Su[(size_t)i * dk + j] * Su[(size_t)i * dk + j];", "a += fabs(Su[(size_t)i * dk + j]);"),
    "tie_to_higher_index": ("score[c] > score[best]", "score[c] >= score[best]"),
    "smoothing_without_sqrt": ("s = (float)sqrt(a);", "s = (float)a;"),
    "scale_divisor": ("ORC_FMT_E4M3 ? 448.0 : 127.0", "ORC_FMT_E4M3 ? 448.0 : 128.0"),
    "e4m3_scale_divisor": ("ORC_FMT_E4M3 ? 448.0 : 127.0", "ORC_FMT_E4M3 ? 240.0 : 127.0"),
    "e4m3_exponent_bias": ("ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)"),
    "e4m3_subnormal_scale": ("ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)"),
    "e4m3_ties_away": ("nearbyint(ldexp(a, 3 - E))", "round(ldexp(a, 3 - E))"),
    "e4m3_no_subnormal_floor": ("if (E < -6) E = -6;", "if (E < -9) E = -9;"),
    "e4m3_carry_dropped": ("e = E + 8;", "e = E + 7;"),
    "fp16_ties_away": ("nearbyint(ldexp(a, 10 - E))", "round(ldexp(a, 10 - E))"),
    "fp16_nine_mantissa_bits": ("ldexp(nearbyint(ldexp(a, 10 - E)), E - 10)", "ldexp(nearbyint(ldexp(a, 9 - E)), E - 9)"),
    "fp16_no_subnormal_floor": ("if (E < -14) E = -14;", "if (E < -24) E = -24;"),
    "fp16_no_saturation": ("if (a > 65504.0) a = 65504.0;", "if (a > 65536.0) a = 65536.0;"),
    "fp16_buffer_keeps_raw_v": ("vt = vr;", "vt = vt;"),
    "ties_away_from_zero": ("double c = nearbyint(x);", "double c = round(x);"),
    "column_slot_unmasked": ("row_sel[i] ? 0.0f : (float)Su", "0 ? 0.0f : (float)Su"),
    "replay_forward_order": ("for (int i = n_ent - 1; i >= 0; --i)", "for (int i = 0; i < n_ent; ++i)"),
    "replay_gate_dropped": ("r[j] = gj * (r[j] - b * c * (double)ki[j]);", "r[j] = (r[j] - b * c * (double)ki[j]);"),
    "replay_acc_without_beta": ("acc[e] += b * c * (double)vi[e];", "acc[e] += c * (double)vi[e];"),
    "row_slot_to_column": ("for (int j = 0; j < dk; ++j) Su[(size_t)c * dk + j] += (double)cv[j];",
                           "for (int j = 0; j < dk && j < dv; ++j) Su[(size_t)j * dk + c] += (double)cv[j];"),
    "flush_one_early": ("if (fill == W || forced)", "if (fill == W - 1 || forced)"),
    "smoothing_switch_ignored": ("if (smooth_enable && a > 0.0)", "if (a > 0.0)"),
    "smoothing_switch_inverted": ("if (smooth_enable && a > 0.0)", "if (!smooth_enable && a > 0.0)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_fail_on_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    mutated = src.replace(old, new, 1)
    csrc = tmp_path / "mutant.c"
    csrc.write_text(mutated)
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(csrc), "-o",
                    str(lib), "-lm"], check=True)
    env = dict(os.environ, LQ_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"pins passed with mutant {name}:\n{r.stdout[-2000:]}"


def test_control_unmutated_copy_passes(tmp_path):
    # the same harness with the source unchanged must pass, so the failures
    # above come from the planted mistakes and not from the harness
    csrc = tmp_path / "control.c"
    csrc.write_text(open(SRC).read())
    lib = tmp_path / "libcontrol.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(csrc), "-o",
                    str(lib), "-lm"], check=True)
    env = dict(os.environ, LQ_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:]
