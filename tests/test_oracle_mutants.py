"""Plant plausible mistakes in copies of the oracle (on the CPU only) and
check that the pins catch every one of them: a pin set that a wrong oracle
also passes would prove nothing."""
import os
import subprocess
import sys

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "nm_oracle.c")

# The ranking helpers of the saliency keep-mask and the hybrid row choice, as
# they stand in nm_oracle.c (replaced whole by the NaN-placement mutants).
RANK_HELPERS = "static int rank_above(double a, double b)\n{\n    if (isnan(a))\n        return 0;\n    return isnan(b) || a > b;\n}\n\nstatic int rank_equal(double a, double b)\n{\n    if (isnan(a) || isnan(b))\n        return isnan(a) && isnan(b);\n    return a == b;\n}"

# (name, text in nm_oracle.c, replacement) -- each is a mistake someone could make.
MUTANTS = [
    ("tie_goes_to_highest_index", "mag[j] > mag[best]", "mag[j] >= mag[best]"),
    ("bitmap_msb_first", "mrow[c / 8] |= (uint8_t)(1u << (c % 8));", "mrow[c / 8] |= (uint8_t)(0x80u >> (c % 8));"),
    ("group_step_assumes_half", "int64_t next = g * N;", "int64_t next = g * M / 2;"),
    ("values_descending_in_expand", "Wt[r * K + c] = values[r * vrow + g * N + k];",
     "Wt[r * K + c] = values[r * vrow + g * N + (N - 1 - k)];"),
    ("last_column_dropped", "for (int64_t c = 0; c < K; ++c) {\n            double p", "for (int64_t c = 0; c + 1 < K; ++c) {\n            double p"),
    ("abs_sum_signed", "sa += fabs(p);", "sa += p;"),
    ("x_transposed", "orc_to_double(x[b * K + c], dtype)", "orc_to_double(x[c * B + b], dtype)"),
    ("ties_away_from_zero", "(r == 0.5 && fmod(n, 2.0) != 0.0)", "(r == 0.5)"),
    ("fp16_subnormal_scale", "v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    ("bf16_exponent_bias", "v = ldexp((double)(128 + f), e - 134);", "v = ldexp((double)(128 + f), e - 133);"),
    ("keep_count_not_checked", "return count == N ? ORC_OK : ORC_BAD_MASK;", "return ORC_OK;"),
    ("nan_not_rejected", "if (isnan(v))\n            return ORC_NONFINITE;", "if (0)\n            return ORC_NONFINITE;"),
    ("signed_magnitude", "mag[j] = fabs(v);", "mag[j] = v;"),
    ("overflow_not_detected", "if (q + fbits > emax)", "if (q + fbits > emax + 1)"),
    ("silu_sign_flipped", "return t / (1.0 + exp(-t));", "return t / (1.0 + exp(t));"),
    ("silu_is_sigmoid", "return t / (1.0 + exp(-t));", "return 1.0 / (1.0 + exp(-t));"),
    ("swiglu_gate_up_swapped", "h[i] = orc_silu(g[i]) * u[i];", "h[i] = orc_silu(u[i]) * g[i];"),
    ("calib_prefill_not_excluded", "if (decode && !decode[t])", "if (0 && decode && !decode[t])"),
    ("calib_diagonal_only", "double p = row[i] * row[j];", "double p = row[i] * row[i];"),
    ("saliency_abs_w", "double s = w * w * h[c];", "double s = fabs(w) * h[c];"),
    ("saliency_ignores_h", "double s = w * w * h[c];", "double s = w * w;"),
    ("saliency_tie_to_highest", "(best < 0 || rank_above(sal[j], sal[best]))", "(best < 0 || !rank_above(sal[best], sal[j]))"),
    # NaN placed elsewhere in the ranking order: above every number, at -1, and
    # equal to -inf (the reading not taken: NaN then ties with -inf)
    ("nan_ranks_high", "        return 0;\n    return isnan(b) || a > b;", "        return !isnan(b);\n    return a > b;"),
    ("nan_at_minus_one", RANK_HELPERS, "static int rank_above(double a, double b)\n{\n    return (isnan(a) ? -1.0 : a) > (isnan(b) ? -1.0 : b);\n}\n\nstatic int rank_equal(double a, double b)\n{\n    return (isnan(a) ? -1.0 : a) == (isnan(b) ? -1.0 : b);\n}"),
    ("nan_equals_minus_inf", RANK_HELPERS, "static int rank_above(double a, double b)\n{\n    return (isnan(a) ? -INFINITY : a) > (isnan(b) ? -INFINITY : b);\n}\n\nstatic int rank_equal(double a, double b)\n{\n    return (isnan(a) ? -INFINITY : a) == (isnan(b) ? -INFINITY : b);\n}"),
    ("hybrid_loss_counts_kept", "                if (chosen[j])\n                    continue;\n                double v",
     "                if (!chosen[j])\n                    continue;\n                double v"),
    ("hybrid_loss_ignores_h", "double hv = h ? h[g * M + j] : 1.0;", "double hv = 1.0;"),
    ("hybrid_select_ascending", "if (rank_above(loss[s], loss[r]) ||", "if (rank_above(loss[r], loss[s]) ||"),
    ("hybrid_select_ties_to_higher", "(rank_equal(loss[s], loss[r]) && s < r)", "(rank_equal(loss[s], loss[r]) && s > r)"),
]


def _failing_pins():
    failures = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except Exception as e:                      # noqa: BLE001 -- any failure counts as caught
            failures.append((getattr(pin, "__name__", "?"), type(e).__name__))
    return failures


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not unique/found"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-ffp-contract=off", str(src), "-o", str(lib), "-lm"],
                   check=True)
    # The pins run in a child process: a planted out-of-bounds write may abort
    # it, which also counts as caught.
    code = ("import sys, oracle, test_oracle_mutants as t; oracle.use_library(sys.argv[1]); "
            "f = t._failing_pins(); print(f); sys.exit(1 if f else 0)")
    tests_dir = os.path.dirname(os.path.abspath(__file__))
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([os.path.dirname(tests_dir), tests_dir]))
    proc = subprocess.run([sys.executable, "-c", code, str(lib)], env=env, capture_output=True, text=True, timeout=300)
    assert proc.returncode != 0, f"planted mistake {name} passed every pin"


def test_real_oracle_passes_every_pin():
    assert _failing_pins() == []
