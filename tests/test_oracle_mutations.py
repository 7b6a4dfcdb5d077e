"""Planted mistakes: each plausible slip in the oracle (a flipped tie rule, a
wrong summation order, a dropped rounding point, a transposed operand, a
swapped nibble, ...) is compiled into a throw-away copy of the oracle on the
CPU, and the pin suite must fail against it.  Shows the pins pin."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTANTS = {
    "ties_to_higher_id": ("(best < 0 || l[e] > l[best])", "(best < 0 || l[e] >= l[best])"),
    "reversed_tree": ("for (int step = 32; step >= 1; step >>= 1)", "for (int step = 1; step <= 32; step <<= 1)"),
    "silu_sign": ("g / (1.0 + exp(-g))", "g / (1.0 + exp(g))"),
    "no_bf16_rounding_of_a": ("if (round_a_bf16) a[f]", "if (0) a[f]"),
    "transposed_down": ("weight_value(wd, sd, w_dt, e, H, F, h, f)", "weight_value(wd, sd, w_dt, e, F, H, f, h)"),
    "swapped_nibbles": ("((c & 1) ? (byte >> 4) : (byte & 15))", "((c & 1) ? (byte & 15) : (byte >> 4))"),
    "softmax_without_max": ("exp((double)l[id[k]] - m) / s", "exp((double)l[id[k]]) / s"),
    "rank_ties_to_higher_id": ("(c[f] == c[e] && f < e)", "(c[f] == c[e] && f > e)"),
    "unstable_permutation": ("for (int64_t s = 0; s < n; s++) {           /* ascending",
                             "for (int64_t s = n - 1; s >= 0; s--) {           /* ascending"),
    "dropped_residual": ("acc[h] + (res ?", "acc[h] + (0 ?"),
    "bias_ignored": ("if (bias) l = l + bias[e];", ";"),
    "up_used_twice": ("u += xv * weight_value(wu, su,", "u += xv * weight_value(wg, sg,"),
    "int2_byte_and_pair_swapped": ("int u = (row[word * 4 + j] >> (2 * k)) & 3;", "int u = (row[word * 4 + k] >> (2 * j)) & 3;"),
    "int3_third_bit_order": ("(third[word3 * 4 + j3] >> (4 * g + k3)) & 1", "(third[word3 * 4 + j3] >> (4 * k3 + g)) & 1"),
    "lowbit_zero_point_off_by_one": ("c) - (1 << (bits - 1));", "c) - (1 << (bits - 1)) + 1;"),
    "keep_map_by_rank": ("if (r[e] < keep) keep_map[(int64_t)l * keep + n++] = e;",
                         "if (r[e] < keep) keep_map[(int64_t)l * keep + r[e]] = e;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(SRC).read()
    a, b = MUTANTS[name]
    assert src.count(a) == 1, f"mutation anchor for {name} not found exactly once"
    c = tmp_path / "mutant.c"
    so = tmp_path / "libmutant.so"
    c.write_text(src.replace(a, b))
    subprocess.run(["gcc", "-std=c11", "-O1", "-ffp-contract=off", "-fPIC", "-shared", "-o", str(so), str(c), "-lm"],
                   check=True)
    env = dict(os.environ, MOE_ORACLE_LIB_OVERRIDE=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        "-q", "-x", "-p", "no:cacheprovider"], env=env, cwd=ROOT, capture_output=True, text=True)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
