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


# The numpy half of the oracle (expert profile and steering projection): each
# mistake goes into a copy of the oracle package, and the pins of those parts
# run against the copy from a scratch tree that mirrors the repository.
PY_MUTANTS = {
    "steer_sign": ("steer.py", "return h - np.multiply.outer(h @ v, v)", "return h + np.multiply.outer(h @ v, v)"),
    "steer_slot_major_inverse": ("steer.py", "inv = np.asarray(inv).reshape(T, K)", "inv = np.asarray(inv).reshape(K, T).T"),
    "steer_residual_dropped": ("steer.py", "if residual is not None:", "if False:"),
    "profile_ties_to_higher_index": ("profile.py", "(-int(flat[i]), i)", "(-int(flat[i]), -i)"),
    "profile_hits_one_pair_too_many": ("profile.py", "np.asarray(pairs)[:S]", "np.asarray(pairs)[:S + 1]"),
    "profile_remap_keeps_pruned": ("profile.py", "j = new_index[l].get(e)", "j = new_index[l].get(e, e)"),
    "profile_inverse_off_by_one": ("profile.py", "inv[l, e] = r", "inv[l, e] = r + 1"),
    "strp_pair_fields_swapped": ("profile.py", 'struct.pack("<HH", l, e)', 'struct.pack("<HH", e, l)'),
}
PY_PINS = "profile or strp or steer"


def _run_py_pins(tmp_path, mutant):
    import shutil
    import oracle
    oracle.build()
    tree = tmp_path / "tree"
    shutil.copytree(os.path.join(ROOT, "oracle"), tree / "oracle", ignore=shutil.ignore_patterns("_build", "__pycache__"))
    (tree / "tests").mkdir()
    for f in ("conftest.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tree / "tests" / f)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tree / "tests" / "golden")
    os.symlink(os.path.join(ROOT, "routed_expert_ffn_amd"), tree / "routed_expert_ffn_amd")
    if mutant is not None:
        fname, a, b = mutant
        p = tree / "oracle" / fname
        src = p.read_text()
        assert src.count(a) == 1, f"mutation anchor {a!r} not found exactly once in {fname}"
        p.write_text(src.replace(a, b))
    env = dict(os.environ, MOE_ORACLE_LIB_OVERRIDE=oracle.LIB)
    return subprocess.run([sys.executable, "-m", "pytest", str(tree / "tests" / "test_oracle_pins.py"), "-q", "-x",
                           "-k", PY_PINS, "-p", "no:cacheprovider"], env=env, cwd=str(tree),
                          capture_output=True, text=True)


def test_python_pins_pass_on_the_unmutated_copy(tmp_path):
    r = _run_py_pins(tmp_path, None)
    assert r.returncode == 0 and " passed" in r.stdout, r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_python_pins_catch_planted_mistake(name, tmp_path):
    r = _run_py_pins(tmp_path, PY_MUTANTS[name])
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
    assert " failed" in r.stdout, r.stdout[-2000:]   # a failing pin, not a broken copy
