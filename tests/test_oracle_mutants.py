"""Plausible mistakes planted in copies of the oracle (CPU only): each mutant
must fail at least one pin, which shows the pins would catch that mistake in
the real oracle."""
import os
import shutil

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gspn_oracle.c")

# (name, original text, replacement, occurrences to replace (0 = all))
MUTANTS = [
    ("zero_padded_normalisation",
     "if (q < 0 || q >= n_o) continue;\n          sig[k]",
     "if (q < 0 || q >= n_o) { S += sigmoid(load_value(j->l[k], j->dt, idx)); continue; }\n          sig[k]", 1),
    ("neighbour_index_reversed", "const int64_t q = o + k - 1;", "const int64_t q = o - k + 1;", 0),
    ("no_local_restart", "return (p / G) != (prev / G);", "return 0;", 1),
    ("groups_relative_to_scan_start", "return (p / G) != (prev / G);", "return (s % G) == 0;", 1),
    ("lambda_dropped", "load_value(j->lam, j->dt, idx + doff) *", "", 1),
    ("reverse_directions_swapped", "(d == 0 || d == 2) ? s : n_s - 1 - s",
     "(d == 0 || d == 3) ? s : n_s - 1 - s", 1),
    ("directions_overwrite", "y[r * W + c] +=", "y[r * W + c] =", 1),
    ("unnormalised_sigmoid", "acc += (sig[k] / S) * h_prev[q];", "acc += sig[k] * h_prev[q];", 1),
    ("gate_missing", "y[r * W + c] += m * load_value(j->u, j->dt, idx + doff) * h_cur[o];",
     "y[r * W + c] += m * h_cur[o];", 1),
    ("sigmoid_sign_flipped", "return 1.0 / (1.0 + exp(-v));", "return 1.0 / (1.0 + exp(v));", 1),
]


@pytest.mark.parametrize("name,old,new,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new, count):
    text = open(SRC, encoding="utf-8").read()
    assert old in text, f"mutation anchor for {name} not found"
    mutated = text.replace(old, new) if count == 0 else text.replace(old, new, count)
    src = tmp_path / "mutant.c"
    src.write_text(mutated, encoding="utf-8")
    shutil.copy(os.path.join(os.path.dirname(SRC), "gspn_oracle.h"), tmp_path / "gspn_oracle.h")
    lib = oracle.load(oracle.build(force=True, src=str(src), out=str(tmp_path / "mutant.so")))

    def prop(*a, **kw):
        return oracle.propagate(*a, lib=lib, **kw)

    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check(prop)
        except (AssertionError, ValueError):
            failed.append(check.__name__)
    assert failed, f"mutant {name} passed every pin"
