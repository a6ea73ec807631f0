"""The backward pass of the fp64 oracle against its pins (CPU only), and
plausible mistakes planted in copies of it, each of which must fail a pin."""
import os
import shutil

import pytest

import oracle
import pins_backward

SRC = os.path.join(os.path.dirname(oracle.__file__), "gspn_oracle.c")


@pytest.mark.parametrize("check", pins_backward.ALL_BWD_CHECKS, ids=lambda c: c.__name__)
def test_backward_pin(check):
    check(oracle.backward)


def test_backward_rejects_bad_arguments():
    import numpy as np
    a = np.zeros((1, 1, 2, 2))
    with pytest.raises(ValueError):
        oracle.backward(a, a, a, a, a, a, a, dirs=0)
    with pytest.raises(ValueError):
        oracle.backward(a, a, a, a, a, a, a, group_rows=-1)
    with pytest.raises(TypeError):
        oracle.backward(a, a, a, a, a, a, a.astype(np.float32))


# (name, original text, replacement, occurrences to replace (0 = all))
MUTANTS = [
    ("adjoint_neighbour_mirrored", "const int64_t op = o - k + 1;", "const int64_t op = o + k - 1;", 1),
    ("adjoint_ignores_restart",
     "const int next_reads = s + 1 < n_s && !restarts(d, n_s, s + 1, j->G);",
     "const int next_reads = s + 1 < n_s;", 1),
    ("adjoint_weights_of_wrong_line", "lin + pixel_offset(j, d, s + 1, op)",
     "lin + pixel_offset(j, d, s, op)", 1),
    ("error_term_without_gate",
     "double e = m * load_value(j->u, j->dt, doff + idx) * load_value(j->gy, j->dt, idx);",
     "double e = m * load_value(j->gy, j->dt, idx);", 1),
    ("sigmoid_slope_missing", "dl[k][lbase + pix] += dsig * sig[k] * (1.0 - sig[k]);",
     "dl[k][lbase + pix] += dsig * sig[k];", 1),
    ("normalisation_term_dropped", "const double dsig = dw[k] / S - t / (S * S);",
     "const double dsig = dw[k] / S;", 1),
    ("gate_gradient_uses_current_line", "dw[k] = e * h[(s - 1) * n_o + o + k - 1];",
     "dw[k] = e * h[s * n_o + o + k - 1];", 1),
    ("gate_gradient_on_restart_lines", "      if (!restarts(d, n_s, s, j->G)) {\n        double sig[3], dw[3]",
     "      if (s > 0) {\n        double sig[3], dw[3]", 1),
    ("du_keeps_last_direction", "hsum[pix] += h[s * n_o + o];", "hsum[pix] = h[s * n_o + o];", 1),
    ("dx_without_lambda", "j->dx[base + i] = load_value(j->lam, j->dt, base + i) * dphi[i];",
     "j->dx[base + i] = dphi[i];", 1),
    ("dlambda_uses_lambda", "j->dlam[base + i] = load_value(j->x, j->dt, base + i) * dphi[i];",
     "j->dlam[base + i] = load_value(j->lam, j->dt, base + i) * dphi[i];", 1),
]


@pytest.mark.parametrize("name,old,new,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_backward_mutant_is_caught(tmp_path, name, old, new, count):
    text = open(SRC, encoding="utf-8").read()
    assert old in text, f"mutation anchor for {name} not found"
    mutated = text.replace(old, new) if count == 0 else text.replace(old, new, count)
    src = tmp_path / "mutant.c"
    src.write_text(mutated, encoding="utf-8")
    shutil.copy(os.path.join(os.path.dirname(SRC), "gspn_oracle.h"), tmp_path / "gspn_oracle.h")
    lib = oracle.load(oracle.build(force=True, src=str(src), out=str(tmp_path / "mutant.so")))

    def bwd(*a, **kw):
        return oracle.backward(*a, lib=lib, **kw)

    failed = []
    for check in pins_backward.ALL_BWD_CHECKS:
        try:
            check(bwd)
        except (AssertionError, ValueError):
            failed.append(check.__name__)
    assert failed, f"mutant {name} passed every pin"
