"""The fp64 oracle's backward pass of the per-direction layer against its
pins, and plausible mistakes planted in copies of the oracle, each of which
must fail at least one pin (CPU only)."""
import os
import shutil

import numpy as np
import pytest

import oracle
import pins_dirs_backward

SRC = os.path.join(os.path.dirname(oracle.__file__), "gspn_oracle.c")


@pytest.mark.parametrize("check", pins_dirs_backward.ALL_DIRS_BACKWARD_CHECKS,
                         ids=lambda c: c.__name__)
def test_dirs_backward_pin(check):
    check(oracle.backward_dirs)


def test_dirs_backward_rejects_bad_arguments():
    x = np.zeros((1, 2, 3, 3))
    d = np.zeros((4, 1, 2, 3, 3))
    with pytest.raises(ValueError):
        oracle.backward_dirs(x, d, d, d, d, d, x, merge=np.ones((4, 3)))
    with pytest.raises(ValueError):
        oracle.backward_dirs(x, d[:3], d, d, d, d, x)
    with pytest.raises(ValueError):
        oracle.backward_dirs(x, d, d, d, d, d, x, dirs=0)
    with pytest.raises(TypeError):
        oracle.backward_dirs(x, d, d, d, d, d, x.astype(np.float32))


MUTANTS = [
    ("error_term_without_merge",
     "double e = m * load_value(j->u, j->dt, doff + idx) * load_value(j->gy, j->dt, idx);",
     "double e = load_value(j->u, j->dt, doff + idx) * load_value(j->gy, j->dt, idx);"),
    ("forward_lambda_of_direction_0",
     "acc + load_value(j->lam, j->dt, doff + idx) * load_value(j->x, j->dt, idx);",
     "acc + load_value(j->lam, j->dt, idx) * load_value(j->x, j->dt, idx);"),
    ("logits_of_direction_0", "const int64_t lin = lbase + doff;", "const int64_t lin = lbase;"),
    ("dx_with_lambda_of_direction_0",
     "j->dx[base + i] += load_value(j->lam, j->dt, doff + base + i) * dphi[i];",
     "j->dx[base + i] += load_value(j->lam, j->dt, base + i) * dphi[i];"),
    ("du_without_merge", "j->du[go + base + i] = m * g * hsum[i];",
     "j->du[go + base + i] = g * hsum[i];"),
    ("merge_gradient_without_gate",
     "j->dmerge[d * j->C + c] += load_value(j->u, j->dt, doff + base + i) * g * hsum[i];",
     "j->dmerge[d * j->C + c] += g * hsum[i];"),
    ("merge_gradient_scaled_by_merge",
     "j->dmerge[d * j->C + c] += load_value(j->u, j->dt, doff + base + i) * g * hsum[i];",
     "j->dmerge[d * j->C + c] += m * load_value(j->u, j->dt, doff + base + i) * g * hsum[i];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_dirs_backward_mutant_is_caught(tmp_path, name, old, new):
    text = open(SRC, encoding="utf-8").read()
    assert text.count(old) == 1, f"mutation anchor for {name} not found once"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new), encoding="utf-8")
    shutil.copy(os.path.join(os.path.dirname(SRC), "gspn_oracle.h"), tmp_path / "gspn_oracle.h")
    lib = oracle.load(oracle.build(force=True, src=str(src), out=str(tmp_path / "mutant.so")))

    def bwd(*a, **kw):
        return oracle.backward_dirs(*a, lib=lib, **kw)

    failed = []
    for check in pins_dirs_backward.ALL_DIRS_BACKWARD_CHECKS:
        try:
            check(bwd)
        except (AssertionError, ValueError):
            failed.append(check.__name__)
    assert failed, f"mutant {name} passed every pin"
