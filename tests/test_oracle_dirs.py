"""The fp64 oracle's per-direction parameters and per-channel merger against
their pins, and plausible mistakes planted in copies of the oracle, each of
which must fail at least one pin (CPU only)."""
import os
import shutil

import numpy as np
import pytest

import oracle
import pins_dirs

SRC = os.path.join(os.path.dirname(oracle.__file__), "gspn_oracle.c")


@pytest.mark.parametrize("check", pins_dirs.ALL_DIRS_CHECKS, ids=lambda c: c.__name__)
def test_dirs_pin(check):
    check(oracle.propagate_dirs)


def test_dirs_rejects_bad_arguments():
    x = np.zeros((1, 2, 3, 3))
    d = np.zeros((4, 1, 2, 3, 3))
    with pytest.raises(ValueError):
        oracle.propagate_dirs(x, d, d, d, d, d, merge=np.ones((4, 3)))
    with pytest.raises(ValueError):
        oracle.propagate_dirs(x, d[:3], d, d, d, d)
    with pytest.raises(ValueError):
        oracle.propagate_dirs(x, d, d, d, d, d, dirs=0)


MUTANTS = [
    ("logits_not_per_direction", "lbase = logit_plane(plane, j->C, j->Cl) * H * W + doff;",
     "lbase = logit_plane(plane, j->C, j->Cl) * H * W;"),
    ("lambda_not_per_direction", "load_value(j->lam, j->dt, idx + doff)",
     "load_value(j->lam, j->dt, idx)"),
    ("gate_not_per_direction", "m * load_value(j->u, j->dt, idx + doff)",
     "m * load_value(j->u, j->dt, idx)"),
    ("merge_index_transposed", "j->merge[d * j->C + plane % j->C]",
     "j->merge[(plane % j->C) * 4 + d]"),
    ("merge_ignored", "y[r * W + c] += m * load_value", "y[r * W + c] += load_value"),
    ("merge_of_first_direction", "j->merge[d * j->C + plane % j->C]",
     "j->merge[plane % j->C]"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_dirs_mutant_is_caught(tmp_path, name, old, new):
    text = open(SRC, encoding="utf-8").read()
    assert text.count(old) == 1, f"mutation anchor for {name} not found once"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new), encoding="utf-8")
    shutil.copy(os.path.join(os.path.dirname(SRC), "gspn_oracle.h"), tmp_path / "gspn_oracle.h")
    lib = oracle.load(oracle.build(force=True, src=str(src), out=str(tmp_path / "mutant.so")))

    def prop(*a, **kw):
        return oracle.propagate_dirs(*a, lib=lib, **kw)

    failed = []
    for check in pins_dirs.ALL_DIRS_CHECKS:
        try:
            check(prop)
        except (AssertionError, ValueError):
            failed.append(check.__name__)
    assert failed, f"mutant {name} passed every pin"
