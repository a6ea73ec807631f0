"""The fp64 oracle's module prologue against its pins, and plausible mistakes
planted in copies of the oracle, each of which must fail at least one pin
(CPU only)."""
import os
import shutil

import numpy as np
import pytest

import oracle
import pins_prologue

SRC = os.path.join(os.path.dirname(oracle.__file__), "gspn_oracle.c")


@pytest.mark.parametrize("check", pins_prologue.ALL_PROLOGUE_CHECKS, ids=lambda c: c.__name__)
def test_prologue_pin(check):
    check(oracle.prologue)


def test_prologue_rejects_bad_arguments():
    x = np.zeros((1, 3, 2, 2))
    with pytest.raises(ValueError):
        oracle.prologue(x, np.zeros((2, 4)), None, np.zeros((10, 2)), None)   # Cin mismatch
    with pytest.raises(ValueError):
        oracle.prologue(x, np.zeros((2, 3)), None, np.zeros((8, 2)), None)    # not 5C rows
    with pytest.raises(TypeError):
        oracle.prologue(x, np.zeros((2, 3), np.float32), None, np.zeros((10, 2)), None)


MUTANTS = [
    ("reduce_weight_transposed", "load_value(j->w_r, j->dt, c * Cin + k)",
     "load_value(j->w_r, j->dt, k * C + c)"),
    ("reduce_bias_dropped", "double acc = j->b_r ? load_value(j->b_r, j->dt, c) : 0.0;",
     "double acc = 0.0;"),
    ("parameters_read_unrounded_x", "load_value(j->w_p, j->dt, q * C + c) * xr[c];",
     "load_value(j->w_p, j->dt, q * C + c) * j->x_out[(b * C + c) * HW + px];"),
    ("parameter_channels_interleaved", "const int64_t t = q / C, c = q % C;",
     "const int64_t t = q % 5, c = q / 5;"),
    ("bf16_rounding_missing", "return ldexp(nearbyint(ldexp(m, 8)), e - 8);", "return v;"),
    ("bf16_rounding_truncates", "return ldexp(nearbyint(ldexp(m, 8)), e - 8);",
     "return ldexp(trunc(ldexp(m, 8)), e - 8);"),
    ("bf16_ties_away", "return ldexp(nearbyint(ldexp(m, 8)), e - 8);",
     "return ldexp(round(ldexp(m, 8)), e - 8);"),
    ("parameter_bias_dropped", "double acc = j->b_p ? load_value(j->b_p, j->dt, q) : 0.0;",
     "double acc = 0.0;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_prologue_mutant_is_caught(tmp_path, name, old, new):
    text = open(SRC, encoding="utf-8").read()
    assert text.count(old) == 1, f"mutation anchor for {name} not found once"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new), encoding="utf-8")
    shutil.copy(os.path.join(os.path.dirname(SRC), "gspn_oracle.h"), tmp_path / "gspn_oracle.h")
    lib = oracle.load(oracle.build(force=True, src=str(src), out=str(tmp_path / "mutant.so")))

    def prol(*a, **kw):
        return oracle.prologue(*a, lib=lib, **kw)

    failed = []
    for check in pins_prologue.ALL_PROLOGUE_CHECKS:
        try:
            check(prol)
        except (AssertionError, ValueError):
            failed.append(check.__name__)
    assert failed, f"mutant {name} passed every pin"
