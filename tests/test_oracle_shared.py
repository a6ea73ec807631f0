"""Channel-shared logits in the fp64 oracle: pins (CPU only), argument
checks, and planted mistakes that must each fail a pin."""
import os
import shutil

import numpy as np
import pytest

import oracle
import pins_shared

SRC = os.path.join(os.path.dirname(oracle.__file__), "gspn_oracle.c")


def test_shared_forward_pin():
    pins_shared.check_shared_forward(oracle.propagate)


@pytest.mark.parametrize("check", pins_shared.SHARED_BWD_CHECKS, ids=lambda c: c.__name__)
def test_shared_backward_pin(check):
    check(oracle.backward)


def test_shared_rejects_non_dividing_channels():
    x = np.zeros((1, 4, 3, 3))
    lg = np.zeros((1, 3, 3, 3))
    with pytest.raises(ValueError):
        oracle.propagate(x, lg, lg, lg, x, x)
    with pytest.raises(ValueError):
        oracle.backward(x, lg, lg, lg, x, x, x)


MUTANTS = [
    ("channel_modulo_instead_of_group", "return b * Cl + c / (C / Cl);", "return b * Cl + c % Cl;"),
    ("group_gradient_not_cleared",
     "      for (int64_t i = 0; i < H * W; ++i) j->dl[k][grp * H * W + i] = 0.0;\n",
     "      for (int64_t i = 0; i < H * W; ++i) j->dl[k][grp * H * W + i] *= 1.0;\n"),
    ("forward_logits_of_own_plane", "load_value(j->l[k], j->dt, lbase + r * W + c)",
     "load_value(j->l[k], j->dt, base % (j->B * j->Cl * H * W) + r * W + c)"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_shared_mutant_is_caught(tmp_path, name, old, new):
    text = open(SRC, encoding="utf-8").read()
    assert old in text, f"mutation anchor for {name} not found"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new), encoding="utf-8")
    shutil.copy(os.path.join(os.path.dirname(SRC), "gspn_oracle.h"), tmp_path / "gspn_oracle.h")
    lib = oracle.load(oracle.build(force=True, src=str(src), out=str(tmp_path / "mutant.so")))
    failed = []
    try:
        pins_shared.check_shared_forward(lambda *a, **kw: oracle.propagate(*a, lib=lib, **kw))
    except (AssertionError, ValueError):
        failed.append("forward")
    for check in pins_shared.SHARED_BWD_CHECKS:
        try:
            check(lambda *a, **kw: oracle.backward(*a, lib=lib, **kw))
        except (AssertionError, ValueError):
            failed.append(check.__name__)
    assert failed, f"mutant {name} passed every pin"
