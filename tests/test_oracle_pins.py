"""The fp64 oracle against its pins (CPU only). See tests/pins.py."""
import numpy as np
import pytest

import oracle
import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(oracle.propagate)


def test_gmatrix_reference_on_golden():
    """The explicit G-matrix construction itself reproduces the hand examples,
    so the two independent routes agree with hand arithmetic."""
    import os
    for case in pins.load_golden(os.path.join(pins.GOLDEN, "hand_examples.txt")):
        got = pins.gmatrix_reference(*case["inputs"], case["dirs"], case["G"])
        assert np.allclose(got, case["y"], rtol=1e-13, atol=1e-13), case["name"]


def test_input_decoding_exact():
    """float32 and bf16 inputs are decoded exactly: the oracle on them equals
    the oracle on their float64 values, bitwise."""
    rng = np.random.default_rng(3)
    shape = (2, 2, 5, 6)
    f32 = [rng.standard_normal(shape).astype(np.float32) for _ in range(6)]
    y32 = oracle.propagate(*f32, dirs=15)
    y64 = oracle.propagate(*[a.astype(np.float64) for a in f32], dirs=15)
    assert np.array_equal(y32, y64)
    # bf16: keep the upper half of each float32 (truncation is fine here: any
    # bit pattern is a valid input)
    bf = [(a.view(np.uint32) >> 16).astype(np.uint16) for a in f32]
    dec = [(b.astype(np.uint32) << 16).view(np.float32).astype(np.float64) for b in bf]
    assert np.array_equal(oracle.propagate(*bf, dirs=15), oracle.propagate(*dec, dirs=15))


def test_threads_do_not_change_result():
    rng = np.random.default_rng(5)
    args = [rng.standard_normal((3, 5, 7, 4)) for _ in range(6)]
    a = oracle.propagate(*args, dirs=15, group_rows=3, nthreads=1)
    b = oracle.propagate(*args, dirs=15, group_rows=3, nthreads=8)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("kw", [dict(dirs=0), dict(dirs=16), dict(group_rows=-1)])
def test_oracle_rejects_bad_arguments(kw):
    args = [np.zeros((1, 1, 2, 2))] * 6
    kw = dict(dict(dirs=15, group_rows=0), **kw)
    with pytest.raises(ValueError):
        oracle.propagate(*args, **kw)


def test_empty_batch():
    args = [np.zeros((0, 3, 4, 4))] * 6
    assert oracle.propagate(*args).shape == (0, 3, 4, 4)
