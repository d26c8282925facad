"""The parity comparison itself: a NaN or an out-of-tolerance value anywhere in
a GPU result must fail the check (CPU only; synthetic arrays)."""
import numpy as np
import pytest

import parity_utils as pu


def _ref(seed=0):
    r = np.random.default_rng(seed)
    return dict(o=r.normal(size=(6, 2, 4)), final=r.normal(size=(1, 2, 4, 4)),
                A=r.normal(size=(2, 2, 4, 4)), B=r.normal(size=(2, 2, 4, 4)),
                C=r.normal(size=(2, 2, 4, 4)))


def test_identical_results_pass():
    ref = _ref()
    errs = pu.compare({k: v.copy() for k, v in ref.items()}, ref, "same")
    assert all(v == 0.0 for k, v in errs.items() if k != "A_max")


@pytest.mark.parametrize("key", ["o", "final", "A", "B", "C"])
def test_nan_anywhere_fails(key):
    ref = _ref()
    got = {k: v.copy() for k, v in ref.items()}
    got[key].flat[3] = np.nan
    with pytest.raises(AssertionError):
        pu.compare(got, ref, "nan")


def test_nan_in_state_is_infinite_error():
    ref = _ref()
    got = ref["B"].copy()
    got[1, 0, 2, 2] = np.nan
    assert pu.state_errors(got, ref["B"]) == float("inf")


@pytest.mark.parametrize("key,delta", [("o", 3e-3), ("B", 1e-3), ("C", 1e-3), ("final", 1e-3)])
def test_out_of_tolerance_fails(key, delta):
    ref = _ref()
    got = {k: v.copy() for k, v in ref.items()}
    scale = np.abs(ref[key]).max()
    got[key].flat[5] += delta * (1.0 if key == "o" else scale)
    with pytest.raises(AssertionError):
        pu.compare(got, ref, "tol")
