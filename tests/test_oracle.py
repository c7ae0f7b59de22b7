"""The CPU oracle against its pins, and the pins against planted mistakes."""
import os
import tempfile

import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


# Planted mistakes compiled into separate copies of the oracle (CPU only):
# 1 drops the last k term, 2 reads B transposed, 3 flips the sign of the
# beta term, 4 ignores the leading dimension of C0, 5 indexes the epilogue's
# bias by row, 6 applies the ReLU before adding the bias.
@pytest.mark.parametrize("mutant", [1, 2, 3, 4, 5, 6])
def test_pins_catch_planted_mistake(mutant):
    with tempfile.TemporaryDirectory() as d:
        path = oracle.build(os.path.join(d, f"liboracle_m{mutant}.so"), mutant=mutant)
        lib = oracle.load(path)
        caught = []
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(lib)
            except AssertionError:
                caught.append(pin.__name__)
        assert caught, f"planted mistake {mutant} passed every pin"


def test_within_tolerance_rule():
    import numpy as np
    ref = np.array([1.0, 2.0, np.nan])
    bnd = np.array([1.0, 1.0, 1.0])
    ok, worst = oracle.within_tolerance(np.array([1.0 + 5e-5, 2.0, np.nan]), ref, bnd)
    assert ok and worst == pytest.approx(0.5)
    ok, _ = oracle.within_tolerance(np.array([1.0 + 2e-4, 2.0, np.nan]), ref, bnd)
    assert not ok
    ok, _ = oracle.within_tolerance(np.array([1.0, np.inf, np.nan]), ref, bnd)
    assert not ok


def test_within_tolerance_matches_non_finite_reference():
    """Where the reference is NaN or +-Inf, the result must be the same
    non-finite value: a finite value, a NaN for an infinity, or an infinity
    of the other sign all fail."""
    import numpy as np
    ref = np.array([np.nan, np.inf, -np.inf, 3.0])
    bnd = np.array([1.0, 1.0, 1.0, 1.0])
    ok, worst = oracle.within_tolerance(np.array([np.nan, np.inf, -np.inf, 3.0]), ref, bnd)
    assert ok and worst == 0.0
    for bad in ([0.0, np.inf, -np.inf, 3.0],       # NaN turned finite
                [np.nan, 1e30, -np.inf, 3.0],      # +Inf turned finite
                [np.nan, -np.inf, -np.inf, 3.0],   # +Inf of the wrong sign
                [np.nan, np.inf, np.nan, 3.0],     # -Inf turned NaN
                [np.inf, np.inf, -np.inf, 3.0]):   # NaN turned Inf
        ok, _ = oracle.within_tolerance(np.array(bad), ref, bnd)
        assert not ok, bad
