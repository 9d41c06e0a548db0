"""Pins of the parity measure every tolerance test uses: oracle.rel_err.

rel_err(got, ref) is max|got - ref| / max|ref| over two arrays of one shape.
Each case below has a value worked out by hand, and the cases are chosen so
that the plausible slips -- dividing by max|got|, subtracting the maxima
instead of the elements, averaging instead of taking the maximum, dropping
the absolute value, returning 0 for an all-zero reference, broadcasting
arrays of different shapes -- each give a different number (the last test
plants every one of them and checks that some pin fails).
"""
import math

import numpy as np
import pytest

from oracle import moe_oracle as O


def pin_known_ratio():
    # largest error (1.0, at index 1) is not where |ref| is largest (4.0, index 2)
    ref = np.array([1.0, -2.0, 4.0, 0.5])
    got = np.array([1.0, -1.0, 3.75, 0.5])
    assert O.rel_err(got, ref) == 0.25


def pin_sign_of_error_is_ignored():
    ref = np.array([2.0, -8.0])
    assert O.rel_err(np.array([2.0, -6.0]), ref) == 0.25     # got above ref
    assert O.rel_err(np.array([2.0, -10.0]), ref) == 0.25    # got below ref
    assert O.rel_err(-ref, ref) == 2.0                       # every sign flipped


def pin_scale_invariant_and_exact():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((7, 5))
    got = ref.copy()
    assert O.rel_err(got, ref) == 0.0
    got[3, 2] += 1e-3
    want = 1e-3 / np.abs(ref).max()
    assert math.isclose(O.rel_err(got, ref), want, rel_tol=1e-9)
    assert math.isclose(O.rel_err(1024.0 * got, 1024.0 * ref), want, rel_tol=1e-9)


def pin_zero_reference_is_absolute():
    z = np.zeros((3, 4))
    assert O.rel_err(z, z) == 0.0
    got = z.copy()
    got[1, 2] = -3e-4
    assert O.rel_err(got, z) == 3e-4


def pin_empty_is_zero():
    assert O.rel_err(np.zeros((0, 5)), np.zeros((0, 5))) == 0.0


def pin_nan_fails_every_tolerance():
    got = np.array([1.0, np.nan, 2.0])
    err = O.rel_err(got, np.array([1.0, 1.0, 2.0]))
    assert not (err <= 1e-2)


def pin_shapes_must_match():
    with pytest.raises(ValueError):
        O.rel_err(np.zeros(3), np.zeros((1, 3)))
    with pytest.raises(ValueError):
        O.rel_err(np.array([5.0]), np.array([1.0, 2.0, 3.0]))   # would broadcast


def pin_max_not_mean():
    ref = np.ones(100)
    got = ref.copy()
    got[17] = 1.5
    assert O.rel_err(got, ref) == 0.5


PINS = [pin_known_ratio, pin_sign_of_error_is_ignored, pin_scale_invariant_and_exact,
        pin_zero_reference_is_absolute, pin_empty_is_zero, pin_nan_fails_every_tolerance,
        pin_shapes_must_match, pin_max_not_mean]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_rel_err_pin(pin):
    pin()


def _as64(got, ref):
    return np.asarray(got, np.float64), np.asarray(ref, np.float64)


def _by_got(got, ref):            # divides by max|got|
    got, ref = _as64(got, ref)
    if ref.size == 0:
        return 0.0
    den = np.abs(got).max()
    return float(np.abs(got - ref).max() / den) if den else float(np.abs(got - ref).max())


def _diff_of_maxima(got, ref):    # compares the maxima, not the elements
    got, ref = _as64(got, ref)
    if ref.size == 0:
        return 0.0
    den = np.abs(ref).max()
    num = abs(np.abs(got).max() - np.abs(ref).max())
    return float(num / den) if den else float(num)


def _zero_ref_is_zero(got, ref):  # an all-zero reference passes anything
    got, ref = _as64(got, ref)
    if ref.size == 0 or not np.abs(ref).max():
        return 0.0
    return float(np.abs(got - ref).max() / np.abs(ref).max())


def _mean_error(got, ref):        # mean instead of max
    got, ref = _as64(got, ref)
    if ref.size == 0:
        return 0.0
    den = np.abs(ref).max()
    num = np.abs(got - ref).mean()
    return float(num / den) if den else float(num)


def _signed(got, ref):            # no absolute value
    got, ref = _as64(got, ref)
    if ref.size == 0:
        return 0.0
    den = np.abs(ref).max()
    num = (got - ref).max()
    return float(num / den) if den else float(num)


def _broadcasting(got, ref):      # no shape check
    got, ref = _as64(got, ref)
    if ref.size == 0:
        return 0.0
    den = np.abs(ref).max()
    num = np.abs(got - ref).max()
    return float(num / den) if den else float(num)


def _nan_blind(got, ref):         # nanmax skips NaN
    got, ref = _as64(got, ref)
    if got.shape != ref.shape:
        raise ValueError("shape")
    if ref.size == 0:
        return 0.0
    den = np.nanmax(np.abs(ref))
    num = np.nanmax(np.abs(got - ref))
    return float(num / den) if den else float(num)


@pytest.mark.parametrize("slip", [_by_got, _diff_of_maxima, _zero_ref_is_zero, _mean_error,
                                  _signed, _broadcasting, _nan_blind], ids=lambda f: f.__name__)
def test_planted_checker_mistakes_fail_a_pin(slip, monkeypatch):
    for pin in PINS:
        pin()                     # the real measure passes every pin
    monkeypatch.setattr(O, "rel_err", slip)
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, pytest.fail.Exception):   # a failed assertion, or an
            failed.append(pin.__name__)                    # expected ValueError that did not come
    assert failed, f"{slip.__name__} passes every pin"
