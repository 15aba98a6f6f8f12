"""Pins of the oracle's checker, ``relative_frobenius_error``.

Every Newton-Schulz parity assertion on the GPU goes through this one
function (directly, or through the GPU tests' ``rel`` helper), so a mistake
in it would loosen every tolerance at once: a dropped square root squares
each error, so a true 0.17 would read 0.029 and pass the 3e-2 bf16 gate.
The pins below hold it to values worked out by hand on integer matrices
whose Frobenius norms are exact, and the last test plants plausible
mistakes in it (on the CPU) and checks that a pin catches each one.
"""

import math

import numpy as np
import pytest

from oracle import oracle as O

W = np.array([[1.0, 2.0], [2.0, 4.0]])          # ||W||_F = 5
D = np.array([[0.0, 0.0], [0.0, 1.0]])          # ||D||_F = 1, max|D| = 1


def test_double_of_want_is_exactly_one():
    # ||2W - W|| / ||W|| = 1; normalising by ||got|| would give 1/2
    assert O.relative_frobenius_error(2.0 * W, W) == 1.0


def test_perturbation_by_hand():
    # ||D|| / ||W|| = 1/5.  Squared norms would give 1/25; max-abs entries
    # 1/4; normalising by ||W + D|| = sqrt(34), 1/sqrt(34).
    assert O.relative_frobenius_error(W + D, W) == pytest.approx(0.2, rel=1e-15)
    # a scaled perturbation: delta * ||D|| / ||W||
    for delta in (1e-6, 3e-2, 7.0):
        assert O.relative_frobenius_error(W + delta * D, W) == pytest.approx(delta / 5.0, rel=1e-12)


def test_zero_want_gives_the_norm_of_got():
    # ||got||_F of [[3, 4], [0, 0]] is 5; a mean over entries would give sqrt(25/4)
    got = np.array([[3.0, 4.0], [0.0, 0.0]])
    assert O.relative_frobenius_error(got, np.zeros((2, 2))) == 5.0
    assert O.relative_frobenius_error(np.zeros((2, 2)), np.zeros((2, 2))) == 0.0


def test_exact_match_and_element_pairing():
    assert O.relative_frobenius_error(W, W) == 0.0
    # entries are paired by position: the transpose of a non-symmetric
    # matrix is not a match (||A^T - A||^2 = 2 * (3 - 0)^2 = 18, ||A||^2 = 34)
    A = np.array([[1.0, 3.0], [0.0, 4.0]]) + np.array([[0.0, 0.0], [0.0, 1.0]])
    assert O.relative_frobenius_error(A.T, A) == pytest.approx(math.sqrt(18.0 / 35.0), rel=1e-15)


def test_shapes_must_agree():
    # (2, 1) against (1, 2) would broadcast to a 2 x 2 difference
    with pytest.raises(ValueError):
        O.relative_frobenius_error(np.ones((2, 1)), np.ones((1, 2)))
    with pytest.raises(ValueError):
        O.relative_frobenius_error(np.ones((3, 4)), np.ones((4, 3)))


def _run_checker_pins():
    fails = []
    for fn in (test_double_of_want_is_exactly_one, test_perturbation_by_hand,
               test_zero_want_gives_the_norm_of_got, test_exact_match_and_element_pairing,
               test_shapes_must_agree):
        try:
            fn()
        except (AssertionError, ValueError, pytest.fail.Exception):
            fails.append(fn.__name__)
    return fails


def _no_sqrt(got, want):
    g, w = np.asarray(got, float), np.asarray(want, float)
    den = float(np.sum(w * w))
    num = float(np.sum((g - w) ** 2))
    return num if den == 0.0 else num / den


def _by_norm_of_got(got, want):
    g, w = np.asarray(got, float), np.asarray(want, float)
    den = math.sqrt(float(np.sum(g * g)))
    num = math.sqrt(float(np.sum((g - w) ** 2)))
    return num if den == 0.0 else num / den


def _max_abs(got, want):
    g, w = np.asarray(got, float), np.asarray(want, float)
    den = float(np.max(np.abs(w)))
    num = float(np.max(np.abs(g - w)))
    return num if den == 0.0 else num / den


def _mean_squares(got, want):
    g, w = np.asarray(got, float), np.asarray(want, float)
    den = math.sqrt(float(np.mean(w * w)))
    num = math.sqrt(float(np.mean((g - w) ** 2)))
    return num if den == 0.0 else num / den


def _absolute(got, want):
    g, w = np.asarray(got, float), np.asarray(want, float)
    return math.sqrt(float(np.sum((g - w) ** 2)))


def _broadcasting(got, want):
    g, w = np.asarray(got, float), np.asarray(want, float)
    den = math.sqrt(float(np.sum(w * w)))
    num = math.sqrt(float(np.sum((g - w) ** 2)))
    return num if den == 0.0 else num / den


def _transposed_pairing(got, want):
    g, w = np.asarray(got, float), np.asarray(want, float)
    if g.shape != w.shape:
        raise ValueError("shapes differ")
    den = math.sqrt(float(np.sum(w * w)))
    num = math.sqrt(float(np.sum((g.T - w) ** 2)))
    return num if den == 0.0 else num / den


@pytest.mark.parametrize("mutant", [_no_sqrt, _by_norm_of_got, _max_abs, _mean_squares, _absolute,
                                    _broadcasting, _transposed_pairing])
def test_planted_checker_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(O, "relative_frobenius_error", mutant)
    assert _run_checker_pins(), f"no pin caught planted mistake {mutant.__name__}"
