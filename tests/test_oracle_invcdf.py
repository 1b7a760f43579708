"""Pins of the oracle's inverse-CDF draw: the target-generation phase samples a
token from a row's distribution ("Accelerating Sonar through speculation",
section "Spekulatives Decoding", phase "Zielgenerierung"). The convention
(smallest v whose cumulative weight exceeds u*S) is checked against numpy's
searchsorted, against a chi-square fit, and on edge cases."""
import numpy as np
import pytest

import oracle
from tests import _np_ref as R


def test_matches_numpy_searchsorted():
    rng = np.random.default_rng(5)
    for trial in range(300):
        n = int(rng.integers(1, 60))
        w = rng.exponential(size=n) * (rng.random(n) < 0.7)
        if w.sum() == 0:
            w[int(rng.integers(n))] = 1.0
        u = float(rng.random())
        y, lo, hi = oracle.invcdf(w, u)
        c = np.cumsum(w)
        want = int(np.searchsorted(c, u * c[-1], side="right"))
        if want < n:
            assert y == want, (trial, w, u)
            assert w[y] > 0
            assert lo <= u < hi or abs(u - hi) < 1e-12


def test_edge_cases():
    # u = 0 skips leading zero-mass entries
    assert oracle.invcdf([0.0, 0.0, 2.0, 1.0], 0.0)[0] == 2
    # the largest uniform the generator can emit lands in the last positive bin
    assert oracle.invcdf([1.0, 1.0, 1.0, 0.0], 1.0 - 2.0 ** -24)[0] == 2
    # a single non-zero entry takes every draw
    for u in (0.0, 0.3, 0.999999):
        assert oracle.invcdf([0.0, 0.0, 5.0, 0.0, 0.0], u)[0] == 2
    # zero total mass: no draw
    assert oracle.invcdf([0.0, 0.0], 0.5)[0] == -1
    # bin edges are reported
    y, lo, hi = oracle.invcdf([1.0, 3.0], 0.25)
    assert (y, lo, hi) == (1, 0.25, 1.0)


def test_chi_square_against_weights():
    rng = np.random.default_rng(9)
    w = np.array([0.1, 0.0, 2.0, 0.7, 1.2, 0.0, 0.05])
    us = rng.random(40000)
    ys = np.array([oracle.invcdf(w, u)[0] for u in us])
    counts = np.bincount(ys, minlength=len(w))
    assert counts[1] == 0 and counts[5] == 0
    assert R.chi2_pvalue(counts, w / w.sum()) > 1e-4


def test_planted_off_by_one_is_caught():
    with oracle.mutation(oracle.MUT_INVCDF_GE):
        assert oracle.invcdf([0.0, 0.0, 2.0, 1.0], 0.0)[0] != 2


def test_rounding_fallback_takes_the_last_positive_bin():
    # u = 1 leaves no bin whose cumulative weight exceeds u*S (the case rounding can
    # produce): the draw is the last entry of positive weight, trailing zeros skipped
    w = [0.5, 2.0, 0.0, 1.5, 0.0, 0.0]
    y, lo, hi = oracle.invcdf(w, 1.0)
    assert y == 3
    assert (lo, hi) == (2.5 / 4.0, 1.0)
    assert oracle.invcdf([1.0, 1.0, 0.0, 0.0], 1.0)[0] == 1
    # u just below 1 still crosses normally
    assert oracle.invcdf(w, 1.0 - 2.0 ** -24)[0] == 3
