"""Pins of the oracle's row statistics (softmax normaliser, log-sum-exp, argmax)
against library routines and closed forms.

The row softmax at temperature T is what every acceptance decision compares
("Accelerating Sonar through speculation", section "Ziel-Entwurf": acceptance
compares the full draft and target distributions; Medusa page, section 二: the
head output is a softmax over the vocabulary)."""
import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
from tests import _np_ref as R

DTYPES = [R.DT_F32, R.DT_BF16, R.DT_F16]


def _rows(rng, dtype, rows, V, sigma=3.0):
    x = rng.normal(0.0, sigma, size=(rows, V))
    if dtype == R.DT_BF16:
        x = R.decode(R.DT_F32, x.astype(np.float32))
        bits = x.astype(np.float32).view(np.uint32)
        bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000   # any bf16 value will do
        x = bits.view(np.float32).astype(np.float64)
    enc = R.encode(dtype, x)
    return enc, R.decode(dtype, enc)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("T", [0.7, 1.0, 2.5])
def test_lse_matches_scipy_logsumexp(dtype, T):
    rng = np.random.default_rng(1000 + dtype)
    enc, x = _rows(rng, dtype, 6, 3001)
    got = oracle.row_stats(enc, 3001, dtype, T)
    want = logsumexp(x / T, axis=1)
    np.testing.assert_allclose(got["lse"], want, rtol=1e-13, atol=1e-12)
    np.testing.assert_array_equal(got["max"], x.max(axis=1))
    assert np.all(got["err"] == 0)


def test_two_token_row_is_logistic():
    # V = 2: p_0 = 1 / (1 + exp((x_1 - x_0)/T)), the logistic function.
    from scipy.special import expit
    rng = np.random.default_rng(7)
    x = rng.normal(0, 4, size=(50, 2))
    for T in (0.5, 1.0, 3.0):
        got = oracle.row_stats(x.astype(np.float32), 2, R.DT_F32, T)
        xf = x.astype(np.float32).astype(np.float64)
        p0 = np.exp(xf[:, 0] / T - got["lse"])
        np.testing.assert_allclose(p0, expit((xf[:, 0] - xf[:, 1]) / T), rtol=1e-12)


@pytest.mark.parametrize("dtype", DTYPES)
def test_argmax_lowest_index_on_ties(dtype):
    rng = np.random.default_rng(11)
    V = 997
    x = np.round(rng.normal(0, 2, size=(40, V)) * 4) / 4    # many duplicates, exact in all dtypes
    for r in range(40):
        top = x[r].max() + 1.0
        pos = sorted(rng.choice(V, size=1 + r % 3, replace=False))
        x[r, pos] = top
    enc = R.encode(dtype, x)
    got = oracle.row_stats(enc, V, dtype, 1.0)
    np.testing.assert_array_equal(got["argmax"], np.argmax(R.decode(dtype, enc), axis=1))


def test_argmax_skips_nan_and_flags_unusable_rows():
    V = 8
    x = np.array([
        [np.nan, 1.0, 3.0, 3.0, -np.inf, 0, 0, 0],
        [-np.inf] * 8,
        [np.nan] * 8,
        [0, 0, 0, 0, 0, 0, 0, 0],
    ], dtype=np.float32)
    got = oracle.row_stats(x, V, R.DT_F32, 1.0)
    assert got["argmax"][0] == 2
    assert got["argmax"][3] == 0
    assert list(got["err"]) == [2, 2, 2, 0]       # row 0: the NaN poisons the normaliser
    assert got["argmax"][1] == -1 and got["argmax"][2] == -1


def test_masked_entries_have_zero_mass():
    x = np.array([[1.0, -np.inf, 2.0, -np.inf]], dtype=np.float32)
    got = oracle.row_stats(x, 4, R.DT_F32, 1.0)
    np.testing.assert_allclose(got["lse"], [np.logaddexp(1.0, 2.0)], rtol=1e-15)
    assert got["err"][0] == 0


@pytest.mark.parametrize("mut", [oracle.MUT_LSE_WITHOUT_MAX, oracle.MUT_TEMPERATURE_IGNORED])
def test_planted_row_mistakes_are_caught(mut):
    rng = np.random.default_rng(3)
    enc, x = _rows(rng, R.DT_F32, 4, 500)
    with oracle.mutation(mut):
        got = oracle.row_stats(enc, 500, R.DT_F32, 0.7)
    want = logsumexp(x / 0.7, axis=1)
    assert not np.allclose(got["lse"], want, rtol=1e-6)


@pytest.mark.parametrize("dtype", DTYPES)
def test_lse_matches_two_pass_long_double(dtype):
    # the textbook two-pass form: m = max x, then m/T + log(sum exp((x - m)/T)),
    # each row summed in extended precision
    rng = np.random.default_rng(2000 + dtype)
    enc, x = _rows(rng, dtype, 5, 4099)
    for T in (0.7, 1.3):
        got = oracle.row_stats(enc, 4099, dtype, T)
        for r in range(x.shape[0]):
            xl = x[r].astype(np.longdouble)
            m = xl.max()
            want = m / np.longdouble(T) + np.log(np.sum(np.exp((xl - m) / np.longdouble(T))))
            assert abs(float(got["lse"][r] - want)) <= 1e-13 * max(1.0, abs(float(want)))
