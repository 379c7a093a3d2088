"""CPU pins of the near-tie index-set checker (tests/support_rules.check_row).

Every GPU index-set verdict runs through check_row, so it is tested here on
hand-made rows whose correct verdict follows from the comparison rule alone:
a selected set of a row is correct iff it holds exactly min(k, units)
distinct ascending unit ids inside the causal range, every unit more than
the band above the k-th largest score, none more than the band below it,
and -1 in every slot after the count. Units within the band of the k-th
score may go either way (gist.science page, Technischer Bericht section 2.1:
top-k of the head-averaged distribution under budget k; the 1e-6 band is the
tolerance this build compares index sets with).
"""
import math

import numpy as np
import pytest

import oracle
from tests.support_rules import check_row

BAND = 1e-6
# Seven units, budget 3. Sorted: 0.5, 0.3+5e-7, 0.3, 0.3-5e-7, 0.2, 0.1, 0.05,
# so the k-th score is 0.3, unit 1 must be in, units 2, 3, 4 lie in the band,
# units 0, 5, 6 must be out.
SCORE = np.array([0.1, 0.5, 0.3, 0.3 + 5e-7, 0.3 - 5e-7, 0.05, 0.2])
K = 3


def _check(units, count, score=SCORE, k=K):
    return check_row(np.asarray(units, dtype=np.int32), count, score,
                     oracle.kth_score(score, k), k, band=BAND)


def test_fixture_boundary():
    assert oracle.kth_score(SCORE, K) == 0.3


@pytest.mark.parametrize("units", [[1, 2, 3], [1, 2, 4], [1, 3, 4]])
def test_accepts_every_choice_inside_the_band(units):
    ok, msg, n_band = _check(units + [-1, -1], count=3)
    assert ok, msg
    assert n_band == 3


@pytest.mark.parametrize("units, count, why", [
    ([2, 3, 4, -1, -1], 3, "missing must-in"),          # unit 1 (0.5) left out
    ([1, 2, 6, -1, -1], 3, "selected must-out"),        # unit 6 (0.2) is below the band
    ([0, 1, 2, -1, -1], 3, "selected must-out"),        # unit 0 (0.1)
    ([1, 2, 2, -1, -1], 3, "not strictly ascending"),   # duplicate
    ([1, 3, 2, -1, -1], 3, "not strictly ascending"),   # unsorted
    ([1, 2, 7, -1, -1], 3, "out of causal range"),      # id past the row (7 units: 0..6)
    ([-1, 1, 2, -1, -1], 3, "out of causal range"),     # negative id inside the count
    ([1, 2, -1, -1, -1], 2, "count"),                   # too few
    ([1, 2, 3, 4, -1], 4, "count"),                     # too many
    ([1, 2, 3, 0, -1], 3, "padding"),                   # padding is not -1
    ([1, 2, 3, -1, 5], 3, "padding"),
])
def test_rejects(units, count, why):
    ok, msg, _ = _check(units, count=count)
    assert not ok
    assert why in msg, msg


def test_exact_ties_at_the_boundary():
    """Four units tie exactly at the k-th score: any two of them complete the set."""
    score = np.array([0.25, 0.125, 0.25, 0.5, 0.25, 0.25, 0.0])
    kth = oracle.kth_score(score, 3)
    assert kth == 0.25
    for a in (0, 2, 4, 5):
        for b in (0, 2, 4, 5):
            if a < b:
                ok, msg, n_band = check_row(np.array(sorted([3, a, b]) + [-1]), 3, score, kth, 3, BAND)
                assert ok, msg
                assert n_band == 4
    ok, msg, _ = check_row(np.array([1, 3, 5, -1]), 3, score, kth, 3, BAND)
    assert not ok and "must-out" in msg


def test_row_with_at_most_k_units_keeps_everything():
    score = np.array([0.7, 0.2, 0.1])
    for k in (3, 4, 10):
        kth = oracle.kth_score(score, k)
        assert kth == -math.inf
        ok, msg, _ = check_row(np.array([0, 1, 2] + [-1] * (k - 3)), 3, score, kth, k, BAND)
        assert ok, msg
        ok, msg, _ = check_row(np.array([0, 2] + [-1] * (k - 2)), 2, score, kth, k, BAND)
        assert not ok and "count" in msg
        ok, msg, _ = check_row(np.array([0, 1, 1] + [-1] * (k - 3)), 3, score, kth, k, BAND)
        assert not ok


def test_band_is_measured_against_the_kth_score():
    """A unit 2e-6 above the k-th score is must-in; 2e-6 below is must-out."""
    score = np.array([0.4, 0.3 + 2e-6, 0.3, 0.3 - 2e-6, 0.0])
    kth = oracle.kth_score(score, 3)
    assert kth == 0.3
    assert check_row(np.array([0, 1, 2]), 3, score, kth, 3, BAND)[0]
    ok, msg, _ = check_row(np.array([0, 2, 3]), 3, score, kth, 3, BAND)
    assert not ok and "must-in" in msg
    score2 = np.array([0.4, 0.35, 0.3, 0.3 - 2e-6, 0.0])
    ok, msg, _ = check_row(np.array([0, 1, 3]), 3, score2, oracle.kth_score(score2, 3), 3, BAND)
    assert not ok and "must-out" in msg


def test_oracle_support_always_passes_its_own_check():
    rng = np.random.default_rng(3)
    for _ in range(50):
        n = int(rng.integers(1, 60))
        score = rng.integers(0, 9, size=n) / 16.0
        k = int(rng.integers(1, 20))
        units = oracle.top_units(score, k)
        row = np.full(k, -1, dtype=np.int64)
        row[: units.size] = units
        ok, msg, _ = check_row(row, units.size, score, oracle.kth_score(score, k), k, BAND)
        assert ok, msg
