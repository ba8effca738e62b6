"""Pins for O4 (LiveEdit's active-row mask and active-row attention), CPU
only.  Each test pins the oracle to something other than itself: a hand
worked example, a library routine (numpy's norm and stable argsort), or a
closed form.  The comment on each test names the mistake it catches."""
import numpy as np
import pytest

from oracle import liveedit as O4


def test_hand_worked_distances():
    # z_src = 0, z_edit row i = (i, 0, 0): distance i, squared i^2.  tau = 2.5
    # keeps rows 3 and 4; keep = 2 keeps the two largest.  (catches a wrong
    # sign, a missing square, summing the wrong axis)
    zs = np.zeros((5, 3))
    ze = np.zeros((5, 3))
    ze[:, 0] = np.arange(5)
    np.testing.assert_array_equal(O4.distance_sq(zs, ze), [0, 1, 4, 9, 16])
    np.testing.assert_array_equal(O4.active_rows_threshold(zs, ze, 2.5), [3, 4])
    np.testing.assert_array_equal(O4.active_rows_topk(zs, ze, 2), [3, 4])
    # the threshold is strict: a distance equal to tau is not above it
    np.testing.assert_array_equal(O4.active_rows_threshold(zs, ze, 3.0), [4])


def test_distance_matches_numpy_norm():
    # against a library routine (catches a dropped channel or term)
    rng = np.random.default_rng(0)
    zs = rng.standard_normal((300, 16))
    ze = rng.standard_normal((300, 16))
    ref = np.linalg.norm(ze - zs, axis=1) ** 2
    np.testing.assert_allclose(O4.distance_sq(zs, ze), ref, rtol=1e-13)


def test_threshold_matches_the_l2_definition_away_from_ties():
    # ||e - s||_2 > tau on data with no distance within 1e-6 of tau
    rng = np.random.default_rng(1)
    zs = rng.standard_normal((2000, 48))
    ze = zs + rng.standard_normal((2000, 48)) * rng.uniform(0, 1, (2000, 1))
    dist = np.linalg.norm(ze - zs, axis=1)
    for tau in (0.5, 2.0, 4.0):
        assert np.abs(dist - tau).min() > 1e-6
        np.testing.assert_array_equal(O4.active_rows_threshold(zs, ze, tau),
                                      np.flatnonzero(dist > tau))


@pytest.mark.parametrize("keep", [0, 1, 137, 600, 2000, 5000])
def test_topk_matches_stable_argsort(keep):
    # the keep largest by numpy's stable sort of the negated distances (ties:
    # lower index first), returned ascending (catches an off-by-one in keep,
    # picking the smallest, unsorted output)
    rng = np.random.default_rng(2)
    zs = rng.standard_normal((2000, 16))
    ze = rng.standard_normal((2000, 16))
    dsq = O4.distance_sq(zs, ze)
    ref = np.sort(np.argsort(-dsq, kind="stable")[:keep])
    got = O4.active_rows_topk(zs, ze, keep)
    np.testing.assert_array_equal(got, ref)
    assert len(got) == min(keep, 2000)


def test_topk_ties_rank_by_index():
    # rows 1, 3, 4 have the same largest distance: keep = 2 takes rows 1 and 3
    zs = np.zeros((6, 2))
    ze = np.zeros((6, 2))
    ze[[1, 3, 4], 0] = 5.0
    ze[5, 1] = 1.0
    np.testing.assert_array_equal(O4.active_rows_topk(zs, ze, 2), [1, 3])
    np.testing.assert_array_equal(O4.active_rows_topk(zs, ze, 4), [1, 3, 4, 5])


def test_nan_distance_is_never_active_first():
    zs = np.zeros((4, 2))
    ze = np.ones((4, 2))
    ze[2, 0] = np.nan
    assert O4.distance_sq(zs, ze)[2] == -1.0
    np.testing.assert_array_equal(O4.active_rows_threshold(zs, ze, 0.0), [0, 1, 3])
    np.testing.assert_array_equal(O4.active_rows_topk(zs, ze, 3), [0, 1, 3])
    np.testing.assert_array_equal(O4.active_rows_topk(zs, ze, 4), [0, 1, 2, 3])


def test_rows_output_replaces_only_active_rows():
    prev = np.full((5, 2, 3), 7.0)
    full = np.arange(30, dtype=np.float64).reshape(5, 2, 3)
    out = O4.rows_output(prev, full, [0, 3])
    np.testing.assert_array_equal(out[[0, 3]], full[[0, 3]])
    np.testing.assert_array_equal(out[[1, 2, 4]], prev[[1, 2, 4]])
