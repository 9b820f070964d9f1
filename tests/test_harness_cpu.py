"""The acceptance helpers of the GPU parity tests, on the CPU: which chosen
sets count as correct when the k-th and (k+1)-th biased scores lie within
the near-tie tolerance, and which set the oracle's output is then computed
under."""
import itertools

import numpy as np
import pytest

from tests.gpu_harness import NEAR_TIE, acceptable_sets, check_routing, expected_ids


def _brute_acceptable(beta, k, tol):
    E = len(beta)
    out = []
    for S in itertools.combinations(range(E), k):
        rest = np.delete(beta, S)
        if beta[list(S)].min() >= (rest.max() if rest.size else -np.inf) - tol:
            out.append(tuple(S))
    return out


@pytest.mark.parametrize("seed", range(6))
def test_acceptable_sets_match_brute_force(seed):
    rng = np.random.default_rng(seed)
    E, k = 9, 3
    for _ in range(50):
        beta = rng.choice([0.1, 0.2, 0.2 + 4e-6, 0.3, 0.3 + 2e-5, 0.5], E).astype(np.float64)
        assert sorted(acceptable_sets(beta, k)) == _brute_acceptable(beta, k, NEAR_TIE)


def test_acceptable_sets_clear_margin_is_unique():
    beta = np.array([0.9, 0.1, 0.8, 0.2, 0.7], np.float64)
    assert acceptable_sets(beta, 2) == [(0, 2)]
    assert acceptable_sets(beta, 5) == [(0, 1, 2, 3, 4)]


def test_check_routing_accepts_only_valid_near_tie_flips():
    # Token 0 has a near tie between experts 1 and 3 at the k-th place; token
    # 1 a clear margin.
    beta = np.array([[0.9, 0.5, 0.1, 0.5 - 3e-6], [0.9, 0.6, 0.1, 0.2]], np.float32)
    o_ids = np.array([[0, 1], [0, 1]], np.int32)
    o_w = np.full((2, 2), 0.5, np.float32)
    o_gap = np.array([3e-6, 0.4], np.float32)
    E = 4
    flipped = np.array([[0, 3], [0, 1]], np.int32)
    cnt = np.bincount(flipped.ravel(), minlength=E)
    same, near = check_routing(flipped, o_w, o_gap, cnt, o_ids, o_w, o_gap, E, beta=beta)
    assert near == 1 and list(same) == [False, True]
    np.testing.assert_array_equal(expected_ids(flipped, o_ids, beta), flipped)
    with pytest.raises(AssertionError):   # no flips allowed with exact=True
        check_routing(flipped, o_w, o_gap, cnt, o_ids, o_w, o_gap, E, beta=beta, exact=True)
    wrong = np.array([[0, 2], [0, 1]], np.int32)   # expert 2 is far below the k-th score
    with pytest.raises(AssertionError):
        check_routing(wrong, o_w, o_gap, np.bincount(wrong.ravel(), minlength=E), o_ids, o_w, o_gap, E, beta=beta)


def test_check_output_own_rounding_bound():
    # A heavy-tailed output (a few elements at 8 times the RMS) stored as
    # bf16: the stored values alone can miss the plain 3e-2 * RMS bar, and
    # pass once each element's bound takes its own half-ulp; an error of a
    # tenth of the RMS on one element fails either way.
    from tests._util import bf16_round
    from tests.gpu_harness import check_output
    rng = np.random.default_rng(3)
    ref = rng.standard_normal((64, 256))
    ref[0, :4] = np.ldexp(1.0 + 2.0 ** -8 - 1e-6, 3) * np.array([1.0, -1.0, 1.0, -1.0])  # just below a tie above 8
    got = bf16_round(ref)
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.abs(got - ref).max() > 3e-2 * rms
    with pytest.raises(AssertionError):
        check_output(got, ref, "plain bar")
    check_output(got, ref, "own rounding", own_rounding=True)
    bad = got.copy()
    bad[5, 7] += 0.1 * rms
    with pytest.raises(AssertionError):
        check_output(bad, ref, "planted error", own_rounding=True)
