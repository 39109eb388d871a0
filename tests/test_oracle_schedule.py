"""Pins for the oracle's hardware-aware prefix scheduler (no GPU).

Pins: closed forms of the survival product; special SPS tables whose
answer is known; brute-force optimality over every (l_1..l_R) when SPS is
linear (then Theta along the ranked list is concave, so stopping at the
first non-rise is the global optimum of the pages' objective); the
marginal form of the stop rule from [xhh] (survival probability must beat
expected output times the slowdown ratio); and the non-anticipation property
([billytse] 7, [xhh]): whether position j is verified cannot depend on
confidences of later positions of the same request.
"""

import itertools

import numpy as np
import pytest

import oracle as O


def test_survival_closed_forms():
    c = np.array([[0.5] * 6, [1.0, 0.25, 1.0, 0.5, 0.0, 1.0]])
    a = O.survival(c)
    np.testing.assert_array_equal(a[0], [0.5 ** (j + 1) for j in range(6)])
    np.testing.assert_array_equal(a[1], [1.0, 0.25, 0.25, 0.125, 0.0, 0.0])


def test_flat_profile_verifies_everything():
    rng = np.random.default_rng(0)
    c = rng.uniform(0.01, 1.0, (5, 4))
    s = O.schedule(c, np.full(100, 7.0))
    assert list(s["ell"]) == [4] * 5 and s["n_admitted"] == 20


def test_no_capacity_verifies_nothing():
    c = np.full((3, 4), 0.99)
    sps = np.zeros(30)
    sps[3] = 50.0          # Bt = R only
    s = O.schedule(c, sps)
    assert list(s["ell"]) == [0, 0, 0]
    assert s["theta"] == 3 * 50.0


def _theta(ell, a, sps):
    """The pages' objective for an arbitrary choice of verify lengths."""
    R = len(ell)
    Bt = sum(1 + l for l in ell)
    if Bt >= len(sps) or sps[Bt] <= 0:
        return -np.inf
    tau = sum(1 + sum(a[r, :l]) for r, l in enumerate(ell))
    return tau * sps[Bt]


@pytest.mark.parametrize("seed", range(40))
def test_greedy_is_global_optimum_for_linear_profile(seed):
    rng = np.random.default_rng(seed)
    R, gamma = rng.integers(1, 4), rng.integers(1, 4)
    c = rng.uniform(0.0, 1.0, (R, gamma))
    slope = rng.uniform(0.005, 0.2)
    bt = np.arange(R * (gamma + 1) + 2, dtype=float)
    sps = 100.0 * (1.0 - slope * bt)
    sps[0] = 0.0
    a = O.survival(c)
    s = O.schedule(c, sps)
    best = max(itertools.product(range(gamma + 1), repeat=R), key=lambda l: _theta(l, a, sps))
    best_val = _theta(best, a, sps)
    assert abs(s["theta"] - best_val) <= 1e-12 * abs(best_val)
    assert abs(_theta(tuple(s["ell"]), a, sps) - s["theta"]) <= 1e-12 * abs(best_val)
    ties = [l for l in itertools.product(range(gamma + 1), repeat=R)
            if abs(_theta(l, a, sps) - best_val) <= 1e-12 * abs(best_val)]
    if len(ties) == 1:
        assert tuple(s["ell"]) == best


@pytest.mark.parametrize("seed", range(25))
def test_stop_rule_matches_marginal_condition(seed):
    # [xhh]: admit iff a > tau * (S(Bt) - S(Bt+1)) / S(Bt+1)
    rng = np.random.default_rng(100 + seed)
    R, gamma = 6, 5
    c = rng.uniform(0.2, 1.0, (R, gamma))
    sps = rng.uniform(50, 100, R * (gamma + 1) + 1)   # jagged profile
    sps[0] = 0.0
    s = O.schedule(c, sps)
    a = O.survival(c).reshape(-1)
    Bt, tau = R, float(R)
    for n, i in enumerate(s["order"]):
        if Bt + 1 >= len(sps):
            break
        gain = a[i] * sps[Bt + 1]
        cost = tau * (sps[Bt] - sps[Bt + 1])
        if n < s["n_admitted"]:
            assert gain > cost * (1 - 1e-12)
            Bt, tau = Bt + 1, tau + a[i]
        else:
            assert not (gain > cost * (1 + 1e-12))
            break


def test_order_is_survival_descending_with_index_ties():
    c = np.array([[1.0, 0.5, 1.0], [0.5, 1.0, 1.0], [1.0, 1.0, 0.25]])
    s = O.schedule(c, np.full(20, 1.0))
    # survival: [1, .5, .5], [.5, .5, .5], [1, 1, .25]
    assert list(s["order"]) == [0, 6, 7, 1, 2, 3, 4, 5, 8]


@pytest.mark.parametrize("seed", range(30))
def test_admitted_sets_are_prefixes_and_counts_match(seed):
    rng = np.random.default_rng(200 + seed)
    R, gamma = 5, 6
    c = rng.uniform(0.0, 1.0, (R, gamma))
    c[rng.random((R, gamma)) < 0.2] = 1.0
    sps = rng.uniform(10, 100, R * (gamma + 1) + 1)
    sps[0] = 0
    s = O.schedule(c, sps)
    admitted = s["order"][: s["n_admitted"]]
    for r in range(R):
        js = sorted(int(i) % gamma for i in admitted if int(i) // gamma == r)
        assert js == list(range(s["ell"][r]))


@pytest.mark.parametrize("seed", range(40))
def test_non_anticipating(seed):
    # Changing confidences after position j of a request never changes
    # whether position j of that request is verified.
    rng = np.random.default_rng(300 + seed)
    R, gamma = 4, 5
    c = rng.uniform(0.05, 1.0, (R, gamma))
    sps = rng.uniform(20, 100, R * (gamma + 1) + 1)
    sps[0] = 0
    base = O.schedule(c, sps)["ell"]
    for _ in range(5):
        r, j = rng.integers(R), rng.integers(gamma)
        c2 = c.copy()
        c2[r, j + 1:] = rng.uniform(0.0, 1.0, gamma - j - 1)
        ell2 = O.schedule(c2, sps)["ell"]
        assert (base[r] >= j + 1) == (ell2[r] >= j + 1)


def test_exact_tie_is_not_admitted():
    # [xhh] scheduler Q&A: grow the verify set until Theta no longer rises, so
    # an addition that leaves Theta exactly unchanged is refused.
    # R = 1, a = 0.5: Theta(0) = 1 * 150, Theta(1) = 1.5 * 100 = 150.
    s = O.schedule(np.array([[0.5, 0.5]]), np.array([0.0, 150.0, 100.0, 90.0]))
    assert s["ell"][0] == 0 and s["n_admitted"] == 0
    # a hair more survival and it is admitted
    s = O.schedule(np.array([[0.5 + 2 ** -40, 0.5]]), np.array([0.0, 150.0, 100.0, 10.0]))
    assert s["ell"][0] == 1


def test_tau_is_exact_sum_rounded_once():
    # Ten survivals of 0.1 (not exact in binary) starting from R = 1: the
    # sequential fp64 sum drifts, the exact sum rounded once does not.
    s = O.schedule(np.ones((1, 10)), np.full(30, 5.0))
    assert s["tau"] == 11.0
    from fractions import Fraction
    a = O.survival(np.full((2, 3), 0.1))
    s = O.schedule(np.full((2, 3), 0.1), np.full(30, 5.0))
    exact = Fraction(2) + sum(Fraction(float(x)) for x in a.reshape(-1))
    assert s["tau"] == float(exact)


@pytest.mark.parametrize("seed", range(6))
def test_verify_length_falls_as_load_rises(seed):
    # [xhh] scheduler note / [billytse] 6: the admission bar rises with load.
    # With SPS(B) = c (1 - s B), admitting candidate n needs
    # a (1 - s (Bt + 1)) > tau s, harder for every candidate as s grows, so
    # no request's verify length can grow with the slope; and more requests
    # (a larger starting batch) shorten the same requests' prefixes.
    rng = np.random.default_rng(700 + seed)
    R, gamma = 48, 8
    c = rng.uniform(0.4, 1.0, (R, gamma))
    n = 4096
    prev = None
    for s in [0.0, 1e-4, 5e-4, 2e-3, 8e-3, 3e-2]:
        sps = 2400.0 * (1.0 - s * np.arange(n))
        sps[sps <= 0] = 0.0
        ell = O.schedule(c, sps)["ell"]
        if prev is not None:
            assert np.all(ell <= prev)
        prev = ell
    assert prev.sum() < R * gamma   # the steepest table really cuts
    # the same 48 requests inside a batch of 4 x 48 requests: no longer prefixes
    sps = 2400.0 * (1.0 - 5e-4 * np.arange(n))
    alone = O.schedule(c, sps)["ell"]
    crowd = O.schedule(np.concatenate([c] + [rng.uniform(0.4, 1.0, (R, gamma))
                                             for _ in range(3)]), sps)["ell"][:R]
    assert np.all(crowd <= alone) and crowd.sum() < alone.sum()
