"""Pins for the oracle's two further scheduler modes (no GPU).

* capacity (two-step causal barrier, [billytse] 7 and [weigao] part 4): the
  number K of verified positions is fixed from older information and the
  current candidates are ranked by their latest survival.
* threshold ([billytse] 8 threshold sweep; [xhh] scheduler Q&A): every
  position whose survival reaches a fixed threshold is verified.

Pins: the exchange characterisation of a top-K set (checked pairwise, not
by re-sorting), agreement of capacity K = n with the Theta rule whose own
count is n (the Theta rule is pinned by brute force elsewhere), exact
rational products against the threshold, closed-form edge cases, the
non-anticipation property for both modes, and exhaustive enumeration of the
step's output law with each mode in the loop (lossless).
"""

import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from enum_harness import TinyStep, enumerate_law, max_law_gap, product_target_law


def _admitted(ell, gamma):
    return {r * gamma + j for r in range(len(ell)) for j in range(int(ell[r]))}


@pytest.mark.parametrize("seed", range(30))
def test_capacity_is_the_top_k_set(seed):
    rng = np.random.default_rng(900 + seed)
    R, gamma = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    # a coarse grid makes equal survivals (ties) common
    c = rng.choice([0.0, 0.25, 0.5, 0.75, 1.0], (R, gamma))
    a = O.survival(c).reshape(-1)
    for K in range(R * gamma + 2):
        s = O.schedule_capacity(c, K)
        S = _admitted(s["ell"], gamma)
        assert len(S) == min(K, R * gamma) == s["n_admitted"]
        # every taken candidate ranks ahead of every one left out
        for x in S:
            for y in set(range(R * gamma)) - S:
                assert a[x] > a[y] or (a[x] == a[y] and x < y)


@pytest.mark.parametrize("seed", range(20))
def test_capacity_equal_to_theta_count_reproduces_theta_rule(seed):
    rng = np.random.default_rng(1000 + seed)
    R, gamma = 5, 4
    c = rng.uniform(0.05, 1.0, (R, gamma))
    sps = np.concatenate([[0.0], np.sort(rng.uniform(20, 100, R * (gamma + 1)))[::-1]])
    g = O.schedule(c, sps)
    s = O.schedule_capacity(c, float(g["n_admitted"]))
    np.testing.assert_array_equal(s["ell"], g["ell"])
    np.testing.assert_array_equal(s["order"], g["order"])
    assert s["tau"] == g["tau"]


def test_capacity_edge_values():
    c = np.array([[0.9, 0.8, 0.1], [0.7, 0.6, 0.5]])
    assert O.schedule_capacity(c, 0)["ell"].tolist() == [0, 0]
    assert O.schedule_capacity(c, -3)["ell"].tolist() == [0, 0]
    assert O.schedule_capacity(c, float("nan"))["ell"].tolist() == [0, 0]
    assert O.schedule_capacity(c, 6)["ell"].tolist() == [3, 3]
    assert O.schedule_capacity(c, 1e9)["ell"].tolist() == [3, 3]
    # survivals: r0 0.9, 0.72, 0.072; r1 0.7, 0.42, 0.21 -> ranked 0.9, 0.72, 0.7, ...
    assert O.schedule_capacity(c, 2.99)["ell"].tolist() == [2, 0]
    assert O.schedule_capacity(c, 3)["ell"].tolist() == [2, 1]
    s = O.schedule_capacity(c, 3)
    assert s["tau"] == float(Fraction(2) + Fraction(0.9) + Fraction(0.9 * 0.8) + Fraction(0.7))
    assert np.isnan(s["theta"])


@pytest.mark.parametrize("seed", range(20))
def test_threshold_against_exact_products(seed):
    # dyadic confidences: every fp64 product is exact, so the rational
    # product decides the same comparison independently of fp64 rounding
    rng = np.random.default_rng(1100 + seed)
    R, gamma = 4, 5
    c = rng.integers(0, 9, (R, gamma)) / 8.0
    for thr in [0.0, 1 / 64, 0.1, 0.25, 0.3, 0.5, 0.75, 1.0]:
        s = O.schedule_threshold(c, thr)
        for r in range(R):
            prod, L = Fraction(1), 0
            for j in range(gamma):
                prod *= Fraction(c[r, j])
                if prod >= Fraction(thr):
                    L = j + 1
                else:
                    break
            assert s["ell"][r] == L


def test_threshold_edge_values():
    c = np.array([[1.0, 0.5, 0.0], [0.25, 1.0, 1.0]])
    assert O.schedule_threshold(c, 0.0)["ell"].tolist() == [3, 3]     # a >= 0 always
    assert O.schedule_threshold(c, -1.0)["ell"].tolist() == [3, 3]
    assert O.schedule_threshold(c, 1.0)["ell"].tolist() == [1, 0]     # equality admits
    assert O.schedule_threshold(c, np.nextafter(1.0, 2.0))["ell"].tolist() == [0, 0]
    assert O.schedule_threshold(c, float("nan"))["ell"].tolist() == [0, 0]
    assert O.schedule_threshold(c, 0.25)["ell"].tolist() == [2, 3]


@pytest.mark.parametrize("mode", ["capacity", "threshold"])
@pytest.mark.parametrize("seed", range(15))
def test_modes_are_non_anticipating(mode, seed):
    # whether position j of request r is verified never depends on the
    # confidences of its later positions (with K or the threshold fixed)
    rng = np.random.default_rng(1200 + seed)
    R, gamma = 4, 5
    c = rng.uniform(0.05, 1.0, (R, gamma))
    run = ((lambda cc: O.schedule_capacity(cc, 9)) if mode == "capacity"
           else (lambda cc: O.schedule_threshold(cc, 0.3)))
    base = run(c)["ell"]
    for _ in range(8):
        r, j = rng.integers(R), rng.integers(gamma)
        c2 = c.copy()
        c2[r, j + 1:] = rng.uniform(0.0, 1.0, gamma - j - 1)
        assert (base[r] >= j + 1) == (run(c2)["ell"][r] >= j + 1)


def test_modes_order_matches_theta_rule_order():
    rng = np.random.default_rng(5)
    c = rng.choice([0.2, 0.5, 1.0], (6, 3))
    ref = O.schedule(c, np.full(40, 1.0))["order"]
    np.testing.assert_array_equal(O.schedule_capacity(c, 4)["order"], ref)
    np.testing.assert_array_equal(O.schedule_threshold(c, 0.3)["order"], ref)


@pytest.mark.parametrize("mode", ["capacity", "threshold"])
def test_lossless_with_mode_in_the_loop(mode):
    # two requests, verify lengths from the confidence head (reads the
    # previous drafted token) and the mode under test: the joint output law
    # is still the product of the targets
    R, gamma, V, rank, H = 2, 2, 3, 2, 2
    W1 = np.array([[2.0, 0.0], [0.0, 2.0], [-1.0, -1.0]])
    hidden = np.zeros((R, gamma, H))
    w = np.array([0.0, 0.0, 1.5, -1.5])
    sched = ((lambda c, sps: O.schedule_capacity(c, 2)["ell"]) if mode == "capacity"
             else (lambda c, sps: O.schedule_threshold(c, 0.45)["ell"]))
    step = TinyStep(R=R, gamma=gamma, V=V, rank=rank, seed=12, T=1.0, W1=W1, anchor=[0, 2],
                    sched=sched)
    step.conf = lambda tokens: O.confidence(hidden, step.W1, step.anchor, tokens, w)
    law = enumerate_law(step)
    ref = product_target_law(step)
    assert max_law_gap(law, ref) < 1e-12
    ells = {tuple(v[1]) for v in step._draft_cache.values()}
    assert len(ells) > 1     # the verify lengths really vary with the drafts


def test_look_ahead_capacity_rule_is_not_lossless():
    # a planted anticipating variant (rank by the survival of the NEXT
    # position, which reads the token just drafted) shifts the law: the
    # enumeration distinguishes it, so the lossless test above has teeth
    R, gamma, V, rank, H = 2, 2, 3, 2, 2
    W1 = np.array([[2.0, 0.0], [0.0, 2.0], [-1.0, -1.0]])
    hidden = np.zeros((R, gamma, H))
    w = np.array([0.0, 0.0, 1.5, -1.5])

    def peek(c, sps):
        a = O.survival(c)
        key = np.concatenate([a[:, 1:], a[:, -1:]], axis=1).reshape(-1)
        order = sorted(range(key.size), key=lambda i: (-key[i], i))
        ell = np.zeros(R, dtype=int)
        for i in order[:1]:
            ell[i // gamma] = max(ell[i // gamma], i % gamma + 1)
        return ell

    step = TinyStep(R=R, gamma=gamma, V=V, rank=rank, seed=12, T=1.0, W1=W1, anchor=[0, 2],
                    sched=peek)
    step.conf = lambda tokens: O.confidence(hidden, step.W1, step.anchor, tokens, w)
    assert max_law_gap(enumerate_law(step), product_target_law(step)) > 1e-3
