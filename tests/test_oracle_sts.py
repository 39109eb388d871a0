"""Pins of the oracle's sequential temperature scaling (STS).

[billytse] 5.2: the raw confidence head ranks well (ROC-AUC 0.81-0.90) but is
overconfident (ECE 3-8%); STS calibrates the cumulative probability from
left to right and brings the mean ECE to about 1%.  [weigao] part 3: the
scheduler needs absolute probabilities.  The pages give no formula; the
reading is one temperature per block position dividing that position's
logit, fitted left to right against the cumulative survival.

Pins: T = 1 is the identity, closed-form values, the limits, the prefix
and non-anticipation properties with calibrated survival, the fit recovering
known temperatures from synthetic calibration drafts (and lowering the ECE
of the cumulative survival), and exhaustive enumeration with calibrated
confidences driving the scheduler (lossless to 1e-12).
"""

import math

import numpy as np

import oracle as O
from enum_harness import TinyStep, enumerate_law, max_law_gap, product_target_law


def _head(seed, B=3, gamma=4, H=8, V=11, r=4):
    rng = np.random.default_rng(seed)
    return (rng.normal(size=(B, gamma, H)), rng.normal(size=(V, r)), rng.integers(0, V, B),
            rng.integers(0, V, (B, gamma)), rng.normal(0.0, 0.7, H + r))


def test_unit_temperature_is_the_plain_head():
    h, W1, anchor, tokens, w = _head(0)
    a = O.confidence(h, W1, anchor, tokens, w, 0.3)
    b = O.confidence_sts(h, W1, anchor, tokens, w, 0.3, np.ones(4))
    np.testing.assert_allclose(a, b, rtol=1e-15, atol=0)


def test_closed_form_values():
    # sigmoid(2 ln 3 / 2) = 3/4; sigmoid(-ln 4 / 0.5) = 1/17; sigmoid(0 / T) = 1/2
    z = np.array([[2.0 * math.log(3.0), -math.log(4.0), 0.0]])
    c = O.sts_apply(z, [2.0, 0.5, 7.0])
    np.testing.assert_allclose(c[0], [0.75, 1.0 / 17.0, 0.5], rtol=0, atol=1e-15)


def test_limits():
    z = np.array([[1.3, -0.4]])
    np.testing.assert_allclose(O.sts_apply(z, [1e9, 1e9]), [[0.5, 0.5]], atol=1e-9)
    np.testing.assert_allclose(O.sts_apply(z, [1e-9, 1e-9]), [[1.0, 0.0]], atol=1e-12)


def test_calibrated_survival_keeps_prefixes_and_reads_no_later_position():
    rng = np.random.default_rng(2)
    z = rng.normal(0.0, 2.0, (20, 6))
    T = np.array([0.7, 1.0, 1.8, 2.5, 3.0, 0.4])
    c = O.sts_apply(z, T)
    a = O.survival(c)
    assert np.all(np.diff(a, axis=1) <= 0.0)
    ell = O.schedule(c, 2400.0 * (1 - 0.55 * np.arange(200) / 200.0))["ell"]
    assert np.all((ell >= 0) & (ell <= 6))
    # position j's calibrated value depends on z_j and T_j alone
    z2 = z.copy()
    z2[:, 3:] += 5.0
    T2 = T.copy()
    T2[3:] = 9.0
    np.testing.assert_array_equal(O.sts_apply(z2, T2)[:, :3], c[:, :3])


def _calibration_drafts(seed, N, t_true):
    """Synthetic calibration drafts of an overconfident head: the target
    accepts position j (given the earlier ones) with probability
    sigmoid(z_j / T*_j) while the raw head reports sigmoid(z_j)."""
    rng = np.random.default_rng(seed)
    gamma = len(t_true)
    z = rng.normal(1.5, 2.0, (N, gamma))
    p = O.sts_apply(z, t_true)
    u = rng.random((N, gamma))
    passed = u < p
    n_acc = np.where(passed.all(axis=1), gamma, np.argmin(passed, axis=1))
    return z, n_acc


def test_fit_recovers_known_temperatures_and_lowers_ece():
    t_true = np.array([1.5, 2.0, 2.6, 3.2])
    z, n_acc = _calibration_drafts(7, 40000, t_true)
    T = O.sts_fit(z, n_acc)
    np.testing.assert_allclose(T, t_true, rtol=0.08)
    labels = np.stack([(n_acc > j) for j in range(4)], axis=1).astype(float)
    raw = O.survival(O.sts_apply(z, np.ones(4)))
    cal = O.survival(O.sts_apply(z, T))
    assert O.ece(raw, labels) > 0.03
    assert O.ece(cal, labels) < 0.01


def test_ece_closed_form():
    # one bin at 0.8 with 3 of 4 labels positive: |0.75 - 0.8| = 0.05
    assert abs(O.ece([0.8, 0.8, 0.8, 0.8], [1, 1, 1, 0], bins=10) - 0.05) < 1e-15
    assert O.ece([0.25, 0.75], [0.0, 1.0], bins=2) == 0.25


def test_calibrated_confidences_keep_the_step_lossless():
    # the scheduler driven by STS-calibrated confidences of the previous token
    # (non-anticipating): the emitted tokens keep the target's law exactly
    rng = np.random.default_rng(11)
    V, gamma = 3, 2
    zt = rng.normal(0.0, 2.0, V)
    T = np.array([0.6, 2.2])

    def conf(tokens):
        R = tokens.shape[0]
        z = np.zeros((R, gamma))
        for r in range(R):
            z[r, 0] = zt[(r + 1) % V]
            z[r, 1] = zt[int(tokens[r, 0])]
        return O.sts_apply(z, T)

    sps = np.array([0.0, 100.0, 90.0, 70.0, 52.0, 40.0, 30.0])
    step = TinyStep(2, gamma, V, 2, seed=12, T=1.0, conf=conf, sps=sps)
    assert max_law_gap(enumerate_law(step), product_target_law(step)) < 1e-12
