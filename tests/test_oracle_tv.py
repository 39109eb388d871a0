"""Pins for the oracle's acceptance label c*_k = 1 - TV(p^d_k, p^t_k) (no GPU).

[weigao] part 3 and [billytse] 5.1: the label is one minus the total
variation between the draft and target distributions of the position, which
is the probability that the accept-or-resample test keeps the drafted token.

Pins: the label equals the accept mass sum_x q(x) min(1, p(x)/q(x)) (the
acceptance rule's own expectation, [billytse] 1); it equals the empirical
acceptance rate of the oracle's verification, which draws through the
Markov-biased draft, over many seeded uniforms; closed cases (p = q gives 1,
disjoint supports give 0, greedy rows give 1 exactly when the draft token is
the target argmax); symmetry and range; and which drafted token it reads (the
previous one, through the Markov bias).
"""

import math

import numpy as np
import pytest

import oracle as O


def _softmax(y):
    w = np.exp(y - y.max())
    return w / w.sum()


def _case(seed, B=3, gamma=3, V=7, rank=3, T=1.0, w=0.7, noise=0.8):
    rng = np.random.default_rng(seed)
    U = rng.normal(0, 1.0, (B, gamma, V))
    W1 = rng.normal(0, w, (V, rank))
    W2 = rng.normal(0, w, (V, rank)).T
    target = np.concatenate([U, rng.normal(0, 1.0, (B, 1, V))], axis=1)
    target = target + rng.normal(0, noise, target.shape)
    anchor = rng.integers(0, V, B)
    tokens = rng.integers(0, V, (B, gamma))
    temp = np.full(B, T)
    return U, W1, W2, target, anchor, tokens, temp


@pytest.mark.parametrize("seed", range(10))
def test_label_is_the_accept_mass(seed):
    U, W1, W2, target, anchor, tokens, temp = _case(seed, T=[0.6, 1.0, 1.7][seed % 3])
    out = O.tv_label(target, U, W1, W2, anchor, tokens, temp)
    B, gamma, V = U.shape
    for b in range(B):
        for k in range(gamma):
            prev = anchor[b] if k == 0 else tokens[b, k - 1]
            z = U[b, k] + W1[prev] @ W2
            q = _softmax(z / temp[b])
            p = _softmax(target[b, k] / temp[b])
            mass = math.fsum(q[x] * min(1.0, p[x] / q[x]) for x in range(V))
            assert abs(out["label"][b, k] - mass) < 1e-13
            assert 0.0 <= out["tv"][b, k] <= 1.0


def test_label_matches_empirical_acceptance_of_verification():
    # one request, one drafted position: the oracle's own draft and
    # verification, run on many seeded uniform sets; the drafted token
    # varies with the draw, the label is its average accept probability
    rng = np.random.default_rng(3)
    V, rank = 6, 2
    U = rng.normal(0, 1.0, (1, 1, V))
    W1 = rng.normal(0, 0.9, (V, rank))
    W2 = rng.normal(0, 0.9, (V, rank)).T
    target = rng.normal(0, 1.2, (1, 2, V))
    anchor = np.array([2])
    temp = np.array([0.9])
    n = 20000
    acc = 0
    lab = 0.0
    for _ in range(n):
        uni = rng.random((1, 2, 2))
        d = O.draft_block(U, W1, W2, anchor, temp, uni)
        v = O.verify(target, U, W1, W2, anchor, d["tokens"], d["q_tok"], temp, uni,
                     np.array([1]))
        acc += int(v["n_accepted"][0])
    # the label does not depend on which token was drafted at k = 0
    lab = O.tv_label(target, U, W1, W2, anchor, np.zeros((1, 1), dtype=int), temp)["label"][0, 0]
    rate = acc / n
    sigma = math.sqrt(lab * (1 - lab) / n)
    assert abs(rate - lab) < 5 * sigma, (rate, lab, sigma)


def test_equal_distributions_give_one_and_disjoint_give_zero():
    V = 5
    U = np.zeros((1, 2, V))
    U[0, 0] = [0.1, 0.5, -0.3, 0.2, 0.0]
    U[0, 1] = [-40.0, 40.0, -40.0, -40.0, -40.0]
    W1 = np.zeros((V, 2))
    W2 = np.zeros((2, V))
    target = np.zeros((1, 3, V))
    target[0, 0] = U[0, 0]                               # p == q
    target[0, 1] = [40.0, -40.0, -40.0, -40.0, -40.0]    # mass on another token
    out = O.tv_label(target, U, W1, W2, np.array([0]), np.array([[1, 1]]), np.array([1.0]))
    assert abs(out["label"][0, 0] - 1.0) < 1e-15
    assert out["label"][0, 1] < 1e-30


def test_greedy_rows_compare_argmaxes():
    V = 4
    U = np.zeros((2, 2, V))
    target = np.zeros((2, 3, V))
    target[:, :, 2] = 1.0
    target[1, 1, 3] = 5.0
    out = O.tv_label(target, U, np.zeros((V, 1)), np.zeros((1, V)), np.array([0, 0]),
                     np.array([[2, 2], [2, 2]]), np.array([0.0, 0.0]))
    assert out["label"].tolist() == [[1.0, 1.0], [1.0, 0.0]]


def test_total_variation_is_symmetric():
    # with no Markov bias, swapping draft and target logits keeps the label
    U, W1, W2, target, anchor, tokens, temp = _case(5)
    Z1, Z2 = np.zeros_like(W1), np.zeros_like(W2)
    a = O.tv_label(target, U, Z1, Z2, anchor, tokens, temp)["tv"]
    swapped_target = np.concatenate([U, target[:, -1:]], axis=1)
    b = O.tv_label(swapped_target, target[:, :-1], Z1, Z2, anchor, tokens, temp)["tv"]
    np.testing.assert_allclose(a, b, atol=1e-14)


def test_label_reads_the_previous_drafted_token():
    U, W1, W2, target, anchor, tokens, temp = _case(8, w=1.5)
    base = O.tv_label(target, U, W1, W2, anchor, tokens, temp)["label"]
    t2 = tokens.copy()
    t2[:, 1] = (t2[:, 1] + 1) % U.shape[2]
    moved = O.tv_label(target, U, W1, W2, anchor, t2, temp)["label"]
    # position 1's own token does not enter its label; position 2 reads it
    np.testing.assert_array_equal(base[:, :2], moved[:, :2])
    assert np.all(np.abs(base[:, 2] - moved[:, 2]) > 1e-9)
