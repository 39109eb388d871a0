"""Pins for the oracle's confidence head (no GPU).

The head is a linear layer on [h_k ; W1[prev]] followed by a sigmoid
([weigao] part 3, [billytse] 5).  The pins use exact sigmoid values, weight
vectors that read off one input coordinate, and an embedding that encodes
the token id, which shows which token feeds each position ([xhh] note on
non-anticipating truncation: position k reads x_{k-1}, never x_k).
"""

import numpy as np

import oracle as O


def _setup(B=2, gamma=4, H=6, V=10, r=3, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.normal(size=(B, gamma, H)), rng.normal(size=(V, r)),
            rng.integers(0, V, B), rng.integers(0, V, (B, gamma)))


def test_zero_weight_gives_one_half():
    h, W1, anchor, tok = _setup()
    c = O.confidence(h, W1, anchor, tok, np.zeros(6 + 3))
    assert np.all(c == 0.5)


def test_exact_sigmoid_values():
    # logit log 3 -> 3/4 exactly up to rounding; logit -log 3 -> 1/4
    B, gamma, H, V, r = 1, 2, 1, 4, 1
    h = np.array([[[np.log(3.0)], [-np.log(3.0)]]])
    c = O.confidence(h, np.zeros((V, r)), [0], [[0, 0]], np.array([1.0, 0.0]))
    np.testing.assert_allclose(c[0], [0.75, 0.25], rtol=0, atol=1e-15)
    c2 = O.confidence(h, np.zeros((V, r)), [0], [[0, 0]], np.array([1.0, 0.0]), b0=np.log(3.0))
    np.testing.assert_allclose(c2[0], [0.9, 0.5], rtol=0, atol=1e-15)


def test_hidden_part_reads_the_position_hidden_state():
    h, W1, anchor, tok = _setup()
    for j in range(6):
        w = np.zeros(9)
        w[j] = 1.0
        c = O.confidence(h, W1, anchor, tok, w)
        np.testing.assert_allclose(np.log(c / (1 - c)), h[:, :, j], rtol=0, atol=1e-12)


def test_markov_part_reads_previous_token_not_current():
    # W1[v] = (v, 0, 0): the Markov part of the logit equals the prev id.
    B, gamma, H, V, r = 3, 5, 2, 12, 3
    W1 = np.zeros((V, r))
    W1[:, 0] = np.arange(V) * 0.25
    w = np.zeros(H + r)
    w[H] = 4.0
    h = np.zeros((B, gamma, H))
    anchor = np.array([7, 0, 11])
    tok = np.array([[1, 2, 3, 4, 5], [11, 10, 9, 8, 7], [0, 0, 6, 6, 2]])
    c = O.confidence(h, W1, anchor, tok, w)
    prev_ids = np.log(c / (1 - c))
    expect = np.concatenate([anchor[:, None], tok[:, :-1]], axis=1)
    np.testing.assert_allclose(prev_ids, expect, rtol=0, atol=1e-9)


def test_sigmoid_symmetry_and_range():
    h, W1, anchor, tok = _setup(seed=3)
    rng = np.random.default_rng(9)
    w = rng.normal(size=9) * 3
    c = O.confidence(h, W1, anchor, tok, w)
    c_neg = O.confidence(h, W1, anchor, tok, -w)
    np.testing.assert_allclose(c + c_neg, 1.0, rtol=0, atol=1e-15)
    assert np.all((c > 0) & (c < 1))
