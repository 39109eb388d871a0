"""Pins of the oracle's RNN head (the recurrent sequential bias).

[weigao] part 2 describes the head's step: the previous state, the previous
token's embedding and the position's hidden state go through one linear
layer whose output splits into gate, candidate and output;
state_k = gate * state_{k-1} + (1 - gate) * candidate; the position's bias
is W2 applied to tanh(output).  [billytse] 3.3: the recurrence lets each
position remember the whole block prefix.  The activations of gate and
candidate, the sizes, the layer's column order and the initial state are
readings (sigmoid, tanh, state size r, columns [state; embedding; hidden],
zero state at the start of each block).

Pins: a two-step recurrence worked out by hand from those definitions (exact
fractions), exhaustive enumeration showing that drafting with the RNN head
keeps the step lossless (the verify recompute at a reject uses the same
projected vector), the prefix memory the Markov head cannot have, and two
reductions (W2 = 0: the parallel drafter; gate saturated at 1: a Markov head
whose embedding is tanh of a linear map of W1).
"""

import math

import numpy as np

import oracle as O
from enum_harness import TinyStep, enumerate_law, max_law_gap, product_target_law

LN3, LN2 = math.log(3.0), math.log(2.0)


def _hand_case():
    # r = 1, H = 1, V = 2.  Columns of Wr: [state, embedding, hidden];
    # rows: [gate, candidate, output].
    W1 = np.array([[1.0], [0.0]])            # token 0 embeds to 1, token 1 to 0
    hidden = np.array([[[0.0], [1.0]]])      # h_1 = 0, h_2 = 1
    Wr = np.array([[8.0, LN3, -1.0],
                   [-8.0 * LN2, LN3 / 2.0, 0.0],
                   [0.0, LN3 / 2.0, LN2]])
    br = np.zeros(3)
    return W1, hidden, Wr, br


def test_two_steps_worked_by_hand():
    # step 1 (state 0, embedding of the anchor 0 = 1, h = 0):
    #   gate = sigmoid(ln 3) = 3/4, candidate = tanh(ln(3)/2) = 1/2,
    #   output = tanh(ln(3)/2) = 1/2, state = 3/4 * 0 + 1/4 * 1/2 = 1/8
    # step 2 (state 1/8, embedding of token 1 = 0, h = 1):
    #   gate = sigmoid(8/8 - 1) = 1/2, candidate = tanh(-ln 2) = -3/5,
    #   output = tanh(ln 2) = 3/5, state = 1/2 * 1/8 + 1/2 * (-3/5) = -19/80
    W1, hidden, Wr, br = _hand_case()
    out = O.rnn_forced(W1, hidden, Wr, br, anchor=[0], tokens=np.array([[1, 0]]))
    np.testing.assert_allclose(out["emb"][0, :, 0], [0.5, 0.6], rtol=0, atol=1e-15)
    np.testing.assert_allclose(out["state"][0, :, 0], [1.0 / 8.0, -19.0 / 80.0], rtol=0,
                               atol=1e-15)
    s1, o1 = O.rnn_step(np.zeros(1), W1[0], hidden[0, 0], Wr, br)
    assert abs(s1[0] - 0.125) < 1e-15 and abs(o1[0] - 0.5) < 1e-15


def test_drafted_bias_is_the_output_through_w2():
    # the draft's logits at each position are U + tanh(output) @ W2: with U = 0
    # and V = 2 the drafted probabilities follow from the hand values
    W1, hidden, Wr, br = _hand_case()
    W2 = np.array([[1.0, -1.0]])             # r x V
    U = np.zeros((1, 2, 2))
    uni = np.array([[[0.999, 0.5], [0.0, 0.5], [0.5, 0.5]]])
    d = O.rnn_draft_block(U, W1, W2, hidden, Wr, br, [0], [1.0], uni)
    # position 1: logits (1/2, -1/2): q(token 1) = 1 / (1 + e), drawn by u = 0.999
    assert d["tokens"][0, 0] == 1
    assert abs(d["q_tok"][0, 0] - 1.0 / (1.0 + math.e)) < 1e-15
    # position 2 (previous token 1): logits (3/5, -3/5), u = 0 draws token 0
    assert d["tokens"][0, 1] == 0
    assert abs(d["q_tok"][0, 1] - 1.0 / (1.0 + math.exp(-1.2))) < 1e-15
    np.testing.assert_allclose(d["emb"][0, :, 0], [0.5, 0.6], atol=1e-15)


def _rnn_weights(rng, r, H, scale=1.2):
    return dict(Wr=rng.normal(0.0, scale, (3 * r, 2 * r + H)), br=rng.normal(0.0, 0.5, 3 * r))


def test_rnn_head_keeps_the_step_lossless():
    # drafting with the RNN head, verifying with the q recompute from the same
    # projected vector: the emitted prefix completed by the target has the
    # target's law exactly ([billytse] 1; [xhh] acceptance rule)
    for seed, T, ell in ((3, 1.0, 2), (4, 0.7, 2), (5, 1.4, 1)):
        rng = np.random.default_rng(seed)
        R, gamma, V, r, H = 1, 2, 3, 2, 1
        w = _rnn_weights(rng, r, H)
        hidden = rng.normal(0.0, 1.0, (R, gamma, H))
        step = TinyStep(R, gamma, V, r, seed=seed, T=T, ell=[ell], w_scale=1.0,
                        rnn=dict(hidden=hidden, **w))
        law = enumerate_law(step)
        ref = product_target_law(step)
        assert max_law_gap(law, ref) < 1e-12


def test_rnn_head_lossless_for_greedy_requests():
    rng = np.random.default_rng(6)
    R, gamma, V, r, H = 1, 2, 3, 2, 1
    w = _rnn_weights(rng, r, H)
    step = TinyStep(R, gamma, V, r, seed=6, T=0.0, ell=[2], w_scale=1.0,
                    rnn=dict(hidden=rng.normal(0.0, 1.0, (R, gamma, H)), **w))
    assert max_law_gap(enumerate_law(step), product_target_law(step)) < 1e-12


def test_state_carries_the_prefix_beyond_the_previous_token():
    # two drafts that differ only in the token two positions back: the RNN
    # head's position-2 vector differs; with the state columns of the layer
    # zeroed it is a function of the previous token and h alone
    rng = np.random.default_rng(7)
    V, r, H = 6, 3, 2
    W1 = rng.normal(0.0, 1.0, (V, r))
    w = _rnn_weights(rng, r, H)
    hidden = rng.normal(0.0, 1.0, (2, 3, H))
    hidden[1] = hidden[0]
    tokens = np.array([[1, 4, 0], [2, 4, 0]])
    a = O.rnn_forced(W1, hidden, w["Wr"], w["br"], [3, 3], tokens)
    assert np.all(np.abs(a["emb"][0, 2] - a["emb"][1, 2]) > 1e-9)
    Wr0 = w["Wr"].copy()
    Wr0[:, :r] = 0.0
    b = O.rnn_forced(W1, hidden, Wr0, w["br"], [3, 3], tokens)
    np.testing.assert_array_equal(b["emb"][0, 2], b["emb"][1, 2])


def test_w2_zero_reduces_to_the_parallel_drafter():
    rng = np.random.default_rng(8)
    B, gamma, V, r, H = 3, 4, 9, 3, 2
    U = rng.normal(0.0, 1.0, (B, gamma, V))
    W1 = rng.normal(0.0, 1.0, (V, r))
    w = _rnn_weights(rng, r, H)
    hidden = rng.normal(0.0, 1.0, (B, gamma, H))
    uni = rng.random((B, gamma + 1, 2))
    T = np.array([1.0, 0.6, 0.0])
    a = O.rnn_draft_block(U, W1, np.zeros((r, V)), hidden, w["Wr"], w["br"], [0, 1, 2], T, uni)
    b = O.draft_block(U, W1, np.zeros((r, V)), [0, 1, 2], T, uni)
    np.testing.assert_array_equal(a["tokens"], b["tokens"])
    np.testing.assert_array_equal(a["q_tok"], b["q_tok"])


def test_saturated_gate_is_a_markov_head_with_a_transformed_embedding():
    # gate = 1 (sigmoid(60) rounds to 1.0) keeps the zero initial state; with
    # no hidden or state input the output is tanh(A W1[prev] + c), i.e. the
    # Markov head with embedding table tanh(W1 A^T + c)
    rng = np.random.default_rng(9)
    B, gamma, V, r, H = 2, 4, 7, 3, 2
    U = rng.normal(0.0, 1.0, (B, gamma, V))
    W1 = rng.normal(0.0, 1.0, (V, r))
    W2 = rng.normal(0.0, 1.0, (r, V))
    A = rng.normal(0.0, 1.0, (r, r))
    c = rng.normal(0.0, 0.3, r)
    Wr = np.zeros((3 * r, 2 * r + H))
    Wr[r:2 * r] = rng.normal(0.0, 1.0, (r, 2 * r + H))   # candidate: anything (gated out)
    Wr[2 * r:, r:2 * r] = A
    br = np.concatenate([np.full(r, 60.0), rng.normal(0.0, 1.0, r), c])
    hidden = rng.normal(0.0, 1.0, (B, gamma, H))
    uni = rng.random((B, gamma + 1, 2))
    T = np.array([1.0, 0.8])
    a = O.rnn_draft_block(U, W1, W2, hidden, Wr, br, [2, 5], T, uni)
    M = np.tanh(W1 @ A.T + c)
    b = O.draft_block(U, M, W2, [2, 5], T, uni)
    np.testing.assert_array_equal(a["tokens"], b["tokens"])
    np.testing.assert_allclose(a["q_tok"], b["q_tok"], rtol=1e-13)
    assert np.all(a["state"] == 0.0)


def test_bf16_rounding_of_the_projected_vector():
    # ties to even at the 8th significant bit, directly from float64
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -0.3, 0.0, 2.0 ** -130 * 1.5])
    np.testing.assert_array_equal(O.bf16_round(x),
                                  [1.0, 1.0 + 2.0 ** -6, -0.30078125, 0.0, 2.0 ** -130 * 1.5])
