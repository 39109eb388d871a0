"""Pins for the oracle's Markov-head drafting (no GPU).

Each test checks the oracle against something other than itself: an
explicit V x V transition matrix, probabilities fixed by construction
(logits = log of integer weights), the deterministic chain a dominant
transition forces, and the W2 = 0 special case (a purely parallel drafter).
"""

import numpy as np
import pytest

import oracle as O


def test_bias_is_row_of_explicit_transition_matrix():
    # [weigao] part 2 / [billytse] 3.3: the low-rank head stands for a V x V
    # transition matrix M = W1 @ W2; the bias for prev is M's row prev.
    rng = np.random.default_rng(1)
    V, r = 13, 5
    A = rng.normal(size=(V, r))
    Bm = rng.normal(size=(r, V))          # the r x V projection
    M = np.zeros((V, V))
    for a in range(V):                     # explicit transition matrix, entry by entry
        for b in range(V):
            M[a, b] = sum(A[a, i] * Bm[i, b] for i in range(r))
    W2 = Bm                               # stored [r, V]
    for prev in range(V):
        np.testing.assert_allclose(O.markov_bias(A, W2, prev), M[prev], rtol=0, atol=1e-12)


def test_bias_full_rank_identity_embedding_recovers_matrix():
    # With r = V and W1 = I the head is an arbitrary (non-symmetric) transition
    # matrix; a transposed operand would return columns instead of rows.
    rng = np.random.default_rng(2)
    V = 9
    M = rng.normal(size=(V, V))
    for prev in range(V):
        np.testing.assert_array_equal(O.markov_bias(np.eye(V), M, prev), M[prev])


def _cells(fn, n):
    """Black-box: lengths of the u-intervals selecting each index 0..n-1,
    found by bisecting the switch points of the monotone map u -> index."""
    lengths = np.zeros(n)
    top = np.nextafter(1.0, 0.0)
    start, cur = 0.0, fn(0.0)
    while fn(top) != cur:
        a, b = start, top
        while True:
            mid = 0.5 * (a + b)
            if mid <= a or mid >= b:
                break
            if fn(mid) == cur:
                a = mid
            else:
                b = mid
        lengths[cur] += b - start
        start, cur = b, fn(b)
    lengths[cur] += 1.0 - start
    return lengths


@pytest.mark.parametrize("T,power", [(1.0, 1), (0.5, 2), (2.0, 0.5)])
def test_inverse_cdf_draw_has_the_softmax_probabilities(T, power):
    # logits = log(w) make softmax(logits / T) = w**(1/T) / sum, a closed form.
    w = np.array([1.0, 2.0, 3.0, 4.0, 0.5])
    p = w ** power / np.sum(w ** power)
    z = np.log(w)
    lengths = _cells(lambda u: O.draft_row(z, T, u)["x"], len(w))
    np.testing.assert_allclose(lengths, p, rtol=0, atol=1e-13)
    for u in (0.0, 0.3, 0.77, 1 - 2 ** -24):
        d = O.draft_row(z, T, u)
        assert abs(d["q"] - p[d["x"]]) < 1e-14
        assert abs(d["m"] - np.max(z) / T) < 1e-14
        assert abs(d["logZ"] - np.log(np.sum(w ** power) / np.max(w) ** power)) < 1e-13
        assert d["lo"] <= u < d["hi"]


def test_lowest_index_convention_and_zero_weight_never_drawn():
    w = np.array([0.0, 1.0, 0.0, 3.0])
    x, lo, hi, _ = O.inverse_cdf(w, 0.0)
    assert (x, lo, hi) == (1, 0.0, 0.25)
    assert O.inverse_cdf(w, 0.25)[0] == 3      # boundary belongs to the next cell
    assert O.inverse_cdf(w, 0.2499999)[0] == 1


def test_greedy_is_lowest_index_argmax():
    z = np.array([0.1, 2.0, -1.0, 2.0])
    for u in (0.0, 0.5, 0.999):
        d = O.draft_row(z, 0.0, u)
        assert d["x"] == 1 and d["q"] == 1.0 and d["m"] == 2.0


def test_block_follows_a_dominant_transition_chain():
    # [billytse] 3.3 loop: the bias at position k comes from the token sampled
    # at k-1 (the anchor at k = 0).  A transition matrix that sends a -> a+3
    # with overwhelming weight forces the chain anchor+3, anchor+6, ...
    V, gamma, B = 11, 6, 3
    M = np.full((V, V), -60.0)
    for a in range(V):
        M[a, (a + 3) % V] = 60.0
    U = np.zeros((B, gamma, V))
    anchor = np.array([0, 4, 10])
    rng = np.random.default_rng(3)
    uni = rng.random((B, gamma + 1, 2))
    out = O.draft_block(U, np.eye(V), M, anchor, np.ones(B), uni)
    for b in range(B):
        expect = [(anchor[b] + 3 * (k + 1)) % V for k in range(gamma)]
        assert list(out["tokens"][b]) == expect


def test_w2_zero_is_a_parallel_drafter():
    # [billytse] 2.2: without the sequential head every position is an
    # independent softmax of its base logits; the anchor and earlier draws
    # cannot matter, and the interval of each draw is the softmax mass.
    rng = np.random.default_rng(4)
    B, gamma, V, r = 2, 4, 6, 3
    wts = rng.integers(1, 9, size=(B, gamma, V)).astype(float)
    U = np.log(wts)
    W1 = rng.normal(size=(V, r))
    uni = rng.random((B, gamma + 1, 2))
    a = O.draft_block(U, W1, np.zeros((r, V)), np.array([0, 1]), np.ones(B), uni)
    b = O.draft_block(U, W1, np.zeros((r, V)), np.array([5, 2]), np.ones(B), uni)
    np.testing.assert_array_equal(a["tokens"], b["tokens"])
    for bb in range(B):
        for k in range(gamma):
            p = wts[bb, k] / wts[bb, k].sum()
            x = a["tokens"][bb, k]
            assert abs(a["q_tok"][bb, k] - p[x]) < 1e-14
            assert abs(a["lo"][bb, k] - p[:x].sum()) < 1e-14
            assert abs(a["hi"][bb, k] - p[: x + 1].sum()) < 1e-14


def test_forced_draft_matches_free_draft_on_its_own_tokens():
    rng = np.random.default_rng(5)
    B, gamma, V, r = 3, 4, 17, 4
    U = rng.normal(size=(B, gamma, V))
    W1, W2 = rng.normal(size=(V, r)), rng.normal(size=(V, r)).T
    anchor = rng.integers(0, V, B)
    T = np.array([1.0, 0.6, 0.0])
    uni = rng.random((B, gamma + 1, 2))
    free = O.draft_block(U, W1, W2, anchor, T, uni)
    forced = O.draft_forced(U, W1, W2, anchor, T, free["tokens"], uniforms=uni)
    for d in forced:
        b, k = d["b"], d["k"]
        assert d["x_oracle"] == free["tokens"][b, k]
        assert d["q"] == free["q_tok"][b, k]
        assert d["m"] == free["row_max"][b, k] and d["logZ"] == free["row_logZ"][b, k]


def test_bf16_decode_is_exact():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x7F7F, 0x0001], dtype=np.uint16)
    vals = O.f64(bits)
    assert vals[0] == 1.0 and vals[1] == -2.0 and vals[2] == 0.0
    assert vals[3] == float(np.float32(3.3895313892515355e38))
    assert vals[4] == 2.0 ** -133
