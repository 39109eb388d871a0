"""Pins for the oracle's lossless verification (no GPU).

* Exhaustive enumeration (tests/enum_harness.py): the emitted tokens,
  completed by the target, have exactly the target's sequence law (1e-12),
  for several temperatures, verify lengths, greedy rows, and with the
  confidence head and greedy scheduler in the loop across two requests.
* The acceptance identity  sum_x q(x) min(1, p(x)/q(x)) = 1 - TV(p, q)
  ([weigao] part 3, [billytse] 5.1), exact by enumeration and statistical at
  V = 64.
* The pages' printed counterexample ([xhh]): non-anticipating truncation
  keeps the first token at (0.7, 0.3); a look-ahead rule moves it to
  (0.85, 0.15) (tests/golden/non_anticipation_toy.json).
* Greedy rows reduce to argmax comparison; p == q accepts every verified
  token; a residual without mass falls back to p and is flagged.
"""

import itertools
import json
import os

import numpy as np
import pytest

import oracle as O
from enum_harness import TinyStep, enumerate_law, max_law_gap, product_target_law

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("T,ell,seed", [(1.0, 3, 0), (0.7, 3, 1), (1.6, 2, 2), (1.0, 1, 3), (1.0, 0, 4)])
def test_lossless_by_enumeration_single_request(T, ell, seed):
    step = TinyStep(R=1, gamma=3, V=4, rank=2, seed=seed, T=T, ell=[ell])
    law = enumerate_law(step)
    ref = product_target_law(step)
    assert abs(sum(law.values()) - 1.0) < 1e-12
    assert max_law_gap(law, ref) < 1e-12


def test_lossless_by_enumeration_greedy():
    step = TinyStep(R=1, gamma=3, V=4, rank=2, seed=7, T=0.0, ell=[3])
    law = enumerate_law(step)
    ref = product_target_law(step)
    assert max_law_gap(law, ref) < 1e-12


def test_lossless_with_confidence_and_scheduler_in_the_loop():
    # Two requests share the target batch; their verify lengths come from the
    # confidence head (which reads the previous drafted token) and the greedy
    # scheduler.  The joint output law must still be the product of targets.
    R, gamma, V, rank, H = 2, 2, 3, 2, 2
    # Markov embeddings chosen so the confidence swings with the previous token
    W1 = np.array([[2.0, 0.0], [0.0, 2.0], [-1.0, -1.0]])
    hidden = np.zeros((R, gamma, H))
    w = np.array([0.0, 0.0, 1.5, -1.5])
    step = TinyStep(R=R, gamma=gamma, V=V, rank=rank, seed=12, T=1.0, W1=W1, anchor=[0, 2])
    step.conf = lambda tokens: O.confidence(hidden, step.W1, step.anchor, tokens, w)
    step.sps = np.array([0.0, 100.0, 100.0, 96.0, 92.0, 80.0, 70.0, 60.0])
    law = enumerate_law(step)
    ref = product_target_law(step)
    assert max_law_gap(law, ref) < 1e-12
    # the scheduler really varies ell across draft outcomes in this setup
    ells = {tuple(v[1]) for v in step._draft_cache.values()}
    assert len(ells) > 1


def _tv(p, q):
    return 0.5 * np.abs(p - q).sum()


@pytest.mark.parametrize("seed", range(4))
def test_acceptance_identity_exact(seed):
    step = TinyStep(R=1, gamma=1, V=5, rank=2, seed=20 + seed, T=1.0, ell=[1])
    # draft distribution of position 1 and target of slot 1, by construction
    z = step.U[0, 0] + step.W1[step.anchor[0]] @ step.W2
    q = np.exp(z - z.max())
    q /= q.sum()
    p = step.ptab[0][()]
    law = enumerate_law(step)     # completed length-2 sequences
    # P(accept) integrated exactly over the cells of the draft uniform
    total = 0.0
    t = 0.0
    while t < 1.0:
        u = np.array([[[t, 0.5], [0.5, 0.5]]])
        d = O.draft_block(step.U, step.W1, step.W2, step.anchor, step.T, u)
        lo, hi = d["lo"][0, 0], d["hi"][0, 0]
        v = O.verify(step.target_logits(d["tokens"]), step.U, step.W1, step.W2, step.anchor,
                     d["tokens"], d["q_tok"], step.T, u, [1])
        total += (hi - lo) * min(1.0, v["ratio"][0, 0])
        t = hi if hi > t else np.nextafter(t, 2)
    assert abs(total - (1.0 - _tv(p, q))) < 1e-12
    assert abs(sum(law.values()) - 1.0) < 1e-12


def test_acceptance_rate_statistical_matches_closed_form():
    # W2 = 0 and a prefix-independent target: E[n_acc | ell] is
    # sum_{j<=ell} prod_{i<=j} alpha_i with alpha_i = 1 - TV(p_i, q_i).
    rng = np.random.default_rng(30)
    N, gamma, V, r = 4000, 3, 64, 4
    Ub = rng.normal(0, 1.0, (gamma, V))
    tgt = (np.concatenate([Ub, rng.normal(size=(1, V))], axis=0)
           + rng.normal(0, 0.8, (gamma + 1, V)))[None]
    U = np.broadcast_to(Ub, (N, gamma, V))
    target = np.broadcast_to(np.concatenate([tgt[0]]), (N, gamma + 1, V))
    W1 = rng.normal(size=(V, r))
    W2 = np.zeros((r, V))
    anchor = rng.integers(0, V, N)
    T = np.ones(N)
    uni = rng.random((N, gamma + 1, 2))
    d = O.draft_block(U, W1, W2, anchor, T, uni)
    v = O.verify(target, U, W1, W2, anchor, d["tokens"], d["q_tok"], T, uni, np.full(N, gamma))
    alpha = []
    for k in range(gamma):
        q = np.exp(Ub[k] - Ub[k].max()); q /= q.sum()
        p = np.exp(tgt[0, k] - tgt[0, k].max()); p /= p.sum()
        alpha.append(1.0 - _tv(p, q))
    expect = sum(np.prod(alpha[: j + 1]) for j in range(gamma))
    n = v["n_accepted"]
    se = n.std() / np.sqrt(N)
    assert abs(n.mean() - expect) < 5 * se, (n.mean(), expect, se)
    # per-position conditional acceptance
    for k in range(gamma):
        reached = n >= k
        acc = (n[reached] > k).mean()
        se_k = np.sqrt(alpha[k] * (1 - alpha[k]) / reached.sum())
        assert abs(acc - alpha[k]) < 5 * se_k


def test_non_anticipation_counterexample_printed_numbers():
    g = json.load(open(os.path.join(GOLDEN, "non_anticipation_toy.json")))
    st = g["setup"]
    V, gamma = st["V"], st["gamma"]
    U = np.zeros((1, gamma, V))
    U[0, 0] = np.log(st["q1"])
    ptab = [{(): np.array(st["p1"])}]
    rng = np.random.default_rng(40)
    for n in (1, 2):
        for pre in itertools.product(range(V), repeat=n):
            ptab[0][pre] = rng.dirichlet(np.ones(V))
    sps = np.array(st["sps"])

    def conf(tokens):
        return np.array([[st["c1"], st["c2_after"][int(tokens[0, 0])]]])

    def look_ahead(c, sps_):
        # anticipating variant: pick the best prefix of the ranked list
        # with hindsight (global maximum instead of stopping early)
        a = O.survival(c)
        flat = a.reshape(-1)
        order = sorted(range(flat.size), key=lambda i: (-flat[i], i))
        best_n, best = 0, 1.0 * sps_[1]
        tau = 1.0
        for n, i in enumerate(order, start=1):
            tau += flat[i]
            if 1 + n < len(sps_) and tau * sps_[1 + n] > best:
                best, best_n = tau * sps_[1 + n], n
        ell = np.zeros(1, dtype=int)
        for i in order[:best_n]:
            ell[i // gamma] += 1
        return ell

    kw = dict(R=1, gamma=gamma, V=V, rank=1, seed=41, T=1.0, U=U, W1=np.zeros((V, 1)),
              W2=np.zeros((1, V)), ptab=ptab, anchor=[0], sps=sps)
    early = enumerate_law(TinyStep(conf=conf, **kw))
    ahead = enumerate_law(TinyStep(conf=conf, sched=look_ahead, **kw))

    def first(law):
        f = np.zeros(V)
        for (seq,), pr in law.items():
            f[seq[0]] += pr
        return f

    np.testing.assert_allclose(first(early), g["printed"]["lossless_first_token_law"], atol=1e-12)
    np.testing.assert_allclose(first(ahead), g["printed"]["look_ahead_first_token_law"], atol=1e-12)


def test_greedy_rows_reduce_to_argmax_comparison():
    rng = np.random.default_rng(50)
    B, gamma, V, r = 6, 4, 9, 3
    U = rng.normal(size=(B, gamma, V))
    W1, W2 = rng.normal(size=(V, r)), rng.normal(size=(V, r)).T
    anchor = rng.integers(0, V, B)
    target = U[:, [0, 1, 2, 3, 3]] + rng.normal(0, 0.7, (B, gamma + 1, V))
    T = np.zeros(B)
    uni = rng.random((B, gamma + 1, 2))
    d = O.draft_block(U, W1, W2, anchor, T, uni)
    ell = rng.integers(0, gamma + 1, B)
    v = O.verify(target, U, W1, W2, anchor, d["tokens"], d["q_tok"], T, uni, ell)
    for b in range(B):
        n = 0
        while n < ell[b] and d["tokens"][b, n] == np.argmax(target[b, n]):
            n += 1
        assert v["n_accepted"][b] == n
        assert v["out_tokens"][b, n] == np.argmax(target[b, n])
        assert list(v["out_tokens"][b, :n]) == list(d["tokens"][b, :n])


def test_identical_draft_and_target_accept_everything():
    rng = np.random.default_rng(60)
    B, gamma, V, r = 5, 4, 11, 2
    U = rng.normal(size=(B, gamma, V))
    target = np.concatenate([U, rng.normal(size=(B, 1, V))], axis=1)
    W1 = rng.normal(size=(V, r))
    T = np.array([1.0, 0.5, 2.0, 1.0, 0.0])
    uni = rng.random((B, gamma + 1, 2))
    anchor = rng.integers(0, V, B)
    d = O.draft_block(U, W1, np.zeros((r, V)), anchor, T, uni)
    ell = np.array([4, 3, 0, 2, 4])
    v = O.verify(target, U, W1, np.zeros((r, V)), anchor, d["tokens"], d["q_tok"], T, uni, ell)
    np.testing.assert_array_equal(v["n_accepted"], ell)


def test_degenerate_residual_falls_back_to_target():
    # A q_tok inconsistent with the draft row (twice the true value) makes a
    # rejection possible while p == q, leaving a residual with no mass.
    V, gamma = 6, 1
    w = np.array([1.0, 2.0, 3.0, 1.0, 1.0, 2.0])
    U = np.log(w)[None, None]
    target = np.log(np.stack([w, w]))[None]
    uni = np.array([[[0.3, 0.9], [0.55, 0.0]]])
    d = O.draft_block(U, np.zeros((V, 1)), np.zeros((1, V)), [0], [1.0], uni)
    v = O.verify(target, U, np.zeros((V, 1)), np.zeros((1, V)), [0], d["tokens"],
                 2 * d["q_tok"], [1.0], uni, [1])
    assert v["n_accepted"][0] == 0 and v["degenerate"][0]
    # u = 0.55 falls in token 3's cell of p = w / 10 ([0.6, ...) is token 3's end)
    assert v["out_tokens"][0, 0] == 2
