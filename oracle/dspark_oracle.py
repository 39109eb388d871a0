"""Plain, slow fp64 CPU oracle of one DSpark draft-and-verify sampling step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything under
``oracle/``.  The GPU library never calls it and shares no code with it.

Sources (three web pages on DSpark; cited by site and section):

* [weigao]   weigao.cc, "DSpark 与 MTP：DeepSeek 投机解码调研",
             section "DSpark 的核心设计" (parts 2 Markov head, 3 confidence
             head, 4 hardware-aware prefix scheduler).
* [billytse] billytse.dev, "DSpark：DeepSeek 點樣「一次估多個、驗證前綴、
             錯咗即修正」", sections 1 (Guess -> Verify -> Fix), 3.2/3.3
             (sequential head, Markov head and its sampling loop), 5
             (confidence head), 6 (hardware-aware prefix scheduler), 7
             (lossless scheduling).
* [xhh]      xhh.club, "DeepSeek-V4.1 模型结构（6）：解码，DSpark", the
             Q&A on the acceptance rule and on the scheduler, and the
             note on non-anticipating truncation.

Everything is computed in float64 from the exact values of the stored
inputs (bf16 bit patterns are decoded exactly).  Positions are 0-based in
storage: draft position k (0..gamma-1) draws token x_{k+1} of the pages.

Uniform layout (the pages fix none; this is the reading used throughout):
``uniforms[b, k, 0]`` draws draft token k, ``uniforms[b, k, 1]`` is the
accept test of draft token k, ``uniforms[b, gamma, 0]`` draws the single
final token (residual or bonus); ``uniforms[b, gamma, 1]`` is unused.

Every function below is pinned by tests under ``tests/test_oracle_*.py``
against values the pages print, closed forms, textbook special cases and
exhaustive enumeration; no function here is "parity unpinned".
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

__all__ = [
    "f64",
    "markov_bias",
    "inverse_cdf",
    "draft_row",
    "draft_block",
    "draft_forced",
    "confidence",
    "survival",
    "schedule",
    "schedule_capacity",
    "schedule_threshold",
    "target_probs",
    "verify",
    "tv_label",
    "bf16_round",
    "rnn_step",
    "rnn_draft_block",
    "rnn_forced",
    "confidence_logits",
    "sts_apply",
    "confidence_sts",
    "sts_fit",
    "ece",
]


# ----------------------------------------------------------------------------
# input decoding
# ----------------------------------------------------------------------------

def f64(a) -> np.ndarray:
    """Exact float64 value of an input array.

    ``uint16`` arrays are bf16 bit patterns: the bf16 value is the float32
    whose upper 16 bits are the pattern and whose lower 16 bits are zero.
    """
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


# ----------------------------------------------------------------------------
# (1) semi-autoregressive block drafting with the vanilla Markov head
# ----------------------------------------------------------------------------

def markov_bias(W1, W2, prev: int) -> np.ndarray:
    """Transition bias B(prev, .) = W1[prev] @ W2 over the whole vocabulary.

    [weigao] part 2 and [billytse] 3.3: the V x V first-order transition
    matrix is replaced by a rank-r product; the row for the previous token is
    the previous token's r-vector times the r x V projection ``W2`` [r, V],
    so bias[v] = sum_i W1[prev, i] * W2[i, v].
    """
    W1 = f64(W1) if not (isinstance(W1, np.ndarray) and W1.dtype == np.float64) else W1
    W2 = f64(W2) if not (isinstance(W2, np.ndarray) and W2.dtype == np.float64) else W2
    return W1[int(prev)] @ W2


def inverse_cdf(weights: np.ndarray, u: float):
    """Inverse-CDF draw from non-negative ``weights`` with one uniform ``u``.

    Returns ``(x, lo, hi, total)``: x is the lowest index whose cumulative
    weight exceeds u * total; [lo, hi) is the interval of u (in probability
    units) that selects x.  Index order is ascending, so a zero-weight entry
    can never be drawn.
    """
    C = np.cumsum(weights)
    total = C[-1]
    target = u * total
    x = int(np.searchsorted(C, target, side="right"))
    if x >= len(C):  # only reachable through rounding when u is 1 - ulp
        x = int(np.nonzero(weights > 0)[0][-1])
    lo = (C[x - 1] if x > 0 else 0.0) / total
    hi = C[x] / total
    return x, lo, hi, total


def draft_row(z: np.ndarray, temperature: float, u: float):
    """Sample one draft position from full logits z = U_k + bias.

    [billytse] 3.2: p_k = softmax(U_k + B_k).  Temperature T divides the
    logits; T == 0 is greedy (lowest-index argmax, q one-hot).
    Returns dict with x, q (probability of x), m (max of z/T), logZ
    (log of sum exp(z/T - m)), and the selecting interval [lo, hi) of u.
    """
    if temperature > 0.0:
        y = z / temperature
        m = float(np.max(y))
        w = np.exp(y - m)
        x, lo, hi, Z = inverse_cdf(w, u)
        return dict(x=x, q=float(w[x] / Z), m=m, logZ=float(np.log(Z)), lo=lo, hi=hi)
    m = float(np.max(z))
    x = int(np.argmax(z))  # first maximum
    return dict(x=x, q=1.0, m=m, logZ=0.0, lo=0.0, hi=1.0)


def draft_block(U, W1, W2, anchor, temperature, uniforms):
    """Sequential Markov sampling over a block, per request.

    [billytse] 3.3 sampling loop: start from the anchor token; at each block
    position add the bias of the previous sampled token to the position's
    base logits, take the softmax, sample, and make the sample the next
    previous token.

    U: [B, gamma, V]; W1: [V, r]; W2: [r, V]; anchor: [B]; temperature: [B];
    uniforms: [B, gamma+1, 2].  Returns arrays tokens [B,gamma] int64,
    q_tok, row_max, row_logZ, lo, hi, margin [B,gamma] float64.  ``margin``
    is the distance of u from the nearest edge of x's interval.
    """
    U = f64(U)
    W1 = f64(W1)
    W2 = f64(W2)
    uni = np.asarray(uniforms, dtype=np.float64)
    B, gamma, V = U.shape
    out = {k: np.zeros((B, gamma)) for k in ("q_tok", "row_max", "row_logZ", "lo", "hi", "margin")}
    tokens = np.zeros((B, gamma), dtype=np.int64)
    for b in range(B):
        prev = int(anchor[b])
        T = float(temperature[b])
        for k in range(gamma):
            z = U[b, k] + markov_bias(W1, W2, prev)
            u = float(uni[b, k, 0])
            r = draft_row(z, T, u)
            tokens[b, k] = r["x"]
            out["q_tok"][b, k] = r["q"]
            out["row_max"][b, k] = r["m"]
            out["row_logZ"][b, k] = r["logZ"]
            out["lo"][b, k] = r["lo"]
            out["hi"][b, k] = r["hi"]
            whole = r["lo"] <= 0.0 and r["hi"] >= 1.0
            out["margin"][b, k] = np.inf if whole else min(u - r["lo"], r["hi"] - u)
            prev = r["x"]
    out["tokens"] = tokens
    return out


def draft_forced(U, W1, W2, anchor, temperature, tokens, uniforms=None, rows=None, emb=None):
    """Draft statistics with the sampled tokens given (teacher forcing).

    Computes, for the listed (b, k) rows (all rows if ``rows`` is None), the
    draft distribution of position k with prev = tokens[b, k-1] (anchor for
    k == 0), and reports q at tokens[b, k], the row stats, the interval of u
    that selects tokens[b, k] and, when uniforms are given, the token the
    oracle itself would draw with uniforms[b, k, 0] and its margin.

    ``emb`` [B, gamma, r] (optional): the vector each position projects
    through W2 (the RNN head's output); the bias of (b, k) is then
    emb[b, k] @ W2 instead of the Markov head's W1[prev] @ W2.
    """
    U_is64 = isinstance(U, np.ndarray) and U.dtype == np.float64
    W1 = W1 if (isinstance(W1, np.ndarray) and W1.dtype == np.float64) else f64(W1)
    W2 = W2 if (isinstance(W2, np.ndarray) and W2.dtype == np.float64) else f64(W2)
    B, gamma = np.asarray(tokens).shape
    if rows is None:
        rows = [(b, k) for b in range(B) for k in range(gamma)]
    res = []
    for b, k in rows:
        prev = int(anchor[b]) if k == 0 else int(tokens[b, k - 1])
        Urow = U[b, k] if U_is64 else f64(U[b, k])
        z = Urow + (markov_bias(W1, W2, prev) if emb is None else f64(emb[b, k]) @ W2)
        T = float(temperature[b])
        x = int(tokens[b, k])
        if T > 0:
            y = z / T
            m = float(np.max(y))
            w = np.exp(y - m)
            C = np.cumsum(w)
            Z = C[-1]
            lo = (C[x - 1] if x > 0 else 0.0) / Z
            hi = C[x] / Z
            d = dict(b=b, k=k, q=float(w[x] / Z), m=m, logZ=float(np.log(Z)), lo=lo, hi=hi)
            if uniforms is not None:
                u = float(uniforms[b, k, 0])
                xo, lo2, hi2, _ = inverse_cdf(w, u)
                whole = lo2 <= 0.0 and hi2 >= 1.0
                d.update(x_oracle=xo, margin=np.inf if whole else min(u - lo2, hi2 - u))
        else:
            m = float(np.max(z))
            am = int(np.argmax(z))
            d = dict(b=b, k=k, q=1.0 if x == am else 0.0, m=m, logZ=0.0, lo=0.0, hi=1.0)
            if uniforms is not None:
                d.update(x_oracle=am, margin=np.inf)
        res.append(d)
    return res


# ----------------------------------------------------------------------------
# (2) confidence head
# ----------------------------------------------------------------------------

def confidence(hidden, W1, anchor, tokens, w, b0: float = 0.0) -> np.ndarray:
    """c[b,k] = sigmoid(w . [h_k ; W1[prev_k]] + b0).

    [weigao] part 3 and [billytse] 5: a linear layer on the concatenation of
    the position's hidden state and the Markov embedding of the previous
    token, squashed to a probability.  [xhh] (non-anticipating truncation):
    the previous token is x_{k-1}, never x_k; the anchor for the first
    position.  The Markov embedding is the W1 row of the previous token.
    """
    h = f64(hidden)
    W1 = f64(W1)
    w = f64(w)
    B, gamma, H = h.shape
    tokens = np.asarray(tokens)
    c = np.zeros((B, gamma))
    for b in range(B):
        for k in range(gamma):
            prev = int(anchor[b]) if k == 0 else int(tokens[b, k - 1])
            feat = np.concatenate([h[b, k], W1[prev]])
            logit = float(np.dot(w, feat)) + b0
            c[b, k] = 1.0 / (1.0 + np.exp(-logit))
    return c


# ----------------------------------------------------------------------------
# (3) hardware-aware prefix scheduler
# ----------------------------------------------------------------------------

def survival(c) -> np.ndarray:
    """a[r, j] = prod_{i <= j} c[r, i], accumulated left to right in fp64.

    [weigao] part 4 / [billytse] 5: only a contiguous prefix can be accepted,
    so a draft position survives only if it and every earlier one pass.
    """
    c = np.asarray(c, dtype=np.float64)
    R, gamma = c.shape
    a = np.zeros((R, gamma))
    for r in range(R):
        acc = 1.0
        for j in range(gamma):
            acc = acc * c[r, j]
            a[r, j] = acc
    return a


def schedule(c, sps):
    """Greedy verify-length choice maximising Theta = tau * SPS(Bt).

    [billytse] 6: Bt = sum_r (1 + l_r) target tokens, tau = sum_r (1 + sum_{j
    <= l_r} a_{r,j}) expected committed tokens; rank every extendable
    position by survival, add them one at a time, and stop as soon as adding
    the next one would not raise Theta ([xhh] scheduler Q&A: stop when Theta
    no longer rises, so admission needs a strict rise; [billytse] 7: stop
    early, never revise an earlier decision).

    Ties in survival are broken by flat index r*gamma + j ascending.  SPS
    entries that are absent (Bt beyond the table) or not positive are
    inadmissible: the scan stops there.  tau is the exact (rational) sum of
    R and the admitted survivals, rounded once to fp64, so it does not depend
    on any summation order; Theta = tau * SPS[Bt] is one fp64 product.

    c: [R, gamma] (any float), sps: 1-D table indexed by Bt.
    Returns dict(ell [R] int64, order [R*gamma] int64, n_admitted, tau,
    theta, a [R, gamma]).
    """
    a = survival(c)
    R, gamma = a.shape
    sps = np.asarray(sps, dtype=np.float64)
    flat = a.reshape(-1)
    order = sorted(range(R * gamma), key=lambda i: (-flat[i], i))
    Bt = R
    exact = Fraction(R)
    tau = float(R)
    theta = tau * sps[Bt] if Bt < len(sps) else 0.0
    ell = np.zeros(R, dtype=np.int64)
    n = 0
    for i in order:
        nb = Bt + 1
        if nb >= len(sps) or not (sps[nb] > 0.0):
            break
        exact_new = exact + Fraction(float(flat[i]))
        tau_new = float(exact_new)
        theta_new = tau_new * sps[nb]
        if theta_new > theta:
            ell[i // gamma] += 1
            Bt, tau, theta, exact = nb, tau_new, theta_new, exact_new
            n += 1
        else:
            break
    return dict(ell=ell, order=np.asarray(order, dtype=np.int64), n_admitted=n,
                tau=tau, theta=theta, a=a)


def _ranked(a):
    """Flat ids of every candidate by survival descending, flat id ascending."""
    flat = a.reshape(-1)
    return flat, sorted(range(flat.size), key=lambda i: (-flat[i], i))


def _admit_prefix(a, order, n):
    """ell and tau when the first n ranked candidates are verified."""
    R, gamma = a.shape
    flat = a.reshape(-1)
    ell = np.zeros(R, dtype=np.int64)
    exact = Fraction(R)
    for i in order[:n]:
        ell[i // gamma] += 1
        exact += Fraction(float(flat[i]))
    return ell, float(exact)


def schedule_capacity(c, capacity):
    """Verify the top-K candidates, K fixed beforehand (two-step barrier).

    [billytse] 7 and [weigao] part 4 (asynchronous scheduling): the size of
    the next target batch is decided from the predictions of two steps
    earlier, so it is known before the current drafts exist; the current
    candidates are still ranked by their latest cumulative confidence, and
    the old information only fixes how many of them (K) are taken.  Whether
    candidate (r, j) is taken then depends only on how many candidates rank
    ahead of it, none of which is a later position of request r.

    capacity: K as a real number (the count an earlier Theta-greedy admitted,
    for example); it is floored and clamped to [0, R*gamma]; NaN or negative
    means 0.  Returns the fields of ``schedule`` with theta = NaN (no SPS
    table is involved).
    """
    a = survival(c)
    R, gamma = a.shape
    _, order = _ranked(a)
    K = float(capacity)
    n = 0 if not (K >= 1.0) else int(min(np.floor(K), R * gamma))
    ell, tau = _admit_prefix(a, order, n)
    return dict(ell=ell, order=np.asarray(order, dtype=np.int64), n_admitted=n, tau=tau,
                theta=float("nan"), a=a)


def schedule_threshold(c, threshold):
    """Verify every candidate whose survival is at least a fixed threshold.

    [billytse] 8 (offline threshold sweep on confidence) and [xhh] scheduler
    Q&A (a fixed threshold, unlike the Theta rule, does not follow the
    load): candidate (r, j) is verified iff a[r, j] >= threshold.  Survival
    never rises along a request's positions, so each request's verified set
    is a prefix, and the decision for (r, j) reads only c[r, :j+1].
    A NaN threshold verifies nothing.  Returns the fields of ``schedule``
    with theta = NaN.
    """
    a = survival(c)
    R, gamma = a.shape
    flat, order = _ranked(a)
    thr = float(threshold)
    n = 0
    for i in order:
        if not (flat[i] >= thr):
            break
        n += 1
    ell, tau = _admit_prefix(a, order, n)
    return dict(ell=ell, order=np.asarray(order, dtype=np.int64), n_admitted=n, tau=tau,
                theta=float("nan"), a=a)


# ----------------------------------------------------------------------------
# (4) lossless verification
# ----------------------------------------------------------------------------

def target_probs(trow: np.ndarray, temperature: float) -> np.ndarray:
    """Target distribution of one slot: softmax(t / T), or one-hot at the
    lowest-index argmax when T == 0 (greedy)."""
    if temperature > 0.0:
        y = trow / temperature
        w = np.exp(y - np.max(y))
        return w / np.sum(w)
    p = np.zeros_like(trow)
    p[int(np.argmax(trow))] = 1.0
    return p


def _draft_probs(z: np.ndarray, temperature: float) -> np.ndarray:
    if temperature > 0.0:
        y = z / temperature
        w = np.exp(y - np.max(y))
        return w / np.sum(w)
    q = np.zeros_like(z)
    q[int(np.argmax(z))] = 1.0
    return q


def verify(target, U, W1, W2, anchor, tokens, q_tok, temperature, uniforms, ell,
           requests=None, keep_final=False, emb=None):
    """Speculative rejection sampling over each request's verified prefix.

    [billytse] 1 and [xhh] acceptance-rule Q&A: draft token x_k (drawn from
    q) is accepted with probability min(1, p(x)/q(x)); the scan stops at the
    first rejection, where one token is drawn from the normalised residual
    max(0, p - q); if every verified token passes, one bonus token is drawn
    from the target slot after the last verified one.  The emitted tokens
    are the accepted prefix plus that one token.

    ``q_tok[b, k]`` is the draft probability of tokens[b, k].  At a reject
    the full draft row q is recomputed from U, W1, W2 and the previous
    token.  Accept iff u < p/q (written u*q < p; a ratio >= 1 always passes
    since u < 1).  A residual with no mass (reachable only by rounding) falls
    back to p and is flagged in ``degenerate``.

    target: [B, gamma+1, V] slot logits (slot k verifies tokens[:, k]; slot
    ell_b is the bonus slot).  Returns dict(out_tokens [B, gamma+1] (-1
    padded), n_accepted [B], ratio [B, gamma] (NaN where untested),
    final_lo, final_hi, final_margin [B], degenerate [B] bool).
    ``requests`` restricts the work to those request indices (others stay at
    their fill values); ``keep_final`` also returns, per processed request,
    the normalised cumulative distribution of the final draw (``final_cdf``).
    ``emb`` [B, gamma, r]: the drafter's projected vectors (RNN head); the
    q recompute at a reject j then uses emb[b, j] @ W2 as its bias.
    """
    W1 = W1 if (isinstance(W1, np.ndarray) and W1.dtype == np.float64) else f64(W1)
    W2 = W2 if (isinstance(W2, np.ndarray) and W2.dtype == np.float64) else f64(W2)
    tokens = np.asarray(tokens)
    B, gamma = tokens.shape
    q_tok = np.asarray(q_tok, dtype=np.float64)
    uni = np.asarray(uniforms, dtype=np.float64)
    out = np.full((B, gamma + 1), -1, dtype=np.int64)
    n_acc = np.zeros(B, dtype=np.int64)
    ratio = np.full((B, gamma), np.nan)
    f_lo = np.zeros(B)
    f_hi = np.zeros(B)
    f_margin = np.zeros(B)
    degenerate = np.zeros(B, dtype=bool)
    final_cdf = {}
    for b in (range(B) if requests is None else requests):
        T = float(temperature[b])
        L = int(ell[b])
        uf = float(uni[b, gamma, 0])
        rejected_at = -1
        for k in range(L):
            p = target_probs(f64(target[b, k]), T)
            x = int(tokens[b, k])
            ratio[b, k] = p[x] / q_tok[b, k]
            if uni[b, k, 1] * q_tok[b, k] < p[x]:
                continue
            rejected_at = k
            break
        if rejected_at >= 0:
            j = rejected_at
            prev = int(anchor[b]) if j == 0 else int(tokens[b, j - 1])
            z = f64(U[b, j]) + (markov_bias(W1, W2, prev) if emb is None
                                else f64(emb[b, j]) @ W2)
            q = _draft_probs(z, T)
            res = np.maximum(0.0, p - q)
            if not (np.sum(res) > 0.0):
                res = p
                degenerate[b] = True
            y, lo, hi, _ = inverse_cdf(res, uf)
            if keep_final:
                final_cdf[b] = np.cumsum(res) / np.sum(res)
            out[b, :j] = tokens[b, :j]
            out[b, j] = y
            n_acc[b] = j
        else:
            p = target_probs(f64(target[b, L]), T)
            y, lo, hi, _ = inverse_cdf(p, uf)
            if keep_final:
                final_cdf[b] = np.cumsum(p) / np.sum(p)
            out[b, :L] = tokens[b, :L]
            out[b, L] = y
            n_acc[b] = L
        f_lo[b], f_hi[b] = lo, hi
        f_margin[b] = np.inf if (lo <= 0.0 and hi >= 1.0) else min(uf - lo, hi - uf)
    return dict(out_tokens=out, n_accepted=n_acc, ratio=ratio, final_lo=f_lo,
                final_hi=f_hi, final_margin=f_margin, degenerate=degenerate,
                final_cdf=final_cdf)


# ----------------------------------------------------------------------------
# (5) acceptance label: total variation between draft and target
# ----------------------------------------------------------------------------

def tv_label(target, U, W1, W2, anchor, tokens, temperature, rows=None, emb=None):
    """Per-position acceptance label from the total variation distance.

    [weigao] part 3 (the confidence head's training target) and [billytse]
    5.1: c*_k = 1 - 0.5 * ||p^d_k - p^t_k||_1, the draft distribution of
    position k against the target distribution of the same position; the
    total variation equals one minus the probability that the
    accept-or-resample test keeps the drafted token ([billytse] 1).

    The draft distribution is the one the token was sampled from: softmax of
    (U[b, k] + W1[prev] W2) / T with prev the anchor (k = 0) or the drafted
    token k - 1; the target distribution is softmax(target[b, k] / T).  A
    greedy request (T <= 0) has one-hot q at its drafted token (the argmax
    it drew) and one-hot p at the target's lowest-index argmax, so its label
    is 1 when they agree, else 0.

    rows: optional list of (b, k) to compute (others are NaN).  ``emb``
    [B, gamma, r]: the RNN head's projected vectors (bias emb[b, k] @ W2).
    Returns dict(tv [B, gamma], label [B, gamma]).
    """
    B, gamma, V = np.asarray(U).shape
    U = f64(U)
    target = f64(target)
    tv = np.full((B, gamma), np.nan)
    todo = [(b, k) for b in range(B) for k in range(gamma)] if rows is None else rows
    for b, k in todo:
        T = float(temperature[b])
        x = int(tokens[b, k])
        if not (T > 0.0):
            tv[b, k] = 0.0 if int(np.argmax(target[b, k])) == x else 1.0
            continue
        prev = int(anchor[b]) if k == 0 else int(tokens[b, k - 1])
        bias = markov_bias(W1, W2, prev) if emb is None else f64(emb[b, k]) @ f64(W2)
        q = _draft_probs(U[b, k] + bias, T)
        p = target_probs(target[b, k], T)
        tv[b, k] = 0.5 * math.fsum(np.abs(p - q))
    return dict(tv=tv, label=1.0 - tv)


# ----------------------------------------------------------------------------
# (6) RNN head: a recurrent sequential bias
# ----------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """Nearest bf16 value of each entry (ties to even), as float64.

    bf16 keeps 8 significant bits and float32's exponent range; the rounding
    is done directly from the float64 value (no float32 step).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                 # below 2^-126 the quantum stays 2^-133
    return np.ldexp(np.round(np.ldexp(x, 8 - e)), e - 8)


def _sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def rnn_step(state, emb, h, Wr, br):
    """One step of the RNN head.

    [weigao] part 2 (the ``_rnn_step`` description): the previous state, the
    previous token's embedding and the position's hidden state are
    concatenated and passed through one linear layer, whose output is split
    into gate, candidate and output; state_k = gate * state_{k-1} + (1 -
    gate) * candidate, and the position's bias is W2 applied to tanh(output).
    [billytse] 3.3: the recurrence lets each position see the whole block
    prefix.

    Readings (the pages give the split, not the activations or sizes): the
    three parts each have the state size r (tanh(output) enters the same
    r -> V projection W2 as the Markov head's W1 row); gate = sigmoid,
    candidate = tanh; the linear layer is Wr [3r, 2r + H] (rows: gate,
    candidate, output; columns: state, embedding, hidden) plus br [3r].

    Returns (state_k, tanh(output)).
    """
    state = np.asarray(state, dtype=np.float64)
    r = state.shape[0]
    x = np.concatenate([state, np.asarray(emb, dtype=np.float64), np.asarray(h, dtype=np.float64)])
    pre = np.asarray(Wr, dtype=np.float64) @ x + np.asarray(br, dtype=np.float64)
    gate = _sigmoid(pre[:r])
    cand = np.tanh(pre[r:2 * r])
    out = np.tanh(pre[2 * r:3 * r])
    return gate * state + (1.0 - gate) * cand, out


def rnn_forced(W1, hidden, Wr, br, anchor, tokens):
    """The RNN head's recurrence with the drafted tokens given.

    Position k's embedding is the W1 row of the previous token (the anchor
    for k = 0; the Markov embedding the pages' heads share), its state input
    is the state after position k - 1 (zero before the first position: the
    recurrence runs within one block).  Returns dict(emb [B, gamma, r]: the
    vectors tanh(output) each position projects, state [B, gamma, r]: the
    state after each position), float64, unrounded.
    """
    W1 = f64(W1)
    h = f64(hidden)
    Wr = f64(Wr)
    br = np.asarray(br, dtype=np.float64)
    tokens = np.asarray(tokens)
    B, gamma = tokens.shape
    r = W1.shape[1]
    emb = np.zeros((B, gamma, r))
    st = np.zeros((B, gamma, r))
    for b in range(B):
        s = np.zeros(r)
        for k in range(gamma):
            prev = int(anchor[b]) if k == 0 else int(tokens[b, k - 1])
            s, o = rnn_step(s, W1[prev], h[b, k], Wr, br)
            emb[b, k] = o
            st[b, k] = s
    return dict(emb=emb, state=st)


def rnn_draft_block(U, W1, W2, hidden, Wr, br, anchor, temperature, uniforms, emb_round=None):
    """Sequential sampling over a block with the RNN head.

    The [billytse] 3.3 loop with the RNN head's bias: at each position the
    head steps its recurrence on the previous sampled token (rnn_step), the
    bias tanh(output) @ W2 is added to the position's base logits, and the
    token is drawn from the softmax exactly as with the Markov head
    (draft_row).  ``emb_round="bf16"`` rounds each projected vector to bf16
    before the projection (the precision in which a bf16 step feeds it to
    the matrix cores); None keeps float64.

    Returns the fields of draft_block plus emb [B, gamma, r] (the projected
    vectors, after rounding) and state [B, gamma, r].
    """
    U = f64(U)
    W1 = f64(W1)
    W2 = f64(W2)
    h = f64(hidden)
    Wr = f64(Wr)
    br = np.asarray(br, dtype=np.float64)
    uni = np.asarray(uniforms, dtype=np.float64)
    B, gamma, V = U.shape
    r = W1.shape[1]
    out = {k: np.zeros((B, gamma)) for k in ("q_tok", "row_max", "row_logZ", "lo", "hi", "margin")}
    tokens = np.zeros((B, gamma), dtype=np.int64)
    emb = np.zeros((B, gamma, r))
    st = np.zeros((B, gamma, r))
    for b in range(B):
        prev = int(anchor[b])
        s = np.zeros(r)
        T = float(temperature[b])
        for k in range(gamma):
            s, o = rnn_step(s, W1[prev], h[b, k], Wr, br)
            if emb_round == "bf16":
                o = bf16_round(o)
            emb[b, k] = o
            st[b, k] = s
            z = U[b, k] + o @ W2
            u = float(uni[b, k, 0])
            d = draft_row(z, T, u)
            tokens[b, k] = d["x"]
            out["q_tok"][b, k] = d["q"]
            out["row_max"][b, k] = d["m"]
            out["row_logZ"][b, k] = d["logZ"]
            out["lo"][b, k] = d["lo"]
            out["hi"][b, k] = d["hi"]
            whole = d["lo"] <= 0.0 and d["hi"] >= 1.0
            out["margin"][b, k] = np.inf if whole else min(u - d["lo"], d["hi"] - u)
            prev = d["x"]
    out["tokens"] = tokens
    out["emb"] = emb
    out["state"] = st
    return out


# ----------------------------------------------------------------------------
# (7) sequential temperature scaling (STS) of the confidence head
# ----------------------------------------------------------------------------

def confidence_logits(hidden, W1, anchor, tokens, w, b0: float = 0.0) -> np.ndarray:
    """z[b, k] = w . [h_k ; W1[prev_k]] + b0: the confidence head's logit
    (confidence() is sigmoid(z))."""
    h = f64(hidden)
    W1 = f64(W1)
    w = f64(w)
    B, gamma, H = h.shape
    tokens = np.asarray(tokens)
    z = np.zeros((B, gamma))
    for b in range(B):
        for k in range(gamma):
            prev = int(anchor[b]) if k == 0 else int(tokens[b, k - 1])
            z[b, k] = float(np.dot(w, np.concatenate([h[b, k], W1[prev]]))) + b0
    return z


def sts_apply(z, temps) -> np.ndarray:
    """Calibrated conditional confidence c^[b, j] = sigmoid(z[b, j] / T_j).

    [billytse] 5.2: the raw head ranks well but is overconfident; sequential
    temperature scaling calibrates the cumulative survival left to right.
    [weigao] part 3: the scheduler needs absolute probabilities.  Reading
    (the pages give no formula): one temperature per block position divides
    that position's logit; the survival the scheduler ranks by is the running
    product of the calibrated conditionals, so it stays non-increasing along
    a request and admitted sets stay prefixes.  T_j = 1 leaves c unchanged.
    """
    z = np.asarray(z, dtype=np.float64)
    T = np.asarray(temps, dtype=np.float64)
    return _sigmoid(z / T[None, :])


def confidence_sts(hidden, W1, anchor, tokens, w, b0, temps) -> np.ndarray:
    """The confidence head followed by STS: sigmoid(z[b, k] / T_k)."""
    return sts_apply(confidence_logits(hidden, W1, anchor, tokens, w, b0), temps)


def _nll(p, y):
    p = np.clip(p, 1e-300, 1.0 - 1e-16)
    return -float(np.sum(y * np.log(p) + (1.0 - y) * np.log1p(-p)))


def sts_fit(z, n_accepted, t_lo: float = 0.05, t_hi: float = 50.0, iters: int = 100):
    """Fit the per-position temperatures left to right on calibration data.

    z [N, gamma]: the head's logits of N calibration drafts; n_accepted [N]:
    how many leading positions the target accepted.  The survival label of
    position j is [n_accepted > j].  Position by position, with the earlier
    temperatures fixed, T_j minimises the binary negative log-likelihood of
    the cumulative survival a^_j = a^_{j-1} sigmoid(z_j / T_j) against those
    labels (the quantity the scheduler uses, [billytse] 5.2: calibrate the
    cumulative probability from left to right).  One-dimensional golden-
    section search over log T in [t_lo, t_hi].  Returns temps [gamma].
    """
    z = np.asarray(z, dtype=np.float64)
    n = np.asarray(n_accepted)
    N, gamma = z.shape
    temps = np.ones(gamma)
    prev = np.ones(N)
    g = (math.sqrt(5.0) - 1.0) / 2.0
    for j in range(gamma):
        y = (n > j).astype(np.float64)

        def f(lt):
            return _nll(prev * _sigmoid(z[:, j] / math.exp(lt)), y)

        a, b = math.log(t_lo), math.log(t_hi)
        c, d = b - g * (b - a), a + g * (b - a)
        fc, fd = f(c), f(d)
        for _ in range(iters):
            if fc < fd:
                b, d, fd = d, c, fc
                c = b - g * (b - a)
                fc = f(c)
            else:
                a, c, fc = c, d, fd
                d = a + g * (b - a)
                fd = f(d)
        temps[j] = math.exp(0.5 * (a + b))
        prev = prev * _sigmoid(z[:, j] / temps[j])
    return temps


def ece(prob, label, bins: int = 15) -> float:
    """Expected calibration error: equal-width bins of the predicted
    probability; the share-weighted mean of |mean label - mean prediction|."""
    p = np.asarray(prob, dtype=np.float64).reshape(-1)
    y = np.asarray(label, dtype=np.float64).reshape(-1)
    idx = np.minimum((p * bins).astype(np.int64), bins - 1)
    err = 0.0
    for i in range(bins):
        m = idx == i
        if np.any(m):
            err += m.mean() * abs(float(y[m].mean()) - float(p[m].mean()))
    return err
