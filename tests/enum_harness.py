"""Exact enumeration of the oracle's output law on tiny problems.

The oracle is driven by uniforms.  Its output is piecewise constant in each
uniform, and every piece boundary is a monotone switch (inverse-CDF draws
move to the next token, accept tests flip from accept to reject).  This
harness walks the uniforms in the order the step consumes them (draft draws,
then accept tests, then the final draw), finds the cells of each uniform
from the interval the oracle reports, probes both ends of every cell to
confirm that the oracle really behaves that way, and integrates the cell
lengths.  The result is the exact (to ~1e-15) law of the emitted tokens,
obtained only by running the oracle, so it checks the oracle's actual
uniform-driven code rather than a restatement of its formulas.

Losslessness is then the statement that the emitted prefix, completed by
sampling the target distribution to a fixed length, has exactly the law of
sampling the target distribution directly ([billytse] section 1; [xhh]
acceptance-rule Q&A, which shows accept-plus-residual mass equals p).
"""

from __future__ import annotations

import itertools
from collections import defaultdict

import numpy as np

import oracle as O

PROBE = 1e-13


class TinyStep:
    """R requests, block gamma, vocabulary V, rank r, prefix-conditioned targets.

    ``ptab[r][prefix]`` is the target distribution of request r after the
    given committed prefix (tuple of token ids); target logits handed to the
    oracle are T*log(p), so softmax(logits / T) == p.  When ``greedy`` is set
    every request runs at T = 0 and the target is the argmax of that table.
    """

    def __init__(self, R, gamma, V, rank, seed, T=1.0, ell=None, conf=None, sps=None,
                 w_scale=0.8, U=None, W1=None, W2=None, ptab=None, anchor=None, sched=None,
                 rnn=None):
        rng = np.random.default_rng(seed)
        self.R, self.gamma, self.V = R, gamma, V
        self.U = rng.normal(0.0, 1.0, (R, gamma, V)) if U is None else np.asarray(U, dtype=np.float64)
        self.W1 = rng.normal(0.0, w_scale, (V, rank)) if W1 is None else np.asarray(W1, dtype=np.float64)
        self.W2 = rng.normal(0.0, w_scale, (V, rank)).T if W2 is None else np.asarray(W2, dtype=np.float64)
        self.anchor = rng.integers(0, V, R) if anchor is None else np.asarray(anchor)
        self.T = np.full(R, float(T))
        if ptab is None:
            ptab = []
            for _ in range(R):
                tab = {}
                for n in range(gamma + 1):
                    for pre in itertools.product(range(V), repeat=n):
                        tab[pre] = rng.dirichlet(np.full(V, 1.5))
                ptab.append(tab)
        self.ptab = ptab
        self.ell = None if ell is None else np.asarray(ell)
        self.conf = conf          # callable tokens [R, gamma] -> c [R, gamma]
        self.sps = sps
        self.sched = sched        # callable (c, sps) -> ell; default: the oracle's greedy
        self.rnn = rnn            # dict(hidden, Wr, br): draft with the RNN head instead
        self._draft_cache = {}

    # -- the step under test -------------------------------------------------
    def target_logits(self, tokens):
        out = np.zeros((self.R, self.gamma + 1, self.V))
        for r in range(self.R):
            for k in range(self.gamma + 1):
                p = self.ptab[r][tuple(int(t) for t in tokens[r, :k])]
                out[r, k] = np.log(p) * (self.T[r] if self.T[r] > 0 else 1.0)
        return out

    def run(self, uni):
        key = np.ascontiguousarray(uni[:, : self.gamma, 0]).tobytes()
        if key not in self._draft_cache:
            if self.rnn is None:
                d = O.draft_block(self.U, self.W1, self.W2, self.anchor, self.T, uni)
            else:
                d = O.rnn_draft_block(self.U, self.W1, self.W2, self.rnn["hidden"],
                                      self.rnn["Wr"], self.rnn["br"], self.anchor, self.T, uni)
            if self.ell is not None:
                ell = self.ell
            else:
                c = self.conf(d["tokens"])
                ell = (self.sched(c, self.sps) if self.sched is not None
                       else O.schedule(c, self.sps)["ell"])
            self._draft_cache[key] = (d, ell)
        d, ell = self._draft_cache[key]
        v = O.verify(self.target_logits(d["tokens"]), self.U, self.W1, self.W2, self.anchor,
                     d["tokens"], d["q_tok"], self.T, uni, ell,
                     emb=None if self.rnn is None else d["emb"])
        return d, ell, v

    # -- reference law --------------------------------------------------------
    def cond(self, r, prefix):
        p = self.ptab[r][tuple(prefix)]
        if self.T[r] > 0:
            return p
        g = np.zeros(self.V)
        g[int(np.argmax(p))] = 1.0
        return g

    def target_law(self, r, L):
        law = {}
        for seq in itertools.product(range(self.V), repeat=L):
            pr = 1.0
            for i in range(L):
                pr *= self.cond(r, seq[:i])[seq[i]]
            law[seq] = pr
        return law

    def complete(self, r, emitted, L):
        """Law of emitted + target continuation up to length L."""
        out = {}
        n = len(emitted)
        for tail in itertools.product(range(self.V), repeat=L - n):
            seq = tuple(emitted) + tail
            pr = 1.0
            for i in range(n, L):
                pr *= self.cond(r, seq[:i])[seq[i]]
            out[seq] = pr
        return out


def _monotone_cells(evalf):
    """Cells of a monotone token map t -> (token, lo, hi) on [0, 1)."""
    cells = []
    t = 0.0
    prev_tok = None
    while t < 1.0:
        tok, lo, hi = evalf(t)
        nudge = 0
        while tok == prev_tok and nudge < 8:   # boundary value rounded into the old cell
            t = np.nextafter(t, 2.0)
            tok, lo, hi = evalf(t)
            nudge += 1
        assert tok != prev_tok, "token map did not advance past a reported boundary"
        assert lo <= t + 1e-15 and t < hi + 1e-15, (lo, t, hi)
        if hi - lo > 4 * PROBE:
            assert evalf(lo + PROBE)[0] == tok, "reported cell start disagrees with behaviour"
            assert evalf(hi - PROBE)[0] == tok, "reported cell end disagrees with behaviour"
        if hi > lo:
            cells.append((lo, hi, 0.5 * (lo + hi)))
        prev_tok = tok
        t = hi
    return cells


def enumerate_law(step: TinyStep, L=None):
    """Exact joint law of the requests' completed output sequences.

    Returns dict: tuple(seq_0, ..., seq_{R-1}) -> probability, where each
    seq_r is the emitted tokens completed by the target to length L.
    """
    R, g = step.R, step.gamma
    L = g + 1 if L is None else L
    coords = [("d", r, k) for r in range(R) for k in range(g)]
    coords += [("a", r, k) for r in range(R) for k in range(g)]
    coords += [("f", r, g) for r in range(R)]
    law = defaultdict(float)

    def uni_of(vals):
        u = np.full((R, g + 1, 2), 0.5)
        for (kind, r, k), val in zip(coords, vals):
            u[r, k, 0 if kind in ("d", "f") else 1] = val
        return u

    def rec(vals, weight):
        i = len(vals)
        if i == len(coords):
            d, ell, v = step.run(uni_of(vals))
            parts = []
            for r in range(R):
                n = int(v["n_accepted"][r])
                emitted = [int(t) for t in v["out_tokens"][r, : n + 1]]
                parts.append(step.complete(r, emitted, L))
            for combo in itertools.product(*[p.items() for p in parts]):
                pr = weight
                for _, q in combo:
                    pr *= q
                law[tuple(s for s, _ in combo)] += pr
            return
        kind, r, k = coords[i]

        def at(t):
            return step.run(uni_of(vals + [t]))

        if kind == "d":
            def ev(t):
                d, _, _ = at(t)
                return int(d["tokens"][r, k]), float(d["lo"][r, k]), float(d["hi"][r, k])
            cells = _monotone_cells(ev)
        elif kind == "f":
            def ev(t):
                _, _, v = at(t)
                n = int(v["n_accepted"][r])
                return int(v["out_tokens"][r, n]), float(v["final_lo"][r]), float(v["final_hi"][r])
            cells = _monotone_cells(ev)
        else:
            _, _, v = at(0.5)
            ratio = float(v["ratio"][r, k])
            if np.isnan(ratio):
                cells = [(0.0, 1.0, 0.5)]
            else:
                thr = min(ratio, 1.0)
                cells = []
                if thr > 0:
                    if thr > 2 * PROBE:
                        assert at(thr - PROBE)[2]["n_accepted"][r] > k, "accept below threshold"
                    cells.append((0.0, thr, 0.5 * thr))
                if thr < 1:
                    if thr < 1 - 2 * PROBE:
                        assert at(thr + PROBE)[2]["n_accepted"][r] == k, "reject above threshold"
                    cells.append((thr, 1.0, 0.5 * (thr + 1.0)))
        for lo, hi, rep in cells:
            rec(vals + [rep], weight * (hi - lo))

    rec([], 1.0)
    return dict(law)


def product_target_law(step: TinyStep, L=None):
    L = step.gamma + 1 if L is None else L
    laws = [step.target_law(r, L) for r in range(step.R)]
    out = {}
    for combo in itertools.product(*[lw.items() for lw in laws]):
        pr = 1.0
        for _, q in combo:
            pr *= q
        out[tuple(s for s, _ in combo)] = pr
    return out


def max_law_gap(a, b):
    keys = set(a) | set(b)
    return max(abs(a.get(k, 0.0) - b.get(k, 0.0)) for k in keys)
