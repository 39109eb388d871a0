"""Stage-wise comparison of device outputs with the fp64 oracle.

TEST INFRASTRUCTURE ONLY (imported by tests/, __graft_entry__.smoke()).

Each oracle stage is fed the device's upstream discrete outputs (tokens,
verify lengths), so one near-tie cannot cascade.  Matching rules:

* tokens: identical wherever the oracle's uniform lies more than BAND = 1e-5
  (probability units) from a boundary of the drawn token's interval;
  otherwise the device token's own oracle interval must lie within BAND of u;
* accept decisions / accepted lengths: identical wherever |u - p/q| > BAND;
* verify lengths, scheduler order and admitted count: bit-exact;
* probabilities, ratios, confidences, row statistics: within 1e-4 absolute
  or 1e-3 relative.
"""

from __future__ import annotations

import numpy as np

from . import dspark_oracle as O

BAND = 1e-5
TOL_ABS = 1e-4
TOL_REL = 1e-3


def close(a, b) -> bool:
    a, b = float(a), float(b)
    if np.isnan(a) and np.isnan(b):
        return True
    d = abs(a - b)
    return d <= TOL_ABS or d <= TOL_REL * abs(b)


class Mismatch(AssertionError):
    pass


def _req(cond, msg):
    if not cond:
        raise Mismatch(msg)


def check_draft(wl, W1_64, W2_64, tokens, q_tok, row_max, row_logZ, rows=None, emb=None):
    """tokens etc. are host numpy arrays of the device outputs; ``emb``: the
    device's RNN-head vectors (the bias of (b, k) is then emb[b, k] @ W2)."""
    forced = O.draft_forced(wl.U, W1_64, W2_64, wl.anchor, wl.temperature, tokens,
                            uniforms=wl.uniforms, rows=rows, emb=emb)
    rep = dict(rows=len(forced), identical=0, band=0)
    for d in forced:
        b, k = d["b"], d["k"]
        x = int(tokens[b, k])
        u = float(wl.uniforms[b, k, 0])
        if x == d["x_oracle"]:
            rep["identical"] += 1
        else:
            _req(d["margin"] <= BAND,
                 f"draft token ({b},{k}): device {x} vs oracle {d['x_oracle']} (margin {d['margin']:.3g})")
            _req(d["lo"] - BAND <= u <= d["hi"] + BAND,
                 f"draft token ({b},{k}): device {x} interval [{d['lo']},{d['hi']}) far from u={u}")
            rep["band"] += 1
        _req(close(q_tok[b, k], d["q"]), f"q_tok ({b},{k}): {q_tok[b, k]} vs {d['q']}")
        _req(close(row_max[b, k], d["m"]), f"row_max ({b},{k}): {row_max[b, k]} vs {d['m']}")
        _req(close(row_logZ[b, k], d["logZ"]), f"row_logZ ({b},{k}): {row_logZ[b, k]} vs {d['logZ']}")
    return rep


def check_rnn(wl, rw, tokens, emb, state, bf16):
    """The RNN head's recurrence on the device's own tokens: the projected
    vectors within the storage rounding (bf16: half a unit in the 8th
    significant bit, plus 2e-5 for the fp32 arithmetic; fp32: the continuous
    tolerance) and the state within 1e-4 absolute."""
    ref = O.rnn_forced(wl.W1, wl.hidden, rw["Wr"], rw["br"], wl.anchor, tokens)
    e_ref, s_ref = ref["emb"], ref["state"]
    lim = (2.0 ** -8 * np.abs(e_ref) + 2e-5) if bf16 else (TOL_ABS + TOL_REL * np.abs(e_ref))
    bad = np.argwhere(np.abs(emb - e_ref) > lim)
    _req(len(bad) == 0, f"rnn emb mismatch at {bad[:4].tolist()}: device "
                        f"{[float(emb[tuple(i)]) for i in bad[:3]]} oracle "
                        f"{[float(e_ref[tuple(i)]) for i in bad[:3]]}")
    out = dict(rows=int(e_ref.shape[0] * e_ref.shape[1]),
               emb_max_abs=float(np.max(np.abs(emb - e_ref))))
    if state is not None:
        ds = np.abs(state - s_ref)
        _req(float(np.max(ds)) <= 1e-4, f"rnn state max |diff| {float(np.max(ds)):.3g}")
        out["state_max_abs"] = float(np.max(ds))
    return out


def check_confidence(wl, tokens, conf):
    c = O.confidence(wl.hidden, wl.W1, wl.anchor, tokens, wl.w, wl.b0)
    bad = [(b, k) for b in range(c.shape[0]) for k in range(c.shape[1]) if not close(conf[b, k], c[b, k])]
    _req(not bad, f"confidence mismatch at {bad[:5]} (device {[conf[i] for i in bad[:3]]}, "
                  f"oracle {[c[i] for i in bad[:3]]})")
    return dict(rows=c.size, max_abs=float(np.max(np.abs(conf - c))))


def check_schedule(conf, sps, ell, order, stats):
    s = O.schedule(conf.astype(np.float64), sps)
    _req(np.array_equal(np.asarray(order, dtype=np.int64), s["order"]), "scheduler order differs")
    _req(np.array_equal(np.asarray(ell, dtype=np.int64), s["ell"]),
         f"ell differs at {np.nonzero(np.asarray(ell) != s['ell'])[0][:8]}")
    _req(int(round(stats[0])) == s["n_admitted"], f"n_admitted {stats[0]} vs {s['n_admitted']}")
    _req(abs(stats[1] - s["tau"]) <= 1e-12 * abs(s["tau"]), f"tau {stats[1]} vs {s['tau']}")
    _req(abs(stats[2] - s["theta"]) <= 1e-12 * abs(s["theta"]), f"theta {stats[2]} vs {s['theta']}")
    return dict(n_admitted=s["n_admitted"], mean_ell=float(np.mean(s["ell"])))


def check_schedule_mode(conf, mode, arg, ell, order, stats):
    """Capacity (arg = K) or threshold (arg = survival threshold) scheduler:
    ell, order and the admitted count bit-exact, tau to 1e-12, Theta NaN."""
    c = conf.astype(np.float64)
    s = O.schedule_capacity(c, arg) if mode == "capacity" else O.schedule_threshold(c, arg)
    _req(np.array_equal(np.asarray(order, dtype=np.int64), s["order"]), "scheduler order differs")
    _req(np.array_equal(np.asarray(ell, dtype=np.int64), s["ell"]),
         f"ell differs at {np.nonzero(np.asarray(ell) != s['ell'])[0][:8]}")
    _req(int(round(stats[0])) == s["n_admitted"], f"n_admitted {stats[0]} vs {s['n_admitted']}")
    _req(abs(stats[1] - s["tau"]) <= 1e-12 * abs(s["tau"]), f"tau {stats[1]} vs {s['tau']}")
    _req(np.isnan(stats[2]), f"theta {stats[2]} should be NaN")
    return dict(n_admitted=s["n_admitted"], mean_ell=float(np.mean(s["ell"])))


def check_verify(wl, W1_64, W2_64, tokens, ell, out_tokens, n_accepted, ratio, requests=None,
                 emb=None):
    B, gamma = tokens.shape
    reqs = list(range(B)) if requests is None else list(requests)
    rows = [(b, k) for b in reqs for k in range(int(ell[b]))]
    q = np.full((B, gamma), np.nan)
    for d in O.draft_forced(wl.U, W1_64, W2_64, wl.anchor, wl.temperature, tokens, rows=rows,
                            emb=emb):
        q[d["b"], d["k"]] = d["q"]
    v = O.verify(wl.target, wl.U, W1_64, W2_64, wl.anchor, tokens, q, wl.temperature,
                 wl.uniforms, ell, requests=reqs, keep_final=True, emb=emb)
    rep = dict(requests=len(reqs), accept_flips=0, final_identical=0, final_band=0)
    for b in reqs:
        L = int(ell[b])
        n_o, n_g = int(v["n_accepted"][b]), int(n_accepted[b])
        _req(0 <= n_g <= L, f"n_accepted[{b}]={n_g} outside [0,{L}]")
        for k in range(min(n_o, n_g, L - 1) + 1 if L > 0 else 0):
            _req(close(ratio[b, k], v["ratio"][b, k]), f"ratio ({b},{k}): {ratio[b, k]} vs {v['ratio'][b, k]}")
        for k in range(gamma):
            if not (k < L and k <= n_g):
                _req(np.isnan(ratio[b, k]), f"ratio ({b},{k}) should be NaN (untested)")
        _req(np.array_equal(out_tokens[b, :n_g], tokens[b, :n_g]), f"accepted prefix of {b} differs")
        _req(np.all(out_tokens[b, n_g + 1:] == -1), f"padding of {b}")
        if n_g != n_o:
            k = min(n_g, n_o)
            gap = abs(float(wl.uniforms[b, k, 1]) - v["ratio"][b, k])
            _req(gap <= BAND, f"accept length of {b}: device {n_g} vs oracle {n_o} (|u-ratio|={gap:.3g})")
            rep["accept_flips"] += 1
            continue
        y_g, y_o = int(out_tokens[b, n_g]), int(v["out_tokens"][b, n_o])
        if y_g == y_o:
            rep["final_identical"] += 1
            continue
        _req(v["final_margin"][b] <= BAND,
             f"final token of {b}: device {y_g} vs oracle {y_o} (margin {v['final_margin'][b]:.3g})")
        cdf = v["final_cdf"][b]
        uf = float(wl.uniforms[b, gamma, 0])
        lo = cdf[y_g - 1] if y_g > 0 else 0.0
        _req(lo - BAND <= uf <= cdf[y_g] + BAND, f"final token of {b}: interval far from u")
        rep["final_band"] += 1
    return rep


def check_tv(wl, W1_64, W2_64, tokens, tv, label, rows=None):
    """Acceptance labels: tv and 1 - tv against the oracle on the GPU's own
    drafted tokens; continuous tolerance, greedy rows exact."""
    B, gamma = tokens.shape
    todo = [(b, k) for b in range(B) for k in range(gamma)] if rows is None else list(rows)
    ref = O.tv_label(wl.target, wl.U, W1_64, W2_64, wl.anchor, tokens, wl.temperature, rows=todo)
    worst = 0.0
    for b, k in todo:
        r = ref["tv"][b, k]
        _req(close(tv[b, k], r), f"tv ({b},{k}): {tv[b, k]} vs {r}")
        if label is not None:
            _req(close(label[b, k], 1.0 - r), f"label ({b},{k}): {label[b, k]} vs {1.0 - r}")
        if not (float(wl.temperature[b]) > 0.0):
            _req(float(tv[b, k]) == r, f"greedy tv ({b},{k}): {tv[b, k]} vs {r}")
        worst = max(worst, abs(float(tv[b, k]) - r))
    return dict(rows=len(todo), max_abs=worst, mean_label=float(np.mean(1.0 - np.array(
        [ref["tv"][b, k] for b, k in todo]))))


def check_end_to_end(wl, out):
    """The oracle's own step from the inputs alone (draft, confidence,
    scheduler or the fixed length, verify), compared with the device step.

    Requests are compared independently.  A request whose drafted tokens
    differ must show the first difference at a draw whose oracle margin is
    within BAND (the device token's interval within BAND of u); its later
    positions and its verification follow different drafts and are not
    compared.  The scheduler is compared when every request drafted the same
    tokens (its verify lengths bit-exact, or an explained near-tie of Theta).
    A request with identical drafts and verify length must accept the same
    count unless |u - p/q| <= BAND at the first difference, and emit the same
    final token unless its final draw's margin is within BAND.
    """
    B, gamma = out["tokens"].shape
    W1_64, W2_64 = O.f64(wl.W1), O.f64(wl.W2)
    d = O.draft_block(wl.U, W1_64, W2_64, wl.anchor, wl.temperature, wl.uniforms)
    rep = dict(requests=B, draft_identical=0, draft_explained=0, conf_rows=0,
               verify_identical=0, verify_explained=0, schedule="compared")
    same = np.zeros(B, dtype=bool)
    for b in range(B):
        diff = np.nonzero(out["tokens"][b] != d["tokens"][b])[0]
        if len(diff) == 0:
            same[b] = True
            rep["draft_identical"] += 1
            for k in range(gamma):
                _req(close(out["q_tok"][b, k], d["q_tok"][b, k]), f"e2e q_tok ({b},{k})")
            continue
        k = int(diff[0])
        _req(d["margin"][b, k] <= BAND,
             f"e2e draft ({b},{k}): device {out['tokens'][b, k]} vs oracle {d['tokens'][b, k]} "
             f"(margin {d['margin'][b, k]:.3g})")
        rep["draft_explained"] += 1
    c = O.confidence(wl.hidden, W1_64, wl.anchor, d["tokens"], wl.w, wl.b0)
    for b in np.nonzero(same)[0]:
        for k in range(gamma):
            _req(close(out["conf"][b, k], c[b, k]), f"e2e confidence ({b},{k})")
            rep["conf_rows"] += 1
    if out["sched"]:
        s = O.schedule(c, wl.sps)
        ell_o = s["ell"]
        if same.all():
            if not np.array_equal(np.asarray(out["ell"], dtype=np.int64), ell_o):
                # only a Theta comparison decided within rounding may differ:
                # the device's fp32 confidences against the oracle's fp64 ones
                s_dev = O.schedule(out["conf"].astype(np.float64), wl.sps)
                _req(np.array_equal(np.asarray(out["ell"], dtype=np.int64), s_dev["ell"]),
                     "e2e scheduler differs from the oracle's on the device's confidences")
                rep["schedule"] = "explained by fp32 confidences"
        else:
            rep["schedule"] = "not compared (drafts differ)"
    else:
        ell_o = np.full(B, gamma, dtype=np.int64)
    v = O.verify(wl.target, wl.U, W1_64, W2_64, wl.anchor, d["tokens"], d["q_tok"],
                 wl.temperature, wl.uniforms, ell_o)
    for b in np.nonzero(same)[0]:
        if int(out["ell"][b]) != int(ell_o[b]):
            continue
        n_o, n_g = int(v["n_accepted"][b]), int(out["n_accepted"][b])
        if n_o != n_g:
            k = min(n_o, n_g)
            gap = abs(float(wl.uniforms[b, k, 1]) - v["ratio"][b, k])
            _req(gap <= BAND, f"e2e accepted length of {b}: device {n_g} vs oracle {n_o}")
            rep["verify_explained"] += 1
            continue
        y_g, y_o = int(out["out_tokens"][b, n_g]), int(v["out_tokens"][b, n_o])
        if y_g != y_o:
            _req(v["final_margin"][b] <= BAND, f"e2e final token of {b}: {y_g} vs {y_o}")
            rep["verify_explained"] += 1
        else:
            rep["verify_identical"] += 1
    return rep
