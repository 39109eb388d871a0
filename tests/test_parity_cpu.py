"""The stage-wise and end-to-end comparison helpers on the CPU: the
oracle's own step passes them, and a planted wrong token far from any draw
boundary is caught (the helpers must not accept everything)."""

import numpy as np
import pytest

import oracle as O
from gen import make_custom
from oracle.parity import Mismatch, check_draft, check_end_to_end


def _oracle_step(wl):
    W1, W2 = O.f64(wl.W1), O.f64(wl.W2)
    d = O.draft_block(wl.U, W1, W2, wl.anchor, wl.temperature, wl.uniforms)
    c = O.confidence(wl.hidden, W1, wl.anchor, d["tokens"], wl.w, wl.b0)
    s = O.schedule(c, wl.sps)
    v = O.verify(wl.target, wl.U, W1, W2, wl.anchor, d["tokens"], d["q_tok"], wl.temperature,
                 wl.uniforms, s["ell"])
    return dict(tokens=d["tokens"].astype(np.int32), q_tok=d["q_tok"], row_max=d["row_max"],
                row_logZ=d["row_logZ"], conf=c.astype(np.float32), ell=s["ell"],
                out_tokens=v["out_tokens"], n_accepted=v["n_accepted"], ratio=v["ratio"],
                sched=True), d


def test_oracle_step_passes_and_a_planted_token_is_caught():
    wl = make_custom(6, 4, 256, 32, 16, "f32", "mixture", seed=3, sps_kind="linear:40",
                     calibrated=True)
    out, d = _oracle_step(wl)
    rep = check_end_to_end(wl, out)
    assert rep["draft_identical"] == 6 and rep["draft_explained"] == 0
    # a token changed where the oracle's draw is far from any boundary
    b, k = np.unravel_index(int(np.argmax(np.where(np.isfinite(d["margin"]), d["margin"], -1))),
                            d["margin"].shape)
    assert d["margin"][b, k] > 1e-3
    bad = dict(out)
    bad["tokens"] = out["tokens"].copy()
    bad["tokens"][b, k] = (bad["tokens"][b, k] + 1) % wl.V
    with pytest.raises(Mismatch):
        check_end_to_end(wl, bad)
    with pytest.raises(Mismatch):
        check_draft(wl, O.f64(wl.W1), O.f64(wl.W2), bad["tokens"], out["q_tok"], out["row_max"],
                    out["row_logZ"])
