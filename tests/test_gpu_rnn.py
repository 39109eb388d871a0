"""RNN-head drafting (dspark_draft_block_rnn) and its verification
(dspark_verify_rnn) on the GPU against the fp64 oracle, stage by stage.

[weigao] part 2 (_rnn_step) and [billytse] 3.3.  The recurrence is checked on
the device's own drafted tokens (projected vectors within their bf16
rounding, state within 1e-4); the draws and the verification are then
checked with the device's projected vectors as the bias rows, so each stage
is compared on identical inputs (tokens identical outside the 1e-5 tie band,
probabilities within 1e-4 absolute or 1e-3 relative).
"""

import numpy as np
import pytest
import torch

import draft_verify_sampling_block_amd as dv
from draft_verify_sampling_block_amd.step import _dev, upload
from gen import make_config, make_custom
from gen.workloads import rnn_weights
from oracle import f64
from oracle.parity import check_draft, check_rnn, check_verify

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[rnn] {msg}", flush=True)


def _run(wl, rw, ell=None, W2=None):
    d = upload(wl, "cuda", scheduler=False)
    if W2 is not None:
        d.W2 = W2
    Wr, br = _dev(rw["Wr"], "cuda"), _dev(rw["br"], "cuda")
    st = torch.zeros((1,), dtype=torch.int32, device="cuda")
    out = dv.dspark_draft_block_rnn(d.U, d.W1, d.W2, d.hidden, Wr, br, d.anchor, d.temperature,
                                    d.uniforms, want_state=True, status=st)
    ell_t = d.fixed_ell if ell is None else torch.from_numpy(np.asarray(ell, np.int32)).cuda()
    ot, na, ratio = dv.dspark_verify_rnn(d.target, d.U, out["emb"], d.W2, d.anchor, out["tokens"],
                                         out["q_tok"], out["row_max"], out["row_logZ"],
                                         d.temperature, d.uniforms, ell_t, status=st)
    torch.cuda.synchronize()
    h = lambda t: t.cpu().numpy()
    res = {k: h(v.float() if v.dtype == torch.bfloat16 else v) for k, v in out.items()}
    res.update(out_tokens=h(ot), n_accepted=h(na), ratio=h(ratio), ell=h(ell_t),
               status=int(st.item()))
    return res


def _check(wl, rw, res, rows=None, requests=None):
    bf = wl.dtype == "bf16"
    assert res["status"] == 0, dv.DEV_FLAGS.get(res["status"], res["status"])
    rep = {"rnn": check_rnn(wl, rw, res["tokens"], res["emb"], res["state"], bf)}
    W1_64, W2_64 = f64(wl.W1), f64(wl.W2)
    emb = res["emb"].astype(np.float64)
    rep["draft"] = check_draft(wl, W1_64, W2_64, res["tokens"], res["q_tok"], res["row_max"],
                               res["row_logZ"], rows=rows, emb=emb)
    rep["verify"] = check_verify(wl, W1_64, W2_64, res["tokens"], res["ell"], res["out_tokens"],
                                 res["n_accepted"], res["ratio"], requests=requests, emb=emb)
    return rep


SMALL = [
    # B, gamma, V, rank, H, dtype, family, T, greedy share
    (5, 4, 2000, 32, 64, "bf16", "mixture", 1.0, 0.0),
    (33, 3, 4096, 256, 128, "bf16", "mixture", 1.0, 0.0),
    (9, 6, 1544, 64, 32, "bf16", "gaussian", 0.7, 0.34),
    (4, 5, 1024, 32, 64, "f32", "gaussian", 1.0, 0.0),
    (3, 7, 777 * 8, 128, 256, "bf16", "two-class", 1.3, 0.0),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"{c[5]}-B{c[0]}-g{c[1]}-V{c[2]}-r{c[3]}" for c in SMALL])
def test_rnn_small_every_row(case):
    B, gamma, V, r, H, dt, fam, T, gf = case
    _say(f"small {case}")
    wl = make_custom(B, gamma, V, r, H, dt, fam, seed=11 + B, temperature=T, greedy_frac=gf)
    rw = rnn_weights(r, H, dt, seed=5)
    res = _run(wl, rw)
    rep = _check(wl, rw, res)
    _say(rep)
    # the RNN bias moves the draws: every row is compared, and most tokens agree exactly
    assert rep["draft"]["identical"] >= rep["draft"]["rows"] - 2


def test_rnn_verify_lengths_below_gamma():
    _say("ell below gamma, ell = 0")
    wl = make_custom(12, 5, 3000, 64, 64, "bf16", "mixture", seed=4)
    rw = rnn_weights(64, 64, "bf16", seed=6)
    ell = np.array([0, 1, 2, 3, 4, 5, 5, 4, 3, 2, 1, 0])
    res = _run(wl, rw, ell=ell)
    rep = _check(wl, rw, res)
    _say(rep)


def test_rnn_with_zero_projection_matches_the_markov_draft():
    # W2 = 0: both heads add no bias, so both drafts are the parallel drafter
    _say("W2 = 0: RNN draft equals the Markov draft")
    wl = make_custom(6, 4, 2048, 32, 64, "bf16", "mixture", seed=8)
    rw = rnn_weights(32, 64, "bf16", seed=7)
    z = torch.zeros((32, 2048), dtype=torch.bfloat16, device="cuda")
    res = _run(wl, rw, W2=z)
    d = upload(wl, "cuda", scheduler=False)
    st = torch.zeros((1,), dtype=torch.int32, device="cuda")
    mk = dv.dspark_draft_block(d.U, d.W1, z, d.anchor, d.temperature, d.uniforms, status=st)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(res["tokens"], mk["tokens"].cpu().numpy())
    np.testing.assert_array_equal(res["q_tok"], mk["q_tok"].cpu().numpy())


def test_rnn_long_proposal_shape():
    # B=128, gamma=15, V=151936, rank 256, H=2560, bf16: the recurrence on
    # every position, the draws and verification on sampled rows
    _say("long-proposal-g15 shape with RNN weights")
    wl = make_config(3)
    rw = rnn_weights(256, 2560, "bf16", seed=3)
    res = _run(wl, rw)
    rng = np.random.default_rng(0)
    reqs = sorted(set(rng.choice(128, 12, replace=False).tolist()) | {0, 127})
    rows = [(b, k) for b in reqs for k in range(15)]
    rep = _check(wl, rw, res, rows=rows, requests=reqs)
    _say(rep)


def test_rnn_rejects_bad_arguments():
    wl = make_custom(2, 3, 1024, 32, 60, "bf16", "gaussian", seed=1)   # H % 8 != 0
    lib = dv.load()
    fake = 4096
    rc = lib.dspark_draft_block_rnn(2, 3, 1024, 32, 60, 1, *([fake] * 15), None, fake, 1 << 30,
                                    None)
    assert rc == -1 and b"H=60" in lib.dspark_last_error()
    assert lib.dspark_verify_rnn(2, 3, 1024, 32, 1, *([fake] * 15), None, fake, 8, None) == -4
    del wl
