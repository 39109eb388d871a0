"""The confidence head with sequential temperature scaling
(dspark_confidence_sts) on the GPU against the fp64 oracle.

[billytse] 5.2; [weigao] part 3.  Every (request, position) at the
long-proposal workload (B=128, gamma=15, H=2560, bf16) and at the tiny fp32
one; unit temperatures reproduce dspark_confidence bit for bit; the
scheduler fed the calibrated confidences matches the oracle's scheduler on
them bit for bit; a temperature that is not finite and positive is flagged
and leaves its position uncalibrated.
"""

import numpy as np
import pytest
import torch

import draft_verify_sampling_block_amd as dv
from draft_verify_sampling_block_amd.step import upload
from gen import make_config
import oracle as O
from oracle.parity import check_schedule, close

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[sts] {msg}", flush=True)


def _tokens(wl, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, wl.V, (wl.B, wl.gamma)).astype(np.int32)


@pytest.mark.parametrize("cfg", [0, 3], ids=["tiny-f32", "long-proposal-g15"])
def test_sts_every_row(cfg):
    _say(f"config {cfg}")
    wl = make_config(cfg)
    d = upload(wl, "cuda")
    tok = _tokens(wl, cfg)
    temps = np.linspace(0.6, 3.0, wl.gamma).astype(np.float32)
    t_dev = torch.from_numpy(temps).cuda()
    st = torch.zeros((1,), dtype=torch.int32, device="cuda")
    conf = dv.dspark_confidence_sts(d.hidden, d.W1, d.anchor, torch.from_numpy(tok).cuda(), d.w,
                                    d.b0, t_dev, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    got = conf.cpu().numpy()
    ref = O.confidence_sts(wl.hidden, wl.W1, wl.anchor, tok, wl.w, wl.b0,
                           temps.astype(np.float64))
    bad = [(b, k) for b in range(wl.B) for k in range(wl.gamma) if not close(got[b, k], ref[b, k])]
    assert not bad, (bad[:4], [got[i] for i in bad[:2]], [ref[i] for i in bad[:2]])
    _say(dict(rows=ref.size, max_abs=float(np.max(np.abs(got - ref)))))
    if wl.sps is not None:
        ell, order, stats = dv.dspark_schedule(conf, d.sps)
        torch.cuda.synchronize()
        rep = check_schedule(got, wl.sps, ell.cpu().numpy(), order.cpu().numpy(),
                             stats.cpu().numpy())
        raw = O.schedule(O.confidence(wl.hidden, wl.W1, wl.anchor, tok, wl.w, wl.b0), wl.sps)
        _say(dict(calibrated=rep, raw_n_admitted=raw["n_admitted"]))


def test_unit_temperatures_reproduce_the_plain_head():
    wl = make_config(3)
    d = upload(wl, "cuda")
    tok = torch.from_numpy(_tokens(wl, 5)).cuda()
    a = dv.dspark_confidence(d.hidden, d.W1, d.anchor, tok, d.w, d.b0)
    b = dv.dspark_confidence_sts(d.hidden, d.W1, d.anchor, tok, d.w, d.b0,
                                 torch.ones((wl.gamma,), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_bad_temperature_is_flagged_and_left_uncalibrated():
    wl = make_config(0)
    d = upload(wl, "cuda")
    tok = torch.from_numpy(_tokens(wl, 6)).cuda()
    temps = torch.tensor([2.0, 0.0, float("nan"), -1.0, 1.0], dtype=torch.float32, device="cuda")
    st = torch.zeros((1,), dtype=torch.int32, device="cuda")
    c = dv.dspark_confidence_sts(d.hidden, d.W1, d.anchor, tok, d.w, d.b0, temps, status=st)
    plain = dv.dspark_confidence(d.hidden, d.W1, d.anchor, tok, d.w, d.b0)
    torch.cuda.synchronize()
    assert int(st.item()) & 16      # DSPARK_DEV_BAD_CONF
    assert torch.equal(c[:, 1:5], plain[:, 1:5])
    assert not torch.equal(c[:, 0], plain[:, 0])
