"""Acceptance statistics of the device path at the real vocabulary.  GPU only.

With the Markov bias switched off (W2 = 0) the draft distribution of each
position no longer depends on the token before it, and with one request's
rows repeated over a large batch every request runs the same experiment
with its own uniforms.  Then position i is accepted with probability
alpha_i = 1 - TV(p_i, q_i) independently of the others ([billytse] 1 and
5.1; [weigao] part 3), so P(n_accepted >= j) = prod_{i<=j} alpha_i and the
batch mean of n_accepted must match sum_j prod_{i<=j} alpha_i within five
standard errors.  alpha comes from the fp64 oracle on the same rows.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
from gen import make_custom
from gen.workloads import to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_verify_sampling_block_amd as dv
    dv.load()


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_mean_accepted_length_matches_closed_form(T):
    import draft_verify_sampling_block_amd as dv
    from draft_verify_sampling_block_amd.step import upload
    print(f"\n[case] acceptance statistics T={T}", flush=True)
    gamma, V, nb = 3, 151936, 512
    one = make_custom(1, gamma, V, 256, 64, "bf16", "mixture", seed=21, temperature=T)
    rng = np.random.default_rng(22)
    wl = dataclasses.replace(
        one, B=nb, U=np.repeat(one.U, nb, axis=0), target=np.repeat(one.target, nb, axis=0),
        hidden=np.repeat(one.hidden, nb, axis=0), anchor=np.repeat(one.anchor, nb),
        temperature=np.repeat(one.temperature, nb),
        uniforms=rng.random((nb, gamma + 1, 2), dtype=np.float32),
        W2=to_bf16_bits(np.zeros((256, V), dtype=np.float32)), requests=np.arange(nb))
    d = upload(wl, "cuda", scheduler=False)
    st = torch.zeros((1,), dtype=torch.int32, device="cuda")
    dr = dv.dspark_draft_block(d.U, d.W1, d.W2, d.anchor, d.temperature, d.uniforms, status=st)
    _, n_acc, _ = dv.dspark_verify(d.target, d.U, d.W1, d.W2, d.anchor, dr["tokens"],
                                   dr["q_tok"], dr["row_max"], dr["row_logZ"], d.temperature,
                                   d.uniforms, d.fixed_ell, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    n = n_acc.cpu().numpy().astype(np.float64)
    # per-position acceptance probabilities of the (prefix-independent) rows
    alpha = O.tv_label(one.target, one.U, O.f64(one.W1), np.zeros((256, V)), one.anchor,
                       np.zeros((1, gamma), dtype=np.int64), one.temperature)["label"][0]
    surv = np.cumprod(alpha)                      # P(n >= j), j = 1..gamma
    mean = surv.sum()
    second = sum((2 * j - 1) * surv[j - 1] for j in range(1, gamma + 1))
    se = np.sqrt((second - mean * mean) / nb)
    print(f"alpha {alpha}, closed form {mean:.4f} +- {se:.4f}, device mean {n.mean():.4f}",
          flush=True)
    assert abs(n.mean() - mean) < 5 * se
