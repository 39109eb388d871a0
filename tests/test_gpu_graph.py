"""The whole step (draft, confidence, schedule, verify) captured in a HIP
graph and replayed: every replay gives the eager step's outputs bit for bit,
with eager steps and host synchronisations between the replays.  GPU only.

The library enqueues only kernels (its flag resets are a kernel, not a
memset), so a caller may capture it; this checks that the cooperative
persistent draft launch, the workspaces and the device status word behave
the same under replay.
"""

import pytest
import torch

from gen import make_config, make_custom

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_verify_sampling_block_amd as dv
    dv.load()


CASES = {
    "bf16-ragged-V1000-B40": lambda: make_custom(40, 4, 1000, 64, 32, "bf16", "mixture", seed=1,
                                                 sps_kind="linear:200", calibrated=True),
    "long-proposal B=128 gamma=15 V=151936 full size": lambda: make_config(3),
}


@pytest.mark.parametrize("name", list(CASES))
def test_step_graph_replay_matches_eager(name):
    from draft_verify_sampling_block_amd.step import Step, upload
    print(f"\n[case] graph replay {name}", flush=True)
    st = Step(upload(CASES[name](), "cuda"))
    st.run()
    torch.cuda.synchronize()
    outs = lambda: [t.clone() for t in (st.tokens, st.q_tok, st.conf, st.ell_used(),
                                        st.out_tokens, st.n_accepted)]
    ref = outs()
    assert int(st.status.item()) == 0
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        st.run()
    for _ in range(3):
        for t in (st.tokens, st.out_tokens, st.n_accepted):
            t.fill_(-7)                      # stale values must be overwritten
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outs()
        for a, b in zip(ref, got):
            assert torch.equal(a, b)
        assert int(st.status.item()) == 0
        st.run()                             # eager work between replays
        torch.cuda.synchronize()
