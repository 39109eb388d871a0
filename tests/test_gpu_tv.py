"""GPU parity of dspark_tv_label (acceptance label 1 - TV per drafted
position) with the fp64 oracle, through the C ABI.  GPU only.

The labels are computed on the device's own drafted tokens and draft row
statistics (dspark_draft_block), as a training pipeline would chain them.
Small shapes are checked on every row (fp32 and bf16, ragged vocabulary
tail and request blocks, greedy rows mixed in, a strong Markov bias, one
request / one position / a vocabulary below one tile); full-size workloads
on sampled rows.
"""

import numpy as np
import pytest
import torch

from gen import SPECS, make_config, make_custom
from oracle import f64
from oracle.parity import check_tv

pytestmark = pytest.mark.gpu


def _workload(i):
    """A workload's name and sizes (for progress lines)."""
    sp = SPECS[i]
    return f"{sp.name} B={sp.B} gamma={sp.gamma} V={sp.V} rank={sp.rank} {sp.dtype}"



def _say(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_verify_sampling_block_amd as dv
    dv.load()


CASES = {
    "fp32-tiny-config0": lambda: make_config(0),
    "bf16-ragged-V1000-B40": lambda: make_custom(40, 4, 1000, 64, 32, "bf16", "mixture", seed=1),
    "bf16-greedy-mix-T0.7": lambda: make_custom(33, 3, 2048, 32, 16, "bf16", "two-class", seed=2,
                                                temperature=0.7, greedy_frac=0.3),
    "bf16-strong-bias": lambda: make_custom(8, 6, 4096, 128, 64, "bf16", "gaussian", seed=3,
                                            w_std=0.25),
    "fp32-strong-bias-ragged": lambda: make_custom(5, 5, 776, 64, 24, "f32", "mixture", seed=4,
                                                   w_std=0.3),
    "bf16-one-request-one-position-V8": lambda: make_custom(1, 1, 8, 32, 8, "bf16", "gaussian",
                                                            seed=5),
    "bf16-temperature-extremes": lambda: _with_temperatures(
        make_custom(45, 5, 3000, 64, 32, "bf16", "mixture", seed=11), [0.05, 0.3, 1.0, 4.0, 0.0]),
    # 97 requests = three full 32-request blocks and one row, ragged tiles
    "bf16-B97-V2000-partial-block": lambda: _with_temperatures(
        make_custom(97, 3, 2000, 64, 16, "bf16", "mixture", seed=13), [1.0, 0.6, 0.0, 1.3]),
}


def _with_temperatures(wl, cycle):
    wl.temperature[:] = np.resize(np.asarray(cycle, dtype=np.float32), wl.B)
    return wl


def _run(wl):
    import draft_verify_sampling_block_amd as dv
    from draft_verify_sampling_block_amd.step import upload
    d = upload(wl, "cuda", scheduler=False)
    st = torch.zeros((1,), dtype=torch.int32, device="cuda")
    dr = dv.dspark_draft_block(d.U, d.W1, d.W2, d.anchor, d.temperature, d.uniforms, status=st)
    tv, label = dv.dspark_tv_label(d.target, d.U, d.W1, d.W2, d.anchor, dr["tokens"],
                                   dr["row_max"], dr["row_logZ"], d.temperature, status=st)
    torch.cuda.synchronize()
    h = lambda t: t.cpu().numpy()
    return h(dr["tokens"]), h(tv), h(label), int(st.item())


@pytest.mark.parametrize("name", list(CASES))
def test_tv_label_small(name):
    _say(f"tv {name}")
    wl = CASES[name]()
    tokens, tv, label, status = _run(wl)
    assert status == 0, status
    rep = check_tv(wl, f64(wl.W1), f64(wl.W2), tokens, tv, label)
    print(rep, flush=True)
    assert np.all((tv >= -1e-6) & (tv <= 1 + 1e-6))


@pytest.mark.parametrize("cfg", [1, 3], ids=lambda i: SPECS[i].name)
def test_tv_label_full_size(cfg):
    _say(f"label {_workload(cfg)}")
    wl = make_config(cfg)
    tokens, tv, label, status = _run(wl)
    assert status == 0, status
    rng = np.random.default_rng(cfg)
    B, g = tokens.shape
    rows = [(int(i) // g, int(i) % g) for i in rng.choice(B * g, 24, replace=False)]
    rep = check_tv(wl, f64(wl.W1), f64(wl.W2), tokens, tv, label, rows=rows)
    print(rep, flush=True)
    assert np.all(np.isfinite(tv))


def test_tv_label_rejects_small_workspace():
    import draft_verify_sampling_block_amd as dv
    lib = dv.load()
    x = torch.zeros(64, dtype=torch.float32, device="cuda")
    p = x.data_ptr()
    assert lib.dspark_tv_label(4, 5, 1000, 32, 0, *([p] * 12), p, 8, None) == -4
    assert lib.dspark_tv_label(4, 5, 1000, 32, 0, *([p] * 9), None, p, p, p, 1 << 30, None) == -1
