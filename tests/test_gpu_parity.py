"""Parity of the HIP path (through the C ABI) with the fp64 oracle.  GPU only.

Small shapes are checked on every row; they span several vocabulary tiles,
a ragged vocabulary tail (V % 256 != 0), ragged request blocks (B % 32 !=
0), fp32 and bf16 inputs, greedy rows mixed with sampled rows, a strong
Markov bias, and the degenerate sizes (one request, one position, a
vocabulary smaller than one tile, verify lengths 0 and gamma).  The five
workloads run at full size in the launch configuration the benchmark times;
there the draft and verify are checked on sampled rows/requests and the
confidence and scheduler on everything.
"""

import numpy as np
import pytest
import torch

from gen import SPECS, make_config, make_custom
from oracle import f64
from oracle.parity import check_confidence, check_draft, check_schedule, check_verify

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
    dv.load()  # fails loudly if the library is missing


def run_step(wl, scheduler=None):
    from draft_verify_sampling_block_amd.step import Step, upload
    d = upload(wl, "cuda", scheduler)
    st = Step(d).run()
    torch.cuda.synchronize()
    h = lambda t: t.detach().cpu().numpy()
    return dict(tokens=h(st.tokens), q_tok=h(st.q_tok), row_max=h(st.row_max),
                row_logZ=h(st.row_logZ), conf=h(st.conf), ell=h(st.ell_used()),
                order=h(st.order), stats=h(st.stats), out_tokens=h(st.out_tokens),
                n_accepted=h(st.n_accepted), ratio=h(st.ratio), status=int(st.status.item()),
                sched=d.sps is not None)


def check_all(wl, out, draft_rows=None, verify_requests=None):
    W1_64, W2_64 = f64(wl.W1), f64(wl.W2)
    rep = {}
    rep["draft"] = check_draft(wl, W1_64, W2_64, out["tokens"], out["q_tok"], out["row_max"],
                               out["row_logZ"], rows=draft_rows)
    rep["conf"] = check_confidence(wl, out["tokens"], out["conf"])
    if out["sched"]:
        rep["sched"] = check_schedule(out["conf"], wl.sps, out["ell"], out["order"], out["stats"])
    rep["verify"] = check_verify(wl, W1_64, W2_64, out["tokens"], out["ell"], out["out_tokens"],
                                 out["n_accepted"], out["ratio"], requests=verify_requests)
    assert out["status"] == 0, f"device status flags {out['status']}"
    print(rep, flush=True)
    return rep


SMALL = {
    "fp32-tiny-config0": lambda: make_config(0),
    "bf16-ragged-V1000-B40": lambda: make_custom(40, 4, 1000, 64, 32, "bf16", "mixture", seed=1,
                                                 sps_kind="linear:200", calibrated=True),
    "bf16-greedy-mix-T0.7": lambda: make_custom(33, 3, 2048, 32, 16, "bf16", "two-class", seed=2,
                                                temperature=0.7, greedy_frac=0.3,
                                                sps_kind="linear:132", calibrated=True),
    "bf16-strong-bias": lambda: make_custom(8, 6, 4096, 128, 64, "bf16", "gaussian", seed=3,
                                            w_std=0.25, sps_kind="linear:64"),
    "fp32-strong-bias-ragged": lambda: make_custom(5, 5, 776, 64, 24, "f32", "mixture", seed=4,
                                                   w_std=0.3, sps_kind="linear:40"),
    "bf16-one-request-one-position-V8": lambda: make_custom(1, 1, 8, 32, 8, "bf16", "gaussian",
                                                            seed=5, sps_kind="linear:4"),
    "bf16-fixed-ell-gamma": lambda: make_custom(37, 5, 1536, 64, 16, "bf16", "mixture", seed=6),
    # the library's largest block and vocabulary (4096 tiles: more than the
    # persistent kernel keeps on chip, so the per-position launches run)
    "bf16-max-gamma64-V262144": lambda: make_custom(2, 64, 262144, 32, 64, "bf16", "mixture",
                                                    seed=12, sps_kind="linear:300",
                                                    calibrated=True),
    "bf16-temperature-extremes": lambda: _with_temperatures(
        make_custom(45, 5, 3000, 64, 32, "bf16", "mixture", seed=11, sps_kind="linear:230",
                    calibrated=True), [0.05, 0.3, 1.0, 4.0, 0.0]),
    # batch sizes at the edges of the verify statistics kernels' forms:
    # 97 = three full 32-request blocks and one row (tile loop), 129 = four
    # full blocks and one row (the per-tile fallback), ragged vocabularies
    "bf16-B97-V2000-tile-loop-edge": lambda: make_custom(97, 3, 2000, 64, 16, "bf16", "mixture",
                                                         seed=13, sps_kind="linear:300",
                                                         calibrated=True),
    "bf16-B129-V1800-fallback-edge": lambda: make_custom(129, 3, 1800, 64, 16, "bf16",
                                                         "mixture", seed=14,
                                                         sps_kind="linear:400", calibrated=True),
}


def _with_temperatures(wl, cycle):
    """Per-request temperatures cycling through `cycle` (very sharp, very
    flat and greedy requests in one batch)."""
    wl.temperature[:] = np.resize(np.asarray(cycle, dtype=np.float32), wl.B)
    return wl


@pytest.mark.parametrize("name", list(SMALL))
def test_small_full_parity(name):
    _say(name)
    wl = SMALL[name]()
    out = run_step(wl)
    check_all(wl, out)


def test_strong_bias_changes_the_draft():
    # the Markov bias must actually move the samples: W2 = 0 gives other tokens
    _say("strong-bias-vs-zero-W2")
    wl = SMALL["bf16-strong-bias"]()
    out = run_step(wl)
    wl0 = SMALL["bf16-strong-bias"]()
    wl0.W2 = np.zeros_like(wl0.W2)
    out0 = run_step(wl0)
    check_draft(wl0, f64(wl0.W1), f64(wl0.W2), out0["tokens"], out0["q_tok"], out0["row_max"],
                out0["row_logZ"])
    assert (out["tokens"] != out0["tokens"]).mean() > 0.3


@pytest.mark.parametrize("ell_value", [0, "gamma"])
def test_verify_extreme_lengths(ell_value):
    _say(f"verify-ell-{ell_value}")
    import draft_verify_sampling_block_amd as dv
    from draft_verify_sampling_block_amd.step import Step, upload
    wl = make_custom(34, 4, 1288, 64, 16, "bf16", "mixture", seed=7)
    d = upload(wl, "cuda", scheduler=False)
    L = 0 if ell_value == 0 else wl.gamma
    d.fixed_ell = torch.full((wl.B,), L, dtype=torch.int32, device="cuda")
    st = Step(d).run()
    torch.cuda.synchronize()
    h = lambda t: t.cpu().numpy()
    rep = check_verify(wl, f64(wl.W1), f64(wl.W2), h(st.tokens), h(d.fixed_ell), h(st.out_tokens),
                       h(st.n_accepted), h(st.ratio))
    if L == 0:
        assert np.all(h(st.n_accepted) == 0)
    print(rep, flush=True)


def test_verify_rejections_past_eight_slots():
    """A 20-slot block verified in full with the target equal to the base
    logits (the Markov bias alone separates p and q): first rejections fall
    on both sides of slot 8, where the accept-flag scan reads its second
    group of eight flags, and one request accepts every slot."""
    _say("verify-long-block")
    from draft_verify_sampling_block_amd.step import Step, upload
    wl = make_custom(24, 20, 1024, 32, 16, "bf16", "mixture", seed=16, w_std=0.3)
    wl.target[:, :wl.gamma] = wl.U
    d = upload(wl, "cuda", scheduler=False)
    d.fixed_ell = torch.full((wl.B,), wl.gamma, dtype=torch.int32, device="cuda")
    st = Step(d).run()
    torch.cuda.synchronize()
    h = lambda t: t.cpu().numpy()
    rep = check_verify(wl, f64(wl.W1), f64(wl.W2), h(st.tokens), h(d.fixed_ell), h(st.out_tokens),
                       h(st.n_accepted), h(st.ratio))
    n = h(st.n_accepted)
    assert np.any(n < 8) and np.any((n > 8) & (n < wl.gamma)) and np.any(n == wl.gamma), n
    print(rep, flush=True)


@pytest.mark.parametrize("seed", range(8))
def test_schedule_random_confidences(seed):
    # sizes on both sides of 4096 candidates (run merging below, bitonic
    # sort above), runs of one position, and one request
    import draft_verify_sampling_block_amd as dv
    rng = np.random.default_rng(seed)
    R, gamma = [(1, 1), (3, 64), (128, 15), (512, 7), (1000, 8), (8192, 1), (4096, 1),
                (273, 15)][seed]
    _say(f"schedule R={R} gamma={gamma}")
    c = rng.uniform(0.0, 1.0, (R, gamma)).astype(np.float32)
    c[rng.random((R, gamma)) < 0.1] = 1.0           # ties in survival
    c[rng.random((R, gamma)) < 0.05] = 0.5
    n = R * (gamma + 1) + 1
    kind = seed % 3
    if kind == 0:
        sps = 2400 * (1 - 0.55 * np.arange(n) / n)
    elif kind == 1:
        sps = rng.uniform(50, 100, n)                 # jagged
    else:
        sps = np.full(n, 10.0)
        sps[: n // 2] = 20.0
    sps = sps.astype(np.float64)
    sps[0] = 0.0
    ell, order, stats = dv.dspark_schedule(torch.from_numpy(c).cuda(), torch.from_numpy(sps).cuda())
    torch.cuda.synchronize()
    print(check_schedule(c, sps, ell.cpu().numpy(), order.cpu().numpy(), stats.cpu().numpy()))


FULL_DRAFT_ROWS = 40
FULL_VERIFY_REQ = 20


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4], ids=lambda i: SPECS[i].name)
def test_full_size_workloads(cfg):
    _say(f"{_workload(cfg)} full size")
    wl = make_config(cfg)
    out = run_step(wl)
    rng = np.random.default_rng(100 + cfg)
    B, g = wl.B, wl.gamma
    if B * g <= 64:
        rows, reqs = None, None
    else:
        flat = rng.choice(B * g, FULL_DRAFT_ROWS, replace=False)
        rows = [(int(i) // g, int(i) % g) for i in flat]
        reqs = sorted(rng.choice(B, min(B, FULL_VERIFY_REQ), replace=False).tolist())
    check_all(wl, out, draft_rows=rows, verify_requests=reqs)
    # properties on every request
    n, ell = out["n_accepted"], out["ell"]
    assert np.all((0 <= n) & (n <= ell))
    for b in range(B):
        assert np.array_equal(out["out_tokens"][b, : n[b]], out["tokens"][b, : n[b]])
        assert 0 <= out["out_tokens"][b, n[b]] < wl.V
    assert np.all((out["tokens"] >= 0) & (out["tokens"] < wl.V))
    print(f"{_workload(cfg)}: mean ell {ell.mean():.2f}, mean accepted {n.mean():.2f}", flush=True)


PATH_CASES = {
    "bf16-ragged-V1000-B40": lambda: SMALL["bf16-ragged-V1000-B40"](),
    "bf16-greedy-mix-T0.7": lambda: SMALL["bf16-greedy-mix-T0.7"](),
    "bf16-strong-bias": lambda: SMALL["bf16-strong-bias"](),
    "bf16-temperature-extremes": lambda: SMALL["bf16-temperature-extremes"](),
    "bf16-B300-rank128-V5000": lambda: make_custom(300, 3, 5000, 128, 16, "bf16", "mixture",
                                                   seed=9, temperature=0.8, greedy_frac=0.2),
    "qwen3-4b-block7 B=32 gamma=7 V=151936 full size": lambda: make_config(1),
}


@pytest.mark.parametrize("name", list(PATH_CASES))
def test_draft_paths_agree(name):
    """The persistent kernel (8 and 4 waves per work-group) and the
    per-position launches give the same bits."""
    import draft_verify_sampling_block_amd as dv
    from draft_verify_sampling_block_amd.step import upload
    wl = PATH_CASES[name]()
    d = upload(wl, "cuda", scheduler=False)
    res = {}
    for path in (1, 3, 4):
        _say(f"{name}: draft path {path}")
        old = dv.dspark_set_draft_path(path)
        try:
            st = torch.zeros((1,), dtype=torch.int32, device="cuda")
            out = dv.dspark_draft_block(d.U, d.W1, d.W2, d.anchor, d.temperature, d.uniforms,
                                        status=st)
            torch.cuda.synchronize()
        finally:
            dv.dspark_set_draft_path(old)
        res[path] = [out[k].cpu().numpy() for k in ("tokens", "q_tok", "row_max", "row_logZ")]
        res[path].append(int(st.item()))
    for path in (3, 4):
        for i, key in enumerate(("tokens", "q_tok", "row_max", "row_logZ")):
            assert np.array_equal(res[1][i], res[path][i]), (path, key)
    assert all(res[p][4] == 0 for p in res), {p: res[p][4] for p in res}
    B, g = wl.B, wl.gamma
    rows = None
    if B * g > 200:
        rng = np.random.default_rng(7)
        rows = [(int(i) // g, int(i) % g) for i in rng.choice(B * g, 40, replace=False)]
    print(check_draft(wl, f64(wl.W1), f64(wl.W2), *res[1][:4], rows=rows), flush=True)


def test_repeat_is_deterministic():
    _say("determinism")
    wl = SMALL["bf16-ragged-V1000-B40"]()
    a, b = run_step(wl), run_step(wl)
    for k in ("tokens", "q_tok", "row_max", "row_logZ", "conf", "ell", "order", "out_tokens",
              "n_accepted"):
        assert np.array_equal(a[k], b[k]), k


def test_bad_token_is_flagged_and_clamped():
    _say("status flags")
    wl = make_custom(4, 2, 512, 32, 8, "bf16", "gaussian", seed=8)
    wl.anchor = wl.anchor.copy()
    wl.anchor[1] = wl.V + 5
    out = run_step(wl, scheduler=False)
    assert out["status"] & 1
    assert np.all((out["tokens"] >= 0) & (out["tokens"] < wl.V))


def test_abi_rejects_bad_arguments_without_launching():
    _say("abi errors")
    import draft_verify_sampling_block_amd as dv
    lib = dv.load()
    x = torch.zeros(64, dtype=torch.float32, device="cuda")
    p = x.data_ptr()
    assert lib.dspark_draft_block(4, 5, 1000, 32, 0, *([p] * 11), p, 0, None) == -4  # workspace
    assert lib.dspark_draft_block(4, 5, 1001, 32, 0, *([p] * 11), p, 1 << 30, None) == -1  # V % 8
    assert lib.dspark_draft_block(4, 5, 1000, 33, 0, *([p] * 11), p, 1 << 30, None) == -1  # rank
    assert lib.dspark_draft_block(4, 5, 1000, 32, 7, *([p] * 11), p, 1 << 30, None) == -2  # dtype
    assert lib.dspark_draft_block(4, 5, 1000, 32, 0, *([p + 4] + [p] * 10), p, 1 << 30, None) == -3
    assert lib.dspark_schedule(9000, 1, p, p, 10, p, p, p, None, None, 0, None) == -5
