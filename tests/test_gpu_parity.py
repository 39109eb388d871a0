"""Parity of the HIP path (through the C ABI) with the fp64 oracle.  GPU only.

Small shapes are checked on every row; they span several vocabulary tiles,
a ragged vocabulary tail (V % 256 != 0), ragged request blocks (B % 32 !=
0), fp32 and bf16 inputs, greedy rows mixed with sampled rows, a strong
Markov bias, and the degenerate sizes (one request, one position, a
vocabulary smaller than one tile, verify lengths 0 and gamma).  The five
workloads run at full size in the launch configuration the benchmark times,
every draft row and every verified request included.  An end-to-end test
also runs the oracle's whole step from the inputs alone and explains every
difference by its recorded margin, and the device's error flags are driven
with non-finite logits, out-of-range verify lengths and bad confidences.
"""

import numpy as np
import pytest
import torch

from gen import SPECS, make_config, make_custom
from oracle import f64
from oracle.parity import (check_confidence, check_draft, check_end_to_end, check_schedule,
                           check_verify)

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


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4], ids=lambda i: SPECS[i].name)
def test_full_size_workloads(cfg):
    # every draft row, every confidence, the whole schedule and every request's
    # verification (greedy requests included) against the oracle
    _say(f"{_workload(cfg)} full size, every row")
    wl = make_config(cfg)
    out = run_step(wl)
    B, g = wl.B, wl.gamma
    check_all(wl, out)
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
    """The earlier persistent kernel (8 and 4 waves per work-group) and the
    per-position launches give the same bits; the pipelined kernel sums the
    group and tile masses in another order,
    so its draws are held to the oracle on every row (tokens outside the
    1e-5 band identical, continuous outputs within tolerance) and its
    tokens agree with the per-position launches outside that band too."""
    import draft_verify_sampling_block_amd as dv
    from draft_verify_sampling_block_amd.step import upload
    wl = PATH_CASES[name]()
    d = upload(wl, "cuda", scheduler=False)
    res = {}
    for path in (1, 3, 4, 5, 6):
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
    # the pipelined kernel by a plain and by a cooperative launch: the same bits
    for i, key in enumerate(("tokens", "q_tok", "row_max", "row_logZ")):
        assert np.array_equal(res[5][i], res[6][i]), key
    assert all(res[p][4] == 0 for p in res), {p: res[p][4] for p in res}
    B, g = wl.B, wl.gamma
    rows = None
    if B * g > 200:
        rng = np.random.default_rng(7)
        rows = [(int(i) // g, int(i) % g) for i in rng.choice(B * g, 40, replace=False)]
    W1, W2 = f64(wl.W1), f64(wl.W2)
    print(check_draft(wl, W1, W2, *res[1][:4], rows=rows), flush=True)
    # every row when the oracle is quick enough, else the sampled rows
    rep = check_draft(wl, W1, W2, *res[5][:4], rows=rows)
    same = float(np.mean(res[5][0] == res[1][0]))
    print(f"pipelined: {rep}, tokens equal to the per-position launches: {same:.4f}", flush=True)


def test_draft_workspace_reuse_across_shapes():
    """One workspace serves calls of changing batch, block length, vocabulary,
    rank and dtype, through the pipelined kernel and the per-position
    launches, with no clearing between them: each call gives the bits a
    fresh zero-filled workspace gives."""
    import draft_verify_sampling_block_amd as dv
    from draft_verify_sampling_block_amd.step import upload
    # (B, gamma, V, rank, dtype, draft path)
    cases = [(96, 5, 20000, 64, "bf16", 5), (40, 4, 20000, 64, "bf16", 5),
             (128, 3, 30000, 256, "bf16", 5), (17, 6, 9000, 128, "bf16", 1),
             (33, 3, 12000, 64, "f32", 0), (17, 6, 9000, 128, "bf16", 5),
             (96, 5, 20000, 64, "bf16", 5)]
    need = max(dv.dspark_draft_block_workspace(B, g, V, r, 1) for B, g, V, r, _, _ in cases)
    shared = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for i, (B, g, V, r, dt, path) in enumerate(cases):
        _say(f"workspace reuse: B={B} gamma={g} V={V} rank={r} {dt} path {path}")
        wl = make_custom(B, g, V, r, 16, dt, "mixture", seed=21 + i % 6, temperature=0.8,
                         greedy_frac=0.2)
        d = upload(wl, "cuda", scheduler=False)
        outs = []
        old = dv.dspark_set_draft_path(path)
        try:
            for ws in (shared, None):
                st = torch.zeros((1,), dtype=torch.int32, device="cuda")
                o = dv.dspark_draft_block(d.U, d.W1, d.W2, d.anchor, d.temperature, d.uniforms,
                                          status=st, workspace=ws)
                torch.cuda.synchronize()
                assert int(st.item()) == 0
                outs.append({k: v.cpu().numpy() for k, v in o.items()})
        finally:
            dv.dspark_set_draft_path(old)
        for k in outs[0]:
            assert np.array_equal(outs[0][k], outs[1][k]), k


CONF_CASES = {
    "bf16-ragged-V1000-B40": lambda: SMALL["bf16-ragged-V1000-B40"](),
    "bf16-greedy-mix-T0.7": lambda: SMALL["bf16-greedy-mix-T0.7"](),
    "fp32-strong-bias-ragged": lambda: SMALL["fp32-strong-bias-ragged"](),
    "bf16-B300-rank128-V5000": lambda: make_custom(300, 3, 5000, 128, 24, "bf16", "mixture",
                                                   seed=9, temperature=0.8, greedy_frac=0.2),
    "qwen3-4b-block7 B=32 gamma=7 V=151936 full size": lambda: make_config(1),
    "long-proposal-g15 B=128 gamma=15 V=151936 full size": lambda: make_config(3),
}


@pytest.mark.parametrize("name", list(CONF_CASES))
def test_draft_block_conf_matches_the_separate_calls(name):
    """dspark_draft_block_conf gives the bits of dspark_draft_block followed by
    dspark_confidence (no temperatures) or dspark_confidence_sts (with them),
    through the pipelined kernel (its draw waves evaluate the head) and
    through the per-position launches (the head's own kernel follows)."""
    import draft_verify_sampling_block_amd as dv
    from draft_verify_sampling_block_amd.step import upload
    wl = CONF_CASES[name]()
    d = upload(wl, "cuda", scheduler=False)
    rng = np.random.default_rng(5)
    temps = torch.tensor(rng.uniform(0.5, 2.0, wl.gamma).astype(np.float32), device="cuda")
    keys = ("tokens", "q_tok", "row_max", "row_logZ")
    for path in (0, 1):
        for tp in (None, temps):
            _say(f"{name}: draft path {path}, temperatures {'given' if tp is not None else 'none'}")
            old = dv.dspark_set_draft_path(path)
            try:
                st = torch.zeros((1,), dtype=torch.int32, device="cuda")
                f = dv.dspark_draft_block_conf(d.U, d.W1, d.W2, d.anchor, d.temperature,
                                               d.uniforms, d.hidden, d.w, d.b0, tp, status=st)
                st2 = torch.zeros((1,), dtype=torch.int32, device="cuda")
                o = dv.dspark_draft_block(d.U, d.W1, d.W2, d.anchor, d.temperature, d.uniforms,
                                          status=st2)
                if tp is None:
                    c = dv.dspark_confidence(d.hidden, d.W1, d.anchor, o["tokens"], d.w, d.b0,
                                             status=st2)
                else:
                    c = dv.dspark_confidence_sts(d.hidden, d.W1, d.anchor, o["tokens"], d.w, d.b0,
                                                 tp, status=st2)
                torch.cuda.synchronize()
            finally:
                dv.dspark_set_draft_path(old)
            assert int(st.item()) == 0 and int(st2.item()) == 0
            for k in keys:
                assert torch.equal(f[k], o[k]), k
            assert torch.equal(f["conf"], c)


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


@pytest.mark.parametrize("case", ["tiny-config0", "qwen3-4b-block7", "long-proposal-g15",
                                  "greedy-mix-small"])
def test_end_to_end_against_the_oracle_step(case):
    """The oracle's whole step from the inputs alone, not fed any device
    output, against the device step; every difference explained by its
    recorded margin at its first occurrence."""
    _say(f"end to end {case}")
    wl = {"tiny-config0": lambda: make_config(0), "qwen3-4b-block7": lambda: make_config(1),
          "long-proposal-g15": lambda: make_config(3),
          "greedy-mix-small": lambda: make_custom(33, 4, 2048, 32, 16, "bf16", "two-class",
                                                  seed=21, temperature=0.7, greedy_frac=0.3,
                                                  sps_kind="linear:132", calibrated=True)}[case]()
    out = run_step(wl)
    rep = check_end_to_end(wl, out)
    print(rep, flush=True)
    # every request is identical or explained; in the long blocks of mixture
    # rows some draw of a request often lands in the 1e-5 band (background
    # tokens have intervals narrower than the band), so only most are identical
    assert rep["draft_identical"] + rep["draft_explained"] == wl.B
    assert rep["draft_identical"] >= wl.B // 2


def _flagged_step(wl, fixed_ell=None, conf_nan=False):
    """A step with the device inputs as given; returns outputs and status."""
    import draft_verify_sampling_block_amd as dv
    from draft_verify_sampling_block_amd.step import Step, upload
    d = upload(wl, "cuda", scheduler=fixed_ell is None)
    if fixed_ell is not None:
        d.sps = None
        d.fixed_ell = torch.from_numpy(np.asarray(fixed_ell, np.int32)).cuda()
    st = Step(d)
    st.run()
    out = None
    if conf_nan:
        conf = st.conf.clone()
        conf[0, 0] = float("nan")
        conf[1, 1] = 1.5
        conf[2, 0] = -0.25
        s2 = torch.zeros((1,), dtype=torch.int32, device="cuda")
        ell, order, stats = dv.dspark_schedule(conf, st.d.sps if st.d.sps is not None else
                                               torch.from_numpy(wl.sps).cuda(), status=s2)
        torch.cuda.synchronize()
        out = dict(ell=ell.cpu().numpy(), status2=int(s2.item()))
    torch.cuda.synchronize()
    h = lambda t: t.cpu().numpy()
    res = dict(tokens=h(st.tokens), q_tok=h(st.q_tok), row_max=h(st.row_max),
               row_logZ=h(st.row_logZ), out_tokens=h(st.out_tokens), n_accepted=h(st.n_accepted),
               ratio=h(st.ratio), ell=h(st.ell_used()), status=int(st.status.item()))
    if out:
        res.update(out)
    return res


def _in_range(wl, res):
    B, g = wl.B, wl.gamma
    assert np.all((res["tokens"] >= 0) & (res["tokens"] < wl.V))
    n = res["n_accepted"]
    assert np.all((n >= 0) & (n <= g))
    for b in range(B):
        assert 0 <= res["out_tokens"][b, n[b]] < wl.V
        assert np.all(res["out_tokens"][b, n[b] + 1:] == -1)


@pytest.mark.parametrize("where", ["U-nan", "U-inf", "U-all-neg-inf", "target-nan"])
def test_nonfinite_logits_are_flagged(where):
    # one request's rows poisoned: the step finishes, NONFINITE is raised,
    # every output stays in range and the other requests match the oracle
    _say(f"non-finite logits: {where}")
    for path in (0, 1):     # the single-launch draft kernel and the per-position launches
        import draft_verify_sampling_block_amd as dv
        wl = make_custom(6, 4, 1536, 32, 16, "bf16", "mixture", seed=31)
        nan16, inf16, ninf16 = np.uint16(0x7FC0), np.uint16(0x7F80), np.uint16(0xFF80)
        if where == "U-nan":
            wl.U[2, 1, 700] = nan16
        elif where == "U-inf":
            wl.U[2, 0, 5] = inf16
        elif where == "U-all-neg-inf":
            wl.U[2, 2, :] = ninf16
        else:
            wl.target[2, :, 100] = nan16
        old = dv.dspark_set_draft_path(path)
        try:
            res = _flagged_step(wl, fixed_ell=np.full(wl.B, wl.gamma))
        finally:
            dv.dspark_set_draft_path(old)
        assert res["status"] & 2, (where, path, res["status"])
        _in_range(wl, res)
        clean = [b for b in range(wl.B) if b != 2]
        rows = [(b, k) for b in clean for k in range(wl.gamma)]
        check_draft(wl, f64(wl.W1), f64(wl.W2), res["tokens"], res["q_tok"], res["row_max"],
                    res["row_logZ"], rows=rows)
        check_verify(wl, f64(wl.W1), f64(wl.W2), res["tokens"], res["ell"], res["out_tokens"],
                     res["n_accepted"], res["ratio"], requests=clean)


def test_out_of_range_verify_lengths_are_flagged_and_clamped():
    _say("verify lengths outside [0, gamma]")
    wl = make_custom(5, 4, 1024, 32, 16, "bf16", "mixture", seed=32)
    ell = np.array([7, -2, 4, 0, 100])
    res = _flagged_step(wl, fixed_ell=ell)
    assert res["status"] & 8
    _in_range(wl, res)
    # clamped lengths give the verification of the clamped values
    import draft_verify_sampling_block_amd as dv
    clamped = np.clip(ell, 0, wl.gamma)
    check_verify(wl, f64(wl.W1), f64(wl.W2), res["tokens"], clamped, res["out_tokens"],
                 res["n_accepted"], np.where(np.isnan(res["ratio"]), np.nan, res["ratio"]))
    del dv


def test_bad_confidences_are_flagged_and_clamped():
    _say("confidence NaN, above 1, below 0")
    wl = make_custom(6, 4, 1024, 32, 16, "bf16", "mixture", seed=33, sps_kind="linear:40",
                     calibrated=True)
    res = _flagged_step(wl, conf_nan=True)
    assert res["status2"] & 16
    assert np.all((res["ell"] >= 0) & (res["ell"] <= wl.gamma))
    # the NaN and the negative value count as 0: those requests verify nothing
    assert res["ell"][0] == 0 and res["ell"][2] == 0
