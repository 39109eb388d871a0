"""GPU parity of the capacity (two-step barrier) and threshold scheduler
modes with the fp64 oracle, through the C ABI.  GPU only.

Shapes span one candidate, single-position runs, both ranking paths (run
merging up to 4096 candidates, bitonic sort above) and the workloads'
R x gamma; confidences carry exact ties (1.0 and 0.5).  The capacity is
read from device memory, including the count an earlier Theta-rule call
wrote (the asynchronous chain), and K / threshold edge values are covered.
"""

import numpy as np
import pytest
import torch

from oracle.parity import check_schedule, check_schedule_mode

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1), (3, 64), (128, 15), (512, 7), (1000, 8), (8192, 1), (4096, 1), (273, 15),
          (128, 5)]


def _say(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_verify_sampling_block_amd as dv
    dv.load()


def _conf(seed, R, gamma):
    rng = np.random.default_rng(seed)
    c = rng.uniform(0.0, 1.0, (R, gamma)).astype(np.float32)
    c[rng.random((R, gamma)) < 0.1] = 1.0
    c[rng.random((R, gamma)) < 0.05] = 0.5
    return c


def _host(*ts):
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in ts]


@pytest.mark.parametrize("si", range(len(SHAPES)))
def test_capacity_matches_oracle(si):
    import draft_verify_sampling_block_amd as dv
    R, gamma = SHAPES[si]
    N = R * gamma
    c = _conf(50 + si, R, gamma)
    cd = torch.from_numpy(c).cuda()
    for K in sorted({0, 1, N // 3, N // 2 + 0.75, N - 1, N, N + 5, float(2 ** 40)}):
        _say(f"capacity R={R} gamma={gamma} K={K}")
        cap = torch.tensor([float(K)], dtype=torch.float64, device="cuda")
        ell, order, stats = dv.dspark_schedule_capacity(cd, cap)
        ell, order, stats = _host(ell, order, stats)
        print(check_schedule_mode(c, "capacity", float(K), ell, order, stats), flush=True)


@pytest.mark.parametrize("si", range(len(SHAPES)))
def test_threshold_matches_oracle(si):
    import draft_verify_sampling_block_amd as dv
    R, gamma = SHAPES[si]
    c = _conf(70 + si, R, gamma)
    cd = torch.from_numpy(c).cuda()
    a = np.cumprod(c.astype(np.float64), axis=1).reshape(-1)
    # thresholds at exact survival values (equality admits), between them,
    # and the edges
    picks = [float(a[len(a) // 2]), float(a[-1]), float(np.median(a))]
    for thr in [0.0, -1.0, 1e-300, 0.25, 0.5, 0.9, 1.0, float(np.nextafter(1.0, 2.0))] + picks:
        _say(f"threshold R={R} gamma={gamma} thr={thr!r}")
        ell, order, stats = dv.dspark_schedule_threshold(cd, thr)
        ell, order, stats = _host(ell, order, stats)
        print(check_schedule_mode(c, "threshold", thr, ell, order, stats), flush=True)


def test_capacity_nan_and_negative_take_nothing():
    import draft_verify_sampling_block_amd as dv
    c = _conf(3, 128, 15)
    cd = torch.from_numpy(c).cuda()
    for K in [float("nan"), -1.0, -1e300, 0.999]:
        _say(f"capacity K={K}")
        cap = torch.tensor([K], dtype=torch.float64, device="cuda")
        ell, order, stats = _host(*dv.dspark_schedule_capacity(cd, cap))
        assert ell.tolist() == [0] * 128
        check_schedule_mode(c, "capacity", K, ell, order, stats)
    ell, order, stats = _host(*dv.dspark_schedule_threshold(cd, float("nan")))
    assert ell.tolist() == [0] * 128
    check_schedule_mode(c, "threshold", float("nan"), ell, order, stats)


def test_two_step_chain_on_device():
    # step t-2: the Theta rule on older confidences writes its count into
    # stats[0]; step t: the capacity mode reads it from device memory while
    # ranking the current confidences -- no host round trip in between
    import draft_verify_sampling_block_amd as dv
    R, gamma = 128, 15
    old, new = _conf(91, R, gamma), _conf(92, R, gamma)
    n = R * (gamma + 1) + 1
    sps = (2400 * (1 - 0.55 * np.arange(n) / 1024)).astype(np.float64)
    sps[0] = 0.0
    _say("chain: schedule(old) -> capacity(new)")
    ell0, order0, stats0 = dv.dspark_schedule(torch.from_numpy(old).cuda(),
                                              torch.from_numpy(sps).cuda())
    ell1, order1, stats1 = dv.dspark_schedule_capacity(torch.from_numpy(new).cuda(), stats0)
    ell0, order0, stats0, ell1, order1, stats1 = _host(ell0, order0, stats0, ell1, order1, stats1)
    check_schedule(old, sps, ell0, order0, stats0)
    K = float(stats0[0])
    assert K > 0
    print(check_schedule_mode(new, "capacity", K, ell1, order1, stats1), flush=True)
    assert int(ell1.sum()) == int(K)


def test_abi_rejects_bad_capacity_pointer():
    import draft_verify_sampling_block_amd as dv
    lib = dv.load()
    x = torch.zeros(64, dtype=torch.float32, device="cuda")
    p = x.data_ptr()
    big = 1 << 20
    assert lib.dspark_schedule_capacity(4, 5, p, None, p, p, p, None, p, big, None) == -1
    assert lib.dspark_schedule_capacity(4, 5, p, p + 4, p, p, p, None, p, big, None) == -3
    assert lib.dspark_schedule_capacity(4, 5, p, p, p, p, p, None, None, 0, None) == -4
    assert lib.dspark_schedule_capacity(9000, 1, p, p, p, p, p, None, None, 0, None) == -5
    assert lib.dspark_schedule_threshold(0, 5, p, 0.5, p, p, p, None, None, 0, None) == -1
