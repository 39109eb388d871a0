"""dspark_schedule_noalloc, the scheduler entry point that allocates nothing
(its ranks live in the library's own per-device scratch), against
dspark_schedule with a caller-supplied workspace, through the C ABI on the
GPU: identical ell, order and (n, tau, Theta) on consecutive calls, the second
with a smaller batch, and on a batch large enough to rank without scratch."""

import numpy as np
import pytest
import torch

import draft_verify_sampling_block_amd as dv

pytestmark = pytest.mark.gpu


def _case(R, gamma, seed):
    rng = np.random.default_rng(seed)
    c = rng.uniform(0.3, 1.0, (R, gamma)).astype(np.float32)
    c[rng.random((R, gamma)) < 0.1] = np.float32(0.75)     # ties across requests
    c[0, :] = 1.0
    n = R * (gamma + 1) + 1
    sps = 2400.0 * (1.0 - 0.55 * np.arange(n) / n)
    sps[0] = 0.0
    return (torch.from_numpy(c).to("cuda"), torch.from_numpy(sps).to("cuda"))


def _host(x):
    return x.cpu().numpy()


def _compare(R, gamma, seed):
    print(f"[no-alloc] R={R} gamma={gamma} seed={seed}", flush=True)
    conf, sps = _case(R, gamma, seed)
    st_a = torch.zeros((1,), dtype=torch.int32, device="cuda")
    st_b = torch.zeros((1,), dtype=torch.int32, device="cuda")
    ell_a, ord_a, sta_a = dv.dspark_schedule(conf, sps, status=st_a)
    ell_b, ord_b, sta_b = dv.dspark_schedule_noalloc(conf, sps, status=st_b)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_host(ell_b), _host(ell_a))
    np.testing.assert_array_equal(_host(ord_b), _host(ord_a))
    np.testing.assert_array_equal(_host(sta_b), _host(sta_a))   # n, tau, Theta bit for bit
    assert int(st_a.item()) == 0 and int(st_b.item()) == 0
    # the admitted sets are prefixes and add up to n
    assert int(_host(ell_b).sum()) == int(_host(sta_b)[0])
    return _host(ell_b)


def test_noalloc_matches_schedule_on_consecutive_calls():
    # 1920 candidates (ranked through the scratch), then 280 (the same scratch,
    # rewritten), then 7200 (ranked inside the one work-group, no scratch)
    e1 = _compare(128, 15, 1)
    e2 = _compare(40, 7, 2)
    assert e1.shape == (128,) and e2.shape == (40,)
    _compare(600, 12, 3)
    _compare(3, 2, 4)


def test_noalloc_without_order_and_stats():
    conf, sps = _case(64, 5, 5)
    ell_a, _, _ = dv.dspark_schedule(conf, sps)
    ell_b = torch.empty((64,), dtype=torch.int32, device="cuda")
    lib = dv.load()
    rc = lib.dspark_schedule_noalloc(64, 5, dv._ptr(conf), dv._ptr(sps), int(sps.numel()),
                                     dv._ptr(ell_b), None, None, None, dv._stream())
    assert rc == 0
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_host(ell_b), _host(ell_a))


def test_noalloc_rejects_bad_sizes_before_launch():
    conf, sps = _case(4, 2, 6)
    lib = dv.load()
    ell = torch.empty((4,), dtype=torch.int32, device="cuda")
    # more candidates than any scheduler entry point supports
    rc = lib.dspark_schedule_noalloc(9000, 1, dv._ptr(conf), dv._ptr(sps), 10, dv._ptr(ell),
                                     None, None, None, dv._stream())
    assert rc == -5 and b"exceeds" in lib.dspark_last_error()
    rc = lib.dspark_schedule_noalloc(4, 2, dv._ptr(conf), dv._ptr(sps), 0, dv._ptr(ell),
                                     None, None, None, dv._stream())
    assert rc == -1
