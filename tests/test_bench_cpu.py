"""The benchmark's byte accounting and counter bookkeeping (no GPU).

The algorithmic bytes are checked against sums written out by hand for a
tiny workload, and the counter traffic is reported only while the draft
kernel's sources hash to the value recorded with the counters.
"""

import os

import numpy as np

import bench
from gen import make_custom


def test_step_bytes_count_each_input_once():
    wl = make_custom(3, 4, 64, 32, 16, "bf16", "gaussian", seed=0)
    ell = np.array([4, 2, 0])
    n_acc = np.array([4, 1, 0])     # request 1 rejects at slot 1; request 2 verifies nothing
    e, B, g, V, r, H = 2, 3, 4, 64, 32, 16
    target_rows = (4 + 1) + (1 + 1) + (0 + 1)      # slots up to the reject or the bonus slot
    u_rows = B * g + 1                             # every base-logit row, and one re-read
    want = (e * V * (u_rows + target_rows) + e * r * V + e * B * g * (H + r)
            + 4 * B * (g + 1) * 2 + 4 * B * g * 4 + 4 * B * (g + 1))
    assert bench.algorithmic_bytes(wl, ell, n_acc) == want


def test_draft_kernel_bytes():
    # every U row, W2 once, one W1 row per (request, position), anchors,
    # temperatures, draw uniforms and four [B, gamma] outputs; the tile
    # statistics are the kernel's intermediates and are not counted
    wl = make_custom(3, 4, 200, 32, 16, "bf16", "gaussian", seed=0, greedy_frac=0.34)
    want = (2 * 3 * 4 * 200 + 2 * 32 * 200 + 2 * 3 * 4 * 32
            + 4 * 3 + 4 * 3 + 4 * 3 * 4 + 4 * 3 * 4 * 4)
    assert bench.draft_kernel_bytes(wl, "pdraft_kernel") == want
    assert bench.draft_kernel_bytes(wl, "pdraft_pipe_kernel") == want
    # with the confidence head in the same launch: the hidden states [B, gamma, H]
    # and the confidences (its W1 rows are the gathered ones)
    assert bench.draft_kernel_bytes(wl, "pdraft_pipe_kernel", with_conf=True) == (
        want + 2 * 3 * 4 * 16 + 4 * 3 * 4)
    nT = (200 + 63) // 64
    greedy = int(np.sum(~(np.asarray(wl.temperature) > 0)))
    assert greedy == 1
    # written once and read once per position: packed (max, sum) words for
    # every request, argmax words for the greedy one
    assert bench.draft_intermediate_bytes(wl, "pdraft_kernel") == 4 * 2 * (8 * 3 * nT + 4 * nT)
    # per-position launches: that position's rows and a 1/gamma share of W2
    assert bench.draft_kernel_bytes(wl, "draft_stats_kernel") == (
        2 * 3 * 200 + 2 * 3 * 32 + 2 * 32 * 200 / 4)


def test_tv_label_bytes():
    wl = make_custom(5, 3, 128, 64, 16, "bf16", "gaussian", seed=0)
    want = 2 * 128 * 2 * 5 * 3 + 2 * 64 * 128 + 2 * 5 * 3 * 64 + 4 * 5 * 3 * 4 + 4 * 5
    assert bench.tv_label_bytes(wl) == want


def test_counter_traffic_follows_the_source_hash(monkeypatch, tmp_path):
    rec = os.path.join(bench.ROOT, "profiles", "pdraft_pipe_kernel-long-proposal-g15.counters.txt")
    kv = dict(line.strip().split("=", 1) for line in open(rec)
              if "=" in line and not line.startswith("#"))
    want = (float(kv["fetch_kib_per_dispatch"]) * float(kv["fetch_scale"])
            + float(kv["write_kib_per_dispatch"]) * float(kv["write_scale"])) * 1024.0
    got = bench.counter_traffic("pdraft_pipe_kernel", "long-proposal-g15")
    if kv["source_sha256"] == bench.kernel_source_hash():
        assert got == want
    else:
        assert got is None
    # a recorded hash that does not match the sources gives no traffic
    fake_root = tmp_path
    (fake_root / "profiles").mkdir()
    text = open(rec).read().replace(kv["source_sha256"], "0" * 64)
    (fake_root / "profiles" / "pdraft_pipe_kernel-long-proposal-g15.counters.txt").write_text(text)
    monkeypatch.setattr(bench, "ROOT", str(fake_root))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "f" * 64)
    assert bench.counter_traffic("pdraft_pipe_kernel", "long-proposal-g15") is None
    assert bench.counter_traffic("pdraft_pipe_kernel", "high-concurrency") is None   # none recorded


def test_kernel_bytes_per_launch():
    wl = make_custom(3, 4, 64, 32, 16, "bf16", "gaussian", seed=0, temperature=1.0)
    ell = np.array([4, 2, 0])
    n_acc = np.array([4, 1, 0])
    kb = bench.kernel_bytes(wl, ell, n_acc)
    # target rows up to the first reject or the bonus slot: 5 + 2 + 1
    assert kb["verify_rows_kernel"] == 2 * 64 * (5 + 2 + 1)
    # the one rejecting request's base-logit row (the q recompute)
    assert kb["verify_tile_stats_kernel"] == 2 * 64 * 1
    assert kb["confidence_kernel"] == 2 * 3 * 4 * (16 + 32) + 4 * 3 * 4
    rd = bench.kernel_bytes_read(wl, ell, n_acc)
    # as built: every slot up to ell (bonus included), the final rows and W2 again
    assert rd["verify_rows_kernel"] == 2 * 64 * (5 + 3 + 1)
    assert rd["verify_tile_stats_kernel"] == 2 * 64 * (3 + 1) + 2 * 32 * 64


def test_rnn_draft_bytes():
    wl = make_custom(3, 4, 64, 32, 16, "bf16", "gaussian", seed=0)
    e, B, g, V, r, H = 2, 3, 4, 64, 32, 16
    want = (e * B * g * V + e * r * V + e * B * g * H + e * 3 * r * (2 * r + H) + 4 * 3 * r
            + e * B * g * r + 4 * B * 2 + 4 * B * g + 4 * B * g * 4 + e * B * g * r
            + 4 * B * g * r)
    assert bench.rnn_draft_bytes(wl) == want
