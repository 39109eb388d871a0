"""Benchmark one decode step of the DSpark sampling path on one MI355X.

A step = dspark_draft_block_conf (the draft and the confidence head in one
call: one launch where the single-launch draft kernel runs, whose draw waves
evaluate the head) -> dspark_schedule (or the fixed verify length) ->
dspark_verify over one batch, inputs resident in HBM.  Prints ONE JSON
line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3]
                    [--no-cpu-baseline] [--cpu-requests N]

value      = B * gamma / (time per step), drafted-and-verified positions/s
roofline   = the draft kernel (pdraft_pipe_kernel, or pdraft_kernel /
             draft_stats_kernel where those run): algorithmic bytes per
             launch / its mean duration, timed with per-launch HIP events in a
             separate pass of K steps (events are kept out of the pass that
             gives `value`)
order      = one step (for the next rows' inputs), the next rows' calls, the
             read ceiling, the per-kernel pass, then the W warm-up and the K
             timed steps: the GPU's clocks rise over the first tens of
             milliseconds of load, and this order times the K steps at the
             clocks a serving loop holds
cpu_baseline = the fp64 oracle on a bounded sample of the same workload
roofline.measured_read_ceiling_gbs = a plain streaming read (torch per-row
             sums over 4 GiB) timed in the same run; the fractions of it sit beside the
             fractions of the published 8 TB/s
next_rows  = per-call times of the scheduler stop-rule variants (capacity,
             threshold) and of the acceptance-label kernels on the first
             step's confidences and drafts (outside `value`)
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "draft+verify positions/sec (B×γ per step) at V=151936; % of HBM peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB, 5 times "
                         "(a reference for hardware byte counters), and exit")
    ap.add_argument("--draft-path", type=int, default=0,
                    help="dspark_set_draft_path value (0 = automatic)")
    ap.add_argument("--cpu-requests", type=int, default=0,
                    help="requests in the oracle sample (0 = sized for ~15 s)")
    return ap.parse_args()


def algorithmic_bytes(wl, ell, n_acc):
    """Bytes the step must move, each input read once: every base-logit row,
    the target rows up to each request's first reject (or its bonus slot), the
    base-logit row again at a reject (the q recompute), W2 once, the hidden
    states and gathered W1 rows, uniforms and outputs."""
    e = 2 if wl.dtype == "bf16" else 4
    B, g, V, r, H = wl.B, wl.gamma, wl.V, wl.rank, wl.H
    rejected = (n_acc < ell)
    j_rows = (n_acc + 1).sum()                      # target slots 0..j_b read
    u_rows = B * g + int(rejected.sum())            # every U row + re-read at rejects
    return (e * V * (u_rows + int(j_rows)) + e * r * V + e * B * g * (H + r)
            + 4 * B * (g + 1) * 2 + 4 * B * g * 4 + 4 * B * (g + 1))


def draft_kernel_bytes(wl, kernel, with_conf=False):
    """Algorithmic bytes of one launch of the draft kernel `kernel`: the
    draft's share of the step's bytes, each input read once.

    pdraft_pipe_kernel / pdraft_kernel (one launch per block of gamma
    positions): every U row, the W2 factor once, the gathered W1 rows (one per
    position and request), the anchors, temperatures and draw uniforms, and
    the four [B, gamma] outputs; with the confidence head evaluated in the
    same launch (with_conf), also the hidden states and the confidences (the
    head's W1 rows are the gathered ones).
    draft_stats_kernel (one launch per position): that position's U rows and
    W1 rows, and 1/gamma of W2 (the per-position launches read W2 again each
    time; the step needs it once).  The kernels' own tile statistics are
    intermediates, reported by draft_intermediate_bytes, not counted here.
    """
    e = 2 if wl.dtype == "bf16" else 4
    B, g, V, r = wl.B, wl.gamma, wl.V, wl.rank
    if kernel in ("pdraft_kernel", "pdraft_pipe_kernel"):
        conf = (e * B * g * wl.H + 4 * B * g) if with_conf else 0
        return (e * B * g * V + e * r * V + e * B * g * r
                + 4 * B + 4 * B + 4 * B * g + 4 * B * g * 4 + conf)
    return e * B * V + e * B * r + e * r * V / g


def draft_intermediate_bytes(wl, kernel):
    """Bytes of the draft kernel's own intermediates per launch: the packed
    per-(request, tile) statistics words (and greedy rows' argmax words)
    written each position and read back by the request's owner."""
    import numpy as np
    nT = (wl.V + 63) // 64
    B, g = wl.B, wl.gamma
    greedy = int(np.sum(~(np.asarray(wl.temperature) > 0)))
    per_pos = 2 * (8 * B * nT + 4 * greedy * nT)
    return g * per_pos if kernel in ("pdraft_kernel", "pdraft_pipe_kernel") else per_pos


KERNEL_SOURCES = ["draft_verify_sampling_block_amd/csrc/draft.hip",
                  "draft_verify_sampling_block_amd/csrc/draft_pipe.hip",
                  "draft_verify_sampling_block_amd/csrc/draft_tile.hpp",
                  "draft_verify_sampling_block_amd/csrc/conf_row.hpp",
                  "draft_verify_sampling_block_amd/csrc/dspark_common.hpp",
                  "draft_verify_sampling_block_amd/csrc/dspark_launch.hpp"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the recorded rocprofv3 counters
    (profiles/<kernel>-<workload>.counters.txt, the workload by name), scaled
    by the plain-copy calibration recorded with them; None when absent or
    when the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}-{workload}.counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#") and "=" in line:
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != kernel_source_hash():
        return None
    return (float(kv["fetch_kib_per_dispatch"]) * float(kv["fetch_scale"])
            + float(kv["write_kib_per_dispatch"]) * float(kv["write_scale"])) * 1024.0


def kernel_bytes(wl, ell, n_acc):
    """Algorithmic bytes per launch of the step's streaming kernels, from the
    realised outcomes (each kernel's share of the step's bytes, nothing
    counted twice): verify_rows_kernel the target rows of slots 0..j_b - 1,
    j_b = n_accepted + 1 (up to the first reject, or the bonus slot); the
    verify statistics the base-logit row of each sampled request that
    rejected (the q recompute); the confidence head the hidden states and the
    gathered W1 rows."""
    import numpy as np
    e = 2 if wl.dtype == "bf16" else 4
    B, g, V, r, H = wl.B, wl.gamma, wl.V, wl.rank, wl.H
    sampled = np.asarray(wl.temperature) > 0
    rejected = (n_acc < ell) & sampled
    stats = e * V * int(rejected.sum())
    return {"verify_rows_kernel": e * V * int((np.asarray(n_acc) + 1).sum()),
            "verify_tile_stats_kernel": stats, "verify_final_stats_kernel": stats,
            "confidence_kernel": e * B * g * (H + r) + 4 * B * g}


def kernel_bytes_read(wl, ell, n_acc):
    """Bytes the same kernels read as built (re-reads included):
    verify_rows_kernel reads every slot up to the verify length ell_b (the
    bonus slot included); the verify statistics read each sampled request's
    final slot row again, the base-logit rows at rejects and W2 again."""
    import numpy as np
    e = 2 if wl.dtype == "bf16" else 4
    V, r = wl.V, wl.rank
    sampled = np.asarray(wl.temperature) > 0
    rejected = (n_acc < ell) & sampled
    stats = e * V * (int(sampled.sum()) + int(rejected.sum())) + e * r * V
    return {"verify_rows_kernel": e * V * int((np.asarray(ell) + 1).sum()),
            "verify_tile_stats_kernel": stats, "verify_final_stats_kernel": stats}


def tv_label_bytes(wl):
    """Algorithmic bytes of one dspark_tv_label call: every drafted
    position's base-logit and target rows once, W2 once, the W1 rows of the
    previous tokens, the draft row statistics, temperatures and the labels."""
    e = 2 if wl.dtype == "bf16" else 4
    B, g, V, r = wl.B, wl.gamma, wl.V, wl.rank
    return e * V * 2 * B * g + e * r * V + e * B * g * r + 4 * B * g * 4 + 4 * B


def rnn_draft_bytes(wl):
    """Algorithmic bytes of one dspark_draft_block_rnn call: every U row, W2
    once, the hidden states, the RNN layer Wr once, the W1 rows of the
    previous tokens, the anchors, temperatures and draw uniforms, and the
    outputs (four [B, gamma] arrays, the projected vectors and the state)."""
    e = 2 if wl.dtype == "bf16" else 4
    B, g, V, r, H = wl.B, wl.gamma, wl.V, wl.rank, wl.H
    return (e * B * g * V + e * r * V + e * B * g * H + e * 3 * r * (2 * r + H) + 4 * 3 * r
            + e * B * g * r + 4 * B * 2 + 4 * B * g + 4 * B * g * 4 + e * B * g * r
            + 4 * B * g * r)


def next_rows(st, wl, reps):
    """Time the scheduler stop-rule variants, the acceptance-label kernels and
    the RNN-head draft on this step's confidences and drafts (events on the
    launch stream)."""
    import torch

    import draft_verify_sampling_block_amd as dv
    from draft_verify_sampling_block_amd.step import _dev
    from gen.workloads import rnn_weights

    d = st.d
    B, g = wl.B, wl.gamma
    dev = d.U.device
    ell = torch.empty((B,), dtype=torch.int32, device=dev)
    order = torch.empty((B * g,), dtype=torch.int32, device=dev)
    stats = torch.empty((3,), dtype=torch.float64, device=dev)
    cap = torch.tensor([float(B * g) / 2.0], dtype=torch.float64, device=dev)
    tv = torch.empty((B, g), dtype=torch.float32, device=dev)
    label = torch.empty((B, g), dtype=torch.float32, device=dev)
    dt = dv.DSPARK_BF16 if wl.dtype == "bf16" else dv.DSPARK_F32
    ws = torch.empty(max(256, dv.dspark_tv_label_workspace(B, g, wl.V, wl.rank, dt)),
                     dtype=torch.uint8, device=dev)
    rw = rnn_weights(wl.rank, wl.H, wl.dtype, seed=wl.spec.index)
    Wr, br = _dev(rw["Wr"], dev), _dev(rw["br"], dev)
    r_out = dict(tokens=torch.empty((B, g), dtype=torch.int32, device=dev),
                 q_tok=torch.empty((B, g), dtype=torch.float32, device=dev),
                 row_max=torch.empty((B, g), dtype=torch.float32, device=dev),
                 row_logZ=torch.empty((B, g), dtype=torch.float32, device=dev),
                 emb=torch.empty((B, g, wl.rank), dtype=d.U.dtype, device=dev))
    ws_rnn = torch.empty(max(256, dv.dspark_draft_block_rnn_workspace(B, g, wl.V, wl.rank, wl.H,
                                                                      dt)),
                         dtype=torch.uint8, device=dev)
    calls = {
        "draft_block_rnn": lambda: dv.dspark_draft_block_rnn(
            d.U, d.W1, d.W2, d.hidden, Wr, br, d.anchor, d.temperature, d.uniforms,
            workspace=ws_rnn, **r_out),
        "schedule_capacity": lambda: dv.dspark_schedule_capacity(st.conf, cap, ell=ell,
                                                                 order=order, stats=stats),
        "schedule_threshold": lambda: dv.dspark_schedule_threshold(st.conf, 0.5, ell=ell,
                                                                   order=order, stats=stats),
        "tv_label": lambda: dv.dspark_tv_label(d.target, d.U, d.W1, d.W2, d.anchor, st.tokens,
                                               st.row_max, st.row_logZ, d.temperature, tv=tv,
                                               label=label, workspace=ws),
    }
    out = {}
    stream = torch.cuda.current_stream()
    for name, fn in calls.items():
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        out[name] = {"us_per_call": us}
    nb = rnn_draft_bytes(wl)
    gbs = nb / (out["draft_block_rnn"]["us_per_call"] / 1e6) / 1e9
    out["draft_block_rnn"].update({"bytes_alg": nb, "hbm_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                                   "path": "per-position launches"})
    nb = tv_label_bytes(wl)
    gbs = nb / (out["tv_label"]["us_per_call"] / 1e6) / 1e9
    out["tv_label"].update({"bytes_alg": nb, "hbm_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                            "mean_label": float(label.mean().item())})
    return out


def read_ceiling_gbs(nbytes=4 << 30, reps=5):
    """Achievable streaming-read rate of this GPU: per-row sums (torch) over a
    4 GiB fp32 tensor viewed as 1024 rows of 1 Mi entries, best of `reps` timed
    runs.  (One reduction to a single value is slower: it measured ~4.0 TB/s
    against ~5.6 TB/s for the per-row form.)"""
    import torch

    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda").view(-1, 1 << 20)
    x.sum(dim=1)
    torch.cuda.synchronize()
    best = float("inf")
    stream = torch.cuda.current_stream()
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        x.sum(dim=1)
        e1.record(stream)
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / 1e3)
    del x
    torch.cuda.empty_cache()
    return nbytes / best / 1e9


def cpu_baseline(cfg, n_req):
    import numpy as np

    import oracle as O
    from gen import make_config

    wl = make_config(cfg, requests=range(n_req))
    # the oracle's loops are single-threaded Python; its vector products run
    # in the BLAS library, so the threads it uses are the BLAS threads
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count() or 1
    def one_pass():
        W1, W2 = O.f64(wl.W1), O.f64(wl.W2)
        d = O.draft_block(wl.U, W1, W2, wl.anchor, wl.temperature, wl.uniforms)
        c = O.confidence(wl.hidden, W1, wl.anchor, d["tokens"], wl.w, wl.b0)
        if wl.spec.scheduler and wl.sps is not None:
            ell = O.schedule(c, wl.sps)["ell"]
        else:
            ell = np.full(wl.B, wl.gamma)
        O.verify(wl.target, wl.U, W1, W2, wl.anchor, d["tokens"], d["q_tok"], wl.temperature,
                 wl.uniforms, ell)

    # whole passes over the sample until about 10 s of CPU work (at most 5)
    t0 = time.perf_counter()
    reps = 0
    while reps < 5 and (reps == 0 or time.perf_counter() - t0 < 10.0):
        one_pass()
        reps += 1
    dt = (time.perf_counter() - t0) / reps
    return {"value": n_req * wl.gamma / dt, "unit": "positions/s", "cores": int(cores),
            "cpu_count": os.cpu_count(), "affinity_cpus": affinity, "blas_threads": int(cores),
            "kind": "oracle",
            "sample": f"first {n_req} of {wl.spec.B} requests of {wl.spec.name} "
                      f"({n_req * wl.gamma} positions; scheduler over the sample), "
                      f"{reps} passes, {dt:.1f} s each"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the sampling path "
              "has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import draft_verify_sampling_block_amd as dv
    from draft_verify_sampling_block_amd.step import Step, upload
    from gen import SPECS, make_config

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_mb:
        n = args.copy_mb << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 5}), flush=True)
        return
    dv.load()
    dv.dspark_set_draft_path(args.draft_path)
    cfg = args.config
    spec = SPECS[cfg]
    t0 = time.perf_counter()
    wl = make_config(cfg)
    print(f"[bench] generated {spec.name} in {time.perf_counter() - t0:.1f}s", file=sys.stderr,
          flush=True)
    st = Step(upload(wl, "cuda"))
    st.run()   # the drafts and confidences the next rows' calls take
    torch.cuda.synchronize()
    # The GPU raises its clocks over the first tens of milliseconds of load,
    # so the bench's other measurements (the next rows' calls, the read
    # ceiling, the per-kernel events) run before the W warm-up and K timed
    # steps: the timed steps then run at the clocks a serving loop holds.
    next_out = next_rows(st, wl, max(3, args.steps // 2))
    ceil = read_ceiling_gbs()
    # per-kernel durations (a pass of K steps with events between launches)
    dv.dspark_trace_enable(True)
    for _ in range(args.steps):
        st.run()
    torch.cuda.synchronize()
    tr = dv.dspark_trace_summary()
    dv.dspark_trace_enable(False)
    print(f"[bench] next rows, read ceiling and per-kernel pass done", file=sys.stderr,
          flush=True)

    for _ in range(args.warmup):
        st.run()
    torch.cuda.synchronize()
    # one device status word per timed step (zeroed beforehand), so a flag
    # raised by any step is seen and traced to that step
    # (16 bytes apart: the library takes 16-byte-aligned pointers)
    step_status = torch.zeros((args.steps, 4), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        st.run(status=step_status[i, :1])
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    print(f"[bench] {args.steps} steps, {ms:.4f} ms/step", file=sys.stderr, flush=True)
    per_step_status = [int(x) for x in step_status[:, 0].cpu().tolist()]
    status = 0
    for x in per_step_status:
        status |= x
    ell = st.ell_used().cpu().numpy()
    n_acc = st.n_accepted.cpu().numpy()

    dom = max(tr, key=lambda k: tr[k][1])
    kern_ms = {k: v[1] / v[0] for k, v in tr.items()}
    per_step_ms = {k: v[1] / args.steps for k, v in tr.items()}
    draft_kernel = next((k for k in ("pdraft_pipe_kernel", "pdraft_kernel") if k in kern_ms),
                        "draft_stats_kernel")
    # the confidence head runs inside the draft launch unless its own kernel ran
    conf_fused = draft_kernel == "pdraft_pipe_kernel" and "confidence_kernel" not in kern_ms
    stats_bytes = draft_kernel_bytes(wl, draft_kernel, with_conf=conf_fused)
    avg_s = kern_ms[draft_kernel] / 1e3
    achieved = stats_bytes / avg_s / 1e9
    traffic = counter_traffic(draft_kernel, spec.name)
    kb_read = kernel_bytes_read(wl, ell, n_acc)
    bytes_step = algorithmic_bytes(wl, ell, n_acc)

    out = {
        "metric": METRIC,
        "value": wl.B * wl.gamma / (ms / 1e3),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; shapes and logit mixtures of the pages' workloads)",
        "config": {"workload": f"{spec.name}: B={wl.B} gamma={wl.gamma} V={wl.V} "
                               f"rank={wl.rank} H={wl.H} {wl.dtype}",
                   "B": wl.B, "gamma": wl.gamma, "V": wl.V, "rank": wl.rank, "H": wl.H,
                   "scheduler": bool(spec.scheduler), "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": draft_kernel, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "traffic_over_alg": None if traffic is None else traffic / stats_bytes,
                     "bytes_per_launch": stats_bytes,
                     "intermediate_bytes": draft_intermediate_bytes(wl, draft_kernel),
                     "confidence_in_launch": conf_fused,
                     "mean_launch_us": avg_s * 1e6},
        "step": {"bytes_alg": bytes_step, "hbm_gbs": bytes_step / (ms / 1e3) / 1e9,
                 "hbm_frac": bytes_step / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                 "mean_ell": float(ell.mean()), "mean_accepted": float(n_acc.mean()),
                 "dominant_kernel": dom,
                 "kernel_gbs": {k: {"bytes_alg": nb, "gbs": nb / (kern_ms[k] / 1e3) / 1e9,
                                    "frac": nb / (kern_ms[k] / 1e3) / 1e9 / HBM_PEAK_GBS,
                                    "bytes_read": kb_read.get(k)}
                                for k, nb in kernel_bytes(wl, ell, n_acc).items()
                                if k in kern_ms},
                 "kernel_ms_per_step": {k: round(v, 5) for k, v in per_step_ms.items()},
                 "device_status": status,
                 "steps_with_status": sum(1 for x in per_step_status if x)},
    }
    out["next_rows"] = next_out
    out["roofline"]["measured_read_ceiling_gbs"] = ceil
    out["roofline"]["frac_of_measured_ceiling"] = achieved / ceil
    out["step"]["hbm_frac_of_measured_ceiling"] = bytes_step / (ms / 1e3) / 1e9 / ceil
    if not args.no_cpu_baseline:
        n_req = args.cpu_requests or {0: 4, 1: 32, 2: 128, 3: 128, 4: 256}[cfg]
        out["cpu_baseline"] = cpu_baseline(cfg, n_req)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
