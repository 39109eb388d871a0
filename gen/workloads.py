"""Seeded synthetic workloads shaped like the pages' DSpark decode steps.

This module only draws random inputs.  It holds none of the method's
arithmetic (no Markov bias, softmax, sampling, survival, scheduling or
verification); both the GPU tests/bench and the CPU oracle consume its
arrays.  All draws use numpy's PCG64 with ``SeedSequence(seed,
spawn_key=(component, request))`` streams, so any subset of requests is
reproducible on its own and generation can run in threads.

Storage: bf16 tensors are returned as ``uint16`` bit patterns (round to
nearest even from float32, done once here); fp32 tensors as ``float32``.

Five workloads (index = default seed):

0  tiny:          B=4,   gamma=5,  V=1024,   r=32,  H=64,   fp32
1  qwen3-4b:      B=32,  gamma=7,  V=151936, r=256, H=2560, bf16, ell = gamma
2  dspark-5:      B=128, gamma=5,  V=129280, r=256, H=4096, bf16, T = 0.7
3  long-proposal: B=128, gamma=15, V=151936, r=256, H=2560, bf16
4  high-conc:     B=512, gamma=7,  V=151936, r=256, H=2560, bf16, 10% T = 0

Logit families:
* gaussian (0):  U ~ N(0, 2); target = U + N(0, 0.5)
* mixture (1,3,4): per row N(0, 1.5) background plus three distinct
  uniformly drawn ids each raised by U(8, 12); target = U + N(0, s_k)
* two-class (2): half the requests low entropy (N(0,1) plus one id at
  +15), half high entropy (N(0,1)); target = U + N(0, 0.5)

Confidence inputs: configs 0/1 draw hidden ~ N(0,1), w ~ N(0, 0.1).  For the
scheduled configs 2-4 the hidden state is projected so that the hidden part
of the confidence logit equals logit(alpha) for a designed conditional
acceptance alpha (falling with position in config 3); the W1 term then adds
a small perturbation.  This only shapes the inputs: alpha is not computed
from the logits.
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# component ids for the seed tree
_C_W1, _C_W2, _C_W, _C_LOGITS, _C_HIDDEN, _C_GLOBAL, _C_RNN = range(7)


@dataclasses.dataclass
class Spec:
    index: int
    name: str
    B: int
    gamma: int
    V: int
    rank: int
    H: int
    dtype: str          # "f32" or "bf16"
    family: str         # "gaussian" | "mixture" | "two-class"
    w_std: float        # std of W1 and W2
    scheduler: bool     # False => ell = gamma for every request
    temperature: float
    greedy_frac: float = 0.0
    sps_kind: str = "none"


SPECS = [
    Spec(0, "tiny", 4, 5, 1024, 32, 64, "f32", "gaussian", 0.05, True, 1.0, sps_kind="tiny"),
    Spec(1, "qwen3-4b-block7", 32, 7, 151936, 256, 2560, "bf16", "mixture", 0.02, False, 1.0),
    Spec(2, "dspark5-production", 128, 5, 129280, 256, 4096, "bf16", "two-class", 0.02, True, 0.7,
         sps_kind="linear1024"),
    Spec(3, "long-proposal-g15", 128, 15, 151936, 256, 2560, "bf16", "mixture", 0.02, True, 1.0,
         sps_kind="linear1024"),
    Spec(4, "high-concurrency", 512, 7, 151936, 256, 2560, "bf16", "mixture", 0.02, True, 1.0,
         greedy_frac=0.1, sps_kind="linear2048"),
]


@dataclasses.dataclass
class Workload:
    spec: Spec
    B: int
    gamma: int
    V: int
    rank: int
    H: int
    dtype: str
    U: np.ndarray          # [B, gamma, V]     uint16 (bf16 bits) or float32
    target: np.ndarray     # [B, gamma+1, V]   slot gamma = bonus slot
    W1: np.ndarray         # [V, rank]
    W2: np.ndarray         # [rank, V]         projection rank -> V
    w: np.ndarray          # [H + rank] float32 confidence weight ([w_h ; w_e])
    b0: float              # confidence bias
    hidden: np.ndarray     # [B, gamma, H]
    anchor: np.ndarray     # [B] int32
    temperature: np.ndarray  # [B] float32
    uniforms: np.ndarray   # [B, gamma+1, 2] float32 in [0, 1)
    sps: np.ndarray | None  # float64 table indexed by target batch Bt (None: no scheduler)
    requests: np.ndarray   # global request ids held here (subset generation)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); return bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 value of bf16 bit patterns (storage format helper)."""
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def sps_table(kind: str) -> np.ndarray | None:
    """Steps-per-second profile SPS[Bt]; entry 0 is unused (set to 0)."""
    if kind == "none":
        return None
    if kind == "tiny":
        bt = np.arange(65, dtype=np.float64)
        t = 1000.0 / (1.0 + bt / 64.0)
    elif kind == "linear1024":
        bt = np.arange(1025, dtype=np.float64)
        t = 2400.0 * (1.0 - 0.55 * bt / 1024.0)
    elif kind == "linear2048":
        bt = np.arange(2049, dtype=np.float64)
        t = 2400.0 * (1.0 - 0.55 * bt / 2048.0)
    else:
        raise ValueError(kind)
    t[0] = 0.0
    return t


def _alpha(spec: Spec, b: int, low_class: np.ndarray) -> np.ndarray:
    """Designed conditional acceptance per position for calibrated configs."""
    g = spec.gamma
    if spec.index == 2:
        return np.full(g, 0.97 if low_class[b] else 0.70)
    if spec.index == 3:
        return 0.84 - (0.84 - 0.57) * np.arange(g) / max(g - 1, 1)
    return np.full(g, 0.74)


def _global_draws(spec: Spec, seed: int):
    r = _rng(seed, _C_GLOBAL)
    anchor = r.integers(0, spec.V, spec.B).astype(np.int32)
    uniforms = r.random((spec.B, spec.gamma + 1, 2), dtype=np.float32)
    low_class = np.zeros(spec.B, dtype=bool)
    if spec.family == "two-class":
        low_class[r.permutation(spec.B)[: spec.B // 2]] = True
    temperature = np.full(spec.B, spec.temperature, dtype=np.float32)
    if spec.greedy_frac > 0:
        n = int(np.floor(spec.greedy_frac * spec.B))
        temperature[r.choice(spec.B, n, replace=False)] = 0.0
    return anchor, uniforms, low_class, temperature


def _noise_std(spec: Spec) -> np.ndarray:
    g1 = spec.gamma + 1
    if spec.index == 0:
        return np.full(g1, 0.5)
    if spec.index == 2:
        return np.full(g1, 0.5)
    if spec.index == 3:
        return 0.4 + 0.05 * np.arange(1, g1 + 1)
    return np.full(g1, 0.7)


def _request_logits(spec: Spec, seed: int, b: int, low: bool):
    r = _rng(seed, _C_LOGITS, b)
    g1, V = spec.gamma + 1, spec.V
    if spec.family == "gaussian":
        base = r.standard_normal((g1, V), dtype=np.float32) * np.float32(2.0)
    elif spec.family == "mixture":
        base = r.standard_normal((g1, V), dtype=np.float32) * np.float32(1.5)
        for k in range(g1):
            ids = r.choice(V, 3, replace=False)
            base[k, ids] += r.uniform(8.0, 12.0, 3).astype(np.float32)
    else:  # two-class
        base = r.standard_normal((g1, V), dtype=np.float32)
        if low:
            for k in range(g1):
                base[k, r.integers(0, V)] += np.float32(15.0)
    std = _noise_std(spec).astype(np.float32)[:, None]
    noise = r.standard_normal((g1, V), dtype=np.float32) * std
    target = base + noise
    return base, target


def _request_hidden(spec: Spec, seed: int, b: int, w_h: np.ndarray, alpha):
    r = _rng(seed, _C_HIDDEN, b)
    h = r.standard_normal((spec.gamma, spec.H)).astype(np.float64)
    if alpha is not None:
        jitter = r.normal(0.0, 0.25, spec.gamma)
        L = np.log(alpha / (1.0 - alpha)) + jitter
        wn2 = float(w_h @ w_h)
        h = h - np.outer((h @ w_h - L) / wn2, w_h)
    return h.astype(np.float32)


def make_config(index: int, seed: int | None = None, requests=None, threads: int | None = None,
                with_target: bool = True) -> Workload:
    """Build workload ``index`` (0..4).

    ``requests``: optional iterable of request ids (subset of range(B)); the
    rows of those requests are identical to the full workload's rows.
    """
    spec = SPECS[index]
    seed = index if seed is None else seed
    req = np.arange(spec.B) if requests is None else np.asarray(list(requests), dtype=np.int64)
    anchor, uniforms, low_class, temperature = _global_draws(spec, seed)

    W1 = _rng(seed, _C_W1).standard_normal((spec.V, spec.rank), dtype=np.float32) * np.float32(spec.w_std)
    # drawn [V, rank] and stored transposed, [rank, V]
    W2 = np.ascontiguousarray((_rng(seed, _C_W2).standard_normal((spec.V, spec.rank), dtype=np.float32)
                               * np.float32(spec.w_std)).T)
    w = (_rng(seed, _C_W).standard_normal(spec.H + spec.rank) * 0.1).astype(np.float32)
    w_h = w[: spec.H].astype(np.float64)

    nb = len(req)
    g, g1, V = spec.gamma, spec.gamma + 1, spec.V
    bf = spec.dtype == "bf16"
    sdt = np.uint16 if bf else np.float32
    U = np.empty((nb, g, V), dtype=sdt)
    target = np.empty((nb, g1, V), dtype=sdt) if with_target else None
    hidden = np.empty((nb, g, spec.H), dtype=sdt)

    def one(i):
        b = int(req[i])
        base, tgt = _request_logits(spec, seed, b, bool(low_class[b]))
        if bf:
            U[i] = to_bf16_bits(base[:g])
            if with_target:
                target[i] = to_bf16_bits(tgt)
        else:
            U[i] = base[:g]
            if with_target:
                target[i] = tgt
        alpha = _alpha(spec, b, low_class) if spec.scheduler and spec.index != 0 else None
        h = _request_hidden(spec, seed, b, w_h, alpha)
        hidden[i] = to_bf16_bits(h) if bf else h

    nthreads = threads or min(16, os.cpu_count() or 1)
    if nb > 1 and nthreads > 1:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(one, range(nb)))
    else:
        for i in range(nb):
            one(i)

    if bf:
        W1s, W2s = to_bf16_bits(W1), to_bf16_bits(W2)
    else:
        W1s, W2s = W1, W2
    return Workload(
        spec=spec, B=nb, gamma=g, V=V, rank=spec.rank, H=spec.H, dtype=spec.dtype,
        U=U, target=target, W1=W1s, W2=W2s, w=w, b0=0.0, hidden=hidden,
        anchor=anchor[req].copy(), temperature=temperature[req].copy(),
        uniforms=uniforms[req].copy(), sps=sps_table(spec.sps_kind), requests=req,
    )


def make_custom(B: int, gamma: int, V: int, rank: int, H: int, dtype: str = "bf16",
                family: str = "mixture", seed: int = 0, temperature: float = 1.0,
                greedy_frac: float = 0.0, sps_kind: str = "none", w_std: float = 0.02,
                calibrated: bool = False, threads: int | None = None) -> Workload:
    """A workload of arbitrary (small) shape drawn with the same recipes.

    Used for parity tests that must span several tiles, a ragged vocabulary
    tail and ragged request blocks while staying cheap for the oracle.
    ``sps_kind`` may also be "linear:<Btmax>" for 2400*(1-0.55*Bt/Btmax).
    """
    spec = Spec(100, "custom", B, gamma, V, rank, H, dtype, family, w_std,
                sps_kind != "none", temperature, greedy_frac=greedy_frac, sps_kind=sps_kind)
    anchor, uniforms, low_class, temp = _global_draws(spec, seed)
    W1 = _rng(seed, _C_W1).standard_normal((V, rank), dtype=np.float32) * np.float32(w_std)
    W2 = np.ascontiguousarray((_rng(seed, _C_W2).standard_normal((V, rank), dtype=np.float32)
                               * np.float32(w_std)).T)
    w = (_rng(seed, _C_W).standard_normal(H + rank) * 0.1).astype(np.float32)
    w_h = w[:H].astype(np.float64)
    bf = dtype == "bf16"
    sdt = np.uint16 if bf else np.float32
    U = np.empty((B, gamma, V), dtype=sdt)
    target = np.empty((B, gamma + 1, V), dtype=sdt)
    hidden = np.empty((B, gamma, H), dtype=sdt)
    for b in range(B):
        base, tgt = _request_logits(spec, seed, b, bool(low_class[b]))
        U[b] = to_bf16_bits(base[:gamma]) if bf else base[:gamma]
        target[b] = to_bf16_bits(tgt) if bf else tgt
        alpha = np.full(gamma, 0.8) if calibrated else None
        h = _request_hidden(spec, seed, b, w_h, alpha)
        hidden[b] = to_bf16_bits(h) if bf else h
    if sps_kind.startswith("linear:"):
        bmax = int(sps_kind.split(":")[1])
        bt = np.arange(bmax + 1, dtype=np.float64)
        sps = 2400.0 * (1.0 - 0.55 * bt / bmax)
        sps[0] = 0.0
    else:
        sps = sps_table(sps_kind)
    return Workload(spec=spec, B=B, gamma=gamma, V=V, rank=rank, H=H, dtype=dtype,
                    U=U, target=target, W1=to_bf16_bits(W1) if bf else W1,
                    W2=to_bf16_bits(W2) if bf else W2, w=w, b0=0.0, hidden=hidden,
                    anchor=anchor, temperature=temp, uniforms=uniforms, sps=sps,
                    requests=np.arange(B))


def rnn_weights(rank: int, H: int, dtype: str = "bf16", seed: int = 0, w_std: float = 0.02):
    """Weights of the RNN head (its own seed stream; no other draw changes).

    Wr [3 rank, 2 rank + H] (rows gate | candidate | output; columns state |
    embedding | hidden) with each column block scaled so that it adds O(1) to
    the pre-activations: state N(0, 1/rank), embedding N(0, 1/(rank w_std^2))
    (the W1 rows it multiplies have std w_std), hidden N(0, 1/H); br [3 rank]
    ~ N(0, 0.1^2), float32.  Returns dict(Wr (bf16 bits or float32), br).
    """
    r = _rng(seed, _C_RNN)
    Wr = np.empty((3 * rank, 2 * rank + H), dtype=np.float32)
    Wr[:, :rank] = r.standard_normal((3 * rank, rank), dtype=np.float32) / np.float32(np.sqrt(rank))
    Wr[:, rank:2 * rank] = (r.standard_normal((3 * rank, rank), dtype=np.float32)
                            / np.float32(np.sqrt(rank) * w_std))
    Wr[:, 2 * rank:] = r.standard_normal((3 * rank, H), dtype=np.float32) / np.float32(np.sqrt(H))
    br = (r.standard_normal(3 * rank) * 0.1).astype(np.float32)
    return dict(Wr=to_bf16_bits(Wr) if dtype == "bf16" else Wr, br=br)
