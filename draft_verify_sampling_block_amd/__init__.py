"""Python binding of libdspark (gfx950 HIP kernels behind a C ABI).

Argument marshalling only: every step of the sampling path runs in the
library's kernels.  torch supplies device memory and the current stream.
The functions carry the C entry points' names:

    dspark_draft_block, dspark_confidence, dspark_schedule, dspark_verify,
    dspark_schedule_capacity, dspark_schedule_threshold, dspark_tv_label

If ``libdspark.so`` is missing the import still succeeds (so the CPU test
suite can run), but every entry point raises ``DsparkError``; nothing falls
back to another implementation.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

__all__ = [
    "DsparkError", "lib_path", "load", "dspark_draft_block", "dspark_confidence",
    "dspark_schedule", "dspark_schedule_noalloc", "dspark_schedule_capacity", "dspark_schedule_threshold", "dspark_verify",
    "dspark_tv_label", "dspark_tv_label_workspace", "dspark_draft_block_workspace",
    "dspark_draft_block_rnn", "dspark_draft_block_rnn_workspace", "dspark_verify_rnn",
    "dspark_confidence_sts", "dspark_draft_block_conf",
    "dspark_verify_workspace", "dspark_schedule_workspace", "exported_names", "header_names",
    "dspark_trace_enable", "dspark_trace_summary", "dspark_set_draft_path",
    "DSPARK_F32", "DSPARK_BF16", "DEV_FLAGS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_HEADER = os.path.join(os.path.dirname(_PKG), "include", "dspark.h")
DSPARK_F32, DSPARK_BF16 = 0, 1
DEV_FLAGS = {1: "BAD_TOKEN", 2: "NONFINITE", 4: "DEGENERATE", 8: "BAD_ELL", 16: "BAD_CONF",
             32: "TIMEOUT"}


class DsparkError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def lib_path() -> str:
    return os.path.join(_PKG, "libdspark.so")


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_SIGS = {
    "dspark_status_str": (ctypes.c_char_p, [_I]),
    "dspark_last_error": (ctypes.c_char_p, []),
    "dspark_version": (ctypes.c_char_p, []),
    "dspark_draft_block_workspace": (_SZ, [_I, _I, _I, _I, _I]),
    "dspark_draft_block": (_I, [_I, _I, _I, _I, _I] + [_P] * 11 + [_P, _SZ, _P]),
    "dspark_draft_block_conf": (_I, [_I] * 6 + [_P] * 8 + [ctypes.c_float] + [_P] * 6
                                + [_P, _P, _SZ, _P]),
    "dspark_confidence": (_I, [_I] * 6 + [_P] * 5 + [ctypes.c_float, _P, _P, _P]),
    "dspark_confidence_sts": (_I, [_I] * 6 + [_P] * 5 + [ctypes.c_float, _P, _P, _P, _P]),
    "dspark_schedule_workspace": (_SZ, [_I, _I]),
    "dspark_schedule": (_I, [_I, _I, _P, _P, _I, _P, _P, _P, _P, _P, _SZ, _P]),
    "dspark_schedule_noalloc": (_I, [_I, _I, _P, _P, _I, _P, _P, _P, _P, _P]),
    "dspark_schedule_capacity": (_I, [_I, _I, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "dspark_schedule_threshold": (_I, [_I, _I, _P, ctypes.c_double, _P, _P, _P, _P, _P, _SZ,
                                       _P]),
    "dspark_verify_workspace": (_SZ, [_I, _I, _I, _I, _I]),
    "dspark_tv_label_workspace": (_SZ, [_I, _I, _I, _I, _I]),
    "dspark_tv_label": (_I, [_I] * 5 + [_P] * 12 + [_P, _SZ, _P]),
    "dspark_verify": (_I, [_I] * 5 + [_P] * 15 + [_P, _P, _SZ, _P]),
    "dspark_draft_block_rnn_workspace": (_SZ, [_I] * 6),
    "dspark_draft_block_rnn": (_I, [_I] * 6 + [_P] * 16 + [_P, _SZ, _P]),
    "dspark_verify_rnn": (_I, [_I] * 5 + [_P] * 15 + [_P, _P, _SZ, _P]),
    "dspark_trace_enable": (_I, [_I]),
    "dspark_trace_summary": (_I, [ctypes.c_char_p, _SZ]),
    "dspark_set_draft_path": (_I, [_I]),
}


def load():
    """Load libdspark.so (once).  Raises DsparkError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise DsparkError(-100, f"{path} is not built; run __graft_entry__.build() or "
                                "python -m draft_verify_sampling_block_amd.build")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def header_names() -> list[str]:
    """Function names declared in include/dspark.h."""
    text = open(_HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(dspark_[a-z_]+)\s*\(",
                                 text, flags=re.M)))


def exported_names() -> list[str]:
    lib = load()
    return [n for n in header_names() if hasattr(lib, n)]


def _check(rc: int):
    if rc != 0:
        lib = load()
        raise DsparkError(rc, f"{lib.dspark_status_str(rc).decode()}: {lib.dspark_last_error().decode()}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DSPARK_BF16
    if t.dtype == torch.float32:
        return DSPARK_F32
    raise DsparkError(-2, f"unsupported tensor dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise DsparkError(-1, f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise DsparkError(-1, f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise DsparkError(-1, f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise DsparkError(-1, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise DsparkError(-2, f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise DsparkError(-1, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _out(t, name: str, dtype, shape, device):
    """A caller-supplied output checked like an input, or a new one."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    return _need(t, name, dtype, shape, device)


def _status(t, device):
    """The optional device status word: None or one int32 on `device`."""
    if t is None:
        return None
    _need(t, "status", torch.int32, None, device)
    if t.numel() != 1:
        raise DsparkError(-1, f"status must hold one int32, got {t.numel()}")
    return t


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def dspark_set_draft_path(path: int) -> int:
    """0 automatic, 1 multi-launch, 2 persistent only; returns the old value."""
    rc = load().dspark_set_draft_path(int(path))
    if rc < 0:
        _check(rc)
    return rc


def dspark_trace_enable(on: bool) -> None:
    _check(load().dspark_trace_enable(1 if on else 0))


def dspark_trace_summary() -> dict:
    """{kernel: (launches, total_ms)} of the launches recorded since enabling."""
    lib = load()
    n = lib.dspark_trace_summary(None, 0)
    if n < 0:
        _check(n)
    buf = ctypes.create_string_buffer(n + 1)
    lib.dspark_trace_summary(buf, n + 1)
    out = {}
    for line in buf.value.decode().splitlines():
        name, cnt, ms = line.split()
        out[name] = (int(cnt), float(ms))
    return out


def dspark_draft_block_workspace(B, gamma, V, rank, dtype) -> int:
    return int(load().dspark_draft_block_workspace(B, gamma, V, rank, dtype))


def dspark_verify_workspace(B, gamma, V, rank, dtype) -> int:
    return int(load().dspark_verify_workspace(B, gamma, V, rank, dtype))


def dspark_schedule_workspace(R, gamma) -> int:
    return int(load().dspark_schedule_workspace(R, gamma))


def _workspace(nbytes: int, device, given=None, zeroed=False):
    """The caller's workspace, checked, or a new one (zero-filled when the call
    needs to find it so: the draft workspace)."""
    if given is not None:
        _need(given, "workspace", torch.uint8, None, device)
        if given.dim() != 1 or given.numel() < nbytes:
            raise DsparkError(-4, f"workspace must be a 1-D uint8 tensor of at least {nbytes} "
                                  f"bytes, got shape {tuple(given.shape)}")
        return given
    alloc = torch.zeros if zeroed else torch.empty
    return alloc(max(nbytes, 256), dtype=torch.uint8, device=device)


def dspark_draft_block(U, W1, W2, anchor, temperature, uniforms, *, tokens=None, q_tok=None,
                       row_max=None, row_logZ=None, status=None, workspace=None):
    """Markov-head block drafting.  U [B,gamma,V]; W1 [V,rank], W2 [rank,V]; returns
    dict(tokens, q_tok, row_max, row_logZ)."""
    lib = load()
    B, gamma, V = U.shape
    rank = W1.shape[1]
    dt = _dtype_code(U)
    dev = U.device
    _need(U, "U"); _need(W1, "W1", U.dtype, (V, rank), dev); _need(W2, "W2", U.dtype, (rank, V), dev)
    _need(anchor, "anchor", torch.int32, (B,), dev)
    _need(temperature, "temperature", torch.float32, (B,), dev)
    _need(uniforms, "uniforms", torch.float32, (B, gamma + 1, 2), dev)
    tokens = _out(tokens, "tokens", torch.int32, (B, gamma), dev)
    q_tok = _out(q_tok, "q_tok", torch.float32, (B, gamma), dev)
    row_max = _out(row_max, "row_max", torch.float32, (B, gamma), dev)
    row_logZ = _out(row_logZ, "row_logZ", torch.float32, (B, gamma), dev)
    status = _status(status, dev)
    need = dspark_draft_block_workspace(B, gamma, V, rank, dt)
    ws = _workspace(need, dev, workspace, zeroed=True)
    _check(lib.dspark_draft_block(B, gamma, V, rank, dt, _ptr(U), _ptr(W1), _ptr(W2), _ptr(anchor),
                                  _ptr(temperature), _ptr(uniforms), _ptr(tokens), _ptr(q_tok),
                                  _ptr(row_max), _ptr(row_logZ), _ptr(status), _ptr(ws),
                                  ws.numel(), _stream()))
    return dict(tokens=tokens, q_tok=q_tok, row_max=row_max, row_logZ=row_logZ)


def dspark_draft_block_conf(U, W1, W2, anchor, temperature, uniforms, hidden, w, bias=0.0,
                            temps=None, *, tokens=None, q_tok=None, row_max=None,
                            row_logZ=None, conf=None, status=None, workspace=None):
    """Markov-head block drafting and the confidence head of the drafted block
    in one call.  As dspark_draft_block, plus hidden [B,gamma,H] (dtype of U),
    w [H+rank] fp32, bias, temps [gamma] fp32 or None; returns dict(tokens,
    q_tok, row_max, row_logZ, conf)."""
    lib = load()
    B, gamma, V = U.shape
    rank = W1.shape[1]
    H = hidden.shape[2]
    dt = _dtype_code(U)
    dev = U.device
    _need(U, "U"); _need(W1, "W1", U.dtype, (V, rank), dev); _need(W2, "W2", U.dtype, (rank, V), dev)
    _need(anchor, "anchor", torch.int32, (B,), dev)
    _need(temperature, "temperature", torch.float32, (B,), dev)
    _need(uniforms, "uniforms", torch.float32, (B, gamma + 1, 2), dev)
    _need(hidden, "hidden", U.dtype, (B, gamma, H), dev)
    _need(w, "w", torch.float32, (H + rank,), dev)
    if temps is not None:
        _need(temps, "temps", torch.float32, (gamma,), dev)
    tokens = _out(tokens, "tokens", torch.int32, (B, gamma), dev)
    q_tok = _out(q_tok, "q_tok", torch.float32, (B, gamma), dev)
    row_max = _out(row_max, "row_max", torch.float32, (B, gamma), dev)
    row_logZ = _out(row_logZ, "row_logZ", torch.float32, (B, gamma), dev)
    conf = _out(conf, "conf", torch.float32, (B, gamma), dev)
    status = _status(status, dev)
    need = dspark_draft_block_workspace(B, gamma, V, rank, dt)
    ws = _workspace(need, dev, workspace, zeroed=True)
    _check(lib.dspark_draft_block_conf(B, gamma, V, rank, H, dt, _ptr(U), _ptr(W1), _ptr(W2),
                                       _ptr(anchor), _ptr(temperature), _ptr(uniforms),
                                       _ptr(hidden), _ptr(w), ctypes.c_float(bias), _ptr(temps),
                                       _ptr(tokens), _ptr(q_tok), _ptr(row_max), _ptr(row_logZ),
                                       _ptr(conf), _ptr(status), _ptr(ws), ws.numel(),
                                       _stream()))
    return dict(tokens=tokens, q_tok=q_tok, row_max=row_max, row_logZ=row_logZ, conf=conf)


def dspark_draft_block_rnn_workspace(B, gamma, V, rank, H, dtype) -> int:
    return int(load().dspark_draft_block_rnn_workspace(B, gamma, V, rank, H, dtype))


def dspark_draft_block_rnn(U, W1, W2, hidden, Wr, br, anchor, temperature, uniforms, *,
                           tokens=None, q_tok=None, row_max=None, row_logZ=None, emb=None,
                           state=None, want_state=False, status=None, workspace=None):
    """Block drafting with the RNN head.  U [B,gamma,V]; W1 [V,rank]; W2 [rank,V];
    hidden [B,gamma,H]; Wr [3 rank, 2 rank + H] (dtype of U); br [3 rank] fp32.
    Returns dict(tokens, q_tok, row_max, row_logZ, emb [B,gamma,rank], state)."""
    lib = load()
    B, gamma, V = U.shape
    rank = W1.shape[1]
    H = hidden.shape[2]
    dt = _dtype_code(U)
    dev = U.device
    _need(U, "U"); _need(W1, "W1", U.dtype, (V, rank), dev); _need(W2, "W2", U.dtype, (rank, V), dev)
    _need(hidden, "hidden", U.dtype, (B, gamma, H), dev)
    _need(Wr, "Wr", U.dtype, (3 * rank, 2 * rank + H), dev)
    _need(br, "br", torch.float32, (3 * rank,), dev)
    _need(anchor, "anchor", torch.int32, (B,), dev)
    _need(temperature, "temperature", torch.float32, (B,), dev)
    _need(uniforms, "uniforms", torch.float32, (B, gamma + 1, 2), dev)
    tokens = _out(tokens, "tokens", torch.int32, (B, gamma), dev)
    q_tok = _out(q_tok, "q_tok", torch.float32, (B, gamma), dev)
    row_max = _out(row_max, "row_max", torch.float32, (B, gamma), dev)
    row_logZ = _out(row_logZ, "row_logZ", torch.float32, (B, gamma), dev)
    emb = _out(emb, "emb", U.dtype, (B, gamma, rank), dev)
    if state is not None or want_state:
        state = _out(state, "state", torch.float32, (B, gamma, rank), dev)
    status = _status(status, dev)
    need = dspark_draft_block_rnn_workspace(B, gamma, V, rank, H, dt)
    ws = _workspace(need, dev, workspace)
    _check(lib.dspark_draft_block_rnn(B, gamma, V, rank, H, dt, _ptr(U), _ptr(W1), _ptr(W2),
                                      _ptr(hidden), _ptr(Wr), _ptr(br), _ptr(anchor),
                                      _ptr(temperature), _ptr(uniforms), _ptr(tokens),
                                      _ptr(q_tok), _ptr(row_max), _ptr(row_logZ), _ptr(emb),
                                      _ptr(state), _ptr(status), _ptr(ws), ws.numel(),
                                      _stream()))
    return dict(tokens=tokens, q_tok=q_tok, row_max=row_max, row_logZ=row_logZ, emb=emb,
                state=state)


def dspark_confidence(hidden, W1, anchor, tokens, w, bias=0.0, *, conf=None, status=None):
    """Confidence head; hidden [B,gamma,H]; w [H+rank] fp32; returns conf [B,gamma]."""
    lib = load()
    B, gamma, H = hidden.shape
    V, rank = W1.shape
    dt = _dtype_code(hidden)
    dev = hidden.device
    _need(hidden, "hidden"); _need(W1, "W1", hidden.dtype, None, dev)
    _need(anchor, "anchor", torch.int32, (B,), dev)
    _need(tokens, "tokens", torch.int32, (B, gamma), dev)
    _need(w, "w", torch.float32, (H + rank,), dev)
    conf = _out(conf, "conf", torch.float32, (B, gamma), dev)
    status = _status(status, dev)
    _check(lib.dspark_confidence(B, gamma, H, V, rank, dt, _ptr(hidden), _ptr(W1), _ptr(anchor),
                                 _ptr(tokens), _ptr(w), ctypes.c_float(bias), _ptr(conf),
                                 _ptr(status), _stream()))
    return conf


def dspark_confidence_sts(hidden, W1, anchor, tokens, w, bias, temps, *, conf=None,
                          status=None):
    """Confidence head with sequential temperature scaling: sigmoid(logit_k / temps[k]);
    temps [gamma] fp32 device tensor.  Returns conf [B,gamma]."""
    lib = load()
    B, gamma, H = hidden.shape
    V, rank = W1.shape
    dt = _dtype_code(hidden)
    dev = hidden.device
    _need(hidden, "hidden"); _need(W1, "W1", hidden.dtype, None, dev)
    _need(anchor, "anchor", torch.int32, (B,), dev)
    _need(tokens, "tokens", torch.int32, (B, gamma), dev)
    _need(w, "w", torch.float32, (H + rank,), dev)
    _need(temps, "temps", torch.float32, (gamma,), dev)
    conf = _out(conf, "conf", torch.float32, (B, gamma), dev)
    status = _status(status, dev)
    _check(lib.dspark_confidence_sts(B, gamma, H, V, rank, dt, _ptr(hidden), _ptr(W1),
                                     _ptr(anchor), _ptr(tokens), _ptr(w), ctypes.c_float(bias),
                                     _ptr(temps), _ptr(conf), _ptr(status), _stream()))
    return conf


def dspark_schedule(conf, sps, *, ell=None, order=None, stats=None, status=None, want_order=True,
                    workspace=None):
    """Prefix scheduler; conf [R,gamma] fp32, sps fp64 table; returns (ell, order, stats)."""
    lib = load()
    R, gamma = conf.shape
    dev = conf.device
    _need(sps, "sps", torch.float64, None, conf.device)
    R, gamma, ell, order, stats, ws = _schedule_outputs(conf, ell, order, stats, want_order,
                                                        workspace)
    status = _status(status, dev)
    _check(lib.dspark_schedule(R, gamma, _ptr(conf), _ptr(sps), int(sps.numel()), _ptr(ell),
                               _ptr(order), _ptr(stats), _ptr(status), _ptr(ws),
                               0 if ws is None else ws.numel(), _stream()))
    return ell, order, stats


def dspark_schedule_noalloc(conf, sps, *, ell=None, order=None, stats=None, status=None,
                            want_order=True):
    """dspark_schedule without a workspace (the library's own per-device
    scratch holds the ranks); calls overlapping on one device race.
    Returns (ell, order, stats)."""
    lib = load()
    R, gamma = conf.shape
    dev = conf.device
    _need(sps, "sps", torch.float64, None, dev)
    _need(conf, "conf", torch.float32)
    ell = _out(ell, "ell", torch.int32, (R,), dev)
    if order is not None or want_order:
        order = _out(order, "order", torch.int32, (R * gamma,), dev)
    stats = _out(stats, "stats", torch.float64, (3,), dev)
    status = _status(status, dev)
    _check(lib.dspark_schedule_noalloc(R, gamma, _ptr(conf), _ptr(sps), int(sps.numel()),
                                       _ptr(ell), _ptr(order), _ptr(stats), _ptr(status),
                                       _stream()))
    return ell, order, stats


def _schedule_outputs(conf, ell, order, stats, want_order, workspace=None):
    R, gamma = conf.shape
    dev = conf.device
    _need(conf, "conf", torch.float32)
    ell = _out(ell, "ell", torch.int32, (R,), dev)
    if order is not None or want_order:
        order = _out(order, "order", torch.int32, (R * gamma,), dev)
    stats = _out(stats, "stats", torch.float64, (3,), dev)
    need = dspark_schedule_workspace(R, gamma)
    ws = _workspace(need, dev, workspace) if need else None
    return R, gamma, ell, order, stats, ws


def dspark_schedule_capacity(conf, capacity, *, ell=None, order=None, stats=None, status=None,
                             want_order=True, workspace=None):
    """Top-K scheduler (two-step barrier); capacity: fp64 device tensor whose first
    element is K (e.g. stats of an earlier dspark_schedule).  Returns (ell, order, stats)."""
    lib = load()
    R, gamma, ell, order, stats, ws = _schedule_outputs(conf, ell, order, stats, want_order,
                                                        workspace)
    status = _status(status, conf.device)
    if not (isinstance(capacity, torch.Tensor) and capacity.dtype == torch.float64
            and capacity.device == conf.device and capacity.numel() >= 1):
        raise DsparkError(-1, "capacity must be a float64 tensor on the device of conf")
    _check(lib.dspark_schedule_capacity(R, gamma, _ptr(conf), _ptr(capacity), _ptr(ell),
                                        _ptr(order), _ptr(stats), _ptr(status), _ptr(ws),
                                        0 if ws is None else ws.numel(), _stream()))
    return ell, order, stats


def dspark_schedule_threshold(conf, threshold, *, ell=None, order=None, stats=None, status=None,
                              want_order=True, workspace=None):
    """Fixed survival threshold scheduler.  Returns (ell, order, stats)."""
    lib = load()
    R, gamma, ell, order, stats, ws = _schedule_outputs(conf, ell, order, stats, want_order,
                                                        workspace)
    status = _status(status, conf.device)
    _check(lib.dspark_schedule_threshold(R, gamma, _ptr(conf), ctypes.c_double(threshold),
                                         _ptr(ell), _ptr(order), _ptr(stats), _ptr(status),
                                         _ptr(ws), 0 if ws is None else ws.numel(), _stream()))
    return ell, order, stats


def dspark_verify(target, U, W1, W2, anchor, tokens, q_tok, row_max, row_logZ, temperature,
                  uniforms, ell, *, out_tokens=None, n_accepted=None, ratio=None, status=None,
                  workspace=None, want_ratio=True):
    """Lossless verification; returns (out_tokens [B,gamma+1], n_accepted [B], ratio [B,gamma])."""
    lib = load()
    B, gamma, V = U.shape
    rank = W1.shape[1]
    dt = _dtype_code(U)
    dev = U.device
    _need(U, "U"); _need(target, "target", U.dtype, (B, gamma + 1, V), dev)
    _need(W1, "W1", U.dtype, (V, rank), dev); _need(W2, "W2", U.dtype, (rank, V), dev)
    for name, t, dtp, shp in (
            ("anchor", anchor, torch.int32, (B,)), ("tokens", tokens, torch.int32, (B, gamma)),
            ("q_tok", q_tok, torch.float32, (B, gamma)),
            ("row_max", row_max, torch.float32, (B, gamma)),
            ("row_logZ", row_logZ, torch.float32, (B, gamma)),
            ("temperature", temperature, torch.float32, (B,)),
            ("uniforms", uniforms, torch.float32, (B, gamma + 1, 2)),
            ("ell", ell, torch.int32, (B,))):
        _need(t, name, dtp, shp, dev)
    out_tokens = _out(out_tokens, "out_tokens", torch.int32, (B, gamma + 1), dev)
    n_accepted = _out(n_accepted, "n_accepted", torch.int32, (B,), dev)
    if ratio is not None or want_ratio:
        ratio = _out(ratio, "ratio", torch.float32, (B, gamma), dev)
    status = _status(status, dev)
    need = dspark_verify_workspace(B, gamma, V, rank, dt)
    ws = _workspace(need, dev, workspace)
    _check(lib.dspark_verify(B, gamma, V, rank, dt, _ptr(target), _ptr(U), _ptr(W1), _ptr(W2),
                             _ptr(anchor), _ptr(tokens), _ptr(q_tok), _ptr(row_max), _ptr(row_logZ),
                             _ptr(temperature), _ptr(uniforms), _ptr(ell), _ptr(out_tokens),
                             _ptr(n_accepted), _ptr(ratio), _ptr(status), _ptr(ws), ws.numel(),
                             _stream()))
    return out_tokens, n_accepted, ratio


def dspark_verify_rnn(target, U, emb, W2, anchor, tokens, q_tok, row_max, row_logZ, temperature,
                      uniforms, ell, *, out_tokens=None, n_accepted=None, ratio=None,
                      status=None, workspace=None, want_ratio=True):
    """dspark_verify for RNN-head drafts: emb [B,gamma,rank] (the drafter's projected
    vectors) replaces W1.  Returns (out_tokens, n_accepted, ratio)."""
    lib = load()
    B, gamma, V = U.shape
    rank = emb.shape[2]
    dt = _dtype_code(U)
    dev = U.device
    _need(U, "U"); _need(target, "target", U.dtype, (B, gamma + 1, V), dev)
    _need(emb, "emb", U.dtype, (B, gamma, rank), dev); _need(W2, "W2", U.dtype, (rank, V), dev)
    for name, t, dtp, shp in (
            ("anchor", anchor, torch.int32, (B,)), ("tokens", tokens, torch.int32, (B, gamma)),
            ("q_tok", q_tok, torch.float32, (B, gamma)),
            ("row_max", row_max, torch.float32, (B, gamma)),
            ("row_logZ", row_logZ, torch.float32, (B, gamma)),
            ("temperature", temperature, torch.float32, (B,)),
            ("uniforms", uniforms, torch.float32, (B, gamma + 1, 2)),
            ("ell", ell, torch.int32, (B,))):
        _need(t, name, dtp, shp, dev)
    out_tokens = _out(out_tokens, "out_tokens", torch.int32, (B, gamma + 1), dev)
    n_accepted = _out(n_accepted, "n_accepted", torch.int32, (B,), dev)
    if ratio is not None or want_ratio:
        ratio = _out(ratio, "ratio", torch.float32, (B, gamma), dev)
    status = _status(status, dev)
    need = dspark_verify_workspace(B, gamma, V, rank, dt)
    ws = _workspace(need, dev, workspace)
    _check(lib.dspark_verify_rnn(B, gamma, V, rank, dt, _ptr(target), _ptr(U), _ptr(emb),
                                 _ptr(W2), _ptr(anchor), _ptr(tokens), _ptr(q_tok), _ptr(row_max),
                                 _ptr(row_logZ), _ptr(temperature), _ptr(uniforms), _ptr(ell),
                                 _ptr(out_tokens), _ptr(n_accepted), _ptr(ratio), _ptr(status),
                                 _ptr(ws), ws.numel(), _stream()))
    return out_tokens, n_accepted, ratio


def dspark_tv_label_workspace(B, gamma, V, rank, dtype) -> int:
    return int(load().dspark_tv_label_workspace(B, gamma, V, rank, dtype))


def dspark_tv_label(target, U, W1, W2, anchor, tokens, row_max, row_logZ, temperature, *,
                    tv=None, label=None, status=None, workspace=None, want_label=True):
    """Acceptance label 1 - TV(draft, target) per drafted position; returns (tv, label)."""
    lib = load()
    B, gamma, V = U.shape
    rank = W1.shape[1]
    dt = _dtype_code(U)
    dev = U.device
    _need(U, "U"); _need(target, "target", U.dtype, (B, gamma + 1, V), dev)
    _need(W1, "W1", U.dtype, (V, rank), dev); _need(W2, "W2", U.dtype, (rank, V), dev)
    for name, t, dtp, shp in (
            ("anchor", anchor, torch.int32, (B,)), ("tokens", tokens, torch.int32, (B, gamma)),
            ("row_max", row_max, torch.float32, (B, gamma)),
            ("row_logZ", row_logZ, torch.float32, (B, gamma)),
            ("temperature", temperature, torch.float32, (B,))):
        _need(t, name, dtp, shp, dev)
    tv = _out(tv, "tv", torch.float32, (B, gamma), dev)
    if label is not None or want_label:
        label = _out(label, "label", torch.float32, (B, gamma), dev)
    status = _status(status, dev)
    need = dspark_tv_label_workspace(B, gamma, V, rank, dt)
    ws = _workspace(need, dev, workspace)
    _check(lib.dspark_tv_label(B, gamma, V, rank, dt, _ptr(target), _ptr(U), _ptr(W1), _ptr(W2),
                               _ptr(anchor), _ptr(tokens), _ptr(row_max), _ptr(row_logZ),
                               _ptr(temperature), _ptr(tv), _ptr(label), _ptr(status), _ptr(ws),
                               ws.numel(), _stream()))
    return tv, label
