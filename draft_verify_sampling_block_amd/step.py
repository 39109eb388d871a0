"""One decode step of the sampling path on the device, through the C ABI.

draft_block -> confidence -> schedule (or a fixed verify length) -> verify,
all enqueued on the current stream with no host synchronisation inside.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import torch

from . import dspark_draft_block_conf, dspark_schedule, dspark_verify


@dataclasses.dataclass
class DeviceInputs:
    B: int
    gamma: int
    V: int
    rank: int
    H: int
    U: torch.Tensor
    target: torch.Tensor
    W1: torch.Tensor
    W2: torch.Tensor
    w: torch.Tensor
    b0: float
    hidden: torch.Tensor
    anchor: torch.Tensor
    temperature: torch.Tensor
    uniforms: torch.Tensor
    sps: torch.Tensor | None
    fixed_ell: torch.Tensor | None


def _dev(a: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:  # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def upload(wl, device="cuda", scheduler: bool | None = None) -> DeviceInputs:
    """Copy a host workload (gen.Workload-like) to device memory."""
    sched = wl.spec.scheduler if scheduler is None else scheduler
    B, g = wl.B, wl.gamma
    return DeviceInputs(
        B=B, gamma=g, V=wl.V, rank=wl.rank, H=wl.H,
        U=_dev(wl.U, device), target=_dev(wl.target, device), W1=_dev(wl.W1, device),
        W2=_dev(wl.W2, device), w=_dev(wl.w.astype(np.float32), device), b0=float(wl.b0),
        hidden=_dev(wl.hidden, device), anchor=_dev(wl.anchor.astype(np.int32), device),
        temperature=_dev(wl.temperature.astype(np.float32), device),
        uniforms=_dev(wl.uniforms.astype(np.float32), device),
        sps=_dev(wl.sps.astype(np.float64), device) if (sched and wl.sps is not None) else None,
        fixed_ell=None if (sched and wl.sps is not None) else torch.full((B,), g, dtype=torch.int32,
                                                                        device=device),
    )


class Step:
    """Holds outputs and workspaces so repeated steps allocate nothing new."""

    def __init__(self, d: DeviceInputs):
        self.d = d
        dev = d.U.device
        B, g = d.B, d.gamma
        self.status = torch.zeros((1,), dtype=torch.int32, device=dev)
        self.tokens = torch.empty((B, g), dtype=torch.int32, device=dev)
        self.q_tok = torch.empty((B, g), dtype=torch.float32, device=dev)
        self.row_max = torch.empty((B, g), dtype=torch.float32, device=dev)
        self.row_logZ = torch.empty((B, g), dtype=torch.float32, device=dev)
        self.conf = torch.empty((B, g), dtype=torch.float32, device=dev)
        self.ell = torch.empty((B,), dtype=torch.int32, device=dev)
        self.order = torch.empty((B * g,), dtype=torch.int32, device=dev)
        self.stats = torch.zeros((3,), dtype=torch.float64, device=dev)
        self.out_tokens = torch.empty((B, g + 1), dtype=torch.int32, device=dev)
        self.n_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
        self.ratio = torch.empty((B, g), dtype=torch.float32, device=dev)
        from . import dspark_draft_block_workspace, dspark_verify_workspace, _dtype_code
        dt = _dtype_code(d.U)
        # the draft workspace starts zero-filled; every draft call leaves it so
        self.ws_draft = torch.zeros(max(256, dspark_draft_block_workspace(B, g, d.V, d.rank, dt)),
                                    dtype=torch.uint8, device=dev)
        self.ws_verify = torch.empty(max(256, dspark_verify_workspace(B, g, d.V, d.rank, dt)),
                                     dtype=torch.uint8, device=dev)
        from . import dspark_schedule_workspace
        self.ws_sched = torch.empty(max(256, dspark_schedule_workspace(B, g)), dtype=torch.uint8,
                                    device=dev)

    def run(self, status: torch.Tensor | None = None):
        """Enqueue one step.  Device flags go to `status` (a (1,) int32
        device tensor the caller cleared) or, when None, to self.status,
        which is cleared first by a fill kernel (no memset node, so the step
        stays capturable in a graph)."""
        d = self.d
        if status is None:
            self.status.zero_()
            status = self.status
        # the draft and the confidence head of the drafted block in one call
        dspark_draft_block_conf(d.U, d.W1, d.W2, d.anchor, d.temperature, d.uniforms, d.hidden,
                                d.w, d.b0, tokens=self.tokens, q_tok=self.q_tok,
                                row_max=self.row_max, row_logZ=self.row_logZ, conf=self.conf,
                                status=status, workspace=self.ws_draft)
        if d.sps is not None:
            dspark_schedule(self.conf, d.sps, ell=self.ell, order=self.order, stats=self.stats,
                            status=status, workspace=self.ws_sched)
            ell = self.ell
        else:
            ell = d.fixed_ell
        dspark_verify(d.target, d.U, d.W1, d.W2, d.anchor, self.tokens, self.q_tok, self.row_max,
                      self.row_logZ, d.temperature, d.uniforms, ell, out_tokens=self.out_tokens,
                      n_accepted=self.n_accepted, ratio=self.ratio, status=status,
                      workspace=self.ws_verify)
        return self

    def ell_used(self) -> torch.Tensor:
        return self.ell if self.d.sps is not None else self.d.fixed_ell
