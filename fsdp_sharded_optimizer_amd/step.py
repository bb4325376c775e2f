"""One rank's sharded optimizer state and its step, on the library's entry points.

The state is plain device buffers: the fp32 master shard, exp_avg and
exp_avg_sq, the fp32 gradient accumulator, the bf16 parameter shard and the
norm scratch.  A step is: ``accumulate`` once per micro-batch (the last one
may form the squared norm in the same pass), then ``step``: the norm (if
not formed yet and requested) and the fused AdamW update with the bf16
re-cast.  Nothing here computes; it orders calls.

``state_dict`` / ``load_state_dict`` carry the step counter and the fp32
master, exp_avg and exp_avg_sq between runs: a resumed run continues bit
for bit (the bf16 parameter is the master's re-cast, rewritten every step).
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _binding as zs


class ShardOptimizer:
    def __init__(self, master: torch.Tensor, *, lr: float, betas=(0.9, 0.999), eps: float = 1e-8,
                 weight_decay: float = 0.0, grad_scale: float = 1.0, max_norm: float = 0.0,
                 param_bf16: Optional[torch.Tensor] = None, compute_norm: Optional[bool] = None):
        if master.dtype != torch.float32 or master.device.type != "cuda":
            raise TypeError("master must be an fp32 GPU tensor")
        n = master.numel()
        dev = master.device
        self.master = master
        self.exp_avg = torch.zeros(n, dtype=torch.float32, device=dev)
        self.exp_avg_sq = torch.zeros(n, dtype=torch.float32, device=dev)
        self.acc = torch.empty(n, dtype=torch.float32, device=dev)
        self.param_bf16 = param_bf16
        self.lr, self.betas, self.eps = lr, betas, eps
        self.weight_decay, self.grad_scale, self.max_norm = weight_decay, grad_scale, max_norm
        self.compute_norm = (max_norm > 0) if compute_norm is None else compute_norm
        self.norm_sq = torch.zeros(1, dtype=torch.float64, device=dev)
        ws = max(zs.grad_norm_sq_workspace_bytes(n), zs.grad_accum_norm_sq_workspace_bytes(n), 8)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
        self._norm_ready = False
        self.t = 0
        self._pending = 0

    def accumulate(self, grad: torch.Tensor, last: bool = False) -> None:
        """Add one micro-batch gradient (fp32 or bf16) into the fp32 buffer.
        With last=True (and a norm wanted) the same pass also forms the
        squared norm, so step() needs no separate read of the buffer."""
        first = self._pending == 0
        if last and self.compute_norm:
            zs.grad_accum_norm_sq(self.acc, grad, first, self.grad_scale, self.norm_sq, self.workspace)
            self._norm_ready = True
        else:
            zs.grad_accum(self.acc, grad, overwrite=first)
            self._norm_ready = False
        self._pending += 1

    def hp(self, extra_norm_sq: float = 0.0) -> zs.AdamWConfig:
        return zs.AdamWConfig(lr=self.lr, beta1=self.betas[0], beta2=self.betas[1], eps=self.eps,
                              weight_decay=self.weight_decay, grad_scale=self.grad_scale,
                              max_norm=self.max_norm, extra_norm_sq=extra_norm_sq, step=self.t)

    def step(self, extra_norm_sq: float = 0.0) -> None:
        """Norm (if clipping or asked for), then the fused AdamW update.  The
        step counter advances only once the update is enqueued."""
        if self._pending == 0:
            raise RuntimeError("step() without an accumulated gradient")
        norm = None
        if self.compute_norm:
            if not self._norm_ready:
                zs.grad_norm_sq(self.acc, self.grad_scale, self.norm_sq, self.workspace)
            norm = self.norm_sq
        hp = self.hp(extra_norm_sq)
        hp.step = self.t + 1
        zs.adamw_step(hp, self.master, self.exp_avg, self.exp_avg_sq, self.acc, self.param_bf16, norm_sq=norm)
        self.t += 1
        self._pending = 0
        self._norm_ready = False

    def state_dict(self) -> dict:
        """The optimizer state: the step counter and the fp32 master,
        exp_avg and exp_avg_sq (the live device tensors, not copies)."""
        return {"step": self.t, "master": self.master, "exp_avg": self.exp_avg, "exp_avg_sq": self.exp_avg_sq}

    def load_state_dict(self, state: dict) -> None:
        """Copy a state_dict's tensors (any device) into this shard's buffers
        and take its step counter; sizes must match.  Drops any pending
        accumulation."""
        names = ("master", "exp_avg", "exp_avg_sq")
        for name in names:   # every check before the first copy: a refused state changes nothing
            src, dst = state[name], getattr(self, name)
            if src.numel() != dst.numel() or src.dtype != torch.float32:
                raise ValueError(f"load_state_dict: {name} must be {dst.numel()} float32 elements")
        t = int(state["step"])
        if t < 0:
            raise ValueError("load_state_dict: step must be >= 0")
        for name in names:
            getattr(self, name).copy_(state[name].reshape(-1))
        self.t = t
        self._pending = 0
        self._norm_ready = False
