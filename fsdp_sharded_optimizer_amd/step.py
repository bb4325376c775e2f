"""One rank's sharded optimizer state and its step, on the library's entry points.

The state is plain device buffers: the fp32 master shard, exp_avg and
exp_avg_sq, the fp32 gradient accumulator, the bf16 parameter shard and the
norm scratch.  A step is: ``accumulate`` once per micro-batch (the last one
may form the squared norm in the same pass), then ``step``: the norm (if
not formed yet and requested) and the fused AdamW update with the bf16
re-cast.  ``step(last_grad=g)`` takes the last micro-batch's gradient
itself instead: its sum with the accumulator is never stored (the norm pass
reads both, and so does AdamW), which saves the accumulator's write and
re-read, 8 B per element; the results are the same bit for bit.  Where a
step's micro-batch gradients are all kept in device memory (2 B per element
each in bf16), ``accumulate_all`` sums them in one pass instead.  Nothing
here computes; it orders calls.

``layout="tiled"`` (the default) keeps master, exp_avg and exp_avg_sq in
one buffer in the library's tiled state layout, which the AdamW step
streams faster than three buffers; the ``master``, ``exp_avg`` and
``exp_avg_sq`` attributes then read fresh split copies back out of it, and
the caller's master tensor only supplies the initial values.
``layout="split"`` steps the caller's master tensor and two moment buffers
in place.  Both layouts give bit-identical results.

``arena=DeviceArena(...)`` takes the optimizer's streamed buffers (the
state and the accumulator, ``arena_parts``) from one physically contiguous
block of device memory, which keeps the step's bandwidth independent of
what the process and others allocated and freed before; the caller takes
its gradient and parameter buffers from the same block.

``state_dict`` / ``load_state_dict`` carry the step counter and the fp32
master, exp_avg and exp_avg_sq between runs: a resumed run continues bit
for bit (the bf16 parameter is the master's re-cast, rewritten every step).
``capture`` records one whole step in a HIP graph that replays every later
step (the AdamW scalars are read from device memory), for shards small
enough that launch overhead counts.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import _binding as zs
from .arena import DeviceArena


_STATE_NAMES = ("master", "exp_avg", "exp_avg_sq")


class ShardOptimizer:
    def __init__(self, master: torch.Tensor, *, lr: float, betas=(0.9, 0.999), eps: float = 1e-8,
                 weight_decay: float = 0.0, grad_scale: float = 1.0, max_norm: float = 0.0,
                 param_bf16: Optional[torch.Tensor] = None, compute_norm: Optional[bool] = None,
                 layout: str = "tiled", arena: Optional[DeviceArena] = None):
        if master.dtype != torch.float32 or master.device.type != "cuda":
            raise TypeError("master must be an fp32 GPU tensor")
        if layout not in ("tiled", "split"):
            raise ValueError("layout must be 'tiled' or 'split'")
        n = master.numel()
        dev = master.device
        if arena is not None and arena.device != dev:
            raise ValueError(f"arena is on {arena.device}, master on {dev}")
        self.n = n
        self.layout = layout
        self.arena = arena

        def take(numel, dtype):
            if arena is not None:
                return arena.take(numel, dtype)
            return torch.empty(numel, dtype=dtype, device=dev)

        parts = iter(self.arena_parts(n, layout))
        if layout == "tiled":
            # the master's values go into the tiled buffer; the moments start at zero
            self.state = take(*next(parts))
            zs.state_tile(master.reshape(-1), None, None, self.state, n=n)
            self._split = None
        else:
            self.state = None
            self._split = {"master": master, "exp_avg": take(*next(parts)).zero_(),
                           "exp_avg_sq": take(*next(parts)).zero_()}
        self.acc = take(*next(parts))
        self.param_bf16 = param_bf16
        self.lr, self.betas, self.eps = lr, betas, eps
        self.weight_decay, self.grad_scale, self.max_norm = weight_decay, grad_scale, max_norm
        self.compute_norm = (max_norm > 0) if compute_norm is None else compute_norm
        # the norm and its partials stay ordinary allocations: the norm pass
        # writes one 8-byte partial per 256 elements, scattered, which ran
        # 5 points slower in a contiguous block
        self.norm_sq = torch.zeros(1, dtype=torch.float64, device=dev)
        ws = max(zs.grad_norm_sq_workspace_bytes(n), zs.grad_accum_norm_sq_workspace_bytes(n),
                 zs.grad_reduce_chunks_norm_sq_workspace_bytes(n), 8)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
        self._norm_ready = False
        self.t = 0
        self._pending = 0

    @staticmethod
    def arena_parts(n: int, layout: str = "tiled") -> list:
        """(numel, dtype) of each streamed buffer the optimizer takes from an
        arena, in order: the state (tiled, or the two moments) and the
        accumulator.  ``DeviceArena.size`` of these, plus the caller's own
        parts (gradients, bf16 parameter), sizes an arena that holds a
        rank's whole streamed working set."""
        state = ([(zs.state_tiled_numel(n), torch.float32)] if layout == "tiled"
                 else [(n, torch.float32), (n, torch.float32)])
        return state + [(n, torch.float32)]

    def _state_tensor(self, name: str) -> torch.Tensor:
        if self._split is not None:
            return self._split[name]
        out = torch.empty(self.n, dtype=torch.float32, device=self.acc.device)
        dst = [out if k == name else None for k in _STATE_NAMES]
        zs.state_untile(self.state, *dst, n=self.n)
        return out

    # split layout: the live buffers; tiled layout: fresh copies read out of the tiled state
    master = property(lambda self: self._state_tensor("master"))
    exp_avg = property(lambda self: self._state_tensor("exp_avg"))
    exp_avg_sq = property(lambda self: self._state_tensor("exp_avg_sq"))

    def _adamw(self, hp: zs.AdamWConfig, norm) -> None:
        if self._split is not None:
            zs.adamw_step(hp, self._split["master"], self._split["exp_avg"], self._split["exp_avg_sq"], self.acc,
                          self.param_bf16, norm_sq=norm)
        else:
            zs.adamw_step_tiled(hp, self.state, self.acc, self.param_bf16, norm_sq=norm)

    def _save(self) -> dict:
        """Device copies of the optimizer state (and bf16 parameter)."""
        saved = {"state": self.state.clone()} if self._split is None else \
            {k: v.clone() for k, v in self._split.items()}
        if self.param_bf16 is not None:
            saved["param_bf16"] = self.param_bf16.clone()
        return saved

    def _restore(self, saved: dict) -> None:
        if self._split is None:
            self.state.copy_(saved["state"])
        else:
            for k in _STATE_NAMES:
                self._split[k].copy_(saved[k])
        if self.param_bf16 is not None:
            self.param_bf16.copy_(saved["param_bf16"])

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

    def accumulate_all(self, grads: list, last: bool = False) -> None:
        """Add several micro-batch gradients held in device memory at once
        (one dtype, fp32 or bf16) into the fp32 buffer in one pass, in list
        order: bit-identical to accumulate() on each in turn, for far fewer
        bytes (the buffer is read and written once, not once per gradient).
        With last=True (and a norm wanted) the same pass also forms the
        squared norm, as accumulate(last=True) does."""
        if not grads:
            raise ValueError("accumulate_all: at least one gradient")
        flat = [g.reshape(-1) for g in grads]
        first = self._pending == 0
        if last and self.compute_norm:
            zs.grad_reduce_chunks_norm_sq(self.acc, flat, first, self.grad_scale, self.norm_sq, self.workspace)
            self._norm_ready = True
        else:
            zs.grad_reduce_chunks(self.acc, flat, overwrite=first)
            self._norm_ready = False
        self._pending += len(grads)

    def hp(self, extra_norm_sq: float = 0.0) -> zs.AdamWConfig:
        return zs.AdamWConfig(lr=self.lr, beta1=self.betas[0], beta2=self.betas[1], eps=self.eps,
                              weight_decay=self.weight_decay, grad_scale=self.grad_scale,
                              max_norm=self.max_norm, extra_norm_sq=extra_norm_sq, step=self.t)

    def step(self, extra_norm_sq: float = 0.0, last_grad: Optional[torch.Tensor] = None) -> None:
        """Norm (if clipping or asked for), then the fused AdamW update.  The
        step counter advances only once the update is enqueued.

        last_grad: the last micro-batch's gradient, not yet accumulated (the
        step is then the same, bit for bit, as accumulate(last_grad,
        last=True) followed by step()).  Its sum with the accumulator is
        formed where it is read and never stored: the norm pass reads the
        accumulator and last_grad (grad_sum_norm_sq), AdamW reads them again
        (adamw_step_tiled_sum, or adamw_step_sum on the split state), and
        the accumulator keeps the earlier micro-batches' sum."""
        if last_grad is not None:
            if self._norm_ready:
                raise RuntimeError("step(last_grad=...) after accumulate(..., last=True)")
            self._step_on_sum(last_grad, extra_norm_sq)
            return
        if self._pending == 0:
            raise RuntimeError("step() without an accumulated gradient")
        norm = None
        if self.compute_norm:
            if not self._norm_ready:
                zs.grad_norm_sq(self.acc, self.grad_scale, self.norm_sq, self.workspace)
            norm = self.norm_sq
        hp = self.hp(extra_norm_sq)
        hp.step = self.t + 1
        self._adamw(hp, norm)
        self.t += 1
        self._pending = 0
        self._norm_ready = False

    def _step_on_sum(self, last_grad: torch.Tensor, extra_norm_sq: float) -> None:
        acc = self.acc if self._pending > 0 else None   # a single micro-batch: its gradient alone
        g = last_grad.reshape(-1)
        norm = None
        if self.compute_norm:
            zs.grad_sum_norm_sq(acc, g, acc is None, self.grad_scale, self.norm_sq, self.workspace)
            norm = self.norm_sq
        hp = self.hp(extra_norm_sq)
        hp.step = self.t + 1
        if self._split is not None:
            zs.adamw_step_sum(hp, self._split["master"], self._split["exp_avg"], self._split["exp_avg_sq"], acc, g,
                              self.param_bf16, norm_sq=norm)
        else:
            zs.adamw_step_tiled_sum(hp, self.state, acc, g, self.param_bf16, norm_sq=norm)
        self.t += 1
        self._pending = 0
        self._norm_ready = False

    def capture(self, grads: list, extra_norm_sq: float = 0.0) -> "CapturedStep":
        """Record one whole step (accumulate every tensor of ``grads`` but
        the last in order, then the last one's norm if wanted and AdamW with
        the bf16 re-cast on the sum, as step(last_grad=) runs them) into a
        HIP graph whose AdamW scalars are read from device memory, so the same
        graph replays every later step.  ``grads`` are fixed device tensors
        the caller refills with each step's micro-batch gradients before
        ``replay()``.  Nothing is allocated at replay; the step counter
        advances on the host and its scalars are copied in by the graph.
        Capturing runs the step once, as graph capture requires, on the
        optimizer's state and restores it after, so it briefly holds a copy
        of the fp32 master and moments (12 B per element, plus the tiled
        layout's padding)."""
        return CapturedStep(self, list(grads), extra_norm_sq)

    def state_dict(self) -> dict:
        """The optimizer state: the step counter and the fp32 master,
        exp_avg and exp_avg_sq as split arrays (split layout: the live
        device tensors; tiled layout: fresh copies read out of the tiled
        buffer), so a checkpoint does not depend on the layout."""
        return {"step": self.t, **{k: self._state_tensor(k) for k in _STATE_NAMES}}

    def load_state_dict(self, state: dict) -> None:
        """Copy a state_dict's tensors (any device) into this shard's buffers
        and take its step counter; sizes must match.  Drops any pending
        accumulation."""
        for name in _STATE_NAMES:   # every check before the first copy: a refused state changes nothing
            src = state[name]
            if src.numel() != self.n or src.dtype != torch.float32:
                raise ValueError(f"load_state_dict: {name} must be {self.n} float32 elements")
        t = int(state["step"])
        if t < 0:
            raise ValueError("load_state_dict: step must be >= 0")
        dev = self.acc.device
        if self._split is None:
            srcs = [state[k].reshape(-1).to(dev).contiguous() for k in _STATE_NAMES]
            zs.state_tile(*srcs, self.state, n=self.n)
        else:
            for name in _STATE_NAMES:
                self._split[name].copy_(state[name].reshape(-1))
        self.t = t
        self._pending = 0
        self._norm_ready = False


class CapturedStep:
    """One ShardOptimizer step captured in a HIP graph (see
    ShardOptimizer.capture).  replay() runs the next step: t + 1, with the
    optimizer's hyperparameters and this capture's extra_norm_sq."""

    def __init__(self, opt: ShardOptimizer, grads: list, extra_norm_sq: float):
        if not grads:
            raise ValueError("capture: at least one gradient buffer")
        self.opt = opt
        self.grads = grads
        self.extra_norm_sq = extra_norm_sq
        dev = opt.acc.device
        nbytes = len(zs.scalars_bytes(zs.AdamWConfig(lr=opt.lr)))
        self._host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        self._dev = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self._done = torch.cuda.Event()
        self._write_scalars(opt.t + 1)
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        # one warm-up run on a side stream, as capture requires; the state it
        # steps is saved first and restored after, so capturing changes nothing
        saved = opt._save()
        with torch.cuda.stream(side):
            self._body()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize(dev)
        opt._restore(saved)
        del saved
        torch.cuda.synchronize(dev)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self._body()
        opt._pending = 0
        opt._norm_ready = False

    def _write_scalars(self, t: int) -> None:
        hp = self.opt.hp(self.extra_norm_sq)
        hp.step = t
        self._host.numpy()[:] = np.frombuffer(zs.scalars_bytes(hp), dtype=np.uint8)

    def _body(self) -> None:
        """The step as ShardOptimizer runs it with step(last_grad=): the last
        gradient folded into the norm pass and AdamW, its sum never stored."""
        opt = self.opt
        last = len(self.grads) - 1
        for k, g in enumerate(self.grads[:last]):
            zs.grad_accum(opt.acc, g, overwrite=(k == 0))
        g = self.grads[last]
        norm = opt.norm_sq if opt.compute_norm else None
        acc = opt.acc if last > 0 else None
        if opt.compute_norm:
            zs.grad_sum_norm_sq(acc, g, acc is None, opt.grad_scale, opt.norm_sq, opt.workspace)
        self._dev.copy_(self._host, non_blocking=True)
        if opt._split is not None:
            s = opt._split
            zs.adamw_step_sum_dev(self._dev, s["master"], s["exp_avg"], s["exp_avg_sq"], acc, g, opt.param_bf16,
                                  norm_sq=norm)
        else:
            zs.adamw_step_tiled_sum_dev(self._dev, opt.state, acc, g, opt.param_bf16, norm_sq=norm)

    def replay(self) -> None:
        """Run the next step.  Waits for the previous replay to have read the
        pinned scalars before rewriting them."""
        self._done.synchronize()
        self._write_scalars(self.opt.t + 1)
        self.graph.replay()
        self._done.record()
        self.opt.t += 1
