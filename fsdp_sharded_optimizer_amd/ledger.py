"""Per-rank memory ledger of ZeRO stages (host arithmetic, no device work).

Bytes per parameter in bf16 mixed precision with AdamW ([Memory page]
ybb.press "大模型分布式训练并行与显存工程实战", §"一、显存账本"; the
[Infra page] "AI/ML 详解：训练基础设施", ZeRO section): 16 B — 2 for the bf16
parameter and 2 for its bf16 gradient (the 4 B every rank needs at some
point), 12 for the optimizer's history (fp32 master, exp_avg, exp_avg_sq).
ZeRO-1 shards the 12 B, ZeRO-2 also the gradient, ZeRO-3 (FSDP FULL_SHARD)
also the parameter, so a rank holds about 16/N B per parameter.

`library_shard_bytes` gives what this library's buffers for one rank's
shard occupy (the fp32 accumulator is an extra 4 B per element).
"""
from __future__ import annotations

from dataclasses import dataclass

PARAM_BYTES = 2      # bf16 parameter
GRAD_BYTES = 2       # bf16 gradient
OPTIM_BYTES = 12     # fp32 master + exp_avg + exp_avg_sq


@dataclass(frozen=True)
class Ledger:
    params: float    # bytes of parameters on one rank
    grads: float
    optim: float

    @property
    def total(self) -> float:
        return self.params + self.grads + self.optim


def per_rank(n_params: float, world: int, stage: int, param_bytes: float = PARAM_BYTES,
             grad_bytes: float = GRAD_BYTES, optim_bytes: float = OPTIM_BYTES) -> Ledger:
    """Model-state bytes one rank holds under ZeRO stage 0 (plain data
    parallel), 1, 2 or 3 (activations and buffers not included)."""
    if world < 1 or stage not in (0, 1, 2, 3):
        raise ValueError("world >= 1 and stage in 0..3")
    p = n_params * param_bytes
    g = n_params * grad_bytes
    o = n_params * optim_bytes
    return Ledger(params=p / world if stage >= 3 else p,
                  grads=g / world if stage >= 2 else g,
                  optim=o / world if stage >= 1 else o)


def redundant_fraction(param_bytes: float = PARAM_BYTES, grad_bytes: float = GRAD_BYTES,
                       optim_bytes: float = OPTIM_BYTES) -> float:
    """Share of the per-parameter bytes that is optimizer history."""
    return optim_bytes / (param_bytes + grad_bytes + optim_bytes)


def cards_to_hold(n_params: float, card_bytes: float, bytes_per_param: float = 16.0) -> float:
    """Cards needed just to hold the model state without sharding savings."""
    return n_params * bytes_per_param / card_bytes


def library_shard_bytes(shard_elems: int, bf16_param: bool = True, grad_buffers: int = 1,
                        grad_bytes: int = GRAD_BYTES) -> int:
    """Bytes of this library's per-rank buffers: fp32 master, exp_avg,
    exp_avg_sq and accumulator, the bf16 parameter shard, and `grad_buffers`
    micro-batch gradients in flight."""
    return shard_elems * (16 + (2 if bf16_param else 0) + grad_buffers * grad_bytes)
