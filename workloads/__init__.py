"""Seeded synthetic inputs for the five ZeRO/FSDP shard-step workloads.

This module is shared by the GPU path's callers (tests, bench) and by the
oracle's callers.  It holds NO arithmetic of the method itself — no shard
range, no flattening, no accumulation, no norm, no optimizer arithmetic —
only workload descriptions (sizes, hyperparameter values, seeds) and random
draws made with ``torch.Generator``.

The shapes follow the model families the pages name: a Llama-7B-shaped and a
LLaMA-13B-shaped flat parameter buffer sharded over 8 ranks, one 70B-style
transformer block as one FSDP unit sharded over 64 ranks, and a 70B model
sharded over 64 ranks (ZeRO-3).  No dataset or trained weight is involved:
parameters are U(-0.1, 0.1) and gradients are scaled standard normals.

Seed of every draw: 0x5EED0000 + 0x1000*cfg + 0x100*purpose + 0x10*step + mb
(purpose 0 = master init, 1 = gradient z, 2 = outlier mask, 3 = unit or model
tensors, 4 = per-tensor gradients; for purposes 3 and 4 ``mb`` is the tensor
index).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

PURPOSE_MASTER = 0
PURPOSE_GRAD = 1
PURPOSE_OUTLIER = 2
PURPOSE_UNIT = 3
PURPOSE_TENSOR_GRAD = 4


def seed_of(cfg: int, purpose: int, step: int = 0, mb: int = 0) -> int:
    return 0x5EED0000 + 0x1000 * cfg + 0x100 * purpose + 0x10 * step + mb


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(seed)
    return g


# ---------------------------------------------------------------------------
# model shapes (parameter counts of the named families; untied output head)
# ---------------------------------------------------------------------------

def llama_tensor_shapes(layers: int, hidden: int, ffn: int, vocab: int):
    """Parameter shapes, in module order, of a Llama-style decoder."""
    shapes = [("embed_tokens", (vocab, hidden))]
    for i in range(layers):
        shapes += [
            (f"layers.{i}.q_proj", (hidden, hidden)),
            (f"layers.{i}.k_proj", (hidden, hidden)),
            (f"layers.{i}.v_proj", (hidden, hidden)),
            (f"layers.{i}.o_proj", (hidden, hidden)),
            (f"layers.{i}.gate_proj", (ffn, hidden)),
            (f"layers.{i}.up_proj", (ffn, hidden)),
            (f"layers.{i}.down_proj", (hidden, ffn)),
            (f"layers.{i}.input_layernorm", (hidden,)),
            (f"layers.{i}.post_attention_layernorm", (hidden,)),
        ]
    shapes += [("norm", (hidden,)), ("lm_head", (vocab, hidden))]
    return shapes


def block70b_tensor_shapes(hidden: int = 8192, ffn: int = 28672, q_heads: int = 64,
                           kv_heads: int = 8, head_dim: int = 128):
    """One 70B-style transformer block in the fixed flatten order
    q, k, v, o, gate, up, down, attn_norm, mlp_norm ([out, in] row-major)."""
    kv = kv_heads * head_dim
    q = q_heads * head_dim
    return [
        ("q_proj", (q, hidden)),
        ("k_proj", (kv, hidden)),
        ("v_proj", (kv, hidden)),
        ("o_proj", (hidden, q)),
        ("gate_proj", (ffn, hidden)),
        ("up_proj", (ffn, hidden)),
        ("down_proj", (hidden, ffn)),
        ("attn_norm", (hidden,)),
        ("mlp_norm", (hidden,)),
    ]


def tiny_model_shapes():
    """A one-layer decoder (hidden 256, ffn 600, vocab 1000) plus an odd
    103x197 output projection: 1,000,003 parameters in 12 tensors, so the
    flat buffer's length is odd and its last tensor ends mid-vector."""
    h, f = 256, 600
    return [
        ("embed_tokens", (1000, h)),
        ("q_proj", (h, h)), ("k_proj", (h, h)), ("v_proj", (h, h)), ("o_proj", (h, h)),
        ("gate_proj", (f, h)), ("up_proj", (f, h)), ("down_proj", (h, f)),
        ("input_layernorm", (h,)), ("post_attention_layernorm", (h,)), ("norm", (h,)),
        ("out_proj", (103, 197)),
    ]


def numel_of(shape) -> int:
    n = 1
    for d in shape:
        n *= int(d)
    return n


# ---------------------------------------------------------------------------
# workload descriptions
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    cfg: int                      # 1..5, used in the seeds
    name: str
    total: int                    # elements of the flat parameter buffer
    world: int                    # ranks the buffer is sharded over
    rank: int                     # the rank whose shard this GPU runs
    steps: int
    micro_batches: int            # gradient micro-batches per step
    grad_dtype: str               # "f32" or "bf16"
    grad_std: float               # std of one micro-batch gradient draw
    lr: float
    beta1: float
    beta2: float
    eps: float
    weight_decay: float
    grad_scale: float             # 1 / (micro_batches * world), a power of two
    max_norm: float               # <= 0: no clip
    bf16_param: bool              # write the bf16 re-cast of the master
    std_multipliers: tuple = ()   # per-step factor on grad_std (empty: 1)
    outlier_frac: float = 0.0     # fraction of gradient entries scaled up
    outlier_mult: float = 1.0
    other_ranks_norm_sq: Optional[float] = None   # fixed stand-in, if any
    unit_shapes: tuple = field(default=())        # FSDP unit tensors (C4)
    param_shapes: tuple = field(default=())       # model tensors of the flat buffer (ZeRO-1 flow)
    description: str = ""

    def std_at(self, step: int) -> float:
        """Gradient std at 1-based step ``step``."""
        if self.std_multipliers:
            return self.grad_std * self.std_multipliers[step - 1]
        return self.grad_std


C3_MULTIPLIERS = (0.6, 1.5, 0.8, 0.7, 2.0, 0.9, 0.5, 1.25, 0.75, 0.85)

TINY = tiny_model_shapes()
LLAMA7B = llama_tensor_shapes(32, 4096, 11008, 32000)
LLAMA13B = llama_tensor_shapes(40, 5120, 13824, 32000)
BLOCK70B = block70b_tensor_shapes()

WORKLOADS = {
    "tiny_zero1": Workload(
        cfg=1, name="tiny_zero1", total=1_000_003, world=8, rank=3, steps=5, micro_batches=1,
        grad_dtype="f32", grad_std=1e-3, lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8,
        weight_decay=0.0, grad_scale=1.0 / 8, max_norm=0.0, bf16_param=False,
        param_shapes=tuple(TINY),
        description="flat fp32 buffer of 1,000,003 params (12 tensors), world 8, rank 3; Adam; "
                    "5 steps"),
    "llama7b_shard": Workload(
        cfg=2, name="llama7b_shard", total=sum(numel_of(s) for _, s in LLAMA7B), world=8, rank=0,
        steps=3, micro_batches=8, grad_dtype="bf16", grad_std=1e-3, lr=3e-4, beta1=0.9,
        beta2=0.95, eps=1e-8, weight_decay=0.1, grad_scale=1.0 / 64, max_norm=0.0,
        bf16_param=True,
        description="Llama-7B-shaped flat buffer (6,738,415,616), world 8: one 842,301,952-element "
                    "shard, 8 bf16 micro-batches accumulated in fp32, AdamW, bf16 re-cast"),
    "llama13b_shard_clip": Workload(
        cfg=3, name="llama13b_shard_clip", total=sum(numel_of(s) for _, s in LLAMA13B), world=8,
        rank=0, steps=10, micro_batches=4, grad_dtype="bf16", grad_std=1.4024e-4, lr=3e-4,
        beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_scale=1.0 / 32, max_norm=1.0,
        bf16_param=True, std_multipliers=C3_MULTIPLIERS,
        description="LLaMA-13B-shaped flat buffer (13,015,864,320), world 8: one shard, 4 bf16 "
                    "micro-batches, global-norm clip 1.0 (steps 2, 5, 8 clip), AdamW"),
    "fsdp_unit_70b_block": Workload(
        cfg=4, name="fsdp_unit_70b_block", total=sum(numel_of(s) for _, s in BLOCK70B), world=64,
        rank=17, steps=1, micro_batches=1, grad_dtype="bf16", grad_std=1e-4, lr=1.5e-4, beta1=0.9,
        beta2=0.95, eps=1e-8, weight_decay=0.1, grad_scale=1.0 / 64, max_norm=0.0,
        bf16_param=True, unit_shapes=tuple(BLOCK70B),
        description="one 70B-style block (855,654,400 params) as one FSDP unit, world 64, rank 17: "
                    "pack, one AdamW step on the shard, unpack"),
    "zero3_70b_shard": Workload(
        cfg=5, name="zero3_70b_shard", total=70_000_000_000, world=64, rank=0, steps=2,
        micro_batches=1, grad_dtype="bf16", grad_std=1e-4, lr=1.5e-4, beta1=0.9, beta2=0.95,
        eps=1e-8, weight_decay=0.1, grad_scale=1.0 / 64, max_norm=1.0, bf16_param=True,
        outlier_frac=1e-3, outlier_mult=100.0, other_ranks_norm_sq=1.8503,
        description="70e9 params over 64 ranks: one 1,093,750,000-element shard, bf16 grads with "
                    "0.1% 100x outliers widened to fp32, clip 1.0, AdamW, 2 steps"),
}


def other_ranks_norm_sq(w: Workload, step: int, shard_len: int) -> float:
    """Stand-in for the other ranks' share of the squared global norm.

    For the 13B workload it is the expected value of the other world-1
    ranks' sums of squares of the scaled gradient at step ``step``
    (each element has variance micro_batches * std^2 * grad_scale^2).
    """
    if w.other_ranks_norm_sq is not None:
        return w.other_ranks_norm_sq
    if w.max_norm <= 0:
        return 0.0
    std = w.std_at(step)
    per_elem = w.micro_batches * std * std * w.grad_scale * w.grad_scale
    return (w.world - 1) * shard_len * per_elem


# ---------------------------------------------------------------------------
# draws
# ---------------------------------------------------------------------------

def master_init(w: Workload, n: int, device="cpu") -> torch.Tensor:
    """fp32 U(-0.1, 0.1) of length n."""
    g = _gen(seed_of(w.cfg, PURPOSE_MASTER), device)
    return torch.rand(n, generator=g, device=device, dtype=torch.float32).mul_(0.2).sub_(0.1)


def grad_draw(w: Workload, n: int, step: int, mb: int, device="cpu") -> torch.Tensor:
    """One micro-batch gradient of length n (fp32 or bf16 per the workload)."""
    g = _gen(seed_of(w.cfg, PURPOSE_GRAD, step, mb), device)
    z = torch.randn(n, generator=g, device=device, dtype=torch.float32)
    z.mul_(w.std_at(step))
    if w.outlier_frac > 0:
        go = _gen(seed_of(w.cfg, PURPOSE_OUTLIER, step, mb), device)
        u = torch.rand(n, generator=go, device=device, dtype=torch.float32)
        z = torch.where(u < w.outlier_frac, z * w.outlier_mult, z)
        del u
    if w.grad_dtype == "bf16":
        return z.to(torch.bfloat16)
    return z


def unit_tensors(w: Workload, device="cpu"):
    """The FSDP unit's parameters: bf16 U(-0.1, 0.1), one tensor per shape."""
    out = []
    for i, (_, shape) in enumerate(w.unit_shapes):
        g = _gen(seed_of(w.cfg, PURPOSE_UNIT, 0, i), device)
        t = torch.rand(shape, generator=g, device=device, dtype=torch.float32).mul_(0.2).sub_(0.1)
        out.append(t.to(torch.bfloat16))
    return out


def param_tensors(w: Workload, device="cpu"):
    """The model's fp32 parameters, U(-0.1, 0.1), one tensor per shape."""
    out = []
    for i, (_, shape) in enumerate(w.param_shapes):
        g = _gen(seed_of(w.cfg, PURPOSE_UNIT, 0, i), device)
        out.append(torch.rand(shape, generator=g, device=device, dtype=torch.float32).mul_(0.2).sub_(0.1))
    return out


def grad_tensors(w: Workload, step: int, device="cpu"):
    """The model's gradients at 1-based step ``step``: fp32 std * z per tensor
    (already the sum over ranks; the workload's grad_scale averages it)."""
    out = []
    for i, (_, shape) in enumerate(w.param_shapes):
        g = _gen(seed_of(w.cfg, PURPOSE_TENSOR_GRAD, step, i), device)
        out.append(torch.randn(shape, generator=g, device=device, dtype=torch.float32).mul_(w.std_at(step)))
    return out


def small_variant(w: Workload, total: int) -> Workload:
    """The same workload at a reduced buffer size (for parity at small sizes)."""
    from dataclasses import replace
    return replace(w, total=total)


def replace_unit(w: Workload, shapes) -> Workload:
    """The same workload over a different list of unit tensor shapes."""
    from dataclasses import replace
    return replace(w, unit_shapes=tuple(shapes), total=sum(numel_of(s) for _, s in shapes))
