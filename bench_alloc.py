#!/usr/bin/env python3
"""Shard length against allocation history, in one process on one GPU.

    python bench_alloc.py [--reps 10] [--rounds 2] [--pad-gib G ...]

Part 1 (shard length): the accumulation (grad_accum, add), the fused last
micro-batch (grad_accum_norm_sq, add) and the clipped tiled AdamW step
(adamw_step_tiled) at the Llama-7B, 70B ZeRO-3 and LLaMA-13B shard lengths,
all on prefixes of one set of buffers sized for the largest shard, in
interleaved rounds: the same physical memory for every length.
Part 2 (allocation history): the AdamW step on the 70B ZeRO-3 and the
Llama-7B shards (bench.py's step rig) allocated fresh, with the other shard
resident, and re-allocated after the other shard's buffers were freed;
each rig's buffers allocated one by one ("separate") and as views of one
physically contiguous block ("arena", bench.py's policy; such a block is
never freed, so a rig made again takes its pooled block back).
Part 3 (--pad-gib): the one-pass step of the Llama-7B rig (bench.py's timed
step, its buffers allocated one by one) allocated behind G GiB of padding
held in device memory, for each G: the same buffers at other physical pages.

One line per measurement: what, shard length, ms per launch (HIP events on
the launch stream) and % of the 8 TB/s HBM peak for the kernel's
algorithmic bytes (10 B/element accumulating, 30 for AdamW).  Run under
rocprofv3 --pmc (e.g. TCP_UTCL1_TRANSLATION_MISS_sum TCP_UTCL1_REQUEST_sum)
to see the address-translation traffic of each launch.
"""
from __future__ import annotations

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

SIZES = {"llama7b_shard": 842_301_952, "zero3_70b_shard": 1_093_750_000, "llama13b_shard_clip": 1_626_983_040}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--rounds", type=int, default=2)
    ap.add_argument("--pad-gib", type=int, nargs="*", default=[])
    args = ap.parse_args()

    import torch
    import workloads
    import fsdp_sharded_optimizer_amd as zs
    from bench import DeviceEvent, StepRig, timed

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(0x5EED)

    def line(what, n, bpe, ms):
        print(f"{what:<44} n={n:>13,} {ms:.4f} ms {bpe * n / (ms * 1e-3) / 8e12 * 100:5.1f} %", flush=True)

    # part 1: prefixes of one allocation
    N = max(SIZES.values())
    state = torch.empty(zs.state_tiled_numel(N), device=dev).uniform_(-0.1, 0.1, generator=gen)
    state.view(-1, 3, zs.STATE_TILE)[:, 2, :].abs_().mul_(1e-6)   # exp_avg_sq: small and positive
    grad = (torch.randn(N, device=dev, generator=gen) * 1e-3).to(torch.bfloat16)
    acc = torch.randn(N, device=dev, generator=gen) * 1e-3
    param = torch.empty(N, dtype=torch.bfloat16, device=dev)
    norm = torch.zeros(1, dtype=torch.float64, device=dev)
    ws = torch.empty(zs.grad_accum_norm_sq_workspace_bytes(N), dtype=torch.uint8, device=dev)
    DeviceEvent.hip()
    for r in range(args.rounds):
        for name, n in SIZES.items():
            g, a, p = grad[:n], acc[:n], param[:n]
            line(f"r{r} prefix {name} grad_accum add", n, 10, timed(lambda: zs.grad_accum(a, g, False), args.reps))
            line(f"r{r} prefix {name} grad_accum_norm_sq add", n, 10,
                 timed(lambda: zs.grad_accum_norm_sq(a, g, False, 1 / 64, norm, ws), args.reps))
            a.mul_(0.5)
            hp = zs.AdamWConfig(lr=1.5e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_scale=1 / 64,
                                max_norm=1.0, extra_norm_sq=1.85, step=1)
            line(f"r{r} prefix {name} adamw_step_tiled", n, 30,
                 timed(lambda: zs.adamw_step_tiled(hp, state, a, p, norm_sq=norm), args.reps))
    del state, grad, acc, param, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    # part 2: allocation history, on bench.py's step rigs
    W7, W70 = workloads.WORKLOADS["llama7b_shard"], workloads.WORKLOADS["zero3_70b_shard"]

    def adamw(rig, what):
        rig.two_call_step(rig.t + 1)   # the stored sum and norm of a real step in place
        rig.t += 1
        line(what, rig.n, 30, timed(lambda: zs.adamw_step_tiled(rig.hp(rig.t), rig.state, rig.acc, rig.param,
                                                                norm_sq=rig.norm), args.reps))

    def free():
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    for r in range(args.rounds):
        for arena in (False, True):
            how = "arena" if arena else "separate"
            a = StepRig(W70, dev, arena)
            adamw(a, f"r{r} {how} 70B shard, fresh")
            b = StepRig(W7, dev, arena)
            adamw(b, f"r{r} {how} 7B shard, fresh, 70B resident")
            adamw(a, f"r{r} {how} 70B shard, 7B resident")
            del a, b
            free()
            b = StepRig(W7, dev, arena)
            adamw(b, f"r{r} {how} 7B shard, re-allocated after a free")
            del b
            free()
            a = StepRig(W70, dev, arena)
            adamw(a, f"r{r} {how} 70B shard, re-allocated after the 7B freed")
            del a
            free()

    # part 3: the one-pass step behind padding
    for gib in args.pad_gib:
        pad = torch.empty(gib << 28, dtype=torch.float32, device=dev) if gib > 0 else None
        rig = StepRig(W7, dev, False)
        res = rig.time_steps(args.reps, 2)
        n = rig.n
        line(f"pad {gib} GiB: one-pass step's AdamW", n, 32, res["adamw_ms"])
        line(f"pad {gib} GiB: accumulation of 7 micro-batches", n, 66, res["accum_ms"])
        del rig, pad
        free()
    print("done", flush=True)


if __name__ == "__main__":
    main()
