"""DeviceArena (one contiguous block of device memory for a rank's buffers)
and ShardOptimizer on it: the views' placement and lifetime, and the same
step results bit for bit as on separately allocated buffers."""
import gc
import weakref

import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_amd as zs
from fsdp_sharded_optimizer_amd.arena import ALIGN, pooled_blocks
from tests.parity import bits_equal, from_np, to_np

pytestmark = pytest.mark.gpu


def test_views_aligned_disjoint_and_typed():
    print("arena views", flush=True)
    parts = [(1000, torch.float32), (3, torch.bfloat16), (0, torch.float32), (ALIGN // 4 + 1, torch.float32),
             (1, torch.float64), (77, torch.uint8)]
    arena = zs.DeviceArena(zs.DeviceArena.size(parts), "cuda")
    assert arena.contiguous                       # a small block on a fresh device
    assert arena.device == torch.device("cuda", torch.cuda.current_device())
    views = [arena.take(n, dt) for n, dt in parts]
    spans = []
    for v, (n, dt) in zip(views, parts):
        assert v.dtype == dt and v.shape == (n,) and v.is_contiguous() and v.device == arena.device
        if n:
            assert (v.data_ptr() - arena.ptr) % ALIGN == 0
            spans.append((v.data_ptr(), v.data_ptr() + n * v.element_size()))
    assert arena.used == arena.nbytes == 6 * ALIGN   # the fourth part spans two alignment units, the empty one none
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 <= b0
    assert spans[-1][1] <= arena.ptr + arena.nbytes
    # every view holds what is written to it, after all were written
    for k, v in enumerate(views):
        if v.numel():
            v.copy_(torch.arange(v.numel(), device="cuda").to(v.dtype) + k)
    torch.cuda.synchronize()
    for k, v in enumerate(views):
        if v.numel():
            want = (torch.arange(v.numel()).to(v.dtype) + k)
            assert torch.equal(v.cpu(), want)


def test_views_keep_the_block_alive_and_the_pool_reuses_it():
    print("arena lifetime and pool", flush=True)
    arena = zs.DeviceArena(2 * ALIGN, "cuda")
    assert arena.contiguous
    alive = weakref.ref(arena)
    block = (arena.capacity, arena.ptr)
    a = arena.take(100, torch.float32)
    b = arena.take(100, torch.bfloat16)
    del arena
    gc.collect()
    assert alive() is not None                    # the views hold the block
    a.fill_(1.5)
    b.fill_(2.5)
    torch.cuda.synchronize()
    assert a.sum().item() == 150.0 and b.float().sum().item() == 250.0
    del a
    gc.collect()
    assert alive() is not None and block not in pooled_blocks()
    del b
    gc.collect()
    assert alive() is None                        # gone with its last view
    assert block in pooled_blocks()               # its block kept for reuse, not freed
    expect = min(b for b in pooled_blocks() if b[0] >= ALIGN)
    again = zs.DeviceArena(ALIGN, "cuda")          # takes the smallest pooled block that holds it
    held = (again.capacity, again.ptr)
    assert again.contiguous and held == expect and held not in pooled_blocks()
    v = again.take(ALIGN // 4, torch.float32)
    v.fill_(3.0)
    torch.cuda.synchronize()
    assert v.sum().item() == 3.0 * (ALIGN // 4)
    del again, v
    gc.collect()
    assert held in pooled_blocks()


def test_take_rejects():
    print("arena rejections", flush=True)
    arena = zs.DeviceArena(ALIGN, "cuda")
    with pytest.raises(TypeError):
        arena.take(4, torch.complex64)
    with pytest.raises(ValueError):
        arena.take(-1, torch.float32)
    with pytest.raises(ValueError):
        arena.take(ALIGN // 4 + 1, torch.float32)
    assert arena.used == 0                        # a rejected take takes nothing
    arena.take(ALIGN // 4, torch.float32)
    with pytest.raises(ValueError):
        arena.take(1, torch.uint8)
    with pytest.raises(ValueError):
        zs.DeviceArena(0, "cuda")


@pytest.mark.parametrize("layout", ["tiled", "split"])
@pytest.mark.parametrize("last_grad", [False, True])
def test_shard_optimizer_in_an_arena_is_bit_identical(layout, last_grad):
    print(f"ShardOptimizer in an arena layout={layout} last_grad={last_grad}", flush=True)
    n, M = 300_007, 3
    rng = np.random.default_rng(23)
    p0 = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    grads = [[torch.from_numpy(rng.standard_normal(n).astype(np.float32) * 0.02).to(torch.bfloat16)
              for _ in range(M)] for _ in range(3)]
    parts = zs.ShardOptimizer.arena_parts(n, layout) + [(n, torch.bfloat16)] * (M + 1)
    arena = zs.DeviceArena(zs.DeviceArena.size(parts), "cuda")
    kw = dict(lr=3e-4, betas=(0.9, 0.95), weight_decay=0.1, grad_scale=1 / 16, max_norm=1.0, layout=layout)
    opts, params = [], []
    for in_arena in (False, True):
        master = from_np(p0.copy())
        if in_arena:
            param = arena.take(n, torch.bfloat16)
            opt = zs.ShardOptimizer(master, param_bf16=param, arena=arena, **kw)
            slots = [arena.take(n, torch.bfloat16) for _ in range(M)]
            for buf in (opt.acc, opt.state if layout == "tiled" else opt._split["exp_avg"], param, *slots):
                assert arena.ptr <= buf.data_ptr() < arena.ptr + arena.nbytes
            for buf in (opt.norm_sq, opt.workspace):   # the norm's scattered partial writes stay outside
                assert not arena.ptr <= buf.data_ptr() < arena.ptr + arena.nbytes
        else:
            param = torch.empty(n, dtype=torch.bfloat16, device="cuda")
            opt = zs.ShardOptimizer(master, param_bf16=param, **kw)
            slots = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(M)]
        opts.append((opt, slots))
        params.append(param)
    assert arena.used == arena.nbytes
    for t, step_grads in enumerate(grads, 1):
        for opt, slots in opts:
            for s, g in zip(slots, step_grads):
                s.copy_(g)
            for k, s in enumerate(slots):
                if not (last_grad and k == M - 1):
                    opt.accumulate(s, last=(not last_grad) and k == M - 1)
            opt.step(extra_norm_sq=0.75, last_grad=slots[-1] if last_grad else None)
        torch.cuda.synchronize()
        a, b = opts[0][0], opts[1][0]
        assert a.t == b.t == t
        for name in ("master", "exp_avg", "exp_avg_sq"):
            assert bits_equal(to_np(getattr(a, name)), to_np(getattr(b, name))), (t, name)
        assert bits_equal(to_np(a.acc), to_np(b.acc))
        assert a.norm_sq.item() == b.norm_sq.item()
        assert torch.equal(params[0].view(torch.int16), params[1].view(torch.int16))


@pytest.mark.parametrize("layout", ["tiled", "split"])
def test_captured_step_in_an_arena_replays_like_eager_steps(layout):
    """ShardOptimizer.capture on an optimizer whose state, accumulator,
    gradients and bf16 parameter are views of one contiguous block: four
    replays with new gradients, bit-identical to the same steps taken
    eagerly on separately allocated buffers."""
    print(f"capture in an arena layout={layout}", flush=True)
    n, M = 70_001, 3
    gen = torch.Generator(device="cuda")
    gen.manual_seed(47)
    p0 = torch.rand(n, generator=gen, device="cuda") * 0.2 - 0.1
    kw = dict(lr=3e-4, betas=(0.9, 0.95), weight_decay=0.1, grad_scale=1 / 24, max_norm=0.5, layout=layout)
    parts = zs.ShardOptimizer.arena_parts(n, layout) + [(n, torch.bfloat16)] * (M + 1)
    arena = zs.DeviceArena(zs.DeviceArena.size(parts), "cuda")
    a = zs.ShardOptimizer(p0.clone(), param_bf16=arena.take(n, torch.bfloat16), arena=arena, **kw)
    grads = [arena.take(n, torch.bfloat16) for _ in range(M)]
    b = zs.ShardOptimizer(p0.clone(), param_bf16=torch.empty(n, dtype=torch.bfloat16, device="cuda"), **kw)
    cap = a.capture(grads, extra_norm_sq=0.02)
    torch.cuda.synchronize()
    assert a.t == 0 and bits_equal(to_np(a.master), to_np(p0))
    for t in range(1, 5):
        for k, g in enumerate(grads):
            g.copy_((torch.randn(n, generator=gen, device="cuda") * 1e-2 * (k + t)).to(torch.bfloat16))
        cap.replay()
        for g in grads[:M - 1]:
            b.accumulate(g)
        b.step(extra_norm_sq=0.02, last_grad=grads[-1])
        torch.cuda.synchronize()
        assert a.t == b.t == t
        for name in ("master", "exp_avg", "exp_avg_sq", "param_bf16", "acc"):
            assert bits_equal(to_np(getattr(a, name)), to_np(getattr(b, name))), (t, name)
        assert a.norm_sq.item() == b.norm_sq.item()
        _ = (b.acc * 2).sum().item()   # unrelated eager work between replays
