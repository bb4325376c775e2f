"""The step captured in a HIP graph (torch.cuda.CUDAGraph) replays exactly.

Every entry point only enqueues kernels on the caller's stream: no
allocation, no memset, no host synchronisation.  So one rank's whole step,
two accumulations, the fused last accumulation with the norm and the
clipped AdamW update, can be captured once and replayed.  Each replay is
checked bit for bit against the same calls run eagerly on a copy of the
state, with the program's own eager work and synchronisations between
replays.  (The step counter is a kernel argument, so a captured step
replays the t it was captured with.)
"""
import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_amd as zs
from tests.parity import bits_equal, to_np

pytestmark = pytest.mark.gpu


def test_captured_step_replays_bit_exact():
    n, M, scale = 100_003, 3, 1 / 24
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    master = (torch.rand(n, generator=gen, device=dev) * 0.2 - 0.1)
    state = {"master": master, "m": torch.zeros(n, device=dev), "v": torch.zeros(n, device=dev),
             "b": torch.empty(n, dtype=torch.bfloat16, device=dev)}
    twin = {k: t.clone() for k, t in state.items()}
    grads = [torch.empty(n, dtype=torch.bfloat16, device=dev) for _ in range(M)]
    acc = torch.empty(n, device=dev)
    norm = torch.zeros(1, dtype=torch.float64, device=dev)
    ws = torch.empty(zs.grad_accum_norm_sq_workspace_bytes(n), dtype=torch.uint8, device=dev)
    hp = zs.AdamWConfig(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_scale=scale,
                        max_norm=0.5, extra_norm_sq=0.01, step=5)

    def step(s):
        for k in range(M - 1):
            zs.grad_accum(acc, grads[k], overwrite=(k == 0))
        zs.grad_accum_norm_sq(acc, grads[M - 1], False, scale, norm, ws)
        zs.adamw_step(hp, s["master"], s["m"], s["v"], acc, s["b"], norm_sq=norm)

    def fresh_grads(r):
        for k, g in enumerate(grads):
            g.copy_((torch.randn(n, generator=gen, device=dev) * (1e-2 * (r + 1) * (k + 1))).to(torch.bfloat16))

    fresh_grads(0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # warm-up outside the capture
        step(twin)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for k in state:                     # both states equal again before the replays
        state[k].copy_(twin[k])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(state)
    torch.cuda.synchronize()
    for r in range(4):
        fresh_grads(r)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {k: to_np(t) for k, t in state.items()}
        norm_graph = norm.item()
        step(twin)                      # the same step, eagerly, on the twin state
        torch.cuda.synchronize()
        assert norm.item() == norm_graph, r
        for k in state:
            assert bits_equal(got[k], to_np(twin[k])), (r, k)
        _ = (acc * 2).sum().item()      # unrelated eager work between replays


def test_one_graph_replays_every_step_with_device_scalars():
    """The scalars of each step (step counter, a learning-rate schedule, a
    changing clip input) are copied from pinned host memory into device
    memory by a copy captured in the graph, and adamw_step_dev reads them
    there: one capture replays steps 1..6, each bit-identical to an eager
    adamw_step with that step's hyperparameters.  Also checked: eager
    adamw_step_dev equals adamw_step."""
    n, M, scale = 100_003, 2, 1 / 16
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    state = {"master": torch.rand(n, generator=gen, device=dev) * 0.2 - 0.1, "m": torch.zeros(n, device=dev),
             "v": torch.zeros(n, device=dev), "b": torch.empty(n, dtype=torch.bfloat16, device=dev)}
    twin = {k: t.clone() for k, t in state.items()}
    grads = [torch.empty(n, dtype=torch.bfloat16, device=dev) for _ in range(M)]
    acc = torch.empty(n, device=dev)
    norm = torch.zeros(1, dtype=torch.float64, device=dev)
    ws = torch.empty(zs.grad_accum_norm_sq_workspace_bytes(n), dtype=torch.uint8, device=dev)
    nbytes = len(zs.scalars_bytes(zs.AdamWConfig(lr=1e-3)))
    host_sc = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dev_sc = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    def hp_at(t):   # warm-up then cosine-like decay; the clip input changes every step
        lr = 3e-4 * min(1.0, t / 3) * (0.5 + 0.5 * np.cos(t / 7))
        return zs.AdamWConfig(lr=lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_scale=scale,
                              max_norm=0.5, extra_norm_sq=0.01 * t, step=t)

    def grads_for(t):
        for k, g in enumerate(grads):
            g.copy_((torch.randn(n, generator=gen, device=dev) * (1e-2 * t * (k + 1))).to(torch.bfloat16))

    def front():
        zs.grad_accum(acc, grads[0], overwrite=True)
        zs.grad_accum_norm_sq(acc, grads[1], False, scale, norm, ws)

    def captured_step(s):
        front()
        dev_sc.copy_(host_sc, non_blocking=True)
        zs.adamw_step_dev(dev_sc, s["master"], s["m"], s["v"], acc, s["b"], norm_sq=norm)

    # eager adamw_step_dev equals adamw_step (scalars copied synchronously)
    grads_for(1)
    host_sc.numpy()[:] = np.frombuffer(zs.scalars_bytes(hp_at(1)), dtype=np.uint8)
    a = {k: t.clone() for k, t in state.items()}
    front()
    dev_sc.copy_(host_sc)
    zs.adamw_step_dev(dev_sc, a["master"], a["m"], a["v"], acc, a["b"], norm_sq=norm)
    front()
    zs.adamw_step(hp_at(1), twin["master"], twin["m"], twin["v"], acc, twin["b"], norm_sq=norm)
    torch.cuda.synchronize()
    for k in state:
        assert bits_equal(to_np(a[k]), to_np(twin[k])), k
    for k in state:
        twin[k].copy_(state[k])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture, on scratch state
        captured_step(a)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured_step(state)
    torch.cuda.synchronize()
    for t in range(1, 7):
        grads_for(t)
        host_sc.numpy()[:] = np.frombuffer(zs.scalars_bytes(hp_at(t)), dtype=np.uint8)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {k: to_np(v) for k, v in state.items()}
        front()
        zs.adamw_step(hp_at(t), twin["master"], twin["m"], twin["v"], acc, twin["b"], norm_sq=norm)
        torch.cuda.synchronize()
        for k in state:
            assert bits_equal(got[k], to_np(twin[k])), (t, k)
        _ = (acc * 3).sum().item()   # unrelated eager work between replays
