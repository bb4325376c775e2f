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


def test_every_other_entry_point_replays_bit_exact():
    """flat_pack (bit copy with padding; widening), grad_reduce_chunks,
    grad_norm_sq, adamw_step_no_master, adam_update, flat_unpack (re-cast),
    flat_apply_update (bf16 and fp32 tensors), adamw_step_tiled on a tiled
    state, state_untile, state_tile, adam_update_tiled and
    adamw_step_no_master_tiled on tiled moments, moments_untile and
    moments_tile captured in one graph and replayed
    four times with fresh inputs, each replay bit-identical to the same
    calls made eagerly on a twin state."""
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    sizes, world = [20_001, 7, 30_000], 8
    T = sum(sizes)
    _, _, _, padded = zs.zero_shard_range(T, world, 0)
    params = [torch.empty(k, dtype=torch.bfloat16, device=dev) for k in sizes]   # shared inputs
    chunks = [torch.empty(T, dtype=torch.bfloat16, device=dev) for _ in range(3)]
    scale = 1 / 24
    hp = zs.AdamWConfig(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_scale=scale,
                        max_norm=0.5, extra_norm_sq=0.01, step=4)
    hu = zs.AdamWConfig(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0, grad_scale=scale,
                        max_norm=0.5, extra_norm_sq=0.01, step=4)

    def side():
        return {"flat": torch.empty(padded, dtype=torch.bfloat16, device=dev),
                "flat32": torch.empty(padded, device=dev),
                "acc": torch.empty(T, device=dev),
                "norm": torch.zeros(1, dtype=torch.float64, device=dev),
                "ws": torch.empty(max(zs.grad_norm_sq_workspace_bytes(T), 8), dtype=torch.uint8, device=dev),
                "p16": (torch.rand(T, generator=gen, device=dev) * 0.2 - 0.1).to(torch.bfloat16),
                "m1": torch.zeros(T, device=dev), "v1": torch.zeros(T, device=dev),
                "m2": torch.zeros(T, device=dev), "v2": torch.zeros(T, device=dev),
                "upd": torch.empty(T, device=dev),
                "outs": [torch.empty(k, dtype=torch.bfloat16, device=dev) for k in sizes],
                "tb": [(torch.rand(k, generator=gen, device=dev) - 0.5).to(torch.bfloat16) for k in sizes],
                "tf": [torch.rand(k, generator=gen, device=dev) - 0.5 for k in sizes],
                "state": tiled(torch.rand(T, generator=gen, device=dev) * 0.2 - 0.1),
                "bt": torch.empty(T, dtype=torch.bfloat16, device=dev),
                "um": torch.empty(T, device=dev), "uv": torch.empty(T, device=dev),
                "state2": torch.empty(zs.state_tiled_numel(T), device=dev),
                "mo": torch.zeros(zs.moments_tiled_numel(T), device=dev),
                "mo2": torch.zeros(zs.moments_tiled_numel(T), device=dev),
                "mo3": torch.empty(zs.moments_tiled_numel(T), device=dev),
                "upd2": torch.empty(T, device=dev), "um2": torch.empty(T, device=dev),
                "p16b": (torch.rand(T, generator=gen, device=dev) * 0.2 - 0.1).to(torch.bfloat16)}

    def tiled(master):
        st = torch.empty(zs.state_tiled_numel(T), device=dev)
        zs.state_tile(master, None, None, st)
        return st

    a = side()
    b = {k: ([t.clone() for t in v] if isinstance(v, list) else v.clone()) for k, v in a.items()}

    def calls(s):
        zs.flat_pack(params, s["flat"], padded)
        zs.flat_pack(params, s["flat32"], padded)
        zs.grad_reduce_chunks(s["acc"], chunks, True)
        zs.grad_norm_sq(s["acc"], scale, s["norm"], s["ws"])
        zs.adamw_step_no_master(hp, s["p16"], s["m1"], s["v1"], s["acc"], norm_sq=s["norm"])
        zs.adam_update(hu, s["m2"], s["v2"], s["acc"], s["upd"], norm_sq=s["norm"])
        zs.flat_unpack(s["flat32"], s["outs"])
        zs.flat_apply_update(s["upd"], s["tb"])
        zs.flat_apply_update(s["upd"], s["tf"])
        zs.adamw_step_tiled(hp, s["state"], s["acc"], s["bt"], norm_sq=s["norm"])
        zs.state_untile(s["state"], None, s["um"], s["uv"], n=T)
        zs.state_tile(s["m1"], None, s["v1"], s["state2"])
        zs.adam_update_tiled(hu, s["mo"], s["acc"], s["upd2"], norm_sq=s["norm"])
        zs.adamw_step_no_master_tiled(hp, s["p16b"], s["mo2"], s["acc"], norm_sq=s["norm"])
        zs.moments_untile(s["mo"], s["um2"], None, n=T)
        zs.moments_tile(s["m2"], s["v2"], s["mo3"])

    def fresh(r):
        for p in params:
            p.copy_((torch.rand(p.numel(), generator=gen, device=dev) - 0.5) * (r + 1))
        for c in chunks:
            c.copy_(torch.randn(T, generator=gen, device=dev) * 1e-2 * (r + 1))

    def flat_bits(s):
        out = {}
        for k, v in s.items():
            if k == "ws":
                continue
            out[k] = [to_np(t) for t in v] if isinstance(v, list) else to_np(v)
        return out

    fresh(0)
    torch.cuda.synchronize()
    warm = torch.cuda.Stream()
    warm.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(warm):       # warm-up outside the capture, on the twin
        calls(b)
    torch.cuda.current_stream().wait_stream(warm)
    torch.cuda.synchronize()
    for k, v in a.items():              # both sides equal again before the replays
        if isinstance(v, list):
            for x, y in zip(v, b[k]):
                x.copy_(y)
        else:
            v.copy_(b[k])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls(a)
    torch.cuda.synchronize()
    for r in range(4):
        print(f"  replay {r}", flush=True)
        fresh(r + 1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = flat_bits(a)
        calls(b)                        # the same calls, eagerly, on the twin
        torch.cuda.synchronize()
        want = flat_bits(b)
        for k in want:
            if isinstance(want[k], list):
                assert all(bits_equal(x, y) for x, y in zip(got[k], want[k])), (r, k)
            else:
                assert bits_equal(got[k], want[k]), (r, k)
        assert not got["flat"][T:].any() and not got["flat32"][T:].view(np.uint32).any()   # padding zero
        _ = (a["acc"] * 2).sum().item()  # unrelated eager work between replays
