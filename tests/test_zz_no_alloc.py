"""grad_accum_norm_sq_noalloc: the fused last-micro-batch accumulation and
norm with its partials in the library's static device scratch, for callers
that cannot allocate.  Checked through the C ABI against the workspace
entry point grad_accum_norm_sq on the same inputs: the accumulator bit for
bit and the squared norm bit for bit (same kernels, same partial layout),
the norm also within the oracle's 1e-5 where the oracle runs.  Calls follow
each other on one stream, each smaller than the one before it, so a later
call reads the scratch a larger call left behind."""
import math

import numpy as np
import pytest
import torch

import oracle
import fsdp_sharded_optimizer_amd as zs
from fsdp_sharded_optimizer_amd import _binding as B
from tests.parity import NORM_TOL, to_np

pytestmark = pytest.mark.gpu


def _inputs(n, bf16, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    acc = torch.randn(n, generator=gen, device="cuda") * 1e-3
    g = torch.randn(n, generator=gen, device="cuda") * 1e-3
    return acc, (g.to(torch.bfloat16) if bf16 else g)


def _both(n, bf16, overwrite, scale, seed):
    """(acc, norm) from the workspace entry point and from the no-alloc one."""
    acc, g = _inputs(n, bf16, seed)
    acc_ws, acc_na = acc.clone(), acc.clone()
    del acc
    norm_ws = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    norm_na = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    zs.grad_accum_norm_sq(acc_ws, g, overwrite, scale, norm_ws)
    L = B.lib()
    rc = L.grad_accum_norm_sq_noalloc(acc_na.data_ptr() if n else None, g.data_ptr() if n else None,
                                      B.ZS_BF16 if bf16 else B.ZS_F32, n, 1 if overwrite else 0, scale,
                                      norm_na.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, (rc, L.zs_strerror(rc))
    torch.cuda.synchronize()
    return acc_ws, acc_na, norm_ws.item(), norm_na.item(), g


CASES = [  # (n, bf16 gradient, overwrite): each call smaller than the one before
    (B.NOALLOC_MAX_ELEMS, True, False),     # the largest call: its partials and stage fill the scratch
    (1_093_750_000, True, True),            # the 70B ZeRO-3 shard's overwriting form (a partial per 1024)
    (5_000_011, False, False),              # fp32 gradient, ragged tail
    (70_001, True, True),
    (257, False, True),
    (1, True, False),
    (0, True, False),
]


def test_noalloc_matches_the_workspace_entry_point_over_calls_of_falling_size():
    for k, (n, bf16, overwrite) in enumerate(CASES):
        print(f"noalloc call {k}: n={n} bf16={bf16} overwrite={overwrite}", flush=True)
        scale = 1 / 64 if n > 10_000_000 else 1 / 8
        acc_ws, acc_na, s_ws, s_na, g = _both(n, bf16, overwrite, scale, seed=100 + k)
        assert torch.equal(acc_ws.view(torch.int32), acc_na.view(torch.int32)), (n, "accumulator")
        assert s_ws == s_na, (n, s_ws, s_na)
        if n == 0:
            assert s_na == 0.0
        elif n <= 10_000_000:   # the oracle on the same seeded inputs: accumulator and norm
            acc0, g0 = _inputs(n, bf16, seed=100 + k)
            ref = to_np(acc0)
            oracle.grad_accum(ref, to_np(g0), oracle.BF16 if bf16 else oracle.F32, overwrite=overwrite)
            assert np.array_equal(ref.view(np.uint32), to_np(acc_na).view(np.uint32))
            S = oracle.grad_norm_sq(ref, scale)
            assert abs(math.sqrt(s_na) - math.sqrt(S)) <= NORM_TOL * math.sqrt(S), (n, s_na, S)
        del acc_ws, acc_na, g
        torch.cuda.empty_cache()


def test_noalloc_binding_and_limits():
    n = 4099
    acc, g = _inputs(n, True, seed=7)
    out = torch.zeros(1, dtype=torch.float64, device="cuda")
    zs.grad_accum_norm_sq_noalloc(acc, g, False, 1 / 8, out)
    ref_acc, _ = _inputs(n, True, seed=7)
    ref_out = torch.zeros(1, dtype=torch.float64, device="cuda")
    zs.grad_accum_norm_sq(ref_acc, g, False, 1 / 8, ref_out)
    torch.cuda.synchronize()
    assert torch.equal(acc.view(torch.int32), ref_acc.view(torch.int32)) and out.item() == ref_out.item()
    L = B.lib()
    # beyond the scratch: rejected before any device call
    assert L.grad_accum_norm_sq_noalloc(acc.data_ptr(), g.data_ptr(), B.ZS_BF16, B.NOALLOC_MAX_ELEMS + 1, 0,
                                        1.0, out.data_ptr(), None) == B.ZS_EINVAL
    # the output overlapping the accumulator: rejected by the shared checks
    assert L.grad_accum_norm_sq_noalloc(acc.data_ptr(), g.data_ptr(), B.ZS_BF16, n, 0, 1.0,
                                        acc.data_ptr() + 16, None) == B.ZS_EOVERLAP


def test_noalloc_step_captured_in_a_graph():
    """The use it is for: a rank's step with no workspace anywhere (two
    accumulations, the fused last one through grad_accum_norm_sq_noalloc,
    the clipped tiled AdamW) captured once in a HIP graph after a first
    eager call on the device, replayed with fresh gradients; every replay
    bit-identical to the same step run eagerly on a twin state with the
    workspace entry point, with eager work between replays."""
    n, M, scale = 300_007, 3, 1 / 24
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(19)
    master = torch.rand(n, generator=gen, device=dev) * 0.2 - 0.1
    states = []
    for _ in range(2):
        st = torch.empty(zs.state_tiled_numel(n), device=dev)
        zs.state_tile(master, None, None, st)
        states.append({"state": st, "b": torch.empty(n, dtype=torch.bfloat16, device=dev),
                       "acc": torch.empty(n, device=dev), "norm": torch.zeros(1, dtype=torch.float64, device=dev)})
    graph_side, eager_side = states
    ws = torch.empty(zs.grad_accum_norm_sq_workspace_bytes(n), dtype=torch.uint8, device=dev)
    grads = [torch.empty(n, dtype=torch.bfloat16, device=dev) for _ in range(M)]
    hp = zs.AdamWConfig(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_scale=scale,
                        max_norm=0.5, extra_norm_sq=0.01, step=3)

    def step(s, noalloc):
        for k in range(M - 1):
            zs.grad_accum(s["acc"], grads[k], overwrite=(k == 0))
        if noalloc:
            zs.grad_accum_norm_sq_noalloc(s["acc"], grads[M - 1], False, scale, s["norm"])
        else:
            zs.grad_accum_norm_sq(s["acc"], grads[M - 1], False, scale, s["norm"], ws)
        zs.adamw_step_tiled(hp, s["state"], s["acc"], s["b"], norm_sq=s["norm"])

    def fresh(r):
        for k, g in enumerate(grads):
            g.copy_((torch.randn(n, generator=gen, device=dev) * (1e-2 * (r + 1) * (k + 1))).to(torch.bfloat16))

    fresh(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # the first call on the device, and torch's warm-up, outside the capture
        step(graph_side, True)
        step(eager_side, False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(graph_side, True)
    torch.cuda.synchronize()
    for r in range(1, 4):
        print(f"noalloc graph replay {r}", flush=True)
        fresh(r)
        torch.cuda.synchronize()
        graph.replay()
        step(eager_side, False)
        torch.cuda.synchronize()
        assert graph_side["norm"].item() == eager_side["norm"].item(), r
        for k in ("state", "b", "acc"):
            a, b = graph_side[k], eager_side[k]
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), (r, k)
        _ = (eager_side["acc"] * 2).sum().item()   # unrelated eager work between replays
