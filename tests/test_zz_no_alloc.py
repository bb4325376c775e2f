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
