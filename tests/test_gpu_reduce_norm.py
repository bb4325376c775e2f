"""grad_reduce_chunks_norm_sq on the GPU against the oracle.

The accumulator is the oracle's left fold of the chunks, bit for bit; the
squared norm is within the tolerance of the fused norms (binary64 partials)
of the oracle's norm of that accumulator, and bit-reproducible.  Sizes span
several 512-element partial tiles with ragged tails; counts cover one pass,
a full pass of 16 and a second pass (19); buffers aligned and not.
"""
import numpy as np
import pytest
import torch

import oracle
import fsdp_sharded_optimizer_amd as zs
from tests.parity import NORM_TOL, bits_equal, from_np, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n,count,overwrite,offset", [
    (1, 1, True, 0), (511, 3, True, 0), (512, 2, False, 0), (5003, 8, True, 0), (3 * 8192 + 77, 16, False, 0),
    (20_001, 19, True, 0), (20_001, 19, False, 0), (4099, 5, True, 1), (4099, 17, False, 3), (1 << 16, 8, True, 0)])
def test_reduce_chunks_norm_sq_matches_the_oracle(dtype, n, count, overwrite, offset):
    print(f"grad_reduce_chunks_norm_sq {dtype} n={n} count={count} overwrite={overwrite} offset={offset}", flush=True)
    rng = np.random.default_rng(n + 7 * count + offset)
    scale = 1.0 / (8 * count)
    odt = oracle.BF16 if dtype == "bf16" else oracle.F32
    chunks_np = []
    for k in range(count):
        x = (rng.standard_normal(n) * 0.05 * (k + 1)).astype(np.float32)
        chunks_np.append(oracle.bf16_rne(x) if dtype == "bf16" else x)
    acc0 = rng.uniform(-1, 1, n).astype(np.float32)
    base = from_np(np.concatenate([np.zeros(offset, np.float32), acc0]))
    acc = base[offset:]                                   # offset > 0: not 16-byte aligned (element path)
    chunks = [from_np(c, bf16=(dtype == "bf16")) for c in chunks_np]
    out = torch.full((1,), -1.0, dtype=torch.float64, device="cuda")
    zs.grad_reduce_chunks_norm_sq(acc, chunks, overwrite, scale, out)
    torch.cuda.synchronize()
    ref = acc0.copy()
    for k, c in enumerate(chunks_np):
        oracle.grad_accum(ref, c, odt, overwrite=(overwrite and k == 0))
    assert bits_equal(to_np(acc), ref)
    S = oracle.grad_norm_sq(ref, scale)
    got = out.item()
    assert abs(got - S) <= NORM_TOL * S, (got, S)
    # bit-reproducible: the same call on the same inputs gives the same bits
    acc.copy_(from_np(acc0))
    out2 = torch.zeros(1, dtype=torch.float64, device="cuda")
    zs.grad_reduce_chunks_norm_sq(acc, chunks, overwrite, scale, out2)
    assert out2.item() == got and bits_equal(to_np(acc), ref)


def test_reduce_chunks_norm_sq_empty_and_special_values():
    """n == 0 writes a zero norm; -0.0 survives an overwriting fold of -0.0
    chunks; a non-finite chunk element makes the norm non-finite."""
    out = torch.full((1,), 5.0, dtype=torch.float64, device="cuda")
    empty = torch.empty(0, device="cuda")
    zs.grad_reduce_chunks_norm_sq(empty, [torch.empty(0, dtype=torch.bfloat16, device="cuda")], True, 1.0, out)
    torch.cuda.synchronize()
    assert out.item() == 0.0
    n = 1000
    acc = torch.ones(n, device="cuda")
    neg0 = torch.full((n,), -0.0, device="cuda")
    zs.grad_reduce_chunks_norm_sq(acc, [neg0, neg0], True, 1.0, out)
    torch.cuda.synchronize()
    assert out.item() == 0.0 and bool(torch.signbit(acc).all())
    bad = torch.zeros(n, device="cuda")
    bad[n - 3] = float("inf")
    zs.grad_reduce_chunks_norm_sq(acc, [neg0, bad], True, 1.0, out)
    torch.cuda.synchronize()
    assert not np.isfinite(out.item())
