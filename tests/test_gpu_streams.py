"""Calls run on the stream they are given.

A side stream is held back by a bounded spin (torch.cuda._sleep) before a
call is enqueued on it; the default stream, which does not wait for the
side stream, then reads the output.  If the library launched on the stream
it was given, the output is still untouched at that point; once the side
stream has drained it holds the result.  A library that ignored the stream
argument (and launched on the default stream) would fail the first check.
"""
import numpy as np
import pytest
import torch

import oracle
import fsdp_sharded_optimizer_amd as zs
from tests.parity import bits_equal, from_np, to_np

pytestmark = pytest.mark.gpu
SPIN = int(4e8)   # GPU clock cycles: ~0.1-0.2 s, far longer than the host reads below


def _held_side_stream():
    if not hasattr(torch.cuda, "_sleep"):
        pytest.skip("torch.cuda._sleep is not available")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        torch.cuda._sleep(SPIN)
    return s


def test_calls_run_on_the_stream_they_are_given():
    print("explicit streams", flush=True)
    n = 1 << 20
    rng = np.random.default_rng(5)
    g_np = oracle.bf16_rne((rng.standard_normal(n) * 1e-2).astype(np.float32))
    g = from_np(g_np, bf16=True)
    acc = torch.zeros(n, device="cuda")
    srcs = [from_np(oracle.bf16_rne(rng.uniform(-1, 1, k).astype(np.float32)), bf16=True) for k in (1000, 5)]
    flat = torch.zeros(1008, dtype=torch.bfloat16, device="cuda")
    master = torch.zeros(n, device="cuda")
    m = torch.zeros(n, device="cuda")
    v = torch.zeros(n, device="cuda")
    torch.cuda.synchronize()

    s = _held_side_stream()
    zs.grad_accum(acc, g, overwrite=True, stream=s)
    zs.flat_pack(srcs, flat, 1008, stream=s)
    hp = zs.AdamWConfig(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, grad_scale=1.0, step=1)
    zs.adamw_step(hp, master, m, v, acc, stream=s)
    early = [to_np(t) for t in (acc, flat, master)]       # the default stream does not wait for s
    assert not early[0].any() and not early[1].any() and not early[2].any(), "a call did not wait on its stream"

    s.synchronize()
    assert bits_equal(to_np(acc), oracle.bf16_widen(g_np))
    assert bits_equal(to_np(flat), oracle.flat_pack([to_np(x) for x in srcs], oracle.BF16, oracle.BF16, 1008))
    p_ref, m_ref, v_ref = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)
    H = oracle.make_hp(1e-3, 0.9, 0.999, 1e-8, 0.0, 1.0, 0.0, 0.0, 1)
    assert oracle.adamw_step(H, p_ref, m_ref, v_ref, oracle.bf16_widen(g_np)) == 0
    assert bits_equal(to_np(master), p_ref) and bits_equal(to_np(m), m_ref) and bits_equal(to_np(v), v_ref)
