"""bench.py's timed configuration computes what the oracle-checked path
computes.  Its step rig holds a rank's streamed buffers as views of one
contiguous block (DeviceArena); the same rig on separately allocated
buffers (the allocation the full-size oracle parity tests use) must give
the same bits at full size: two steps of the one-pass schedule bench.py
times, then one of the two-call schedule, on the Llama-7B and the 70B
ZeRO-3 shards (the latter clipped, on its single bf16 micro-batch)."""
import pytest
import torch

import workloads
from bench import StepRig

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def same_bits(x: torch.Tensor, y: torch.Tensor) -> bool:
    w = torch.int32 if x.element_size() == 4 else torch.int16
    return torch.equal(x.view(w), y.view(w))


@pytest.mark.parametrize("name", ["llama7b_shard", "zero3_70b_shard"])
def test_bench_rig_in_one_block_is_bit_identical(name):
    print(f"bench rig in one block against separate buffers: {name}", flush=True)
    w = workloads.WORKLOADS[name]
    dev = torch.device("cuda", 0)
    a = StepRig(w, dev, True)
    b = StepRig(w, dev, False)
    assert a.arena is not None and a.arena.contiguous and b.arena is None
    for rig in (a, b):
        rig.step(1)
        rig.step(2)
        rig.two_call_step(3)
    torch.cuda.synchronize()
    assert same_bits(a.state, b.state)
    assert same_bits(a.acc, b.acc)
    if w.bf16_param:
        assert same_bits(a.param, b.param)
    assert a.norm.item() == b.norm.item() and torch.isfinite(a.norm).item()
    for ga, gb in zip(a.grads, b.grads):
        assert same_bits(ga, gb)                  # the same seeded draws in both layouts
