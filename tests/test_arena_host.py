"""DeviceArena's and ShardOptimizer's sizing on the host (no GPU needed)."""
import pytest
import torch

import fsdp_sharded_optimizer_amd as zs
from fsdp_sharded_optimizer_amd.arena import ALIGN


def test_size_rounds_each_part_to_the_alignment():
    assert ALIGN == 2 << 20
    assert zs.DeviceArena.size([]) == ALIGN
    assert zs.DeviceArena.size([(0, torch.float32)]) == ALIGN
    assert zs.DeviceArena.size([(1, torch.uint8)]) == ALIGN
    assert zs.DeviceArena.size([(ALIGN // 4, torch.float32)]) == ALIGN
    assert zs.DeviceArena.size([(ALIGN // 4 + 1, torch.float32)]) == 2 * ALIGN
    assert zs.DeviceArena.size([(ALIGN // 2, torch.bfloat16), (1, torch.float64), (3, torch.uint8)]) == 3 * ALIGN
    assert zs.DeviceArena.size([(0, torch.float32), (5, torch.float32)]) == ALIGN


@pytest.mark.parametrize("layout", ["tiled", "split"])
def test_shard_optimizer_arena_parts(layout):
    n = 842_301_952
    parts = zs.ShardOptimizer.arena_parts(n, layout)
    f32 = torch.float32
    if layout == "tiled":
        assert parts[0] == (zs.state_tiled_numel(n), f32)
        rest = parts[1:]
    else:
        assert parts[:2] == [(n, f32), (n, f32)]
        rest = parts[2:]
    assert rest == [(n, f32)]                  # the accumulator
    state_bytes = (zs.state_tiled_numel(n) if layout == "tiled" else 2 * n) * 4
    assert zs.DeviceArena.size(parts) >= state_bytes + 4 * n
    assert zs.DeviceArena.size(parts) < state_bytes + 4 * n + len(parts) * ALIGN


def test_arena_needs_a_gpu_device():
    with pytest.raises(TypeError):
        zs.DeviceArena(ALIGN, "cpu")
