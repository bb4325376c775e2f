"""MI355X-native per-rank ZeRO/FSDP optimizer step (libzshard).

The Python names mirror the C ABI in include/zshard.h:

    zero_shard_range(total, world, rank) -> (chunk, start, end, padded_total)
    flat_pack(src_tensors, flat, padded_total=None)
    flat_unpack(flat, dst_tensors)
    grad_accum(acc, grad, overwrite)
    grad_reduce_chunks(acc, chunks, overwrite)
    grad_reduce_chunks_norm_sq(acc, chunks, overwrite, grad_scale, out, workspace=None)
    grad_accum_norm_sq(acc, grad, overwrite, grad_scale, out, workspace=None)
    grad_accum_norm_sq_noalloc(acc, grad, overwrite, grad_scale, out)   partials in a static device scratch
    grad_norm_sq(grad, grad_scale, out, workspace=None)
    grad_sum_norm_sq(acc, grad, overwrite, grad_scale, out, workspace=None)   grad_accum_norm_sq's norm, no store
    adamw_step(hp, master, exp_avg, exp_avg_sq, grad, param_bf16=None, norm_sq=None)
    adamw_scalars(hp) / scalars_bytes(hp)       the step's binary32 scalars, on the host
    adamw_step_dev(scalars_dev, master, exp_avg, exp_avg_sq, grad, param_bf16=None, norm_sq=None)
    adamw_step_sum(hp, master, exp_avg, exp_avg_sq, acc, grad, param_bf16=None, norm_sq=None)
                                                the step on fl(acc + widen(grad)), the sum not stored
    adamw_step_sum_dev(scalars_dev, master, exp_avg, exp_avg_sq, acc, grad, param_bf16=None, norm_sq=None)
    adamw_step_no_master(hp, param_bf16, exp_avg, exp_avg_sq, grad, norm_sq=None)
    adam_update(hp, exp_avg, exp_avg_sq, grad, update, norm_sq=None)
    flat_apply_update(update, dst_tensors)
    state_tiled_numel(n)                        floats of the tiled optimizer state
    state_tile(master, exp_avg, exp_avg_sq, state, n=None)     split -> tiled (None sources: zeros)
    state_untile(state, master, exp_avg, exp_avg_sq, n=None)   tiled -> split (None: skipped)
    adamw_step_tiled(hp, state, grad, param_bf16=None, norm_sq=None)
    adamw_step_tiled_dev(scalars_dev, state, grad, param_bf16=None, norm_sq=None)
    adamw_step_tiled_sum(hp, state, acc, grad, param_bf16=None, norm_sq=None)   gradient fl(acc + widen(grad))
    adamw_step_tiled_sum_dev(scalars_dev, state, acc, grad, param_bf16=None, norm_sq=None)
    moments_tiled_numel(n) / moments_tile(exp_avg, exp_avg_sq, moments, n=None) / moments_untile(...)
    adam_update_tiled(hp, moments, grad, update, norm_sq=None)
    adamw_step_no_master_tiled(hp, param_bf16, moments, grad, norm_sq=None)

DeviceArena(nbytes, device) holds one physically contiguous block of device
memory and hands out 2 MiB-aligned views of it (ShardOptimizer(arena=...)).

All device work runs in the library's gfx950 HIP kernels on the current
torch stream; torch supplies device memory and the stream only.
"""
from ._binding import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    NOALLOC_MAX_ELEMS,
    STATE_TILE,
    AdamWConfig,
    ZShardError,
    AdamWScalars,
    adam_update,
    adam_update_tiled,
    adamw_scalars,
    adamw_step,
    adamw_step_dev,
    adamw_step_no_master,
    adamw_step_no_master_tiled,
    adamw_step_sum,
    adamw_step_sum_dev,
    adamw_step_tiled,
    adamw_step_tiled_dev,
    adamw_step_tiled_sum,
    adamw_step_tiled_sum_dev,
    flat_apply_update,
    flat_pack,
    flat_unpack,
    grad_accum,
    grad_accum_norm_sq,
    grad_accum_norm_sq_noalloc,
    grad_accum_norm_sq_workspace_bytes,
    grad_reduce_chunks,
    grad_reduce_chunks_norm_sq,
    grad_reduce_chunks_norm_sq_workspace_bytes,
    grad_norm_sq,
    grad_norm_sq_workspace_bytes,
    grad_sum_norm_sq,
    lib,
    moments_tile,
    moments_tiled_numel,
    moments_untile,
    scalars_bytes,
    state_tile,
    state_tiled_numel,
    state_untile,
    zero_shard_range,
)
from .arena import DeviceArena  # noqa: F401
from .step import ShardOptimizer  # noqa: F401
