"""ctypes binding of libzshard.so (include/zshard.h).

Argument marshalling only: torch tensors supply device pointers, sizes and
the current HIP stream; every step of the path runs in the library's HIP
kernels.  There is no fallback: if the library is not built, every call
raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzshard.so")

ZS_F32 = 0
ZS_BF16 = 1
ZS_OK = 0
ZS_EINVAL = -1
ZS_EOVERLAP = -2
ZS_EWORKSPACE = -3
ZS_EHIP = -4

# every symbol include/zshard.h declares
EXPORTS = (
    "zero_shard_range", "flat_pack", "flat_unpack", "grad_accum", "grad_reduce_chunks",
    "grad_norm_sq_workspace_bytes", "grad_norm_sq", "grad_accum_norm_sq_workspace_bytes",
    "grad_accum_norm_sq", "adamw_step", "adamw_scalars", "adamw_step_dev", "adamw_step_no_master", "adam_update",
    "flat_apply_update", "state_tiled_numel", "state_tile", "state_untile", "adamw_step_tiled",
    "adamw_step_tiled_dev", "moments_tiled_numel", "moments_tile", "moments_untile", "adam_update_tiled",
    "adamw_step_no_master_tiled", "grad_reduce_chunks_norm_sq_workspace_bytes", "grad_reduce_chunks_norm_sq",
    "grad_accum_norm_sq_noalloc", "grad_sum_norm_sq", "adamw_step_tiled_sum", "adamw_step_tiled_sum_dev",
    "adamw_step_sum", "adamw_step_sum_dev",
    "zs_strerror", "zs_last_hip_error",
)
NOALLOC_MAX_ELEMS = 2_146_959_360   # ZS_NOALLOC_MAX_ELEMS

STATE_TILE = 8192   # ZS_STATE_TILE: elements per tile of the tiled optimizer state


class ZShardError(RuntimeError):
    def __init__(self, fn: str, code: int, message: str):
        super().__init__(f"{fn}: {message} (code {code})")
        self.code = code


class Shard(ctypes.Structure):
    _fields_ = [("chunk", ctypes.c_int64), ("start", ctypes.c_int64),
                ("end", ctypes.c_int64), ("padded_total", ctypes.c_int64)]

    def as_tuple(self):
        return (self.chunk, self.start, self.end, self.padded_total)


class Tensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("numel", ctypes.c_int64)]


class AdamW(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
        ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double),
        ("grad_scale", ctypes.c_double), ("max_norm", ctypes.c_double),
        ("extra_norm_sq", ctypes.c_double), ("step", ctypes.c_int64),
    ]


class AdamWScalars(ctypes.Structure):
    """zs_adamw_scalars: one step's binary32 scalars (56 bytes)."""
    _fields_ = [(name, ctypes.c_float) for name in (
        "beta1", "beta2", "one_minus_beta1", "one_minus_beta2", "step_size", "bias_correction2_sqrt", "eps",
        "decay", "grad_scale")] + [("clip", ctypes.c_int32), ("max_norm", ctypes.c_double),
                                   ("extra_norm_sq", ctypes.c_double)]


@dataclass
class AdamWConfig:
    """Hyperparameters of one step (``step`` is t >= 1)."""
    lr: float
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    grad_scale: float = 1.0
    max_norm: float = 0.0
    extra_norm_sq: float = 0.0
    step: int = 1

    def c_struct(self) -> AdamW:
        return AdamW(self.lr, self.beta1, self.beta2, self.eps, self.weight_decay,
                     self.grad_scale, self.max_norm, self.extra_norm_sq, int(self.step))


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m fsdp_sharded_optimizer_amd.build` "
                "(or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.zero_shard_range.argtypes = [I64, I32, I32, ctypes.POINTER(Shard)]
        L.zero_shard_range.restype = I32
        L.flat_pack.argtypes = [ctypes.POINTER(Tensor), I32, I32, P, I32, I64, P]
        L.flat_pack.restype = I32
        L.flat_unpack.argtypes = [P, I32, ctypes.POINTER(Tensor), I32, I32, P]
        L.flat_unpack.restype = I32
        L.grad_accum.argtypes = [P, P, I32, I64, I32, P]
        L.grad_accum.restype = I32
        L.grad_reduce_chunks.argtypes = [P, P, I32, I32, I64, I32, P]
        L.grad_reduce_chunks.restype = I32
        L.grad_reduce_chunks_norm_sq_workspace_bytes.argtypes = [I64]
        L.grad_reduce_chunks_norm_sq_workspace_bytes.restype = I64
        L.grad_reduce_chunks_norm_sq.argtypes = [P, P, I32, I32, I64, I32, D, P, P, I64, P]
        L.grad_reduce_chunks_norm_sq.restype = I32
        L.grad_norm_sq_workspace_bytes.argtypes = [I64]
        L.grad_norm_sq_workspace_bytes.restype = I64
        L.grad_norm_sq.argtypes = [P, I64, D, P, P, I64, P]
        L.grad_norm_sq.restype = I32
        L.grad_accum_norm_sq_workspace_bytes.argtypes = [I64]
        L.grad_accum_norm_sq_workspace_bytes.restype = I64
        L.grad_accum_norm_sq.argtypes = [P, P, I32, I64, I32, D, P, P, I64, P]
        L.grad_accum_norm_sq.restype = I32
        L.grad_accum_norm_sq_noalloc.argtypes = [P, P, I32, I64, I32, D, P, P]
        L.grad_accum_norm_sq_noalloc.restype = I32
        L.grad_sum_norm_sq.argtypes = [P, P, I32, I64, I32, D, P, P, I64, P]
        L.grad_sum_norm_sq.restype = I32
        L.adamw_step_tiled_sum.argtypes = [ctypes.POINTER(AdamW), P, P, P, I32, P, I64, P, P]
        L.adamw_step_tiled_sum.restype = I32
        L.adamw_step_tiled_sum_dev.argtypes = [P, P, P, P, I32, P, I64, P, P]
        L.adamw_step_tiled_sum_dev.restype = I32
        L.adamw_step_sum.argtypes = [ctypes.POINTER(AdamW), P, P, P, P, P, I32, P, I64, P, P]
        L.adamw_step_sum.restype = I32
        L.adamw_step_sum_dev.argtypes = [P, P, P, P, P, P, I32, P, I64, P, P]
        L.adamw_step_sum_dev.restype = I32
        L.adamw_step.argtypes = [ctypes.POINTER(AdamW), P, P, P, P, P, I64, P, P]
        L.adamw_step.restype = I32
        L.adamw_scalars.argtypes = [ctypes.POINTER(AdamW), ctypes.POINTER(AdamWScalars)]
        L.adamw_scalars.restype = I32
        L.adamw_step_dev.argtypes = [P, P, P, P, P, P, I64, P, P]
        L.adamw_step_dev.restype = I32
        L.adamw_step_no_master.argtypes = [ctypes.POINTER(AdamW), P, P, P, P, I64, P, P]
        L.adamw_step_no_master.restype = I32
        L.adam_update.argtypes = [ctypes.POINTER(AdamW), P, P, P, P, I64, P, P]
        L.adam_update.restype = I32
        L.flat_apply_update.argtypes = [P, ctypes.POINTER(Tensor), I32, I32, P]
        L.flat_apply_update.restype = I32
        L.state_tiled_numel.argtypes = [I64]
        L.state_tiled_numel.restype = I64
        L.state_tile.argtypes = [P, P, P, P, I64, P]
        L.state_tile.restype = I32
        L.state_untile.argtypes = [P, P, P, P, I64, P]
        L.state_untile.restype = I32
        L.adamw_step_tiled.argtypes = [ctypes.POINTER(AdamW), P, P, P, I64, P, P]
        L.adamw_step_tiled.restype = I32
        L.adamw_step_tiled_dev.argtypes = [P, P, P, P, I64, P, P]
        L.adamw_step_tiled_dev.restype = I32
        L.moments_tiled_numel.argtypes = [I64]
        L.moments_tiled_numel.restype = I64
        L.moments_tile.argtypes = [P, P, P, I64, P]
        L.moments_tile.restype = I32
        L.moments_untile.argtypes = [P, P, P, I64, P]
        L.moments_untile.restype = I32
        L.adam_update_tiled.argtypes = [ctypes.POINTER(AdamW), P, P, P, I64, P, P]
        L.adam_update_tiled.restype = I32
        L.adamw_step_no_master_tiled.argtypes = [ctypes.POINTER(AdamW), P, P, P, I64, P, P]
        L.adamw_step_no_master_tiled.restype = I32
        L.zs_strerror.argtypes = [I32]
        L.zs_strerror.restype = ctypes.c_char_p
        L.zs_last_hip_error.argtypes = []
        L.zs_last_hip_error.restype = I32
        _lib = L
    return _lib


def _check(fn: str, code: int) -> None:
    if code != ZS_OK:
        msg = lib().zs_strerror(code).decode()
        if code == ZS_EHIP:
            msg += f" (hipError {lib().zs_last_hip_error()})"
        raise ZShardError(fn, code, msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return ZS_F32
    if t.dtype == torch.bfloat16:
        return ZS_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _dev(t: Optional[torch.Tensor], name: str, dtype=None) -> int:
    """Device pointer of a contiguous tensor on the current GPU (0 for None).
    Every call runs on the current device's stream, so every buffer must live
    on that device."""
    if t is None:
        return 0
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor, got {t.device}")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name}: on {t.device}, but the current device is cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    if s.device.index != torch.cuda.current_device():
        raise ValueError(f"stream on {s.device}, but the current device is cuda:{torch.cuda.current_device()}")
    return int(s.cuda_stream)


def _norm(norm_sq: Optional[torch.Tensor], fn: str) -> int:
    if norm_sq is None:
        return 0
    if norm_sq.dtype != torch.float64 or norm_sq.numel() < 1:
        raise TypeError(f"{fn}: norm_sq must hold one float64")
    return _dev(norm_sq, "norm_sq")


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def zero_shard_range(total: int, world: int, rank: int):
    """(chunk, start, end, padded_total) of `rank`'s range; host only."""
    out = Shard()
    _check("zero_shard_range", lib().zero_shard_range(int(total), int(world), int(rank), ctypes.byref(out)))
    return out.as_tuple()


def _tensor_list(ts: Sequence[torch.Tensor], name: str):
    arr = (Tensor * max(len(ts), 1))()
    dt = None
    for i, t in enumerate(ts):
        arr[i].ptr = _dev(t, f"{name}[{i}]")
        arr[i].numel = t.numel()
        code = _dtype_code(t)
        if dt is not None and code != dt:
            raise TypeError(f"{name}: all tensors must share one dtype")
        dt = code
    return arr, dt


def flat_pack(src: Sequence[torch.Tensor], flat: torch.Tensor, padded_total: Optional[int] = None,
              stream=None) -> None:
    """flat[o_i + j] = src[i].view(-1)[j]; flat[sum numel:padded_total] = 0."""
    arr, dt = _tensor_list(src, "src")
    if dt is None:
        dt = _dtype_code(flat)
    pt = flat.numel() if padded_total is None else int(padded_total)
    if pt > flat.numel():
        raise ValueError("flat_pack: padded_total exceeds the flat buffer")
    _check("flat_pack", lib().flat_pack(arr, len(src), dt, _dev(flat, "flat"), _dtype_code(flat), pt,
                                        _stream(stream)))


def flat_unpack(flat: torch.Tensor, dst: Sequence[torch.Tensor], stream=None) -> None:
    """dst[i].view(-1)[j] = flat[o_i + j] (padding ignored)."""
    arr, dt = _tensor_list(dst, "dst")
    if dt is None:
        dt = _dtype_code(flat)
    total = sum(t.numel() for t in dst)
    if total > flat.numel():
        raise ValueError("flat_unpack: destinations exceed the flat buffer")
    _check("flat_unpack", lib().flat_unpack(_dev(flat, "flat"), _dtype_code(flat), arr, len(dst), dt,
                                            _stream(stream)))


def flat_apply_update(update: torch.Tensor, dst: Sequence[torch.Tensor], stream=None) -> None:
    """dst[i].view(-1)[j] += update[o_i + j] in place (fp32 or bf16 tensors;
    the update is fp32, its padding ignored)."""
    arr, dt = _tensor_list(dst, "dst")
    if dt is None:
        dt = ZS_F32
    total = sum(t.numel() for t in dst)
    if total > update.numel():
        raise ValueError("flat_apply_update: destinations exceed the update buffer")
    _check("flat_apply_update", lib().flat_apply_update(_dev(update, "update", torch.float32), arr, len(dst), dt,
                                                        _stream(stream)))


def grad_accum(acc: torch.Tensor, grad: torch.Tensor, overwrite: bool, stream=None) -> None:
    """acc = widen(grad) (overwrite) or acc = acc + widen(grad), fp32."""
    if grad.numel() != acc.numel():
        raise ValueError("grad_accum: size mismatch")
    _check("grad_accum", lib().grad_accum(_dev(acc, "acc", torch.float32), _dev(grad, "grad"),
                                          _dtype_code(grad), acc.numel(), 1 if overwrite else 0,
                                          _stream(stream)))


def grad_reduce_chunks(acc: torch.Tensor, chunks: Sequence[torch.Tensor], overwrite: bool, stream=None) -> None:
    """acc = (acc or 0) + chunks[0] + chunks[1] + ... in order, fp32 (reduce-scatter arithmetic)."""
    n = acc.numel()
    ptrs = (ctypes.c_void_p * max(len(chunks), 1))()
    dt = None
    for k, c in enumerate(chunks):
        if c.numel() != n:
            raise ValueError("grad_reduce_chunks: size mismatch")
        code = _dtype_code(c)
        if dt is not None and code != dt:
            raise TypeError("grad_reduce_chunks: all chunks must share one dtype")
        dt = code
        ptrs[k] = _dev(c, f"chunks[{k}]")
    _check("grad_reduce_chunks", lib().grad_reduce_chunks(
        _dev(acc, "acc", torch.float32), ctypes.cast(ptrs, ctypes.c_void_p), len(chunks),
        ZS_BF16 if dt is None else dt, n, 1 if overwrite else 0, _stream(stream)))


def _chunk_ptrs(chunks: Sequence[torch.Tensor], n: int, fn: str):
    ptrs = (ctypes.c_void_p * max(len(chunks), 1))()
    dt = None
    for k, c in enumerate(chunks):
        if c.numel() != n:
            raise ValueError(f"{fn}: size mismatch")
        code = _dtype_code(c)
        if dt is not None and code != dt:
            raise TypeError(f"{fn}: all chunks must share one dtype")
        dt = code
        ptrs[k] = _dev(c, f"chunks[{k}]")
    return ptrs, ZS_BF16 if dt is None else dt


def grad_reduce_chunks_norm_sq_workspace_bytes(n: int) -> int:
    return int(lib().grad_reduce_chunks_norm_sq_workspace_bytes(int(n)))


def grad_reduce_chunks_norm_sq(acc: torch.Tensor, chunks: Sequence[torch.Tensor], overwrite: bool,
                               grad_scale: float, out: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                               stream=None) -> torch.Tensor:
    """grad_reduce_chunks, then out[0] (fp64, device) = squared norm of fl32(acc * scale), in one pass."""
    n = acc.numel()
    ptrs, dt = _chunk_ptrs(chunks, n, "grad_reduce_chunks_norm_sq")
    need = grad_reduce_chunks_norm_sq_workspace_bytes(n)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=acc.device)
    if out.dtype != torch.float64 or out.numel() < 1:
        raise TypeError("grad_reduce_chunks_norm_sq: out must hold one float64")
    _check("grad_reduce_chunks_norm_sq", lib().grad_reduce_chunks_norm_sq(
        _dev(acc, "acc", torch.float32), ctypes.cast(ptrs, ctypes.c_void_p), len(chunks), dt, n,
        1 if overwrite else 0, float(grad_scale), _dev(out, "out"), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def grad_norm_sq_workspace_bytes(n: int) -> int:
    return int(lib().grad_norm_sq_workspace_bytes(int(n)))


def grad_norm_sq(grad: torch.Tensor, grad_scale: float, out: torch.Tensor,
                 workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out[0] (fp64, device) = sum of (fl32(grad * scale))^2 in binary64."""
    n = grad.numel()
    need = grad_norm_sq_workspace_bytes(n)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=grad.device)
    if out.dtype != torch.float64 or out.numel() < 1:
        raise TypeError("grad_norm_sq: out must hold one float64")
    _check("grad_norm_sq", lib().grad_norm_sq(_dev(grad, "grad", torch.float32), n, float(grad_scale),
                                              _dev(out, "out"), _dev(workspace, "workspace"),
                                              workspace.numel() * workspace.element_size(),
                                              _stream(stream)))
    return out


def grad_accum_norm_sq_workspace_bytes(n: int) -> int:
    return int(lib().grad_accum_norm_sq_workspace_bytes(int(n)))


def grad_accum_norm_sq(acc: torch.Tensor, grad: torch.Tensor, overwrite: bool, grad_scale: float,
                       out: torch.Tensor, workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """grad_accum, then out[0] (fp64, device) = squared norm of fl32(acc * scale), in one pass."""
    n = acc.numel()
    if grad.numel() != n:
        raise ValueError("grad_accum_norm_sq: size mismatch")
    need = grad_accum_norm_sq_workspace_bytes(n)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=acc.device)
    if out.dtype != torch.float64 or out.numel() < 1:
        raise TypeError("grad_accum_norm_sq: out must hold one float64")
    _check("grad_accum_norm_sq", lib().grad_accum_norm_sq(
        _dev(acc, "acc", torch.float32), _dev(grad, "grad"), _dtype_code(grad), n, 1 if overwrite else 0,
        float(grad_scale), _dev(out, "out"), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def grad_accum_norm_sq_noalloc(acc: torch.Tensor, grad: torch.Tensor, overwrite: bool, grad_scale: float,
                               out: torch.Tensor, stream=None) -> torch.Tensor:
    """grad_accum_norm_sq with the partials in the library's static device
    scratch: no workspace, nothing allocated (n <= NOALLOC_MAX_ELEMS)."""
    n = acc.numel()
    if grad.numel() != n:
        raise ValueError("grad_accum_norm_sq_noalloc: size mismatch")
    if out.dtype != torch.float64 or out.numel() < 1:
        raise TypeError("grad_accum_norm_sq_noalloc: out must hold one float64")
    _check("grad_accum_norm_sq_noalloc", lib().grad_accum_norm_sq_noalloc(
        _dev(acc, "acc", torch.float32), _dev(grad, "grad"), _dtype_code(grad), n, 1 if overwrite else 0,
        float(grad_scale), _dev(out, "out"), _stream(stream)))
    return out


def grad_sum_norm_sq(acc: Optional[torch.Tensor], grad: torch.Tensor, overwrite: bool, grad_scale: float,
                     out: torch.Tensor, workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out[0] = the squared norm grad_accum_norm_sq(acc, grad, overwrite, ...)
    would form, bit for bit, without writing acc (not read when overwrite)."""
    n = grad.numel()
    if overwrite:
        acc = None
    elif acc is None or acc.numel() != n:
        raise ValueError("grad_sum_norm_sq: acc must hold the gradient's numel unless overwrite")
    need = grad_accum_norm_sq_workspace_bytes(n)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=grad.device)
    if out.dtype != torch.float64 or out.numel() < 1:
        raise TypeError("grad_sum_norm_sq: out must hold one float64")
    _check("grad_sum_norm_sq", lib().grad_sum_norm_sq(
        _dev(acc, "acc", torch.float32), _dev(grad, "grad"), _dtype_code(grad), n, 1 if overwrite else 0,
        float(grad_scale), _dev(out, "out"), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def adamw_step(hp: AdamWConfig, master: torch.Tensor, exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor,
               grad: torch.Tensor, param_bf16: Optional[torch.Tensor] = None,
               norm_sq: Optional[torch.Tensor] = None, stream=None) -> None:
    """Fused AdamW update of the shard (in place), with the bf16 re-cast."""
    n = master.numel()
    for t, nm in ((exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq"), (grad, "grad")):
        if t.numel() != n:
            raise ValueError(f"adamw_step: {nm} size mismatch")
    if param_bf16 is not None and param_bf16.numel() != n:
        raise ValueError("adamw_step: param_bf16 size mismatch")
    c = hp.c_struct()
    _check("adamw_step", lib().adamw_step(
        ctypes.byref(c), _dev(master, "master", torch.float32), _dev(exp_avg, "exp_avg", torch.float32),
        _dev(exp_avg_sq, "exp_avg_sq", torch.float32), _dev(grad, "grad", torch.float32),
        _dev(param_bf16, "param_bf16", torch.bfloat16), n, _norm(norm_sq, "adamw_step"), _stream(stream)))


def adamw_scalars(hp: AdamWConfig) -> AdamWScalars:
    """The binary32 scalars adamw_step forms from hp (host only)."""
    out = AdamWScalars()
    c = hp.c_struct()
    _check("adamw_scalars", lib().adamw_scalars(ctypes.byref(c), ctypes.byref(out)))
    return out


def scalars_bytes(hp: AdamWConfig) -> bytes:
    """adamw_scalars(hp) as the bytes adamw_step_dev reads from device memory."""
    return bytes(adamw_scalars(hp))


def adamw_step_dev(scalars_dev: torch.Tensor, master: torch.Tensor, exp_avg: torch.Tensor,
                   exp_avg_sq: torch.Tensor, grad: torch.Tensor, param_bf16: Optional[torch.Tensor] = None,
                   norm_sq: Optional[torch.Tensor] = None, stream=None) -> None:
    """adamw_step with its scalars read from device memory when the kernels
    run: scalars_dev is a uint8 GPU tensor holding scalars_bytes(hp)."""
    if scalars_dev.dtype != torch.uint8 or scalars_dev.numel() < ctypes.sizeof(AdamWScalars):
        raise TypeError("adamw_step_dev: scalars_dev must be a uint8 tensor of at least "
                        f"{ctypes.sizeof(AdamWScalars)} bytes")
    n = master.numel()
    for t, nm in ((exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq"), (grad, "grad")):
        if t.numel() != n:
            raise ValueError(f"adamw_step_dev: {nm} size mismatch")
    if param_bf16 is not None and param_bf16.numel() != n:
        raise ValueError("adamw_step_dev: param_bf16 size mismatch")
    _check("adamw_step_dev", lib().adamw_step_dev(
        _dev(scalars_dev, "scalars_dev"), _dev(master, "master", torch.float32),
        _dev(exp_avg, "exp_avg", torch.float32), _dev(exp_avg_sq, "exp_avg_sq", torch.float32),
        _dev(grad, "grad", torch.float32), _dev(param_bf16, "param_bf16", torch.bfloat16), n,
        _norm(norm_sq, "adamw_step_dev"), _stream(stream)))


def adamw_step_no_master(hp: AdamWConfig, param_bf16: torch.Tensor, exp_avg: torch.Tensor,
                         exp_avg_sq: torch.Tensor, grad: torch.Tensor, norm_sq: Optional[torch.Tensor] = None,
                         stream=None) -> None:
    """AdamW on a bf16 parameter shard with no fp32 master (in place)."""
    n = param_bf16.numel()
    for t, nm in ((exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq"), (grad, "grad")):
        if t.numel() != n:
            raise ValueError(f"adamw_step_no_master: {nm} size mismatch")
    c = hp.c_struct()
    _check("adamw_step_no_master", lib().adamw_step_no_master(
        ctypes.byref(c), _dev(param_bf16, "param_bf16", torch.bfloat16), _dev(exp_avg, "exp_avg", torch.float32),
        _dev(exp_avg_sq, "exp_avg_sq", torch.float32), _dev(grad, "grad", torch.float32), n,
        _norm(norm_sq, "adamw_step_no_master"), _stream(stream)))


def adam_update(hp: AdamWConfig, exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor, grad: torch.Tensor,
                update: torch.Tensor, norm_sq: Optional[torch.Tensor] = None, stream=None) -> None:
    """ZeRO-1 form: Adam (weight_decay 0) moments in place, the update vector
    -(lr/bc1) * m / den into ``update``."""
    n = update.numel()
    for t, nm in ((exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq"), (grad, "grad")):
        if t.numel() != n:
            raise ValueError(f"adam_update: {nm} size mismatch")
    c = hp.c_struct()
    _check("adam_update", lib().adam_update(
        ctypes.byref(c), _dev(exp_avg, "exp_avg", torch.float32), _dev(exp_avg_sq, "exp_avg_sq", torch.float32),
        _dev(grad, "grad", torch.float32), _dev(update, "update", torch.float32), n,
        _norm(norm_sq, "adam_update"), _stream(stream)))


def state_tiled_numel(n: int) -> int:
    """Floats of the tiled optimizer state of n elements (host only)."""
    out = int(lib().state_tiled_numel(int(n)))
    if out < 0:
        raise ValueError(f"state_tiled_numel: invalid element count {n}")
    return out


def _state_buffer(state: torch.Tensor, n: int, fn: str) -> int:
    if state.numel() < state_tiled_numel(n):
        raise ValueError(f"{fn}: state holds {state.numel()} floats, the tiled layout of {n} elements needs "
                         f"{state_tiled_numel(n)}")
    return _dev(state, "state", torch.float32)


def state_tile(master: Optional[torch.Tensor], exp_avg: Optional[torch.Tensor], exp_avg_sq: Optional[torch.Tensor],
               state: torch.Tensor, n: Optional[int] = None, stream=None) -> None:
    """Split fp32 arrays (None = zeros) into the tiled state buffer."""
    srcs = (master, exp_avg, exp_avg_sq)
    if n is None:
        n = next((t.numel() for t in srcs if t is not None), None)
        if n is None:
            raise ValueError("state_tile: give n when every source is None")
    for t, nm in zip(srcs, ("master", "exp_avg", "exp_avg_sq")):
        if t is not None and t.numel() != n:
            raise ValueError(f"state_tile: {nm} size mismatch")
    _check("state_tile", lib().state_tile(
        _dev(master, "master", torch.float32), _dev(exp_avg, "exp_avg", torch.float32),
        _dev(exp_avg_sq, "exp_avg_sq", torch.float32), _state_buffer(state, n, "state_tile"), int(n),
        _stream(stream)))


def state_untile(state: torch.Tensor, master: Optional[torch.Tensor], exp_avg: Optional[torch.Tensor],
                 exp_avg_sq: Optional[torch.Tensor], n: Optional[int] = None, stream=None) -> None:
    """The tiled state back into split fp32 arrays (None = that stream skipped)."""
    dsts = (master, exp_avg, exp_avg_sq)
    if n is None:
        n = next((t.numel() for t in dsts if t is not None), None)
        if n is None:
            raise ValueError("state_untile: give n when every destination is None")
    for t, nm in zip(dsts, ("master", "exp_avg", "exp_avg_sq")):
        if t is not None and t.numel() != n:
            raise ValueError(f"state_untile: {nm} size mismatch")
    _check("state_untile", lib().state_untile(
        _state_buffer(state, n, "state_untile"), _dev(master, "master", torch.float32),
        _dev(exp_avg, "exp_avg", torch.float32), _dev(exp_avg_sq, "exp_avg_sq", torch.float32), int(n),
        _stream(stream)))


def adamw_step_tiled(hp: AdamWConfig, state: torch.Tensor, grad: torch.Tensor,
                     param_bf16: Optional[torch.Tensor] = None, norm_sq: Optional[torch.Tensor] = None,
                     stream=None) -> None:
    """Fused AdamW update of the shard held in the tiled state layout (in
    place), with the bf16 re-cast; n is the gradient's length."""
    n = grad.numel()
    if param_bf16 is not None and param_bf16.numel() != n:
        raise ValueError("adamw_step_tiled: param_bf16 size mismatch")
    c = hp.c_struct()
    _check("adamw_step_tiled", lib().adamw_step_tiled(
        ctypes.byref(c), _state_buffer(state, n, "adamw_step_tiled"), _dev(grad, "grad", torch.float32),
        _dev(param_bf16, "param_bf16", torch.bfloat16), n, _norm(norm_sq, "adamw_step_tiled"), _stream(stream)))


def adamw_step_tiled_dev(scalars_dev: torch.Tensor, state: torch.Tensor, grad: torch.Tensor,
                         param_bf16: Optional[torch.Tensor] = None, norm_sq: Optional[torch.Tensor] = None,
                         stream=None) -> None:
    """adamw_step_tiled with its scalars read from device memory when the
    kernels run (scalars_dev: uint8 GPU tensor holding scalars_bytes(hp))."""
    if scalars_dev.dtype != torch.uint8 or scalars_dev.numel() < ctypes.sizeof(AdamWScalars):
        raise TypeError("adamw_step_tiled_dev: scalars_dev must be a uint8 tensor of at least "
                        f"{ctypes.sizeof(AdamWScalars)} bytes")
    n = grad.numel()
    if param_bf16 is not None and param_bf16.numel() != n:
        raise ValueError("adamw_step_tiled_dev: param_bf16 size mismatch")
    _check("adamw_step_tiled_dev", lib().adamw_step_tiled_dev(
        _dev(scalars_dev, "scalars_dev"), _state_buffer(state, n, "adamw_step_tiled_dev"),
        _dev(grad, "grad", torch.float32), _dev(param_bf16, "param_bf16", torch.bfloat16), n,
        _norm(norm_sq, "adamw_step_tiled_dev"), _stream(stream)))


def _sum_args(acc: Optional[torch.Tensor], grad: torch.Tensor, param_bf16: Optional[torch.Tensor], fn: str):
    n = grad.numel()
    if acc is not None and acc.numel() != n:
        raise ValueError(f"{fn}: acc size mismatch")
    if param_bf16 is not None and param_bf16.numel() != n:
        raise ValueError(f"{fn}: param_bf16 size mismatch")
    return n


def _split_sum_args(master, exp_avg, exp_avg_sq, acc, grad, param_bf16, fn: str):
    n = _sum_args(acc, grad, param_bf16, fn)
    if master.numel() != n or exp_avg.numel() != n or exp_avg_sq.numel() != n:
        raise ValueError(f"{fn}: size mismatch")
    return n


def adamw_step_sum(hp: AdamWConfig, master: torch.Tensor, exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor,
                   acc: Optional[torch.Tensor], grad: torch.Tensor, param_bf16: Optional[torch.Tensor] = None,
                   norm_sq: Optional[torch.Tensor] = None, stream=None) -> None:
    """adamw_step on the last micro-batch's sum fl(acc + widen(grad))
    (widen(grad) alone when acc is None), formed as it is read: acc is not
    written.  Bit for bit grad_accum then adamw_step."""
    n = _split_sum_args(master, exp_avg, exp_avg_sq, acc, grad, param_bf16, "adamw_step_sum")
    c = hp.c_struct()
    _check("adamw_step_sum", lib().adamw_step_sum(
        ctypes.byref(c), _dev(master, "master", torch.float32), _dev(exp_avg, "exp_avg", torch.float32),
        _dev(exp_avg_sq, "exp_avg_sq", torch.float32), _dev(acc, "acc", torch.float32), _dev(grad, "grad"),
        _dtype_code(grad), _dev(param_bf16, "param_bf16", torch.bfloat16), n, _norm(norm_sq, "adamw_step_sum"),
        _stream(stream)))


def adamw_step_sum_dev(scalars_dev: torch.Tensor, master: torch.Tensor, exp_avg: torch.Tensor,
                       exp_avg_sq: torch.Tensor, acc: Optional[torch.Tensor], grad: torch.Tensor,
                       param_bf16: Optional[torch.Tensor] = None, norm_sq: Optional[torch.Tensor] = None,
                       stream=None) -> None:
    """adamw_step_sum with its scalars read from device memory when the
    kernels run (scalars_dev: uint8 GPU tensor holding scalars_bytes(hp))."""
    if scalars_dev.dtype != torch.uint8 or scalars_dev.numel() < ctypes.sizeof(AdamWScalars):
        raise TypeError("adamw_step_sum_dev: scalars_dev must be a uint8 tensor of at least "
                        f"{ctypes.sizeof(AdamWScalars)} bytes")
    n = _split_sum_args(master, exp_avg, exp_avg_sq, acc, grad, param_bf16, "adamw_step_sum_dev")
    _check("adamw_step_sum_dev", lib().adamw_step_sum_dev(
        _dev(scalars_dev, "scalars_dev"), _dev(master, "master", torch.float32),
        _dev(exp_avg, "exp_avg", torch.float32), _dev(exp_avg_sq, "exp_avg_sq", torch.float32),
        _dev(acc, "acc", torch.float32), _dev(grad, "grad"), _dtype_code(grad),
        _dev(param_bf16, "param_bf16", torch.bfloat16), n, _norm(norm_sq, "adamw_step_sum_dev"), _stream(stream)))


def adamw_step_tiled_sum(hp: AdamWConfig, state: torch.Tensor, acc: Optional[torch.Tensor], grad: torch.Tensor,
                         param_bf16: Optional[torch.Tensor] = None, norm_sq: Optional[torch.Tensor] = None,
                         stream=None) -> None:
    """adamw_step_tiled on the last micro-batch's sum fl(acc + widen(grad))
    (widen(grad) alone when acc is None), formed as it is read: acc is not
    written.  Bit for bit grad_accum then adamw_step_tiled."""
    n = _sum_args(acc, grad, param_bf16, "adamw_step_tiled_sum")
    c = hp.c_struct()
    _check("adamw_step_tiled_sum", lib().adamw_step_tiled_sum(
        ctypes.byref(c), _state_buffer(state, n, "adamw_step_tiled_sum"), _dev(acc, "acc", torch.float32),
        _dev(grad, "grad"), _dtype_code(grad), _dev(param_bf16, "param_bf16", torch.bfloat16), n,
        _norm(norm_sq, "adamw_step_tiled_sum"), _stream(stream)))


def adamw_step_tiled_sum_dev(scalars_dev: torch.Tensor, state: torch.Tensor, acc: Optional[torch.Tensor],
                             grad: torch.Tensor, param_bf16: Optional[torch.Tensor] = None,
                             norm_sq: Optional[torch.Tensor] = None, stream=None) -> None:
    """adamw_step_tiled_sum with its scalars read from device memory when
    the kernels run (scalars_dev: uint8 GPU tensor holding scalars_bytes(hp))."""
    if scalars_dev.dtype != torch.uint8 or scalars_dev.numel() < ctypes.sizeof(AdamWScalars):
        raise TypeError("adamw_step_tiled_sum_dev: scalars_dev must be a uint8 tensor of at least "
                        f"{ctypes.sizeof(AdamWScalars)} bytes")
    n = _sum_args(acc, grad, param_bf16, "adamw_step_tiled_sum_dev")
    _check("adamw_step_tiled_sum_dev", lib().adamw_step_tiled_sum_dev(
        _dev(scalars_dev, "scalars_dev"), _state_buffer(state, n, "adamw_step_tiled_sum_dev"),
        _dev(acc, "acc", torch.float32), _dev(grad, "grad"), _dtype_code(grad),
        _dev(param_bf16, "param_bf16", torch.bfloat16), n, _norm(norm_sq, "adamw_step_tiled_sum_dev"),
        _stream(stream)))


def moments_tiled_numel(n: int) -> int:
    """Floats of the tiled moments (exp_avg, exp_avg_sq) of n elements (host only)."""
    out = int(lib().moments_tiled_numel(int(n)))
    if out < 0:
        raise ValueError(f"moments_tiled_numel: invalid element count {n}")
    return out


def _moments_buffer(moments: torch.Tensor, n: int, fn: str) -> int:
    if moments.numel() < moments_tiled_numel(n):
        raise ValueError(f"{fn}: moments hold {moments.numel()} floats, the tiled layout of {n} elements needs "
                         f"{moments_tiled_numel(n)}")
    return _dev(moments, "moments", torch.float32)


def moments_tile(exp_avg: Optional[torch.Tensor], exp_avg_sq: Optional[torch.Tensor], moments: torch.Tensor,
                 n: Optional[int] = None, stream=None) -> None:
    """Split fp32 moments (None = zeros) into the tiled moments buffer."""
    srcs = (exp_avg, exp_avg_sq)
    if n is None:
        n = next((t.numel() for t in srcs if t is not None), None)
        if n is None:
            raise ValueError("moments_tile: give n when every source is None")
    for t, nm in zip(srcs, ("exp_avg", "exp_avg_sq")):
        if t is not None and t.numel() != n:
            raise ValueError(f"moments_tile: {nm} size mismatch")
    _check("moments_tile", lib().moments_tile(
        _dev(exp_avg, "exp_avg", torch.float32), _dev(exp_avg_sq, "exp_avg_sq", torch.float32),
        _moments_buffer(moments, n, "moments_tile"), int(n), _stream(stream)))


def moments_untile(moments: torch.Tensor, exp_avg: Optional[torch.Tensor], exp_avg_sq: Optional[torch.Tensor],
                   n: Optional[int] = None, stream=None) -> None:
    """The tiled moments back into split fp32 arrays (None = that stream skipped)."""
    dsts = (exp_avg, exp_avg_sq)
    if n is None:
        n = next((t.numel() for t in dsts if t is not None), None)
        if n is None:
            raise ValueError("moments_untile: give n when every destination is None")
    for t, nm in zip(dsts, ("exp_avg", "exp_avg_sq")):
        if t is not None and t.numel() != n:
            raise ValueError(f"moments_untile: {nm} size mismatch")
    _check("moments_untile", lib().moments_untile(
        _moments_buffer(moments, n, "moments_untile"), _dev(exp_avg, "exp_avg", torch.float32),
        _dev(exp_avg_sq, "exp_avg_sq", torch.float32), int(n), _stream(stream)))


def adam_update_tiled(hp: AdamWConfig, moments: torch.Tensor, grad: torch.Tensor, update: torch.Tensor,
                      norm_sq: Optional[torch.Tensor] = None, stream=None) -> None:
    """adam_update on tiled moments: the update vector into ``update``."""
    n = update.numel()
    if grad.numel() != n:
        raise ValueError("adam_update_tiled: grad size mismatch")
    c = hp.c_struct()
    _check("adam_update_tiled", lib().adam_update_tiled(
        ctypes.byref(c), _moments_buffer(moments, n, "adam_update_tiled"), _dev(grad, "grad", torch.float32),
        _dev(update, "update", torch.float32), n, _norm(norm_sq, "adam_update_tiled"), _stream(stream)))


def adamw_step_no_master_tiled(hp: AdamWConfig, param_bf16: torch.Tensor, moments: torch.Tensor,
                               grad: torch.Tensor, norm_sq: Optional[torch.Tensor] = None, stream=None) -> None:
    """adamw_step_no_master on tiled moments (the bf16 parameter in place)."""
    n = param_bf16.numel()
    if grad.numel() != n:
        raise ValueError("adamw_step_no_master_tiled: grad size mismatch")
    c = hp.c_struct()
    _check("adamw_step_no_master_tiled", lib().adamw_step_no_master_tiled(
        ctypes.byref(c), _dev(param_bf16, "param_bf16", torch.bfloat16),
        _moments_buffer(moments, n, "adamw_step_no_master_tiled"), _dev(grad, "grad", torch.float32), n,
        _norm(norm_sq, "adamw_step_no_master_tiled"), _stream(stream)))
