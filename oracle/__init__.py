"""Oracle for the per-rank ZeRO/FSDP optimizer step — TEST INFRASTRUCTURE ONLY.

Thin numpy wrapper over ``oracle/oracle.c`` (plain C, built by ``build()``).
Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package; the GPU library never does, and this
package never imports the GPU library.  The two share nothing but the seeded
input generators in ``workloads``, which hold no arithmetic of the method.

Every function cites the passage of the pages it follows in ``oracle.c``.
bf16 arrays are carried as ``numpy.uint16`` bit patterns (numpy has no bf16).

Parity status: every function is pinned by ``tests/test_oracle_*.py``
(closed forms, brute force, invariants, independent library routines).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F32 = 0
BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile oracle.c with gcc: IEEE binary32/64, no contraction, OpenMP."""
    cmd = [
        "gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
        "-fPIC", "-shared", "-Wall", "-Wextra", "-o", _LIB_PATH + ".tmp", _SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


class AdamWHp(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
        ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double),
        ("grad_scale", ctypes.c_double), ("max_norm", ctypes.c_double),
        ("extra_norm_sq", ctypes.c_double), ("step", ctypes.c_int64),
    ]


class AdamWScalars(ctypes.Structure):
    _fields_ = [(name, ctypes.c_float) for name in (
        "beta1", "beta2", "one_minus_beta1", "one_minus_beta2", "step_size",
        "bias_correction2_sqrt", "eps", "decay", "grad_scale")]


def _configure(L):
    """Declare the C signatures on a loaded oracle library."""
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I32 = ctypes.c_int32
    L.orc_bf16_rne.argtypes = [ctypes.c_float]
    L.orc_bf16_rne.restype = ctypes.c_uint16
    L.orc_bf16_rne_array.argtypes = [P, P, I64]
    L.orc_bf16_rne_array.restype = None
    L.orc_shard_range.argtypes = [I64, I32, I32, P]
    L.orc_shard_range.restype = ctypes.c_int
    L.orc_flat_pack.argtypes = [P, P, I32, I32, P, I32, I64]
    L.orc_flat_pack.restype = ctypes.c_int
    L.orc_flat_unpack.argtypes = [P, I32, P, P, I32, I32]
    L.orc_flat_unpack.restype = ctypes.c_int
    L.orc_grad_accum.argtypes = [P, P, I32, I64, I32]
    L.orc_grad_accum.restype = ctypes.c_int
    L.orc_grad_norm_sq.argtypes = [P, I64, ctypes.c_double]
    L.orc_grad_norm_sq.restype = ctypes.c_double
    L.orc_adamw_scalars_make.argtypes = [ctypes.POINTER(AdamWHp), ctypes.POINTER(AdamWScalars)]
    L.orc_adamw_scalars_make.restype = ctypes.c_int
    L.orc_clip_coef.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double]
    L.orc_clip_coef.restype = ctypes.c_float
    L.orc_adamw_step.argtypes = [ctypes.POINTER(AdamWHp), P, P, P, P, P, I64, P]
    L.orc_adamw_step.restype = ctypes.c_int
    L.orc_adamw_step_no_master.argtypes = [ctypes.POINTER(AdamWHp), P, P, P, P, I64, P]
    L.orc_adamw_step_no_master.restype = ctypes.c_int
    L.orc_adam_update.argtypes = [ctypes.POINTER(AdamWHp), P, P, P, P, I64, P]
    L.orc_adam_update.restype = ctypes.c_int
    L.orc_flat_apply_update.argtypes = [P, P, P, I32, I32]
    L.orc_flat_apply_update.restype = ctypes.c_int
    L.orc_moments_tiled_numel.argtypes = [I64, I64]
    L.orc_moments_tiled_numel.restype = I64
    L.orc_moments_tile.argtypes = [P, P, P, I64, I64]
    L.orc_moments_tile.restype = ctypes.c_int
    L.orc_moments_untile.argtypes = [P, P, P, I64, I64]
    L.orc_moments_untile.restype = ctypes.c_int
    L.orc_state_tiled_numel.argtypes = [I64, I64]
    L.orc_state_tiled_numel.restype = I64
    L.orc_state_tile.argtypes = [P, P, P, P, I64, I64]
    L.orc_state_tile.restype = ctypes.c_int
    L.orc_state_untile.argtypes = [P, P, P, P, I64, I64]
    L.orc_state_untile.restype = ctypes.c_int
    L.orc_num_threads.argtypes = []
    L.orc_num_threads.restype = ctypes.c_int
    L.orc_set_num_threads.argtypes = [ctypes.c_int]
    L.orc_set_num_threads.restype = None
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = _configure(ctypes.CDLL(_LIB_PATH))
    return _lib


class use_library:
    """Context manager: route every oracle call to another build of oracle.c
    (the mutation tests load deliberately broken copies this way)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = lib()
        _lib = _configure(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _need(a: np.ndarray, dtype, name: str):
    if not isinstance(a, np.ndarray) or a.dtype != dtype or not a.flags.c_contiguous:
        raise TypeError(f"{name}: need a C-contiguous numpy {np.dtype(dtype).name} array")


def _np_dtype(code: int):
    return np.float32 if code == F32 else np.uint16


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads the OpenMP loops use from now on (results do not depend on it)."""
    lib().orc_set_num_threads(int(n))


def bf16_rne(x, out: np.ndarray = None) -> np.ndarray:
    """bf16 bit patterns of fp32 values, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if out is None:
        out = np.empty(x.shape, dtype=np.uint16)
    _need(out, np.uint16, "out")
    if out.size != x.size:
        raise ValueError("bf16_rne: out has the wrong size")
    lib().orc_bf16_rne_array(_ptr(x), _ptr(out), x.size)
    return out


def bf16_widen(b: np.ndarray) -> np.ndarray:
    """fp32 values of bf16 bit patterns (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def shard_range(total: int, world: int, rank: int):
    """(chunk, start, end, padded_total); raises ValueError on bad arguments."""
    out = (ctypes.c_int64 * 4)()
    rc = lib().orc_shard_range(total, world, rank, ctypes.cast(out, ctypes.c_void_p))
    if rc != 0:
        raise ValueError("shard_range: invalid arguments")
    return tuple(int(v) for v in out)


def flat_pack(srcs, src_dtype: int, flat_dtype: int, padded_total: int) -> np.ndarray:
    srcs = [np.ascontiguousarray(s, dtype=_np_dtype(src_dtype)).reshape(-1) for s in srcs]
    flat = np.full(padded_total, 0xFF if flat_dtype == BF16 else np.nan,
                   dtype=_np_dtype(flat_dtype))  # poison: every element must be written
    n = len(srcs)
    ptrs = (ctypes.c_void_p * max(n, 1))(*[s.ctypes.data for s in srcs])
    numel = (ctypes.c_int64 * max(n, 1))(*[s.size for s in srcs])
    rc = lib().orc_flat_pack(ctypes.cast(ptrs, ctypes.c_void_p), ctypes.cast(numel, ctypes.c_void_p),
                             n, src_dtype, _ptr(flat), flat_dtype, padded_total)
    if rc != 0:
        raise ValueError("flat_pack: invalid arguments")
    return flat


def flat_unpack(flat: np.ndarray, flat_dtype: int, numels, dst_dtype: int):
    _need(flat, _np_dtype(flat_dtype), "flat")
    dsts = [np.empty(int(k), dtype=_np_dtype(dst_dtype)) for k in numels]
    n = len(dsts)
    ptrs = (ctypes.c_void_p * max(n, 1))(*[d.ctypes.data for d in dsts])
    numel = (ctypes.c_int64 * max(n, 1))(*[d.size for d in dsts])
    rc = lib().orc_flat_unpack(_ptr(flat), flat_dtype, ctypes.cast(ptrs, ctypes.c_void_p),
                               ctypes.cast(numel, ctypes.c_void_p), n, dst_dtype)
    if rc != 0:
        raise ValueError("flat_unpack: invalid arguments")
    return dsts


def grad_accum(acc: np.ndarray, grad: np.ndarray, grad_dtype: int, overwrite: bool) -> None:
    _need(acc, np.float32, "acc")
    _need(grad, _np_dtype(grad_dtype), "grad")
    if grad.size != acc.size:
        raise ValueError("grad_accum: size mismatch")
    rc = lib().orc_grad_accum(_ptr(acc), _ptr(grad), grad_dtype, acc.size, 1 if overwrite else 0)
    if rc != 0:
        raise ValueError("grad_accum: invalid arguments")


def grad_norm_sq(acc: np.ndarray, grad_scale: float) -> float:
    _need(acc, np.float32, "acc")
    return float(lib().orc_grad_norm_sq(_ptr(acc), acc.size, grad_scale))


def make_hp(lr, beta1, beta2, eps, weight_decay, grad_scale, max_norm, extra_norm_sq, step) -> AdamWHp:
    return AdamWHp(lr, beta1, beta2, eps, weight_decay, grad_scale, max_norm, extra_norm_sq, step)


def adamw_scalars(hp: AdamWHp) -> AdamWScalars:
    s = AdamWScalars()
    if lib().orc_adamw_scalars_make(ctypes.byref(hp), ctypes.byref(s)) != 0:
        raise ValueError("adamw_scalars: invalid hyperparameters")
    return s


def clip_coef(norm_sq_local: float, extra_norm_sq: float, max_norm: float) -> float:
    return float(lib().orc_clip_coef(norm_sq_local, extra_norm_sq, max_norm))


def adamw_step(hp: AdamWHp, master, exp_avg, exp_avg_sq, grad, param_bf16=None, norm_sq=None) -> int:
    """In-place step; returns 0 (updated) or 1 (skipped: non-finite norm)."""
    for a, nm in ((master, "master"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq"), (grad, "grad")):
        _need(a, np.float32, nm)
        if a.size != master.size:
            raise ValueError("adamw_step: size mismatch")
    if param_bf16 is not None:
        _need(param_bf16, np.uint16, "param_bf16")
        if param_bf16.size != master.size:
            raise ValueError("adamw_step: size mismatch")
    nsq = None
    if norm_sq is not None:
        nsq = ctypes.c_double(float(norm_sq))
    rc = lib().orc_adamw_step(ctypes.byref(hp), _ptr(master), _ptr(exp_avg), _ptr(exp_avg_sq),
                              _ptr(grad), _ptr(param_bf16), master.size,
                              ctypes.byref(nsq) if nsq is not None else None)
    if rc < 0:
        raise ValueError("adamw_step: invalid arguments")
    return int(rc)


def adamw_step_no_master(hp: AdamWHp, param_bf16, exp_avg, exp_avg_sq, grad, norm_sq=None) -> int:
    """In-place step on a bf16 parameter with no fp32 master; 0 or 1 (skipped)."""
    _need(param_bf16, np.uint16, "param_bf16")
    for a, nm in ((exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq"), (grad, "grad")):
        _need(a, np.float32, nm)
        if a.size != param_bf16.size:
            raise ValueError("adamw_step_no_master: size mismatch")
    nsq = ctypes.c_double(float(norm_sq)) if norm_sq is not None else None
    rc = lib().orc_adamw_step_no_master(ctypes.byref(hp), _ptr(param_bf16), _ptr(exp_avg), _ptr(exp_avg_sq),
                                        _ptr(grad), param_bf16.size,
                                        ctypes.byref(nsq) if nsq is not None else None)
    if rc < 0:
        raise ValueError("adamw_step_no_master: invalid arguments")
    return int(rc)


def adam_update(hp: AdamWHp, exp_avg, exp_avg_sq, grad, update, norm_sq=None) -> int:
    """ZeRO-1 form: exp_avg / exp_avg_sq in place, the update vector into
    ``update``; 0 or 1 (skipped).  weight_decay must be 0."""
    for a, nm in ((exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq"), (grad, "grad"), (update, "update")):
        _need(a, np.float32, nm)
        if a.size != exp_avg.size:
            raise ValueError("adam_update: size mismatch")
    nsq = ctypes.c_double(float(norm_sq)) if norm_sq is not None else None
    rc = lib().orc_adam_update(ctypes.byref(hp), _ptr(exp_avg), _ptr(exp_avg_sq), _ptr(grad), _ptr(update),
                               exp_avg.size, ctypes.byref(nsq) if nsq is not None else None)
    if rc < 0:
        raise ValueError("adam_update: invalid arguments")
    return int(rc)


def flat_apply_update(update: np.ndarray, dsts, dst_dtype: int) -> None:
    """In place: dsts[i] += update[o_i : o_i + numel_i] (fp32 or bf16 tensors)."""
    _need(update, np.float32, "update")
    for d in dsts:
        _need(d, _np_dtype(dst_dtype), "dst")
    if sum(d.size for d in dsts) > update.size:
        raise ValueError("flat_apply_update: update shorter than the tensors")
    n = len(dsts)
    ptrs = (ctypes.c_void_p * max(n, 1))(*[d.ctypes.data for d in dsts])
    numel = (ctypes.c_int64 * max(n, 1))(*[d.size for d in dsts])
    rc = lib().orc_flat_apply_update(_ptr(update), ctypes.cast(ptrs, ctypes.c_void_p),
                                     ctypes.cast(numel, ctypes.c_void_p), n, dst_dtype)
    if rc != 0:
        raise ValueError("flat_apply_update: invalid arguments")


def state_tiled_numel(n: int, tile: int) -> int:
    """Floats of the tiled optimizer state for n elements (-1 if invalid)."""
    return int(lib().orc_state_tiled_numel(int(n), int(tile)))


def state_tile(master, exp_avg, exp_avg_sq, n: int, tile: int) -> np.ndarray:
    """The tiled state buffer of three fp32 arrays of n elements (None = zeros)."""
    srcs = []
    for a, nm in ((master, "master"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq")):
        if a is not None:
            _need(a, np.float32, nm)
            if a.size != n:
                raise ValueError(f"state_tile: {nm} size mismatch")
        srcs.append(a)
    total = state_tiled_numel(n, tile)
    if total < 0:
        raise ValueError("state_tile: invalid arguments")
    state = np.full(total, np.nan, dtype=np.float32)   # poison: every float must be written
    rc = lib().orc_state_tile(_ptr(srcs[0]), _ptr(srcs[1]), _ptr(srcs[2]), _ptr(state), int(n), int(tile))
    if rc != 0:
        raise ValueError("state_tile: invalid arguments")
    return state


def state_untile(state: np.ndarray, n: int, tile: int):
    """(master, exp_avg, exp_avg_sq) fp32 arrays of n elements from a tiled state."""
    _need(state, np.float32, "state")
    total = state_tiled_numel(n, tile)
    if total < 0 or state.size < total:
        raise ValueError("state_untile: state too small or invalid arguments")
    outs = [np.empty(int(n), dtype=np.float32) for _ in range(3)]
    rc = lib().orc_state_untile(_ptr(state), _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]), int(n), int(tile))
    if rc != 0:
        raise ValueError("state_untile: invalid arguments")
    return tuple(outs)


def moments_tiled_numel(n: int, tile: int) -> int:
    """Floats of the tiled moments (exp_avg, exp_avg_sq) for n elements (-1 if invalid)."""
    return int(lib().orc_moments_tiled_numel(int(n), int(tile)))


def moments_tile(exp_avg, exp_avg_sq, n: int, tile: int) -> np.ndarray:
    """The tiled moments buffer of two fp32 arrays of n elements (None = zeros)."""
    srcs = []
    for a, nm in ((exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq")):
        if a is not None:
            _need(a, np.float32, nm)
            if a.size != n:
                raise ValueError(f"moments_tile: {nm} size mismatch")
        srcs.append(a)
    total = moments_tiled_numel(n, tile)
    if total < 0:
        raise ValueError("moments_tile: invalid arguments")
    buf = np.full(total, np.nan, dtype=np.float32)   # poison: every float must be written
    if lib().orc_moments_tile(_ptr(srcs[0]), _ptr(srcs[1]), _ptr(buf), int(n), int(tile)) != 0:
        raise ValueError("moments_tile: invalid arguments")
    return buf


def moments_untile(buf: np.ndarray, n: int, tile: int):
    """(exp_avg, exp_avg_sq) fp32 arrays of n elements from tiled moments."""
    _need(buf, np.float32, "moments")
    total = moments_tiled_numel(n, tile)
    if total < 0 or buf.size < total:
        raise ValueError("moments_untile: buffer too small or invalid arguments")
    outs = [np.empty(int(n), dtype=np.float32) for _ in range(2)]
    if lib().orc_moments_untile(_ptr(buf), _ptr(outs[0]), _ptr(outs[1]), int(n), int(tile)) != 0:
        raise ValueError("moments_untile: invalid arguments")
    return tuple(outs)
