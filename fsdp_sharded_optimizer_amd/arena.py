"""One physically contiguous block of device memory for a rank's buffers.

A rank allocates its optimizer state, accumulator, gradients and parameter
shard once and streams them every step.  On gfx950 the step's bandwidth
depends on where those buffers land in device memory: allocated one by one
after other processes have allocated and freed memory, the same kernels ran
at 79-82 % of the HBM peak where, carved from one physically contiguous
block (hipExtMallocWithFlags with hipDeviceMallocContiguous), they ran at
85 % on a fresh device and after such a process alike (the buffers' offsets
inside the block did not matter).  ``DeviceArena`` holds such a block and
hands out aligned torch views of it; it computes nothing.

Such a block is not cached in the L2 like an ordinary allocation: writing
64 MiB into one made about 3 thousand L2 requests, against about a million
for an ordinary allocation (rocprofv3, TCC_HIT + TCC_MISS).  Freeing device
memory of that kind has left later allocations holding stale values on this
hardware (a fresh tensor read back its pre-kernel contents after arenas had
been freed), so a contiguous block is never returned to the driver: when the
arena and every view of it are gone (each view keeps the arena alive), the
block goes to a per-process pool, and a later arena on the same device that
fits in it reuses it after a device synchronisation (so work still queued
on the old views ends first).  Each device holds
its pooled blocks until the process ends.  When the runtime cannot give a
contiguous block (device memory too fragmented), the arena falls back to an
ordinary allocation of the same size, says so in ``contiguous``, and frees
it normally.
"""
from __future__ import annotations

import ctypes
import sys

import torch

from . import _binding

HIP_DEVICE_MALLOC_DEFAULT = 0x0
HIP_DEVICE_MALLOC_CONTIGUOUS = 0x4
ALIGN = 2 << 20   # every view starts on a 2 MiB boundary of the block

_hip = None


def _runtime() -> ctypes.CDLL:
    """The HIP runtime the library's kernels run on: its symbols resolved
    through the library's own handle (torch loads the same runtime)."""
    global _hip
    if _hip is None:
        torch.cuda.init()
        _binding.lib()   # raises if the library has not been built
        L = ctypes.CDLL(_binding.LIB_PATH)
        L.hipExtMallocWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t, ctypes.c_uint]
        L.hipExtMallocWithFlags.restype = ctypes.c_int
        L.hipFree.argtypes = [ctypes.c_void_p]
        L.hipFree.restype = ctypes.c_int
        L.hipDeviceSynchronize.argtypes = []
        L.hipDeviceSynchronize.restype = ctypes.c_int
        L.hipGetLastError.argtypes = []
        L.hipGetLastError.restype = ctypes.c_int
        _hip = L
    return _hip


class _View:
    """A CUDA-array-interface provider for one slice of the block; holds the
    arena so the block outlives every tensor made from it."""

    def __init__(self, arena: "DeviceArena", ptr: int, numel: int, typestr: str):
        self.arena = arena
        self.__cuda_array_interface__ = {"shape": (numel,), "typestr": typestr, "data": (ptr, False),
                                         "version": 2, "strides": None}


_TYPESTR = {torch.float32: "<f4", torch.float64: "<f8", torch.uint8: "|u1", torch.int16: "<i2"}


_pool = {}   # device index -> [(capacity, ptr)] contiguous blocks held for the process's lifetime


def pooled_blocks(device=None) -> list:
    """(capacity, ptr) of the contiguous blocks pooled for reuse on a device
    (the current one by default)."""
    d = torch.device("cuda") if device is None else torch.device(device)
    return list(_pool.get(torch.cuda.current_device() if d.index is None else d.index, []))


class DeviceArena:
    """``nbytes`` of device memory on ``device`` in one block, physically
    contiguous when the runtime can give it.  ``take(numel, dtype)`` returns
    the next view, starting on a 2 MiB boundary."""

    def __init__(self, nbytes: int, device: torch.device, contiguous: bool = True):
        self.ptr = None
        device = torch.device(device)
        if device.type != "cuda":
            raise TypeError(f"DeviceArena: {device} is not a GPU")
        L = _runtime()
        self.device = torch.device("cuda", torch.cuda.current_device() if device.index is None else device.index)
        self.nbytes = int(nbytes)
        if self.nbytes <= 0:
            raise ValueError("DeviceArena: nbytes must be positive")
        self.contiguous = False
        if contiguous:
            pool = _pool.setdefault(self.device.index, [])
            fits = [b for b in pool if b[0] >= self.nbytes]
            if fits:   # the smallest pooled block that holds the request
                block = min(fits)
                with torch.cuda.device(self.device):
                    rc = L.hipDeviceSynchronize()   # work queued on the block's last views has ended
                if rc != 0:
                    raise RuntimeError(f"DeviceArena: hipDeviceSynchronize returned {rc}")
                pool.remove(block)
                self.capacity, self.ptr = block
                self.contiguous = True
        if self.ptr is None:
            p = ctypes.c_void_p()
            with torch.cuda.device(self.device):
                rc = -1
                if contiguous:
                    rc = L.hipExtMallocWithFlags(ctypes.byref(p), self.nbytes, HIP_DEVICE_MALLOC_CONTIGUOUS)
                    if rc != 0:
                        L.hipGetLastError()   # clear the failed call's error before the fallback
                self.contiguous = contiguous and rc == 0
                if rc != 0:
                    rc = L.hipExtMallocWithFlags(ctypes.byref(p), self.nbytes, HIP_DEVICE_MALLOC_DEFAULT)
                    if rc != 0:
                        L.hipGetLastError()
                        raise torch.cuda.OutOfMemoryError(f"DeviceArena: {self.nbytes} bytes (hipError {rc})")
            self.ptr, self.capacity = p.value, self.nbytes
        self.used = 0

    @staticmethod
    def size(parts) -> int:
        """Bytes an arena needs for views of these (numel, dtype) parts."""
        total = 0
        for numel, dtype in parts:
            total += -(-int(numel) * torch.empty(0, dtype=dtype).element_size() // ALIGN) * ALIGN
        return max(total, ALIGN)

    def take(self, numel: int, dtype: torch.dtype) -> torch.Tensor:
        """The next ``numel`` elements of ``dtype`` (1-D view, uninitialised)."""
        if dtype != torch.bfloat16 and dtype not in _TYPESTR:
            raise TypeError(f"DeviceArena: unsupported dtype {dtype}")
        numel = int(numel)
        if numel < 0:
            raise ValueError("DeviceArena: numel must be >= 0")
        nbytes = numel * torch.empty(0, dtype=dtype).element_size()
        if self.used + nbytes > self.nbytes:
            raise ValueError(f"DeviceArena: {nbytes} more bytes do not fit ({self.used} of {self.nbytes} used)")
        ptr = self.ptr + self.used
        self.used += -(-nbytes // ALIGN) * ALIGN
        if dtype == torch.bfloat16:   # the interface has no bf16 type string: int16, then a view
            return torch.as_tensor(_View(self, ptr, numel, "<i2"), device=self.device).view(torch.bfloat16)
        return torch.as_tensor(_View(self, ptr, numel, _TYPESTR[dtype]), device=self.device)

    def __del__(self):
        ptr, self.ptr = getattr(self, "ptr", None), None
        if ptr is None or sys.is_finalizing():
            return   # nothing held, or the interpreter is shutting down: the process's end frees the block
        if self.contiguous:
            # back to the pool as it is (no synchronisation here, so dropping
            # an arena never blocks); the arena that takes it back synchronises
            _pool.setdefault(self.device.index, []).append((self.capacity, ptr))
            return
        with torch.cuda.device(self.device):
            _hip.hipDeviceSynchronize()   # work queued on the views ends before the block is freed
            _hip.hipFree(ctypes.c_void_p(ptr))
