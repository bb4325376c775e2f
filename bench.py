#!/usr/bin/env python3
"""Benchmark of the per-rank ZeRO/FSDP optimizer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole hot path over one batch of synthetic
input, on one rank's real-size shard (inputs resident in HBM):
  grad_accum over every micro-batch but the last (bf16 -> fp32),
  grad_accum_norm_sq for the last one (the accumulation and this shard's
  squared norm in one pass; the norm is formed every step: it feeds the clip
  when the workload clips and the non-finite skip always), and the fused
  AdamW step with the bf16 re-cast, on the optimizer state held in the
  library's tiled layout (adamw_step_tiled, as ShardOptimizer holds it by
  default).  The same AdamW step on three separate state buffers
  (adamw_step) is timed after the step on the same evolved state.
The shard range is host arithmetic done once at set-up.  Default workload:
the Llama-7B-shaped buffer over 8 ranks, one 842,301,952-element shard,
8 micro-batches.

Prints ONE JSON line: whole-step throughput (shard elements per second),
the roofline of the dominant kernel (adamw_step_tiled, timed live with HIP
events on the launch stream) and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X published HBM3E bandwidth

# HBM bytes per AdamW launch (adamw_step_tiled, the step's kernel, and
# adamw_step, the same step on split buffers), per shard size (the Llama-7B
# shard and the 70B ZeRO-3 shard), from two rocprofv3 --pmc runs of this script for that
# workload (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what
# the same counter reads for the 4 GiB device copy this script also runs
# (FETCH_SIZE reads about 2,097,194 KiB for it: x2.0; WRITE_SIZE reads
# 4,194,304 KiB: x1.0).  Valid only for the kernel source it was taken on: the
# hash covers the kernel file and its header.
PMC_SOURCES = ("csrc/adamw.hip", "csrc/zs_common.h")
PMC_TRAFFIC = {
    "adamw_step_tiled": [
        {"sha256_16": "7122c719bce82d1d", "shard_elems": 842301952,
         "fetch_kib": 6580552.4, "fetch_scale": 2.0, "write_kib": 11515857.7, "write_scale": 1.0},
        {"sha256_16": "7122c719bce82d1d", "shard_elems": 1093750000,
         "fetch_kib": 8545002.6, "fetch_scale": 2.0, "write_kib": 14953618.9, "write_scale": 1.0},
    ],
    "adamw_step": [
        {"sha256_16": "7122c719bce82d1d", "shard_elems": 842301952,
         "fetch_kib": 6580517.5, "fetch_scale": 2.0, "write_kib": 11515853.2, "write_scale": 1.0},
        {"sha256_16": "7122c719bce82d1d", "shard_elems": 1093750000,
         "fetch_kib": 8544955.5, "fetch_scale": 2.0, "write_kib": 14953618.7, "write_scale": 1.0},
    ],
}


def pmc_traffic(kernel: str, n: int):
    """Measured HBM bytes per launch, or None if there is no record for this
    shard size or the kernel changed since it was taken."""
    import hashlib
    recs = [r for r in PMC_TRAFFIC.get(kernel, []) if r["shard_elems"] == n]
    if not recs:
        return None
    rec = recs[0]
    h = hashlib.sha256()
    for rel in PMC_SOURCES:
        with open(os.path.join(ROOT, "fsdp_sharded_optimizer_amd", rel), "rb") as f:
            h.update(f.read())
    if h.hexdigest()[:16] != rec["sha256_16"]:
        return None
    return rec["fetch_kib"] * 1024 * rec["fetch_scale"] + rec["write_kib"] * 1024 * rec["write_scale"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class DeviceEvent:
    """A timing HIP event recorded with a device-scope release
    (hipEventReleaseToDevice).  A default event's system-scope release makes
    its timestamp wait for a write-back of the GPU caches, which lands inside
    the timed interval; with a device-scope release the interval between two
    events is the work between them.  Same interface as torch.cuda.Event;
    created through the HIP runtime torch has loaded (one runtime per
    process).  FLAGS falls back to 0 (a default event) if the runtime
    refuses the flag, and the JSON line says which was used."""
    RELEASE_TO_DEVICE = 0x40000000
    FLAGS = None
    _hip = None

    @classmethod
    def hip(cls):
        if cls._hip is None:
            import ctypes
            import torch
            torch.cuda.init()
            path = None
            with open("/proc/self/maps") as f:
                for line in f:
                    if "libamdhip64.so" in line:
                        path = line.split()[-1]
                        break
            if path is None:
                raise RuntimeError("the HIP runtime is not loaded")
            L = ctypes.CDLL(path)
            L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            L.hipEventDestroy.argtypes = [ctypes.c_void_p]
            for fn in ("hipEventCreateWithFlags", "hipEventRecord", "hipEventElapsedTime", "hipEventDestroy"):
                getattr(L, fn).restype = ctypes.c_int
            probe = ctypes.c_void_p()
            if L.hipEventCreateWithFlags(ctypes.byref(probe), cls.RELEASE_TO_DEVICE) == 0:
                cls.FLAGS = cls.RELEASE_TO_DEVICE
                L.hipEventDestroy(probe)
            else:
                cls.FLAGS = 0
            cls._hip = L
        return cls._hip

    def __init__(self):
        import ctypes
        self._ct = ctypes
        self.h = ctypes.c_void_p()
        rc = self.hip().hipEventCreateWithFlags(ctypes.byref(self.h), self.FLAGS)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags returned {rc}")

    def record(self, stream=None):
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        rc = self.hip().hipEventRecord(self.h, self._ct.c_void_p(s.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord returned {rc}")

    def elapsed_time(self, end: "DeviceEvent") -> float:
        ms = self._ct.c_float()
        rc = self.hip().hipEventElapsedTime(self._ct.byref(ms), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime returned {rc}")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.h:
            self._hip.hipEventDestroy(self.h)


def timing_events() -> str:
    DeviceEvent.hip()
    return "hipEventReleaseToDevice" if DeviceEvent.FLAGS else "default (system-scope release)"


def step_bytes_per_elem(w) -> dict:
    """Algorithmic HBM bytes per shard element of each kernel of one step."""
    g = 2 if w.grad_dtype == "bf16" else 4
    accum_first = g + 4
    accum_next = g + 8
    adamw = 28 + (2 if w.bf16_param else 0)
    # the last micro-batch also forms the norm, without another read
    accum = accum_first + (w.micro_batches - 1) * accum_next
    last = accum_first if w.micro_batches == 1 else accum_next
    return {"grad_accum_first": accum_first, "grad_accum_next": accum_next,
            "grad_accum_norm_sq_last": last, "adamw_step": adamw, "step": accum + adamw}


def step_kernel_rates(bpe: dict, n: int, r: dict) -> dict:
    """Algorithmic bandwidth of each part of the timed step (HIP events on
    the launch stream): the accumulations of every micro-batch but the last
    (one overwriting launch and the rest accumulating, by time the largest
    share of the step), the last micro-batch with the norm, and AdamW."""
    parts = {
        "grad_accum_all_but_last": (bpe["step"] - bpe["grad_accum_norm_sq_last"] - bpe["adamw_step"], r["accum_ms"]),
        "grad_accum_norm_sq_last": (bpe["grad_accum_norm_sq_last"], r["last_ms"]),
        "adamw_step_tiled": (bpe["adamw_step"], r["adamw_ms"]),
    }
    out = {}
    for name, (b, ms) in parts.items():
        gbps = b * n / (ms * 1e-3) / 1e9 if (ms > 0 and b > 0) else None
        out[name] = {"bytes_per_elem": b, "ms": ms, "gbps": gbps,
                     "frac": gbps / HBM_PEAK_GBPS if gbps is not None else None}
    return out


def ceiling_report(ms_by_lds: dict, nbytes: int, adamw_ms: float) -> dict:
    """The AdamW-traffic kernel's time at each residency cap, its best, and
    the AdamW step's bandwidth as a fraction of that best."""
    best = min(ms_by_lds, key=ms_by_lds.get)
    gbps = nbytes / (ms_by_lds[best] * 1e-3) / 1e9
    return {"kernel": "zsc_adamw_traffic", "algorithmic_bytes": nbytes,
            "ms_by_lds_bytes": {str(k): v for k, v in ms_by_lds.items()},
            "best_lds_bytes": best, "gbps": gbps, "frac": gbps / HBM_PEAK_GBPS,
            "adamw_step_of_ceiling": ms_by_lds[best] / adamw_ms}


def shard_len(w) -> int:
    import fsdp_sharded_optimizer_amd as zs
    _, start, end, _ = zs.zero_shard_range(w.total, w.world, w.rank)
    return end - start


# ---------------------------------------------------------------------------
# GPU leg
# ---------------------------------------------------------------------------

def run_gpu(w, steps: int, warmup: int):
    import torch
    import workloads
    import fsdp_sharded_optimizer_amd as zs

    n = shard_len(w)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log(f"[bench] workload={w.name} shard_elems={n} micro_batches={w.micro_batches}")
    master = workloads.master_init(w, n, dev)
    param = master.to(torch.bfloat16) if w.bf16_param else None
    # the step's optimizer state, tiled: master values in, moments zero
    state = torch.empty(zs.state_tiled_numel(n), dtype=torch.float32, device=dev)
    zs.state_tile(master, None, None, state)
    # split buffers: the adamw_step comparison and the no-master variant
    exp_avg = torch.zeros(n, dtype=torch.float32, device=dev)
    exp_avg_sq = torch.zeros(n, dtype=torch.float32, device=dev)
    acc = torch.empty(n, dtype=torch.float32, device=dev)
    grads = [workloads.grad_draw(w, n, 1, mb, dev) for mb in range(w.micro_batches)]
    norm = torch.zeros(1, dtype=torch.float64, device=dev)
    ws = torch.empty(max(zs.grad_accum_norm_sq_workspace_bytes(n), zs.grad_norm_sq_workspace_bytes(n),
                         zs.grad_reduce_chunks_norm_sq_workspace_bytes(n), 8), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs resident: {torch.cuda.memory_allocated() / 2**30:.1f} GiB")

    ev = DeviceEvent
    timing = []   # per step: (start, last micro-batch start, adamw start, adamw end)
    last = len(grads) - 1

    def step_hp(t: int):
        return zs.AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                              weight_decay=w.weight_decay, grad_scale=w.grad_scale,
                              max_norm=w.max_norm, extra_norm_sq=workloads.other_ranks_norm_sq(w, 1, n),
                              step=t)

    def one_step(t: int, record: bool):
        e = [ev() for _ in range(4)] if record else None
        if record:
            e[0].record()
        for mb, g in enumerate(grads[:last]):
            zs.grad_accum(acc, g, overwrite=(mb == 0))
        if record:
            e[1].record()
        zs.grad_accum_norm_sq(acc, grads[last], last == 0, w.grad_scale, norm, ws)
        if record:
            e[2].record()
        zs.adamw_step_tiled(step_hp(t), state, acc, param, norm_sq=norm)
        if record:
            e[3].record()
            timing.append(e)

    t = 0
    for _ in range(warmup):
        t += 1
        one_step(t, record=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        t += 1
        one_step(t, record=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    acc_ms = sum(e[0].elapsed_time(e[1]) for e in timing) / steps
    last_ms = sum(e[1].elapsed_time(e[2]) for e in timing) / steps
    adamw_ms = sum(e[2].elapsed_time(e[3]) for e in timing) / steps
    assert math.isfinite(norm.item()), "non-finite gradient norm in the bench"

    # outside the step: the same step captured once in a HIP graph and
    # replayed (the library allocates, clears and synchronises nothing, so
    # the step captures as is; launch overhead matters for small shards)
    graph_ms = None
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one_step(t + 1, record=False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one_step(t + 1, record=False)
    graph.replay()
    g0, g1 = ev(), ev()
    g0.record()
    for _ in range(steps):
        graph.replay()
    g1.record()
    torch.cuda.synchronize()
    graph_ms = g0.elapsed_time(g1) / steps
    del graph

    # outside the step: the same AdamW step on three separate state buffers
    # (adamw_step), loaded with the tiled state as the timed steps left it so
    # both layouts stream the same values
    zs.state_untile(state, master, exp_avg, exp_avg_sq)
    split_ms = []
    for k in range(steps):
        e0, e1 = ev(), ev()
        e0.record()
        zs.adamw_step(step_hp(t + 1 + k), master, exp_avg, exp_avg_sq, acc, param, norm_sq=norm)
        e1.record()
        split_ms.append((e0, e1))
    torch.cuda.synchronize()
    split_ms = sum(a.elapsed_time(b) for a, b in split_ms) / steps

    # outside the step: the reduce-scatter's arithmetic on this rank's shard,
    # the same buffers read as N rank chunks, in one pass
    reduce_ms = None
    if len(grads) > 1:
        r0, r1 = ev(), ev()
        zs.grad_reduce_chunks(acc, grads, True)
        r0.record()
        for _ in range(3):
            zs.grad_reduce_chunks(acc, grads, True)
        r1.record()
        torch.cuda.synchronize()
        reduce_ms = r0.elapsed_time(r1) / 3

    # outside the step: the same step with the step's micro-batch gradients
    # all kept in device memory (ShardOptimizer.accumulate_all): one pass sums
    # them (bit-identical accumulator) and forms the norm, then the same
    # AdamW on the tiled state
    staged_ms = None
    if len(grads) > 1:
        def staged(tt: int):
            zs.grad_reduce_chunks_norm_sq(acc, grads, True, w.grad_scale, norm, ws)
            zs.adamw_step_tiled(step_hp(tt), state, acc, param, norm_sq=norm)

        staged(t + 1)
        s0, s1 = ev(), ev()
        s0.record()
        for k in range(steps):
            staged(t + 2 + k)
        s1.record()
        torch.cuda.synchronize()
        staged_ms = s0.elapsed_time(s1) / steps
        t += 1 + steps

    # outside the step: the standalone squared norm over the accumulated
    # gradient (4 B/element), as when the gradient arrives from a
    # reduce-scatter instead of this rank's own accumulation
    n0, n1 = ev(), ev()
    zs.grad_norm_sq(acc, w.grad_scale, norm, ws)
    n0.record()
    for _ in range(5):
        zs.grad_norm_sq(acc, w.grad_scale, norm, ws)
    n1.record()
    torch.cuda.synchronize()
    norm_ms = n0.elapsed_time(n1) / 5

    # outside the step: the variant with no fp32 master (24 B/element), on the
    # same buffers (state after the timed steps), then on tiled moments
    no_master_ms = no_master_tiled_ms = None
    if param is not None:
        def time_no_master(fn):
            hp = zs.AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                                grad_scale=w.grad_scale, step=t + 1)
            fn(hp)
            n0, n1 = ev(), ev()
            n0.record()
            for k in range(3):
                hp.step = t + 2 + k
                fn(hp)
            n1.record()
            torch.cuda.synchronize()
            return n0.elapsed_time(n1) / 3

        no_master_ms = time_no_master(lambda hp: zs.adamw_step_no_master(hp, param, exp_avg, exp_avg_sq, acc))
        moments = torch.empty(zs.moments_tiled_numel(n), dtype=torch.float32, device=dev)
        zs.moments_tile(exp_avg, exp_avg_sq, moments)
        no_master_tiled_ms = time_no_master(lambda hp: zs.adamw_step_no_master_tiled(hp, param, moments, acc))
        del moments

    # achievable-bandwidth reference for the AdamW step's own traffic: the
    # same bytes per element and accesses, one addition per stream in place
    # of the update, at several residency caps (run last on these buffers:
    # it changes them)
    ceiling = {lds: _time_adamw_traffic(state, None, None, acc, param, n, lds, tiled=True)
               for lds in CEILING_LDS}
    ceiling_split = {lds: _time_adamw_traffic(master, exp_avg, exp_avg_sq, acc, param, n, lds)
                     for lds in CEILING_LDS}

    # achievable-bandwidth reference: a plain device copy of 4 GiB (also the
    # calibration kernel for the HBM byte counters)
    src = torch.empty(1 << 30, dtype=torch.float32, device=dev)
    src.fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = ev(), ev()
    c0.record()
    for _ in range(5):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_ms = c0.elapsed_time(c1) / 5
    copy_gbps = 2 * src.numel() * 4 / (copy_ms * 1e-3) / 1e9
    del src, dst
    return {"n": n, "wall_s": wall, "accum_ms": acc_ms, "last_ms": last_ms, "adamw_ms": adamw_ms, "graph_ms": graph_ms,
            "split_ms": split_ms, "reduce_ms": reduce_ms, "staged_ms": staged_ms, "chunks": len(grads),
            "no_master_ms": no_master_ms,
            "no_master_tiled_ms": no_master_tiled_ms,
            "copy_gbps": copy_gbps, "ceiling_ms": ceiling, "ceiling_split_ms": ceiling_split, "norm_ms": norm_ms}


CEILING_LDS = (0, 8192, 12288, 14336, 16384, 20480)   # LDS reserved per one-wave workgroup


def _time_adamw_traffic(master, exp_avg, exp_avg_sq, grad, bf16, n: int, lds: int, reps: int = 5,
                        tiled: bool = False) -> float:
    """Average launch time of the AdamW-traffic ceiling kernel
    (libzsceiling.so, built next to libzshard.so), each launch bracketed by
    HIP events on the stream it runs on.  tiled: `master` is the tiled state
    buffer and the kernel walks that layout."""
    import ctypes
    import torch
    from fsdp_sharded_optimizer_amd import build as zbuild

    if not os.path.exists(zbuild.CEILING_LIB):
        raise RuntimeError(f"{zbuild.CEILING_LIB} is not built: run python -m fsdp_sharded_optimizer_amd.build")
    lib = ctypes.CDLL(zbuild.CEILING_LIB)
    stream = torch.cuda.current_stream()
    bptr = bf16.data_ptr() if bf16 is not None else None
    if tiled:
        f = lib.zsc_adamw_traffic_tiled
        f.restype = ctypes.c_int32
        f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]
        args = [master.data_ptr(), grad.data_ptr(), bptr, n, lds, stream.cuda_stream]
    else:
        f = lib.zsc_adamw_traffic
        f.restype = ctypes.c_int32
        f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]
        args = [master.data_ptr(), exp_avg.data_ptr(), exp_avg_sq.data_ptr(), grad.data_ptr(), bptr, n, lds,
                stream.cuda_stream]
    events = []
    for k in range(reps + 1):
        e0, e1 = DeviceEvent(), DeviceEvent()
        e0.record(stream)
        rc = f(*args)
        e1.record(stream)
        if rc != 0:
            raise RuntimeError(f"zsc_adamw_traffic returned {rc}")
        if k:
            events.append((e0, e1))
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in events) / reps


def run_flat(w, reps: int = 10):
    """FSDP unit: time flat_pack of the unit's tensors into the padded flat
    bf16 buffer and flat_unpack back (4 B per element each), then the two
    conversions: the widening pack into an fp32 flat buffer (the master's
    initialisation) and the re-casting unpack from it (6 B per element
    each)."""
    import torch
    import workloads
    import fsdp_sharded_optimizer_amd as zs

    dev = torch.device("cuda", 0)
    params = workloads.unit_tensors(w, dev)
    _, _, _, padded = zs.zero_shard_range(w.total, w.world, w.rank)
    flat = torch.empty(padded, dtype=torch.bfloat16, device=dev)
    outs = [torch.empty_like(p) for p in params]
    ev = DeviceEvent
    zs.flat_pack(params, flat, padded)
    zs.flat_unpack(flat, outs)
    e = [ev() for _ in range(3)]
    e[0].record()
    for _ in range(reps):
        zs.flat_pack(params, flat, padded)
    e[1].record()
    for _ in range(reps):
        zs.flat_unpack(flat, outs)
    e[2].record()
    torch.cuda.synchronize()
    pack_ms = e[0].elapsed_time(e[1]) / reps
    unpack_ms = e[1].elapsed_time(e[2]) / reps
    assert all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(params, outs))
    del flat
    flat32 = torch.empty(padded, dtype=torch.float32, device=dev)
    zs.flat_pack(params, flat32, padded)
    zs.flat_unpack(flat32, outs)
    e[0].record()
    for _ in range(reps):
        zs.flat_pack(params, flat32, padded)
    e[1].record()
    for _ in range(reps):
        zs.flat_unpack(flat32, outs)
    e[2].record()
    torch.cuda.synchronize()
    widen_ms = e[0].elapsed_time(e[1]) / reps
    recast_ms = e[1].elapsed_time(e[2]) / reps
    assert all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(params, outs))
    bytes_ = 4 * w.total
    gbps = lambda b, ms: b / (ms * 1e-3) / 1e9
    return {"tensors": len(params), "elements": w.total, "padded": padded,
            "pack_ms": pack_ms, "unpack_ms": unpack_ms,
            "pack_gbps": gbps(bytes_, pack_ms), "unpack_gbps": gbps(bytes_, unpack_ms),
            "widen_pack_ms": widen_ms, "recast_unpack_ms": recast_ms,
            "widen_pack_gbps": gbps(6 * w.total, widen_ms), "recast_unpack_gbps": gbps(6 * w.total, recast_ms)}


def run_zero1_flow(w, shapes, reps: int = 3):
    """The ZeRO page's ZeRO-1 flow at the same model size: the full fp32
    gradient resident as one flat buffer, this rank's adam_update on its
    slice writing its chunk of the gathered update (24 B per shard element),
    and flat_apply_update of the whole gathered update into every parameter
    tensor of the model: bf16 parameters (8 B per model element) and fp32
    parameters (12 B).  Values are synthetic; the timing has no data
    dependence."""
    import torch
    import fsdp_sharded_optimizer_amd as zs

    dev = torch.device("cuda", 0)
    chunk, start, end, padded = zs.zero_shard_range(w.total, w.world, w.rank)
    n = end - start
    flat_grad = torch.empty(padded, dtype=torch.float32, device=dev).normal_(0.0, 1e-3)
    gathered = torch.empty(padded, dtype=torch.float32, device=dev).normal_(0.0, 1e-5)
    m = torch.zeros(n, dtype=torch.float32, device=dev)
    v = torch.zeros(n, dtype=torch.float32, device=dev)
    mine = gathered[w.rank * chunk:w.rank * chunk + n]
    ev = DeviceEvent

    def timed(fn):
        fn(0)
        e0, e1 = ev(), ev()
        e0.record()
        for k in range(reps):
            fn(k + 1)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def update(k):
        hp = zs.AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=0.0,
                            grad_scale=1.0 / w.world, step=k + 1)
        zs.adam_update(hp, m, v, flat_grad[start:end], mine)

    upd_ms = timed(update)
    # the same update with the rank's moments tiled (two runs per tile)
    moments = torch.empty(zs.moments_tiled_numel(n), dtype=torch.float32, device=dev)
    zs.moments_tile(m, v, moments)

    def update_tiled(k):
        hp = zs.AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=0.0,
                            grad_scale=1.0 / w.world, step=k + 1)
        zs.adam_update_tiled(hp, moments, flat_grad[start:end], mine)

    upd_tiled_ms = timed(update_tiled)
    del m, v, flat_grad, moments
    out = {"workload": f"{w.name} as ZeRO-1: full flat fp32 grad and gathered update of {w.total} elements, "
                       f"rank {w.rank} of {w.world}",
           "tensors": len(shapes),
           "adam_update": {"ms": upd_ms, "elements": n, "bytes_per_elem": 24,
                           "gbps": 24 * n / (upd_ms * 1e-3) / 1e9},
           "adam_update_tiled": {"ms": upd_tiled_ms, "elements": n, "bytes_per_elem": 24,
                                 "gbps": 24 * n / (upd_tiled_ms * 1e-3) / 1e9}}
    from workloads import numel_of
    for dtype, bpe, key in ((torch.bfloat16, 8, "apply_bf16"), (torch.float32, 12, "apply_f32")):
        buf = torch.empty(w.total, dtype=dtype, device=dev).uniform_(-0.1, 0.1)
        params, off = [], 0
        for _, shp in shapes:
            k = numel_of(shp)
            params.append(buf[off:off + k].view(shp))
            off += k
        assert off == w.total
        ms = timed(lambda k: zs.flat_apply_update(gathered, params))
        assert bool(torch.isfinite(buf[:: 1 << 20]).all())
        out[key] = {"ms": ms, "elements": w.total, "bytes_per_elem": bpe,
                    "gbps": bpe * w.total / (ms * 1e-3) / 1e9}
        del params, buf
    del gathered, mine
    return out


# ---------------------------------------------------------------------------
# CPU baseline leg: the oracle as it stands on a bounded sample
# ---------------------------------------------------------------------------

def run_cpu_baseline(w, target_s: float = 10.0, sample: int = 1 << 25):
    import numpy as np
    import torch
    import oracle
    import workloads

    n = sample
    master = workloads.master_init(w, n, "cpu").numpy().copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    bf = np.zeros(n, np.uint16) if w.bf16_param else None
    code = oracle.BF16 if w.grad_dtype == "bf16" else oracle.F32
    grads = []
    for mb in range(w.micro_batches):
        g = workloads.grad_draw(w, n, 1, mb, "cpu")
        grads.append(g.view(torch.int16).numpy().view(np.uint16).copy() if code == oracle.BF16
                     else g.numpy().copy())
    acc = np.empty(n, np.float32)
    done = 0
    phase = {"accumulate": 0.0, "norm": 0.0, "adamw": 0.0}
    t0 = time.perf_counter()
    while True:
        ta = time.perf_counter()
        for mb, g in enumerate(grads):
            oracle.grad_accum(acc, g, code, overwrite=(mb == 0))
        tb = time.perf_counter()
        s = oracle.grad_norm_sq(acc, w.grad_scale)   # the oracle has no fused form
        tc = time.perf_counter()
        hp = oracle.make_hp(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, w.grad_scale, w.max_norm,
                            workloads.other_ranks_norm_sq(w, 1, n), done + 1)
        oracle.adamw_step(hp, master, m, v, acc, bf, norm_sq=s)
        td = time.perf_counter()
        phase["accumulate"] += tb - ta
        phase["norm"] += tc - tb
        phase["adamw"] += td - tc
        done += 1
        el = time.perf_counter() - t0
        if el >= target_s or done >= 1000:
            break
    bpe = step_bytes_per_elem(w)
    accum_bytes = bpe["step"] - bpe["adamw_step"]   # every micro-batch's accumulation
    phases = {
        "accumulate": {"ms_per_step": phase["accumulate"] * 1e3 / done,
                       "gbps": accum_bytes * n * done / phase["accumulate"] / 1e9},
        "norm": {"ms_per_step": phase["norm"] * 1e3 / done, "gbps": 4 * n * done / phase["norm"] / 1e9},
        "adamw": {"ms_per_step": phase["adamw"] * 1e3 / done,
                  "gbps": bpe["adamw_step"] * n * done / phase["adamw"] / 1e9},
    }
    return {"value": n * done / el, "unit": "elements/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{n} elements of the same workload (first {n} of a shard drawn by the same "
                      f"recipe on the CPU), {done} whole steps ({w.micro_batches} micro-batch "
                      f"accumulations + norm + AdamW/bf16) in {el:.1f} s",
            "phases": phases}


def _staged(r, n: int, w) -> dict:
    """The step with its micro-batch gradients staged in device memory: the
    one-pass sum with the norm (gradient bytes per micro-batch + 4 written)
    and AdamW (30), timed back to back over the bench's step count."""
    bpe = r["chunks"] * (2 if w.grad_dtype == "bf16" else 4) + 4 + 30
    gbps = bpe * n / (r["staged_ms"] * 1e-3) / 1e9
    return {"ms": r["staged_ms"], "elements_per_s": n / (r["staged_ms"] * 1e-3), "bytes_per_elem": bpe,
            "gbps": gbps, "frac": gbps / HBM_PEAK_GBPS,
            "staged_grad_bytes_per_elem": r["chunks"] * (2 if w.grad_dtype == "bf16" else 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama7b_shard")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--no-zero1", action="store_true", help="skip the ZeRO-1 flow timing")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU's shard only; --gpus {args.gpus} is not "
              "supported (collectives are out of scope). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import workloads
    if args.workload not in workloads.WORKLOADS:
        sys.exit(f"unknown workload {args.workload}; one of {sorted(workloads.WORKLOADS)}")
    w = workloads.WORKLOADS[args.workload]

    import fsdp_sharded_optimizer_amd as zs
    zs.lib()

    r = run_gpu(w, args.steps, args.warmup)
    n = r["n"]
    flat = None
    if w.unit_shapes:
        import torch
        torch.cuda.empty_cache()
        flat = run_flat(w)
    zero1 = None
    if w.name == "llama7b_shard" and not args.no_zero1:
        import torch
        torch.cuda.empty_cache()
        zero1 = run_zero1_flow(w, workloads.LLAMA7B)
    bpe = step_bytes_per_elem(w)
    ms_per_step = r["wall_s"] * 1e3 / args.steps
    adamw_bytes = bpe["adamw_step"] * n
    achieved = adamw_bytes / (r["adamw_ms"] * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host cores ...")
        cpu = run_cpu_baseline(w, args.cpu_seconds)
    step_gbps = bpe["step"] * n / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": "AdamW shard step: elements/s and achieved HBM GB/s (% of peak) per GPU",
        "value": n / (ms_per_step * 1e-3),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded U(-0.1,0.1) master, N(0,std) bf16 micro-batch grads)",
        "config": {"workload": w.name, "shard_elems": n, "total_params": w.total, "world": w.world,
                   "rank": w.rank, "micro_batches": w.micro_batches, "grad_dtype": w.grad_dtype,
                   "state": "fp32 master/exp_avg/exp_avg_sq (tiled layout) + bf16 param", "clip": w.max_norm > 0},
        "graph_ms_per_step": r["graph_ms"],
        "step_hbm_gbps": step_gbps,
        "step_hbm_frac": step_gbps / HBM_PEAK_GBPS,
        "kernels_ms": {"grad_accum_all_but_last": r["accum_ms"], "grad_accum_norm_sq_last": r["last_ms"],
                       "adamw_step_tiled": r["adamw_ms"]},
        "step_kernels": step_kernel_rates(bpe, n, r),
        "bytes_per_elem": bpe,
        "device_copy_gbps": r["copy_gbps"],
        "timing_events": timing_events(),
        "adamw_traffic_ceiling": ceiling_report(r["ceiling_ms"], adamw_bytes, r["adamw_ms"]),
        "roofline": {"kernel": "adamw_step_tiled", "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": pmc_traffic("adamw_step_tiled", n), "traffic_unit": "bytes/launch",
                     "algorithmic_bytes": adamw_bytes, "launch_ms": r["adamw_ms"]},
        "adamw_step_split": {
            "ms": r["split_ms"], "bytes_per_elem": bpe["adamw_step"],
            "gbps": adamw_bytes / (r["split_ms"] * 1e-3) / 1e9,
            "frac": adamw_bytes / (r["split_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "traffic": pmc_traffic("adamw_step", n),
            "traffic_ceiling": ceiling_report(r["ceiling_split_ms"], adamw_bytes, r["split_ms"])},
        "cpu_baseline": cpu,
        "flat_unit": flat,
        "zero1_flow": zero1,
        "grad_norm_sq": {"ms": r["norm_ms"], "bytes_per_elem": 4,
                         "gbps": 4 * n / (r["norm_ms"] * 1e-3) / 1e9,
                         "frac": 4 * n / (r["norm_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS},
        "adamw_step_no_master": None if r["no_master_ms"] is None else {
            "ms": r["no_master_ms"], "bytes_per_elem": 24,
            "gbps": 24 * n / (r["no_master_ms"] * 1e-3) / 1e9},
        "adamw_step_no_master_tiled": None if r["no_master_tiled_ms"] is None else {
            "ms": r["no_master_tiled_ms"], "bytes_per_elem": 24,
            "gbps": 24 * n / (r["no_master_tiled_ms"] * 1e-3) / 1e9},
        "reduce_chunks": None if r["reduce_ms"] is None else {
            "chunks": r["chunks"], "ms": r["reduce_ms"],
            "gbps": (r["chunks"] * (2 if w.grad_dtype == "bf16" else 4) + 4) * n / (r["reduce_ms"] * 1e-3) / 1e9},
        "staged_step": None if r["staged_ms"] is None else _staged(r, n, w),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
