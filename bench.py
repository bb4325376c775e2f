#!/usr/bin/env python3
"""Benchmark of the per-rank ZeRO/FSDP optimizer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole hot path over one batch of synthetic
input, on one rank's real-size shard (inputs resident in HBM):
  grad_accum over every micro-batch but the last (bf16 -> fp32);
  grad_sum_norm_sq: this shard's squared norm of the last micro-batch's sum
  (accumulator + last gradient, read, not stored; the norm is formed every
  step: it feeds the clip when the workload clips and the non-finite skip
  always); and adamw_step_tiled_sum: the fused AdamW step with the bf16
  re-cast on the optimizer state held in the library's tiled layout,
  forming the same sum again as it reads it (ShardOptimizer's schedule for
  its default layout).  The same step as two calls that store the sum first
  (grad_accum_norm_sq, then adamw_step_tiled) is timed after it, and the
  AdamW step on three separate state buffers (adamw_step) after that.
The shard range is host arithmetic done once at set-up.  Default workload:
the Llama-7B-shaped buffer over 8 ranks, one 842,301,952-element shard,
8 micro-batches; a second shard (the 70B ZeRO-3 one) is timed in the same
process.

Prints ONE JSON line: whole-step throughput (shard elements per second),
the roofline of the dominant kernel (the step's AdamW, timed live with HIP
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

# The kernels whose HBM traffic the JSON line reports, as rocprofv3 names
# them (bench_pmc.py keys each record to the gfx950 code object that
# defines the kernel; a rebuilt kernel reports null until the counters are
# taken again).
K_ADAMW_TILED = "zs::(anonymous namespace)::adamw_kernel<4, 1, 64, false, true, true, 0>"
K_ADAMW_SPLIT = "zs::(anonymous namespace)::adamw_kernel<4, 1, 64, false, false, true, 0>"
# the step's AdamW on the last micro-batch's sum: bf16 gradient alone (1) or onto the accumulator (2)
K_ADAMW_SUM_BF16 = "zs::(anonymous namespace)::adamw_kernel<4, 1, 64, false, true, true, 1>"
K_ADAMW_SUM_ACC_BF16 = "zs::(anonymous namespace)::adamw_kernel<4, 1, 64, false, true, true, 2>"
K_SUM_NORM_ADD = "zs::(anonymous namespace)::sum_norm_kernel<1, 1, 2, true, true, false>"
K_SUM_NORM_FIRST = "zs::(anonymous namespace)::sum_norm_kernel<4, 1, 1, true, true, true>"
K_ACCUM_FIRST = "zs::(anonymous namespace)::accum_kernel<1, 64, true, true, true, false>"
K_ACCUM_ADD = "zs::(anonymous namespace)::accum_kernel<1, 64, true, true, false, false>"
K_ACCUM_NORM_ADD = "zs::(anonymous namespace)::accum_kernel<1, 64, true, true, false, true>"
K_ACCUM_NORM_FIRST = "zs::(anonymous namespace)::accum_kernel<4, 64, true, true, true, true>"


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
    """Algorithmic HBM bytes per shard element of each kernel of one step
    (the norm's binary64 partials, 8 B per 256 elements, come on top of the
    last micro-batch's bytes: 0.03 B per element).  The step folds the last
    micro-batch into AdamW: its norm pass reads the accumulator and the last
    gradient (the gradient alone for a single micro-batch) and AdamW reads
    them again instead of one stored sum.  The *_two_call entries are the
    same step with the sum stored first (grad_accum_norm_sq, then
    adamw_step_tiled on it)."""
    g = 2 if w.grad_dtype == "bf16" else 4
    accum_first = g + 4
    accum_next = g + 8
    M = w.micro_batches
    adamw = 28 + (2 if w.bf16_param else 0)
    acc_read = 4 if M > 1 else 0
    before_last = 0 if M == 1 else accum_first + (M - 2) * accum_next
    norm_last = g + acc_read
    adamw_sum = adamw - 4 + g + acc_read
    last_two_call = accum_first if M == 1 else accum_next
    return {"grad_accum_first": accum_first, "grad_accum_next": accum_next,
            "grad_accum_all_but_last": before_last, "grad_sum_norm_sq_last": norm_last,
            "adamw_step_sum": adamw_sum, "step": before_last + norm_last + adamw_sum,
            "grad_accum_norm_sq_last": last_two_call, "adamw_step": adamw,
            "step_two_call": before_last + last_two_call + adamw}


def fused_norm_partials(w, n: int) -> int:
    """Binary64 partials the last micro-batch's norm pass writes (either
    schedule): one per 256 elements, or per 1024 when the step has a single
    bf16 micro-batch."""
    per = 1024 if (w.micro_batches == 1 and w.grad_dtype == "bf16") else 256
    return (n + per - 1) // per


def step_kernel_rates(bpe: dict, n: int, r: dict, two_call: bool = False) -> dict:
    """Algorithmic bandwidth of each part of the timed step (HIP events on
    the launch stream): the accumulations of every micro-batch but the last
    (one overwriting launch and the rest accumulating, by time the largest
    share of the step), the last micro-batch's norm (with its accumulation,
    two_call) and AdamW."""
    if two_call:
        parts = {"grad_accum_all_but_last": (bpe["grad_accum_all_but_last"], r["accum_ms"]),
                 "grad_accum_norm_sq_last": (bpe["grad_accum_norm_sq_last"], r["last_ms"]),
                 "adamw_step_tiled": (bpe["adamw_step"], r["adamw_ms"])}
    else:
        parts = {"grad_accum_all_but_last": (bpe["grad_accum_all_but_last"], r["accum_ms"]),
                 "grad_sum_norm_sq_last": (bpe["grad_sum_norm_sq_last"], r["last_ms"]),
                 "adamw_step_tiled_sum": (bpe["adamw_step_sum"], r["adamw_ms"])}
    out = {}
    for name, (b, ms) in parts.items():
        if b == 0:
            continue
        gbps = b * n / (ms * 1e-3) / 1e9 if ms > 0 else None
        out[name] = {"bytes_per_elem": b, "ms": ms, "gbps": gbps,
                     "frac": gbps / HBM_PEAK_GBPS if gbps is not None else None}
    return out


def ceiling_report(ms_by_lds: dict, nbytes: int, adamw_ms: float, kernel: str = "zsc_adamw_traffic") -> dict:
    """The AdamW-traffic kernel's time at each residency cap, its best, and
    the AdamW step's bandwidth as a fraction of that best."""
    best = min(ms_by_lds, key=ms_by_lds.get)
    gbps = nbytes / (ms_by_lds[best] * 1e-3) / 1e9
    return {"kernel": kernel, "algorithmic_bytes": nbytes,
            "ms_by_lds_bytes": {str(k): v for k, v in ms_by_lds.items()},
            "best_lds_bytes": best, "gbps": gbps, "frac": gbps / HBM_PEAK_GBPS,
            "adamw_step_of_ceiling": ms_by_lds[best] / adamw_ms}


def shard_len(w) -> int:
    import fsdp_sharded_optimizer_amd as zs
    _, start, end, _ = zs.zero_shard_range(w.total, w.world, w.rank)
    return end - start


def traffic_of(label: str, n: int, digests: dict):
    """Calibrated PMC bytes per launch from bench_pmc.json, or None when no
    record was taken on the code object that is running."""
    import bench_pmc
    return bench_pmc.traffic(label, n, digests)


def rate(nbytes: float, ms: float) -> dict:
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"ms": ms, "gbps": gbps, "frac": gbps / HBM_PEAK_GBPS}


# ---------------------------------------------------------------------------
# GPU legs
# ---------------------------------------------------------------------------

class StepRig:
    """One rank's resident buffers for a workload: the tiled optimizer
    state (master values in, moments zero), the fp32 accumulator, the step's
    micro-batch gradients (seeded draws) and the bf16 parameter, views of
    one physically contiguous DeviceArena (in that order) unless ``arena``
    is false; the norm and its workspace."""

    def __init__(self, w, dev, arena: bool = True):
        import torch
        import workloads
        import fsdp_sharded_optimizer_amd as zs
        self.w, self.dev = w, dev
        self.n = n = shard_len(w)
        log(f"[bench] workload={w.name} shard_elems={n} micro_batches={w.micro_batches}")
        f32, gdt = torch.float32, (torch.bfloat16 if w.grad_dtype == "bf16" else torch.float32)
        ws = max(zs.grad_accum_norm_sq_workspace_bytes(n), zs.grad_norm_sq_workspace_bytes(n),
                 zs.grad_reduce_chunks_norm_sq_workspace_bytes(n), 8)
        parts = ([(zs.state_tiled_numel(n), f32), (n, f32)] + [(n, gdt)] * w.micro_batches
                 + [(n, torch.bfloat16)] * int(w.bf16_param))
        self.arena = zs.DeviceArena(zs.DeviceArena.size(parts), dev) if arena else None

        def take(numel, dtype):
            return self.arena.take(numel, dtype) if arena else torch.empty(numel, dtype=dtype, device=dev)

        self.state = take(*parts[0])
        self.acc = take(*parts[1])
        master = workloads.master_init(w, n, dev)
        zs.state_tile(master, None, None, self.state)
        self.grads = []
        for mb in range(w.micro_batches):
            self.grads.append(take(n, gdt))
            self.grads[-1].copy_(workloads.grad_draw(w, n, 1, mb, dev))
        self.param = take(n, torch.bfloat16).copy_(master) if w.bf16_param else None
        del master
        # the norm and its partials stay ordinary allocations: the norm pass
        # writes one 8-byte partial per 256 elements, scattered, and ran 5
        # points slower with them in the contiguous block
        self.norm = torch.zeros(1, dtype=torch.float64, device=dev)
        self.ws = torch.empty(ws, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()   # the draws' temporaries
        if self.arena is not None:
            log(f"[bench] {w.name}: one {'contiguous' if self.arena.contiguous else 'ordinary'} "
                f"block of {self.arena.nbytes / 2**30:.2f} GiB")
        self.t = 0

    def hp(self, t: int):
        import workloads
        import fsdp_sharded_optimizer_amd as zs
        w = self.w
        return zs.AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                              grad_scale=w.grad_scale, max_norm=w.max_norm,
                              extra_norm_sq=workloads.other_ranks_norm_sq(w, 1, self.n), step=t)

    def step(self, t: int, ev=None):
        """The step as ShardOptimizer runs it on its tiled state: one
        accumulation per micro-batch as its gradient arrives, but the last;
        the last one's norm of the sum (not stored), then AdamW on that sum
        (bf16 re-cast, clip when the workload clips).  ev: four events
        recorded around the parts."""
        import fsdp_sharded_optimizer_amd as zs
        last = len(self.grads) - 1
        if ev:
            ev[0].record()
        for mb, g in enumerate(self.grads[:last]):
            zs.grad_accum(self.acc, g, overwrite=(mb == 0))
        if ev:
            ev[1].record()
        acc = self.acc if last > 0 else None
        zs.grad_sum_norm_sq(acc, self.grads[last], last == 0, self.w.grad_scale, self.norm, self.ws)
        if ev:
            ev[2].record()
        zs.adamw_step_tiled_sum(self.hp(t), self.state, acc, self.grads[last], self.param, norm_sq=self.norm)
        if ev:
            ev[3].record()

    def two_call_step(self, t: int, ev=None):
        """The same step with the last micro-batch's sum stored first: the
        accumulation forming the norm in the same pass, then AdamW reading
        the stored sum (the same results, bit for bit)."""
        import fsdp_sharded_optimizer_amd as zs
        last = len(self.grads) - 1
        if ev:
            ev[0].record()
        for mb, g in enumerate(self.grads[:last]):
            zs.grad_accum(self.acc, g, overwrite=(mb == 0))
        if ev:
            ev[1].record()
        zs.grad_accum_norm_sq(self.acc, self.grads[last], last == 0, self.w.grad_scale, self.norm, self.ws)
        if ev:
            ev[2].record()
        zs.adamw_step_tiled(self.hp(t), self.state, self.acc, self.param, norm_sq=self.norm)
        if ev:
            ev[3].record()

    def staged_step(self, t: int, k: int):
        """The same step with the micro-batch gradients staged k at a time in
        device memory: each group of k is summed in one pass
        (grad_reduce_chunks, the same left fold bit for bit), the last group
        forming the norm (grad_reduce_chunks_norm_sq), then AdamW on the
        stored sum; k = 1 is two_call_step()."""
        import fsdp_sharded_optimizer_amd as zs
        if k == 1:
            return self.two_call_step(t)
        groups = [self.grads[i:i + k] for i in range(0, len(self.grads), k)]
        for j, grp in enumerate(groups[:-1]):
            zs.grad_reduce_chunks(self.acc, grp, j == 0)
        zs.grad_reduce_chunks_norm_sq(self.acc, groups[-1], len(groups) == 1, self.w.grad_scale, self.norm,
                                      self.ws)
        zs.adamw_step_tiled(self.hp(t), self.state, self.acc, self.param, norm_sq=self.norm)

    def sum_ceiling(self) -> dict:
        """The step's AdamW traffic (accumulator + last bf16 gradient, or the
        gradient alone) with trivial arithmetic, at each residency cap (it
        changes the state: run after the timed steps)."""
        last = len(self.grads) - 1
        acc = self.acc if last > 0 else None
        return {lds: _time_adamw_traffic(self.state, None, None, acc, self.param, self.n, lds, tiled=True,
                                         grad_bf16=self.grads[last]) for lds in CEILING_LDS}

    def time_steps(self, steps: int, warmup: int, two_call: bool = False) -> dict:
        """W untimed steps, then K steps bracketed by synchronisations (wall
        clock), each with HIP events around its parts on the launch stream."""
        import math
        import torch
        ev = DeviceEvent
        run = self.two_call_step if two_call else self.step
        for _ in range(warmup):
            self.t += 1
            run(self.t)
        torch.cuda.synchronize()
        timing = []
        t0 = time.perf_counter()
        for _ in range(steps):
            self.t += 1
            e = [ev() for _ in range(4)]
            run(self.t, e)
            timing.append(e)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        assert math.isfinite(self.norm.item()), "non-finite gradient norm in the bench"
        return {"wall_s": wall, "ms_per_step": wall * 1e3 / steps,
                "accum_ms": sum(e[0].elapsed_time(e[1]) for e in timing) / steps,
                "last_ms": sum(e[1].elapsed_time(e[2]) for e in timing) / steps,
                "adamw_ms": sum(e[2].elapsed_time(e[3]) for e in timing) / steps}


def timed(fn, reps: int) -> float:
    """Average ms of fn() over reps calls after one untimed call, HIP events
    on the current stream."""
    import torch
    fn()
    e0, e1 = DeviceEvent(), DeviceEvent()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def run_gpu(rig: StepRig, steps: int, warmup: int):
    import torch
    import fsdp_sharded_optimizer_amd as zs
    from fsdp_sharded_optimizer_amd import ledger

    w, dev = rig.w, rig.dev
    n = rig.n
    torch.cuda.synchronize()
    resident = rig.arena.nbytes if rig.arena is not None else torch.cuda.memory_allocated()
    log(f"[bench] inputs resident: {resident / 2**30:.1f} GiB")
    r = rig.time_steps(steps, warmup)
    r["n"] = n
    r["chunks"] = len(rig.grads)
    r["buffers"] = ("one physically contiguous block (DeviceArena)" if rig.arena is not None and rig.arena.contiguous
                    else "separate allocations" if rig.arena is None else "one ordinary block")
    ev = DeviceEvent

    # outside the step: the same step captured once in a HIP graph and
    # replayed (the library allocates, clears and synchronises nothing, so
    # the step captures as is; launch overhead matters for small shards)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        rig.step(rig.t + 1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        rig.step(rig.t + 1)
    r["graph_ms"] = timed(graph.replay, steps)
    del graph

    # outside the step: the same step with the last micro-batch's sum stored
    # first (grad_accum_norm_sq, then adamw_step_tiled on the stored sum)
    r["two_call"] = rig.time_steps(steps, 1, two_call=True)

    # outside the step: the same AdamW step on three separate state buffers
    # (adamw_step), loaded with the tiled state as the timed steps left it so
    # both layouts stream the same values
    master = torch.empty(n, dtype=torch.float32, device=dev)
    exp_avg = torch.empty(n, dtype=torch.float32, device=dev)
    exp_avg_sq = torch.empty(n, dtype=torch.float32, device=dev)
    zs.state_untile(rig.state, master, exp_avg, exp_avg_sq)
    split_ms = []
    for k in range(steps):
        e0, e1 = ev(), ev()
        e0.record()
        zs.adamw_step(rig.hp(rig.t + 1 + k), master, exp_avg, exp_avg_sq, rig.acc, rig.param, norm_sq=rig.norm)
        e1.record()
        split_ms.append((e0, e1))
    torch.cuda.synchronize()
    r["split_ms"] = sum(a.elapsed_time(b) for a, b in split_ms) / steps
    # and the step's own AdamW (accumulator + last gradient) on those split buffers
    last = len(rig.grads) - 1
    acc_arg = rig.acc if last > 0 else None
    r["split_sum_ms"] = timed(lambda: zs.adamw_step_sum(rig.hp(rig.t + 1), master, exp_avg, exp_avg_sq, acc_arg,
                                                        rig.grads[last], rig.param, norm_sq=rig.norm), steps)

    # outside the step: the one-pass sums of the step's micro-batch
    # gradients alone, without and with the norm (the reduce-scatter's
    # arithmetic on this rank's shard, the same buffers read as N chunks)
    r["reduce_ms"] = r["reduce_norm_ms"] = None
    if len(rig.grads) > 1:
        r["reduce_ms"] = timed(lambda: zs.grad_reduce_chunks(rig.acc, rig.grads, True), 5)
        r["reduce_norm_ms"] = timed(lambda: zs.grad_reduce_chunks_norm_sq(rig.acc, rig.grads, True, w.grad_scale,
                                                                          rig.norm, rig.ws), 5)

    # outside the step: the step with its micro-batch gradients staged k at a
    # time in device memory (ShardOptimizer.accumulate_all over groups of k):
    # fewer passes over the fp32 accumulator for (k - 1) more bf16 gradient
    # buffers resident
    curve = []
    if len(rig.grads) > 1:
        g = 2 if w.grad_dtype == "bf16" else 4
        M = len(rig.grads)
        for k in (1, 2, 4, 8):
            if k > M or M % k:
                continue
            G = M // k
            bpe = (g * k + 4) + (G - 1) * (g * k + 8) + step_bytes_per_elem(w)["adamw_step"]
            t0 = rig.t
            ms = timed(lambda: rig.staged_step(t0 + 1, k), steps)
            extra = ledger.library_shard_bytes(n, grad_buffers=k) - ledger.library_shard_bytes(n, grad_buffers=1)
            curve.append({"k": k, "passes_over_acc": G, "bytes_per_elem": bpe, "elements_per_s": n / (ms * 1e-3),
                          "extra_hbm_bytes": extra, **rate(bpe * n, ms)})
            rig.t += steps + 1
    r["staging_curve"] = curve

    # outside the step: the standalone squared norm over the accumulated
    # gradient (4 B/element), as when the gradient arrives from a
    # reduce-scatter instead of this rank's own accumulation
    r["norm_ms"] = timed(lambda: zs.grad_norm_sq(rig.acc, w.grad_scale, rig.norm, rig.ws), 5)

    # outside the step: the variant with no fp32 master (24 B/element), on the
    # split buffers, then on tiled moments
    r["no_master_ms"] = r["no_master_tiled_ms"] = None
    if rig.param is not None:
        def no_master_hp():
            rig.t += 1
            return zs.AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                                  grad_scale=w.grad_scale, step=rig.t)
        r["no_master_ms"] = timed(lambda: zs.adamw_step_no_master(no_master_hp(), rig.param, exp_avg, exp_avg_sq,
                                                                  rig.acc), 3)
        moments = torch.empty(zs.moments_tiled_numel(n), dtype=torch.float32, device=dev)
        zs.moments_tile(exp_avg, exp_avg_sq, moments)
        r["no_master_tiled_ms"] = timed(lambda: zs.adamw_step_no_master_tiled(no_master_hp(), rig.param, moments,
                                                                              rig.acc), 3)
        del moments

    # achievable-bandwidth reference for the AdamW step's own traffic: the
    # same bytes per element and accesses, one addition per stream in place
    # of the update, at several residency caps (run last on these buffers:
    # it changes them)
    r["ceiling_ms"] = {lds: _time_adamw_traffic(rig.state, None, None, rig.acc, rig.param, n, lds, tiled=True)
                       for lds in CEILING_LDS}
    r["ceiling_sum_ms"] = rig.sum_ceiling()
    r["ceiling_split_ms"] = {lds: _time_adamw_traffic(master, exp_avg, exp_avg_sq, rig.acc, rig.param, n, lds)
                             for lds in CEILING_LDS}
    del rig, master, exp_avg, exp_avg_sq
    torch.cuda.empty_cache()

    # achievable-bandwidth reference: a plain device copy of 4 GiB (also the
    # calibration kernel for the HBM byte counters, which find it as the
    # runtime copy kernel's largest dispatch)
    src = torch.empty(1 << 30, dtype=torch.float32, device=dev)
    src.fill_(1.0)
    dst = torch.empty_like(src)
    copy_ms = timed(lambda: dst.copy_(src), 5)
    r["copy_gbps"] = 2 * src.numel() * 4 / (copy_ms * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return r


def run_step_leg(rig: StepRig, steps: int, warmup: int) -> dict:
    """The timed step alone on another shard (the 70B ZeRO-3 shard): the
    same kernels, the same launch configuration, in the same process."""
    import torch
    torch.cuda.synchronize()
    r = rig.time_steps(steps, warmup)
    r["n"] = rig.n
    r["two_call"] = rig.time_steps(steps, 1, two_call=True)
    r["ceiling_sum_ms"] = rig.sum_ceiling()
    return r


CEILING_LDS = (0, 8192, 12288, 14336, 16384, 20480)   # LDS reserved per one-wave workgroup


def _time_adamw_traffic(master, exp_avg, exp_avg_sq, grad, bf16, n: int, lds: int, reps: int = 5,
                        tiled: bool = False, grad_bf16=None) -> float:
    """Average launch time of the AdamW-traffic ceiling kernel
    (libzsceiling.so, built next to libzshard.so), each launch bracketed by
    HIP events on the stream it runs on.  tiled: `master` is the tiled state
    buffer and the kernel walks that layout.  grad_bf16: the gradient is
    `grad` (an fp32 accumulator, or None) plus this bf16 micro-batch
    gradient, as adamw_step_tiled_sum reads it."""
    import ctypes
    import torch
    from fsdp_sharded_optimizer_amd import build as zbuild

    if not os.path.exists(zbuild.CEILING_LIB):
        raise RuntimeError(f"{zbuild.CEILING_LIB} is not built: run python -m fsdp_sharded_optimizer_amd.build")
    lib = ctypes.CDLL(zbuild.CEILING_LIB)
    stream = torch.cuda.current_stream()
    bptr = bf16.data_ptr() if bf16 is not None else None
    if grad_bf16 is not None:
        f = lib.zsc_adamw_traffic_tiled_sum
        f.restype = ctypes.c_int32
        f.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]
        args = [master.data_ptr(), grad.data_ptr() if grad is not None else None, grad_bf16.data_ptr(), bptr, n, lds,
                stream.cuda_stream]
    elif tiled:
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

def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _mem_available() -> int:
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemAvailable:"):
                    return int(line.split()[1]) * 1024
    except OSError:
        pass
    return 0


def _oracle_threads() -> tuple:
    """Threads for the oracle: every core of the process affinity mask,
    capped by OMP_NUM_THREADS when the environment sets it (the host's CPU
    share); returns (threads, affinity cores)."""
    affinity = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    threads = min(affinity, int(cap)) if cap.isdigit() and int(cap) > 0 else affinity
    return threads, affinity


def run_cpu_baseline(w, target_s: float = 10.0, sample: int = 1 << 25):
    """The oracle as it stands, timed on the host cores on the same
    workload: whole steps (every micro-batch accumulation, the norm, AdamW
    with the bf16 re-cast) over the full shard when the host has the memory
    for it (inputs drawn by the same seeded recipe on the GPU and copied to
    the host), else over the first `sample` elements; as many steps as fit
    in about target_s.  Then the tiny ZeRO-1 workload single-threaded."""
    import numpy as np
    import torch
    import oracle
    import workloads

    threads, affinity = _oracle_threads()
    oracle.set_num_threads(threads)
    n_full = shard_len(w)
    g_bytes = 2 if w.grad_dtype == "bf16" else 4
    need = n_full * (16 + (2 if w.bf16_param else 0) + w.micro_batches * g_bytes)
    full = torch.cuda.is_available() and _mem_available() > 2 * need
    n = n_full if full else sample
    where = "cuda" if full else "cpu"
    master = workloads.master_init(w, n, where).cpu().numpy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    bf = np.zeros(n, np.uint16) if w.bf16_param else None
    code = oracle.BF16 if w.grad_dtype == "bf16" else oracle.F32
    grads = []
    for mb in range(w.micro_batches):
        g = workloads.grad_draw(w, n, 1, mb, where).cpu()
        grads.append(g.view(torch.int16).numpy().view(np.uint16) if code == oracle.BF16 else g.numpy())
        del g
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
    del master, m, v, bf, grads, acc
    bpe = step_bytes_per_elem(w)
    accum_bytes = bpe["step_two_call"] - bpe["adamw_step"]   # every micro-batch's accumulation, stored
    phases = {
        "accumulate": {"ms_per_step": phase["accumulate"] * 1e3 / done,
                       "gbps": accum_bytes * n * done / phase["accumulate"] / 1e9},
        "norm": {"ms_per_step": phase["norm"] * 1e3 / done, "gbps": 4 * n * done / phase["norm"] / 1e9},
        "adamw": {"ms_per_step": phase["adamw"] * 1e3 / done,
                  "gbps": bpe["adamw_step"] * n * done / phase["adamw"] / 1e9},
    }
    mode = "full shard" if full else "sample"
    out = {"value": n * done / el, "unit": "elements/s", "cores": threads, "kind": "oracle",
           "sample": (f"{mode}: {n} elements ({'the whole' if full else 'the first of the'} {n_full}-element "
                      f"{w.name} shard, inputs by the same seeded recipe), {done} whole steps "
                      f"({w.micro_batches} micro-batch accumulations + norm + AdamW/bf16) in {el:.1f} s"),
           "mode": mode, "elements": n, "steps": done, "seconds": el,
           "threads": threads, "affinity_cores": affinity, "cpu_model": _cpu_model(),
           "phases": phases}
    oracle.set_num_threads(1)
    out["single_thread_c1"] = _cpu_tiny_zero1(target_s=2.0)
    oracle.set_num_threads(threads)
    return out


def _cpu_tiny_zero1(target_s: float) -> dict:
    """The tiny ZeRO-1 workload (rank 3's 125,001-element slice, 5 Adam
    steps of fresh fp32 gradients) through the oracle on one thread,
    repeated for about target_s: shard elements stepped per second."""
    import numpy as np
    import oracle
    import workloads
    w = workloads.WORKLOADS["tiny_zero1"]
    _, start, end, _ = oracle.shard_range(w.total, w.world, w.rank)
    n = end - start
    p0 = workloads.master_init(w, w.total).numpy()[start:end].copy()
    grads = [workloads.grad_draw(w, w.total, t, 0).numpy()[start:end].copy() for t in range(1, w.steps + 1)]
    runs = 0
    t0 = time.perf_counter()
    while True:
        p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
        for t, g in enumerate(grads, 1):
            hp = oracle.make_hp(w.lr, w.beta1, w.beta2, w.eps, 0.0, w.grad_scale, 0.0, 0.0, t)
            oracle.adamw_step(hp, p, m, v, g)
        runs += 1
        el = time.perf_counter() - t0
        if el >= target_s:
            break
    return {"value": n * w.steps * runs / el, "unit": "elements/s", "threads": oracle.num_threads(),
            "workload": w.name, "shard_elems": n, "steps_per_run": w.steps, "runs": runs, "seconds": el}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama7b_shard")
    ap.add_argument("--second-workload", default="zero3_70b_shard",
                    help="a second shard timed in the same process after the first ('' to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--no-zero1", action="store_true", help="skip the ZeRO-1 flow timing")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU's shard only; --gpus {args.gpus} is not "
              "supported (collectives are out of scope). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import workloads
    for name in (args.workload, args.second_workload):
        if name and name not in workloads.WORKLOADS:
            sys.exit(f"unknown workload {name}; one of {sorted(workloads.WORKLOADS)}")
    w = workloads.WORKLOADS[args.workload]

    import fsdp_sharded_optimizer_amd as zs
    import bench_pmc
    zs.lib()
    digests = bench_pmc.kernel_digests()

    # both shards' buffers are allocated up front, as a rank allocates its
    # buffers once, each shard's in one physically contiguous block (the
    # timed workload's first): separate allocations made after other
    # processes had allocated and freed device memory streamed up to 6
    # points slower on gfx950, and a block placed behind tens of GiB of
    # other allocations a few points slower
    import torch
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    rig = StepRig(w, dev)
    second_rig = None
    if args.second_workload and args.second_workload != w.name:
        second_rig = StepRig(workloads.WORKLOADS[args.second_workload], dev)
    r = run_gpu(rig, args.steps, args.warmup)
    del rig
    n = r["n"]
    second = None
    if second_rig is not None:
        second = (second_rig.w, run_step_leg(second_rig, args.steps, args.warmup))
        del second_rig
        torch.cuda.empty_cache()
    flat = None
    if w.unit_shapes:
        flat = run_flat(w)
    zero1 = None
    if w.name == "llama7b_shard" and not args.no_zero1:
        zero1 = run_zero1_flow(w, workloads.LLAMA7B)
    bpe = step_bytes_per_elem(w)
    ms_per_step = r["ms_per_step"]
    tc = r["two_call"]
    adamw_bytes = bpe["adamw_step"] * n            # the AdamW step on a stored gradient, either layout
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host cores ...")
        cpu = run_cpu_baseline(w, args.cpu_seconds)
    step_gbps = bpe["step"] * n / (ms_per_step * 1e-3) / 1e9

    # kernels whose HBM traffic has records (bench_pmc.py): label, kernel,
    # shard length, algorithmic bytes per launch
    def entry(label, kernel, nn, nbytes, per_wg=256, workgroups=None):
        # one-wave workgroups of per_wg elements: the launch's grid in work-items
        wgs = -(-nn // per_wg) if workgroups is None else workgroups
        return {"label": label, "kernel": kernel, "shard_elems": nn, "algorithmic_bytes": nbytes,
                "grid": wgs * 64}

    def sum_norm_workgroups(nn, single):
        """grad_sum_norm_sq's one-wave workgroups: 8 x ceil(blocks per XCD
        / blocks per wave), blocks of 1024 elements (single bf16 micro-batch,
        one per wave) or 256 (two per wave)."""
        span, per_wave = (1024, 1) if single else (256, 2)
        blocks = -(-nn // span)
        return 8 * -(-(-(-blocks // 8)) // per_wave)

    def sum_entries(wl, nn):
        """The step's last micro-batch and AdamW (bf16 gradients)."""
        b = step_bytes_per_elem(wl)
        single = wl.micro_batches == 1
        return [entry("adamw_step_tiled_sum", K_ADAMW_SUM_BF16 if single else K_ADAMW_SUM_ACC_BF16, nn,
                      b["adamw_step_sum"] * nn),
                entry("grad_sum_norm_sq_last", K_SUM_NORM_FIRST if single else K_SUM_NORM_ADD, nn,
                      b["grad_sum_norm_sq_last"] * nn + 8 * fused_norm_partials(wl, nn),
                      workgroups=sum_norm_workgroups(nn, single))]

    def two_call_entries(wl, nn):
        b = step_bytes_per_elem(wl)
        single = wl.micro_batches == 1
        return [entry("adamw_step_tiled", K_ADAMW_TILED, nn, b["adamw_step"] * nn),
                entry("grad_accum_norm_sq_last", K_ACCUM_NORM_FIRST if single else K_ACCUM_NORM_ADD, nn,
                      b["grad_accum_norm_sq_last"] * nn + 8 * fused_norm_partials(wl, nn), 1024 if single else 256)]

    bf16_grads = w.grad_dtype == "bf16"
    pmc = [entry("adamw_step", K_ADAMW_SPLIT, n, adamw_bytes)]
    if bf16_grads:
        pmc += sum_entries(w, n) + two_call_entries(w, n)
    if w.micro_batches > 2 and bf16_grads:
        pmc += [entry("grad_accum_first", K_ACCUM_FIRST, n, 6 * n),
                entry("grad_accum_add", K_ACCUM_ADD, n, 10 * n)]

    def roofline(wl, rr, nn):
        """The step's AdamW, on the last micro-batch's sum; its traffic with
        trivial arithmetic at the best residency beside it."""
        b = step_bytes_per_elem(wl)["adamw_step_sum"] * nn
        ach = b / (rr["adamw_ms"] * 1e-3) / 1e9
        return {"kernel": "adamw_step_tiled_sum", "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS,
                "traffic": traffic_of("adamw_step_tiled_sum", nn, digests), "traffic_unit": "bytes/launch",
                "algorithmic_bytes": b, "launch_ms": rr["adamw_ms"],
                "traffic_ceiling": ceiling_report(rr["ceiling_sum_ms"], b, rr["adamw_ms"],
                                                  "zsc_adamw_traffic_tiled_sum")}

    def with_traffic(kernels: dict, nn: int, wl) -> dict:
        """Measured bytes per launch next to the algorithmic ones, for the
        parts that have records."""
        b = step_bytes_per_elem(wl)
        parts = {"grad_sum_norm_sq_last": b["grad_sum_norm_sq_last"] * nn + 8 * fused_norm_partials(wl, nn),
                 "grad_accum_norm_sq_last": b["grad_accum_norm_sq_last"] * nn + 8 * fused_norm_partials(wl, nn),
                 "adamw_step_tiled_sum": b["adamw_step_sum"] * nn, "adamw_step_tiled": b["adamw_step"] * nn}
        for name, nbytes in parts.items():
            if name in kernels:
                kernels[name]["algorithmic_bytes"] = nbytes
                kernels[name]["traffic"] = traffic_of(name, nn, digests) if wl.grad_dtype == "bf16" else None
        return kernels

    def two_call_report(wl, rr, nn):
        b = step_bytes_per_elem(wl)
        t = rr["two_call"]
        return {"ms_per_step": t["ms_per_step"], "elements_per_s": nn / (t["ms_per_step"] * 1e-3),
                "bytes_per_elem": b["step_two_call"], "step_kernels": with_traffic(
                    step_kernel_rates(b, nn, t, two_call=True), nn, wl),
                "one_pass_speedup": t["ms_per_step"] / rr["ms_per_step"]}

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
                   "state": "fp32 master/exp_avg/exp_avg_sq (tiled layout) + bf16 param", "clip": w.max_norm > 0,
                   "buffers": r["buffers"]},
        "graph_ms_per_step": r["graph_ms"],
        "step_hbm_gbps": step_gbps,
        "step_hbm_frac": step_gbps / HBM_PEAK_GBPS,
        "kernels_ms": {"grad_accum_all_but_last": r["accum_ms"], "grad_sum_norm_sq_last": r["last_ms"],
                       "adamw_step_tiled_sum": r["adamw_ms"]},
        "step_kernels": with_traffic(step_kernel_rates(bpe, n, r), n, w),
        "bytes_per_elem": bpe,
        "step_two_call": two_call_report(w, r, n),
        "device_copy_gbps": r["copy_gbps"],
        "timing_events": timing_events(),
        "adamw_traffic_ceiling": ceiling_report(r["ceiling_ms"], adamw_bytes, tc["adamw_ms"],
                                                "zsc_adamw_traffic_tiled"),
        "roofline": roofline(w, r, n),
        "adamw_step_split": {
            "ms": r["split_ms"], "bytes_per_elem": bpe["adamw_step"],
            "gbps": adamw_bytes / (r["split_ms"] * 1e-3) / 1e9,
            "frac": adamw_bytes / (r["split_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "traffic": traffic_of("adamw_step", n, digests),
            "traffic_ceiling": ceiling_report(r["ceiling_split_ms"], adamw_bytes, r["split_ms"])},
        "adamw_step_sum_split": {"ms": r["split_sum_ms"], "bytes_per_elem": bpe["adamw_step_sum"],
                                 **rate(bpe["adamw_step_sum"] * n, r["split_sum_ms"])},
        "cpu_baseline": cpu,
        "flat_unit": flat,
        "zero1_flow": zero1,
        "grad_norm_sq": {"bytes_per_elem": 4, **rate(4 * n, r["norm_ms"])},
        "adamw_step_no_master": None if r["no_master_ms"] is None else {
            "bytes_per_elem": 24, **rate(24 * n, r["no_master_ms"])},
        "adamw_step_no_master_tiled": None if r["no_master_tiled_ms"] is None else {
            "bytes_per_elem": 24, **rate(24 * n, r["no_master_tiled_ms"])},
        "reduce_chunks": None if r["reduce_ms"] is None else {
            "chunks": r["chunks"], "bytes_per_elem": r["chunks"] * (2 if w.grad_dtype == "bf16" else 4) + 4,
            **rate((r["chunks"] * (2 if w.grad_dtype == "bf16" else 4) + 4) * n, r["reduce_ms"])},
        "reduce_chunks_norm_sq": None if r["reduce_norm_ms"] is None else {
            "chunks": r["chunks"], "bytes_per_elem": r["chunks"] * (2 if w.grad_dtype == "bf16" else 4) + 4,
            "of_plain_fold": r["reduce_norm_ms"] / r["reduce_ms"],
            **rate((r["chunks"] * (2 if w.grad_dtype == "bf16" else 4) + 4) * n, r["reduce_norm_ms"])},
        "staging_curve": r["staging_curve"],
    }
    if w.micro_batches > 2 and bf16_grads:
        # measured bytes of the accumulations before the last, from the per-kernel records
        t_first, t_add = (traffic_of(k, n, digests) for k in ("grad_accum_first", "grad_accum_add"))
        sk = out["step_kernels"]
        sk["grad_accum_all_but_last"]["algorithmic_bytes"] = bpe["grad_accum_all_but_last"] * n
        sk["grad_accum_all_but_last"]["traffic"] = (None if t_first is None or t_add is None
                                                    else t_first + (w.micro_batches - 2) * t_add)
    if second is not None:
        w2, r2 = second
        n2 = r2["n"]
        bpe2 = step_bytes_per_elem(w2)
        if w2.grad_dtype == "bf16":
            pmc += sum_entries(w2, n2) + two_call_entries(w2, n2)
        out["roofline_second"] = {"workload": w2.name, **roofline(w2, r2, n2)}
        out["second_workload"] = {
            "workload": w2.name, "shard_elems": n2, "micro_batches": w2.micro_batches, "clip": w2.max_norm > 0,
            "ms_per_step": r2["ms_per_step"], "elements_per_s": n2 / (r2["ms_per_step"] * 1e-3),
            "bytes_per_elem": bpe2, "step_kernels": with_traffic(step_kernel_rates(bpe2, n2, r2), n2, w2),
            "step_two_call": two_call_report(w2, r2, n2)}
    out["pmc_kernels"] = pmc
    out["code_objects_sha256"] = sorted(set(digests.values()))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
