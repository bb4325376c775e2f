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


def _spin_ms() -> float:
    """How long the spin holds a stream on this GPU."""
    s = torch.cuda.Stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        e0.record()
        torch.cuda._sleep(SPIN)
        e1.record()
    s.synchronize()
    return e0.elapsed_time(e1)


def test_calls_run_on_the_stream_they_are_given():
    print("explicit streams", flush=True)
    import time
    if not hasattr(torch.cuda, "_sleep"):
        pytest.skip("torch.cuda._sleep is not available")
    n = 1 << 20
    rng = np.random.default_rng(5)
    g_np = oracle.bf16_rne((rng.standard_normal(n) * 1e-2).astype(np.float32))
    g = from_np(g_np, bf16=True)
    srcs = [from_np(oracle.bf16_rne(rng.uniform(-1, 1, k).astype(np.float32)), bf16=True) for k in (1000, 5)]
    acc = torch.zeros(n, device="cuda")
    flat = torch.zeros(1008, dtype=torch.bfloat16, device="cuda")
    master, m, v = (torch.zeros(n, device="cuda") for _ in range(3))
    state = torch.zeros(zs.state_tiled_numel(n), device="cuda")   # the same step on the tiled layout
    hp = zs.AdamWConfig(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, grad_scale=1.0, step=1)
    spin = _spin_ms()
    observed = False
    for attempt in range(3):   # the check needs the host to read within the spin: retry if it did not
        for t in (acc, flat, master, m, v, state):
            t.zero_()
        torch.cuda.synchronize()
        s = _held_side_stream()
        t0 = time.perf_counter()
        zs.grad_accum(acc, g, overwrite=True, stream=s)
        zs.flat_pack(srcs, flat, 1008, stream=s)
        zs.adamw_step(hp, master, m, v, acc, stream=s)
        zs.adamw_step_tiled(hp, state, acc, stream=s)
        early = [to_np(t) for t in (acc, flat, master, state)]   # the default stream does not wait for s
        host_ms = (time.perf_counter() - t0) * 1e3
        s.synchronize()
        if host_ms < 0.5 * spin:
            assert not any(e.any() for e in early), "a call did not wait on its stream"
            observed = True
            break
        print(f"  attempt {attempt}: host took {host_ms:.1f} ms of a {spin:.1f} ms spin, inconclusive", flush=True)
    if not observed:
        pytest.skip("the host could not read within the spin; ordering not observed")
    assert bits_equal(to_np(acc), oracle.bf16_widen(g_np))
    assert bits_equal(to_np(flat), oracle.flat_pack([to_np(x) for x in srcs], oracle.BF16, oracle.BF16, 1008))
    p_ref, m_ref, v_ref = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)
    H = oracle.make_hp(1e-3, 0.9, 0.999, 1e-8, 0.0, 1.0, 0.0, 0.0, 1)
    assert oracle.adamw_step(H, p_ref, m_ref, v_ref, oracle.bf16_widen(g_np)) == 0
    assert bits_equal(to_np(master), p_ref) and bits_equal(to_np(m), m_ref) and bits_equal(to_np(v), v_ref)
    split = [torch.empty(n, device="cuda") for _ in range(3)]
    zs.state_untile(state, *split)
    for got, want in zip(split, (p_ref, m_ref, v_ref)):
        assert bits_equal(to_np(got), want)


@pytest.mark.parametrize("layout", ["split", "tiled"])
def test_two_host_threads_on_two_streams_match_serial_runs(layout):
    """The library keeps no global state (only a thread-local error code):
    two host threads, each driving its own shard on its own stream through
    ten accumulate / fused-norm / clipped-AdamW steps, end bit-identical to
    the same sequences run one after the other on the default stream."""
    import threading
    print(f"two threads, two streams, {layout} state", flush=True)
    n, M, steps, scale = 300_007, 3, 10, 1 / 24
    gen = torch.Generator(device="cuda")
    gen.manual_seed(99)
    grads = [[(torch.randn(n, generator=gen, device="cuda") * 1e-2 * (k + 1)).to(torch.bfloat16) for k in range(M)]
             for _ in range(2)]
    init = [(torch.rand(n, generator=gen, device="cuda") * 0.2 - 0.1) for _ in range(2)]

    def make(i):
        d = {"master": init[i].clone(), "m": torch.zeros(n, device="cuda"), "v": torch.zeros(n, device="cuda"),
             "b": torch.empty(n, dtype=torch.bfloat16, device="cuda"), "acc": torch.empty(n, device="cuda"),
             "norm": torch.zeros(1, dtype=torch.float64, device="cuda"),
             "ws": torch.empty(zs.grad_accum_norm_sq_workspace_bytes(n), dtype=torch.uint8, device="cuda"),
             "state": torch.empty(zs.state_tiled_numel(n), device="cuda")}
        if layout == "tiled":
            zs.state_tile(d["master"], None, None, d["state"])
        return d

    def run(i, s, stream):
        for t in range(1, steps + 1):
            for k in range(M - 1):
                zs.grad_accum(s["acc"], grads[i][k], overwrite=(k == 0), stream=stream)
            zs.grad_accum_norm_sq(s["acc"], grads[i][M - 1], False, scale, s["norm"], s["ws"], stream=stream)
            hp = zs.AdamWConfig(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_scale=scale,
                                max_norm=0.5, extra_norm_sq=0.01 * i, step=t)
            if layout == "split":
                zs.adamw_step(hp, s["master"], s["m"], s["v"], s["acc"], s["b"], norm_sq=s["norm"], stream=stream)
            else:
                zs.adamw_step_tiled(hp, s["state"], s["acc"], s["b"], norm_sq=s["norm"], stream=stream)
        if layout == "tiled":
            zs.state_untile(s["state"], s["master"], s["m"], s["v"], stream=stream)

    serial = [make(0), make(1)]
    run(0, serial[0], None)
    run(1, serial[1], None)
    torch.cuda.synchronize()

    par = [make(0), make(1)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st_ in streams:
        st_.wait_stream(torch.cuda.current_stream())   # inputs are ready before either thread starts
    errors = []

    def worker(i):
        try:
            torch.cuda.set_device(0)
            run(i, par[i], streams[i])
            streams[i].synchronize()
        except Exception as e:   # re-raised below on the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i in range(2):
        for k in ("master", "m", "v", "b", "acc", "norm"):
            assert bits_equal(to_np(par[i][k]), to_np(serial[i][k])), (i, k)
