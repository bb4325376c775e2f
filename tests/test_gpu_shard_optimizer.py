"""ShardOptimizer (the call-ordering layer) on the GPU against the oracle.

Four bf16 micro-batches per step, a global-norm clip with the other ranks'
share as a stand-in, three steps, on a ragged shard; with the norm formed in
the last accumulation pass, with a separate norm pass, and with the last
micro-batch handed to step() (on the tiled state, its sum with the
accumulator formed where it is read, never stored).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import fsdp_sharded_optimizer_amd as zs
from tests.parity import NORM_TOL, StateCheck, bits_equal, from_np, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("layout", ["tiled", "split"])
@pytest.mark.parametrize("mode", ["fused", "separate", "last_grad"])
def test_shard_optimizer_matches_the_oracle(mode, layout):
    print(f"ShardOptimizer mode={mode} layout={layout}", flush=True)
    fused = mode == "fused"
    n, M, scale, lr, wd = 100_003, 4, 1 / 32, 3e-4, 0.1
    rng = np.random.default_rng(17)
    p0 = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    master = from_np(p0.copy())
    param = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    opt = zs.ShardOptimizer(master, lr=lr, betas=(0.9, 0.95), weight_decay=wd, grad_scale=scale, max_norm=1.0,
                            param_bf16=param, layout=layout)
    p_ref, m_ref, v_ref = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    b_ref = np.zeros(n, np.uint16)
    for t in range(1, 4):
        mbs = [oracle.bf16_rne((rng.standard_normal(n) * 0.05 * t).astype(np.float32)) for _ in range(M)]
        acc_ref = np.empty(n, np.float32)
        for k, g in enumerate(mbs):
            if k == M - 1:
                before_last = acc_ref.copy()
            oracle.grad_accum(acc_ref, g, oracle.BF16, overwrite=(k == 0))
            if mode != "last_grad" or k < M - 1:
                opt.accumulate(from_np(g, bf16=True), last=fused and k == M - 1)
        S = oracle.grad_norm_sq(acc_ref, scale)
        extra = 3.0 * S                                   # the other ranks' share
        prev = {"p": p_ref.copy(), "m": m_ref.copy()}
        H = oracle.make_hp(lr, 0.9, 0.95, 1e-8, wd, scale, 1.0, extra, t)
        assert oracle.adamw_step(H, p_ref, m_ref, v_ref, acc_ref, b_ref, norm_sq=S) == 0
        opt.step(extra_norm_sq=extra, last_grad=from_np(mbs[-1], bf16=True) if mode == "last_grad" else None)
        torch.cuda.synchronize()
        assert opt.t == t
        # the one-pass step never stores the last micro-batch's sum
        stored = before_last if mode == "last_grad" else acc_ref
        assert bits_equal(to_np(opt.acc), stored)
        assert abs(opt.norm_sq.item() - S) <= NORM_TOL * S
        coef = oracle.clip_coef(S, extra, 1.0)
        assert coef < 1.0                                 # every step clips
        g2 = (acc_ref * np.float32(scale)) * np.float32(coef)
        s = oracle.adamw_scalars(H)
        gpu = {"p": to_np(opt.master), "m": to_np(opt.exp_avg), "v": to_np(opt.exp_avg_sq), "b": to_np(param)}
        if layout == "split":
            assert opt.master is master                   # the caller's tensor is stepped in place
        res = StateCheck(0.9, lr, wd, s.step_size).check(gpu, {"p": p_ref, "m": m_ref, "v": v_ref, "b": b_ref},
                                                          prev, g2, f"t={t}")
        print(f"  t={t} norm {math.sqrt(S + extra):.4f} coef {coef:.4f} {res}", flush=True)


def test_shard_optimizer_refuses_a_step_without_gradients():
    opt = zs.ShardOptimizer(torch.zeros(16, device="cuda"), lr=1e-3)
    with pytest.raises(RuntimeError):
        opt.step()
    with pytest.raises(TypeError):
        zs.ShardOptimizer(torch.zeros(16, device="cuda", dtype=torch.float64), lr=1e-3)
    with pytest.raises(ValueError):
        zs.ShardOptimizer(torch.zeros(16, device="cuda"), lr=1e-3, layout="interleaved")


def test_layouts_give_identical_bits():
    """The same five steps under the tiled and the split layout: master,
    moments and bf16 parameter bit-identical after every step."""
    n, M = 3 * zs.STATE_TILE + 1001, 2
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    p0 = torch.rand(n, generator=gen, device="cuda") * 0.2 - 0.1
    kw = dict(lr=3e-4, betas=(0.9, 0.95), weight_decay=0.1, grad_scale=1 / 16, max_norm=1.0)
    opts = [zs.ShardOptimizer(p0.clone(), param_bf16=torch.empty(n, dtype=torch.bfloat16, device="cuda"),
                              layout=lay, **kw) for lay in ("tiled", "split")]
    for t in range(1, 6):
        mbs = [(torch.randn(n, generator=gen, device="cuda") * 0.05 * t).to(torch.bfloat16) for _ in range(M)]
        for opt in opts:
            for k, g in enumerate(mbs):
                opt.accumulate(g, last=k == M - 1)
            opt.step(extra_norm_sq=0.5)
        torch.cuda.synchronize()
        for name in ("master", "exp_avg", "exp_avg_sq", "param_bf16"):
            assert bits_equal(to_np(getattr(opts[0], name)), to_np(getattr(opts[1], name))), (t, name)


@pytest.mark.parametrize("layouts", [("tiled", "tiled"), ("split", "tiled"), ("tiled", "split")])
def test_shard_optimizer_resume_is_bit_identical(layouts):
    """Five steps in one run against two steps, a state_dict copied to the
    host, a fresh optimizer loading it and three more steps: master, moments,
    bf16 parameter and step counter bit-identical, also when the run is
    resumed under the other state layout (checkpoints hold split arrays)."""
    print(f"ShardOptimizer resume {layouts}", flush=True)
    saved_layout, resumed_layout = layouts
    n, M, scale = 70_001, 2, 1 / 16
    rng = np.random.default_rng(23)
    p0 = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    grads = [[oracle.bf16_rne((rng.standard_normal(n) * 0.05).astype(np.float32)) for _ in range(M)]
             for _ in range(5)]
    kw = dict(lr=3e-4, betas=(0.9, 0.95), weight_decay=0.1, grad_scale=scale, max_norm=1.0)

    def run(opt, steps):
        for mbs in steps:
            for k, g in enumerate(mbs):
                opt.accumulate(from_np(g, bf16=True), last=k == M - 1)
            opt.step(extra_norm_sq=0.25)

    whole = zs.ShardOptimizer(from_np(p0.copy()), param_bf16=torch.empty(n, dtype=torch.bfloat16, device="cuda"),
                              **kw)
    run(whole, grads)
    first = zs.ShardOptimizer(from_np(p0.copy()), layout=saved_layout, **kw)
    run(first, grads[:2])
    saved = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in first.state_dict().items()}
    del first
    resumed = zs.ShardOptimizer(torch.empty(n, device="cuda"), layout=resumed_layout,
                                param_bf16=torch.empty(n, dtype=torch.bfloat16, device="cuda"), **kw)
    resumed.load_state_dict(saved)
    assert resumed.t == 2
    run(resumed, grads[2:])
    torch.cuda.synchronize()
    assert resumed.t == whole.t == 5
    for name in ("master", "exp_avg", "exp_avg_sq", "param_bf16"):
        assert bits_equal(to_np(getattr(resumed, name)), to_np(getattr(whole, name))), name
    before = to_np(resumed.master)
    with pytest.raises(ValueError):
        resumed.load_state_dict({**saved, "exp_avg": saved["exp_avg"][:-1]})
    assert resumed.t == 5 and bits_equal(to_np(resumed.master), before)   # a refused state changes nothing


@pytest.mark.parametrize("layout", ["tiled", "split"])
@pytest.mark.parametrize("max_norm", [0.5, 0.0])
def test_captured_step_replays_like_eager_steps(max_norm, layout):
    """ShardOptimizer.capture: one graph, replayed for four steps with new
    gradients each time, bit-identical to the same steps taken eagerly by a
    twin optimizer (step counter, master, moments, bf16 parameter, norm)."""
    print(f"ShardOptimizer capture max_norm={max_norm} layout={layout}", flush=True)
    n, M, scale = 50_003, 3, 1 / 24
    gen = torch.Generator(device="cuda")
    gen.manual_seed(31)
    p0 = torch.rand(n, generator=gen, device="cuda") * 0.2 - 0.1
    kw = dict(lr=3e-4, betas=(0.9, 0.95), weight_decay=0.1, grad_scale=scale, max_norm=max_norm, layout=layout)
    a = zs.ShardOptimizer(p0.clone(), param_bf16=torch.empty(n, dtype=torch.bfloat16, device="cuda"), **kw)
    b = zs.ShardOptimizer(p0.clone(), param_bf16=torch.empty(n, dtype=torch.bfloat16, device="cuda"), **kw)
    grads = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(M)]
    cap = a.capture(grads, extra_norm_sq=0.02)
    # the twin runs the schedule the capture records: the last gradient goes
    # to step() (its sum with the accumulator never stored)
    torch.cuda.synchronize()
    assert a.t == 0 and bits_equal(to_np(a.master), to_np(p0))   # capturing changed nothing
    for t in range(1, 5):
        for k, g in enumerate(grads):
            g.copy_((torch.randn(n, generator=gen, device="cuda") * 1e-2 * (k + t)).to(torch.bfloat16))
        cap.replay()
        for g in grads[:M - 1]:
            b.accumulate(g)
        b.step(extra_norm_sq=0.02, last_grad=grads[-1])
        torch.cuda.synchronize()
        assert a.t == b.t == t
        for name in ("master", "exp_avg", "exp_avg_sq", "param_bf16", "acc"):
            assert bits_equal(to_np(getattr(a, name)), to_np(getattr(b, name))), (t, name)
        if max_norm > 0:
            assert a.norm_sq.item() == b.norm_sq.item()
        _ = (a.acc * 2).sum().item()   # unrelated eager work between replays


@pytest.mark.parametrize("layout", ["tiled", "split"])
@pytest.mark.parametrize("M", [1, 3])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("max_norm", [0.4, 0.0])
def test_step_with_last_grad_equals_accumulate_then_step(layout, M, dtype, max_norm):
    """step(last_grad=g) against accumulate(g, last=True) then step(), over
    four steps of M micro-batches: master, moments, bf16 parameter and norm
    bit-identical; the accumulator keeps the earlier micro-batches' sum (bit
    for bit the oracle's fold of them)."""
    print(f"ShardOptimizer last_grad layout={layout} M={M} dtype={dtype} max_norm={max_norm}", flush=True)
    n = 2 * zs.STATE_TILE + 4099
    rng = np.random.default_rng(M * 7 + (dtype == torch.float32) + int(max_norm * 10))
    p0 = from_np(rng.uniform(-0.1, 0.1, n).astype(np.float32))
    kw = dict(lr=3e-4, betas=(0.9, 0.95), weight_decay=0.1, grad_scale=1 / (4 * M), max_norm=max_norm,
              layout=layout, compute_norm=True)
    a, b = (zs.ShardOptimizer(p0.clone(), param_bf16=torch.empty(n, dtype=torch.bfloat16, device="cuda"), **kw)
            for _ in range(2))
    bf16 = dtype == torch.bfloat16
    for t in range(1, 5):
        mbs = [(rng.standard_normal(n) * 0.05 * (k + t)).astype(np.float32) for k in range(M)]
        mbs = [oracle.bf16_rne(g) for g in mbs] if bf16 else mbs
        gpu = [from_np(g, bf16=bf16) for g in mbs]
        for g in gpu[:-1]:
            a.accumulate(g)
            b.accumulate(g)
        a.step(extra_norm_sq=0.05, last_grad=gpu[-1])
        b.accumulate(gpu[-1], last=True)
        b.step(extra_norm_sq=0.05)
        torch.cuda.synchronize()
        assert a.t == b.t == t
        assert a.norm_sq.item() == b.norm_sq.item(), t
        for name in ("master", "exp_avg", "exp_avg_sq", "param_bf16"):
            assert bits_equal(to_np(getattr(a, name)), to_np(getattr(b, name))), (t, name)
        if M > 1:
            acc_ref = np.empty(n, np.float32)
            for k, g in enumerate(mbs[:-1]):
                oracle.grad_accum(acc_ref, g, oracle.BF16 if bf16 else oracle.F32, overwrite=(k == 0))
            assert bits_equal(to_np(a.acc), acc_ref), t
    with pytest.raises(RuntimeError):   # the last micro-batch handed over twice
        a.accumulate(gpu[0], last=True)
        a.step(last_grad=gpu[0])


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("layout", ["tiled", "split"])
def test_accumulate_all_matches_one_call_per_micro_batch(layout, fused):
    """accumulate_all over a step's staged micro-batch gradients (19 of them:
    more than one pass of 16, and after one accumulate()) against accumulate()
    per micro-batch with the norm formed by step(): accumulator equal to the
    oracle's left fold, and accumulator, norm, master, moments and bf16
    parameter bit-identical between the two over three clipped steps.  With
    fused=True the one pass also forms the norm: the accumulator is still
    bit-identical and the norm within the fused norms' tolerance of the
    oracle's norm of the same accumulator (its last bits, and so the clipped
    step's, may differ from the separate norm pass's).  In both cases the
    master, moments and bf16 parameter of the accumulate_all optimizer are
    bit-identical to the oracle's AdamW stepped from the oracle's
    accumulator with the GPU's own norm."""
    print(f"ShardOptimizer accumulate_all layout={layout} fused={fused}", flush=True)
    n, M = 2 * zs.STATE_TILE + 777, 19
    rng = np.random.default_rng(41)
    p0_host = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    p0 = from_np(p0_host)
    kw = dict(lr=3e-4, betas=(0.9, 0.95), weight_decay=0.1, grad_scale=1 / M, max_norm=0.5, layout=layout)
    a, b = (zs.ShardOptimizer(p0.clone(), param_bf16=torch.empty(n, dtype=torch.bfloat16, device="cuda"), **kw)
            for _ in range(2))
    ref = {"master": p0_host.copy(), "exp_avg": np.zeros(n, np.float32), "exp_avg_sq": np.zeros(n, np.float32),
           "param_bf16": np.zeros(n, np.uint16)}
    for t in range(1, 4):
        mbs = [oracle.bf16_rne((rng.standard_normal(n) * 0.05 * (k + t)).astype(np.float32)) for k in range(M)]
        gpu = [from_np(g, bf16=True) for g in mbs]
        a.accumulate(gpu[0])
        a.accumulate_all(gpu[1:], last=fused)
        for g in gpu:
            b.accumulate(g)
        acc_ref = np.empty(n, np.float32)
        for k, g in enumerate(mbs):
            oracle.grad_accum(acc_ref, g, oracle.BF16, overwrite=(k == 0))
        torch.cuda.synchronize()
        assert bits_equal(to_np(a.acc), acc_ref), t
        a.step(extra_norm_sq=0.1)
        b.step(extra_norm_sq=0.1)
        torch.cuda.synchronize()
        assert oracle.clip_coef(a.norm_sq.item(), 0.1, 0.5) < 1.0   # every step clips
        assert bits_equal(to_np(a.acc), to_np(b.acc))
        hp_orc = oracle.make_hp(3e-4, 0.9, 0.95, 1e-8, 0.1, 1 / M, 0.5, 0.1, t)
        assert oracle.adamw_step(hp_orc, ref["master"], ref["exp_avg"], ref["exp_avg_sq"], acc_ref,
                                 ref["param_bf16"], norm_sq=a.norm_sq.item()) == 0
        for name in ("master", "exp_avg", "exp_avg_sq", "param_bf16"):
            assert bits_equal(to_np(getattr(a, name)), ref[name]), (t, name, "vs the oracle")
        if fused:
            S = oracle.grad_norm_sq(acc_ref, 1 / M)
            assert abs(a.norm_sq.item() - S) <= NORM_TOL * S
            continue
        assert a.norm_sq.item() == b.norm_sq.item()
        for name in ("master", "exp_avg", "exp_avg_sq", "param_bf16"):
            assert bits_equal(to_np(getattr(a, name)), to_np(getattr(b, name))), (t, name)
    with pytest.raises(ValueError):
        a.accumulate_all([])


@pytest.mark.parametrize("layout", ["split", "tiled"])
@pytest.mark.parametrize("k", [1, 4])
def test_ledger_bytes_match_the_device_allocator(layout, k):
    """ledger.library_shard_bytes against what torch's device allocator
    hands out for one rank's buffers: a ShardOptimizer (fp32 master,
    exp_avg, exp_avg_sq and accumulator, split or tiled) with its bf16
    parameter and k bf16 micro-batch gradients in flight.  The allocated
    bytes grow by the ledger's figure plus the norm's fp64 and workspace (and
    the tiled state's last-tile padding), up to the allocator's rounding of
    each buffer to 512 bytes."""
    from fsdp_sharded_optimizer_amd import ledger
    n = (1 << 22) + 12345
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    before = torch.cuda.memory_allocated()
    master = torch.zeros(n, device="cuda")
    opt = zs.ShardOptimizer(master, lr=1e-3, param_bf16=torch.empty(n, dtype=torch.bfloat16, device="cuda"),
                            layout=layout)
    if layout == "tiled":
        del master            # the tiled state holds the values; the caller's tensor may go
    grads = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(k)]
    torch.cuda.synchronize()
    got = torch.cuda.memory_allocated() - before
    want = ledger.library_shard_bytes(n, grad_buffers=k) + 8 + opt.workspace.numel()
    if layout == "tiled":
        want += (zs.state_tiled_numel(n) - 3 * n) * 4
    buffers = 4 + k + (3 if layout == "split" else 2)   # + norm, workspace, param; master / state, acc
    print(f"ledger {layout} k={k}: allocated {got}, ledger + norm scratch {want}", flush=True)
    assert want <= got <= want + 512 * buffers, (got, want)
    del opt, grads
