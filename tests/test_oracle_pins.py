"""Pins of the oracle against things other than itself (CPU only).

Each test names what fixes the expected value: a closed form, brute force
over a small domain, an invariant of the method, a value worked by hand
from the pages' formula (tests/golden/), or an independent library routine
(torch CPU).  Together they are chosen so that a plausible slip in the
oracle — a dropped term, a swapped beta, a wrong sign, an off-by-one in the
step counter or an index — fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import BF16, F32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f32_bits(x) -> int:
    return int(np.array([x], dtype=np.float32).view(np.uint32)[0])


def hp(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.0, scale=1.0, max_norm=0.0, extra=0.0, step=1):
    return oracle.make_hp(lr, beta1, beta2, eps, wd, scale, max_norm, extra, step)


# ---------------------------------------------------------------------------
# bf16 round-to-nearest-even (the re-cast of the fp32 master)
# ---------------------------------------------------------------------------

def test_bf16_rne_exhaustive_vs_torch(orc):
    """All 2^32 fp32 patterns against torch CPU .to(bfloat16) (library pin).
    NaNs: torch's encoding differs; both must be NaN, the oracle's 0x7FC0."""
    chunk = 1 << 24
    base = np.arange(chunk, dtype=np.uint32)
    bits = np.empty(chunk, dtype=np.uint32)       # buffers reused across chunks
    mine = np.empty(chunk, dtype=np.uint16)
    ref = torch.empty(chunk, dtype=torch.bfloat16)
    neq = np.empty(chunk, dtype=bool)
    for c in range((1 << 32) // chunk):
        np.add(base, np.uint32(c * chunk), out=bits)
        x = bits.view(np.float32)
        oracle.bf16_rne(x, out=mine)
        ref.copy_(torch.from_numpy(x))
        np.not_equal(mine, ref.view(torch.int16).numpy().view(np.uint16), out=neq)
        if neq.any():   # only NaN inputs may differ, and the oracle writes 0x7FC0 for them
            diff = np.flatnonzero(neq)
            assert np.all(np.isnan(x[diff])), f"chunk {c}: non-NaN mismatch at {bits[diff[0]]:#x}"
            assert np.all(mine[diff] == 0x7FC0)
    nan_bits = np.array([0x7F800001, 0x7FC00000, 0x7FFFFFFF, 0xFF800001, 0xFFFFFFFF], dtype=np.uint32)
    assert np.all(oracle.bf16_rne(nan_bits.view(np.float32)) == 0x7FC0)


def test_bf16_rne_ties_and_overflow(orc):
    # 1 + 2^-8 is a tie between 1.0 and 1+2^-7: even mantissa wins -> 1.0
    assert oracle.bf16_rne(np.float32(1 + 2**-8))[()] == 0x3F80
    # 1 + 3*2^-8 is a tie between 1+2^-7 (odd) and 1+2^-6 (even) -> 1.015625
    assert oracle.bf16_rne(np.float32(1 + 3 * 2**-8))[()] == 0x3F82
    # just above the tie rounds up
    assert oracle.bf16_rne(np.array([0x3F808001], dtype=np.uint32).view(np.float32))[0] == 0x3F81
    # largest finite fp32 rounds to +inf in bf16; sign carried
    assert oracle.bf16_rne(np.array([0x7F7FFFFF], dtype=np.uint32).view(np.float32))[0] == 0x7F80
    assert oracle.bf16_rne(np.array([0xFF7FFFFF], dtype=np.uint32).view(np.float32))[0] == 0xFF80
    assert oracle.bf16_rne(np.float32(-0.0))[()] == 0x8000
    # every NaN (quiet, signalling, negative, any payload) becomes 0x7FC0
    nans = np.array([0x7FC00000, 0x7F800001, 0xFFC00000, 0x7FFFFFFF, 0xFF812345], dtype=np.uint32)
    assert np.all(oracle.bf16_rne(nans.view(np.float32)) == 0x7FC0)


def test_bf16_widen_all_patterns_vs_torch(orc):
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = oracle.bf16_widen(b)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# ---------------------------------------------------------------------------
# shard range
# ---------------------------------------------------------------------------

def test_shard_range_golden(orc):
    for case in _golden("shard_ranges.json")["cases"]:
        got = oracle.shard_range(case["total"], case["world"], case["rank"])
        assert got == (case["chunk"], case["start"], case["end"], case["padded_total"]), case["name"]


def _shard_brute(max_total: int, max_world: int):
    for T in range(0, max_total + 1):
        for N in range(1, max_world + 1):
            c = 0
            while N * c < T:
                c += 1
            owner = [i // c for i in range(T)] if c else []
            covered = []
            for r in range(N):
                chunk, start, end, padded = oracle.shard_range(T, N, r)
                assert chunk == c and padded == N * c
                mine = [i for i in range(T) if owner[i] == r]
                if mine:
                    assert (start, end) == (mine[0], mine[-1] + 1)
                else:
                    assert start == end and start == min(r * c, T)
                covered += list(range(start, end))
            assert covered == list(range(T))
            assert padded % N == 0 and padded - T < max(N, 1)


def test_shard_range_brute_force(orc):
    """For every T <= 300, N <= 40 and rank: the ranges are exactly the
    index classes {i in [0,T): i // c == r} for the smallest c with N*c >= T,
    found by search, so they tile [0, T) with no overlap."""
    _shard_brute(300, 40)


def test_shard_range_brute_force_small(orc):
    _shard_brute(60, 12)


def test_shard_range_rejects(orc):
    for args in [(10, 0, 0), (10, 4, 4), (10, 4, -1), (-1, 4, 0)]:
        with pytest.raises(ValueError):
            oracle.shard_range(*args)


# ---------------------------------------------------------------------------
# flatten / unflatten
# ---------------------------------------------------------------------------

def _rand_shapes(rng, k):
    return [tuple(int(d) for d in rng.integers(1, 9, size=rng.integers(1, 4))) for _ in range(k)]


@pytest.mark.parametrize("seed", range(6))
def test_flat_pack_matches_concatenate(orc, seed):
    """Library pin: numpy.concatenate of the row-major ravels, then zeros."""
    rng = np.random.default_rng(seed)
    shapes = _rand_shapes(rng, int(rng.integers(0, 9)))
    srcs = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    T = sum(int(np.prod(s)) for s in shapes)
    N = int(rng.integers(1, 7))
    padded = oracle.shard_range(T, N, 0)[3]
    flat = oracle.flat_pack(srcs, F32, F32, padded)
    ref = np.concatenate([s.ravel() for s in srcs] + [np.zeros(padded - T, np.float32)])
    assert np.array_equal(flat.view(np.uint32), ref.view(np.uint32))
    # element (tensor t, index j) sits at prefix-sum offset + j
    off = 0
    for t, s in enumerate(srcs):
        for j in range(s.size):
            assert flat[off + j].view(np.uint32) == s.ravel()[j].view(np.uint32)
        off += s.size
    # unpack is the inverse and never reads the padding
    back = oracle.flat_unpack(flat, F32, [s.size for s in srcs], F32)
    for b, s in zip(back, srcs):
        assert np.array_equal(b.view(np.uint32), s.ravel().view(np.uint32))


def test_flat_pack_bf16_and_widen(orc):
    rng = np.random.default_rng(7)
    srcs = [rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16) for n in (5, 1, 17, 8)]
    T = 31
    flat16 = oracle.flat_pack(srcs, BF16, BF16, 32)
    assert np.array_equal(flat16, np.concatenate(srcs + [np.zeros(1, np.uint16)]))
    flat32 = oracle.flat_pack(srcs, BF16, F32, 34)
    ref = torch.from_numpy(np.concatenate(srcs).view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(flat32[:T]), nan)
    assert np.array_equal(flat32[:T][~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.all(flat32[T:].view(np.uint32) == 0)
    # unpack fp32 -> bf16 is the RNE re-cast
    vals = rng.standard_normal(12).astype(np.float32)
    out = oracle.flat_unpack(vals, F32, [7, 5], BF16)
    torch_b = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(np.concatenate(out), torch_b)


def test_flat_pack_rejects(orc):
    with pytest.raises(ValueError):
        oracle.flat_pack([np.zeros(5, np.float32)], F32, F32, 4)        # padded < total
    with pytest.raises(ValueError):
        oracle.flat_pack([np.zeros(5, np.float32)], F32, BF16, 8)       # narrowing pack
    with pytest.raises(ValueError):
        oracle.flat_unpack(np.zeros(5, np.uint16), BF16, [5], F32)      # widening unpack


def test_fsdp_unit_rank17_maps_into_gate_proj(orc):
    """The 70B block unit: the tensor offsets and the rank-17 range follow
    from the shapes alone; a scaled-down copy of the unit (same order, every
    dimension divided by 128 or 8) checks that the oracle's pack puts every
    element of every tensor at its row-major offset."""
    import workloads
    w = workloads.WORKLOADS["fsdp_unit_70b_block"]
    numels = [workloads.numel_of(s) for _, s in w.unit_shapes]
    offsets = np.concatenate([[0], np.cumsum(numels)]).tolist()
    assert offsets[:8] == [0, 67108864, 75497472, 83886080, 150994944, 385875968, 620756992, 855638016]
    chunk, start, end, padded = oracle.shard_range(w.total, w.world, w.rank)
    assert (start, end, padded) == (227283200, 240652800, 855654400)
    gate = 4
    assert offsets[gate] <= start and end <= offsets[gate + 1]
    assert divmod(start - offsets[gate], 8192) == (9312, 4352)
    assert divmod(end - 1 - offsets[gate], 8192) == (10944, 4607)
    # scaled copy: hidden 64, ffn 224, heads 8 q / 1 kv of width 8
    small = workloads.block70b_tensor_shapes(hidden=64, ffn=224, q_heads=8, kv_heads=1, head_dim=8)
    rng = np.random.default_rng(3)
    srcs = [rng.integers(0, 1 << 16, size=s, dtype=np.uint32).astype(np.uint16) for _, s in small]
    Ts = sum(x.size for x in srcs)
    flat = oracle.flat_pack(srcs, BF16, BF16, oracle.shard_range(Ts, 64, 0)[3])
    off = 0
    for x in srcs:
        if x.ndim == 2:
            r = rng.integers(0, x.shape[0], 50)
            c = rng.integers(0, x.shape[1], 50)
            assert np.array_equal(flat[off + r * x.shape[1] + c], x[r, c])
        else:
            assert np.array_equal(flat[off:off + x.size], x)
        off += x.size


# ---------------------------------------------------------------------------
# gradient accumulation
# ---------------------------------------------------------------------------

def test_grad_accum_closed_form_power_of_two(orc):
    """Adding x eight times gives 8x exactly when every partial sum k*x is
    representable (x has <= 8 significant bits, so k*x has <= 11)."""
    rng = np.random.default_rng(1)
    x16 = oracle.bf16_rne(rng.standard_normal(4096).astype(np.float32) * 1e-3)
    acc = np.empty(4096, np.float32)
    for mb in range(8):
        oracle.grad_accum(acc, x16, BF16, overwrite=(mb == 0))
    assert np.array_equal(acc, oracle.bf16_widen(x16) * np.float32(8))


def test_grad_accum_overwrite_keeps_negative_zero(orc):
    acc = np.full(3, 5.0, np.float32)
    g = np.array([0x8000, 0x0000, 0x3F80], np.uint16)
    oracle.grad_accum(acc, g, BF16, overwrite=True)
    assert acc.view(np.uint32).tolist() == [0x80000000, 0, 0x3F800000]


def test_grad_accum_matches_torch_add(orc):
    """Library pin: the page's own op, acc.add_(grad.float()), on torch CPU."""
    rng = np.random.default_rng(2)
    acc = rng.standard_normal(10000).astype(np.float32)
    g32 = rng.standard_normal(10000).astype(np.float32) * np.float32(1e-3)
    g16 = torch.from_numpy(g32).to(torch.bfloat16)
    ref = torch.from_numpy(acc.copy()).add_(g16.float()).numpy()
    mine = acc.copy()
    oracle.grad_accum(mine, g16.view(torch.int16).numpy().view(np.uint16), BF16, overwrite=False)
    assert np.array_equal(mine.view(np.uint32), ref.view(np.uint32))
    ref32 = torch.from_numpy(acc.copy()).add_(torch.from_numpy(g32)).numpy()
    mine32 = acc.copy()
    oracle.grad_accum(mine32, g32, F32, overwrite=False)
    assert np.array_equal(mine32.view(np.uint32), ref32.view(np.uint32))


def test_grad_accum_error_bound_vs_exact_sum(orc):
    """Against the exact real sum (math.fsum of the widened micro-batches):
    sequential fp32 addition of M terms is within (M-1) u sum|terms|."""
    rng = np.random.default_rng(4)
    M, n = 8, 2000
    mbs = [oracle.bf16_rne(rng.standard_normal(n).astype(np.float32)) for _ in range(M)]
    acc = np.empty(n, np.float32)
    for k, g in enumerate(mbs):
        oracle.grad_accum(acc, g, BF16, overwrite=(k == 0))
    wide = np.stack([oracle.bf16_widen(g).astype(np.float64) for g in mbs])
    exact = np.array([math.fsum(wide[:, i]) for i in range(n)])
    bound = (M - 1) * 2.0**-24 * np.abs(wide).sum(0) * (1 + 1e-6)
    assert np.all(np.abs(acc - exact) <= bound)
    # and the sum is of all M terms, not M-1
    assert np.max(np.abs(acc - (exact - wide[-1]))) > 1e-3


# ---------------------------------------------------------------------------
# scaled squared norm and the clip coefficient
# ---------------------------------------------------------------------------

def test_norm_sq_closed_forms(orc):
    # constant 2^-7 with scale 1/8 -> g1 = 2^-10; 2^20 elements -> S = 1 exactly
    acc = np.full(1 << 20, 2.0**-7, np.float32)
    assert oracle.grad_norm_sq(acc, 1.0 / 8) == 1.0
    # crosses the 2^20 block boundary: 2^20 + 3 elements
    acc = np.full((1 << 20) + 3, 2.0**-7, np.float32)
    assert oracle.grad_norm_sq(acc, 1.0 / 8) == 1.0 + 3 * 2.0**-20
    # one-hot
    acc = np.zeros(1000, np.float32)
    acc[637] = 2.0
    assert oracle.grad_norm_sq(acc, 1.0) == 4.0
    assert oracle.grad_norm_sq(acc, 1.0 / 8) == 1.0 / 16
    assert oracle.grad_norm_sq(acc[:0], 1.0) == 0.0


def test_norm_sq_vs_exact_sum(orc):
    """math.fsum of the exact squares of g1 = fl32(acc * s): the oracle's
    binary64 sum is within n * 2^-53 relative."""
    rng = np.random.default_rng(5)
    acc = (rng.standard_normal(300_000) * 1e-3).astype(np.float32)
    s = 1.0 / 64
    g1 = acc * np.float32(s)     # one binary32 multiply per element
    exact = math.fsum((g1.astype(np.float64) ** 2).tolist())
    got = oracle.grad_norm_sq(acc, s)
    assert abs(got - exact) <= 300_000 * 2.0**-53 * exact
    # the scale enters squared: the same buffer at scale 1 is 4096x larger
    assert abs(oracle.grad_norm_sq(acc, 1.0) / got - 4096.0) < 1e-9


def test_clip_coef_vs_torch_clip_grad_norm(orc):
    """Library pin: torch.nn.utils.clip_grad_norm_ on the same scaled grads,
    spread over several tensors; total norm and the scaled grads agree."""
    rng = np.random.default_rng(6)
    for target in (2.0, 0.5, 1.37):
        parts = [rng.standard_normal(n).astype(np.float32) for n in (100, 1000, 37)]
        flat = np.concatenate(parts)
        flat *= np.float32(target / np.linalg.norm(flat.astype(np.float64)))
        S = oracle.grad_norm_sq(flat, 1.0)
        params = [torch.nn.Parameter(torch.zeros(p.size)) for p in parts]
        off = 0
        for p, a in zip(params, parts):
            p.grad = torch.from_numpy(flat[off:off + a.size].copy())
            off += a.size
        total = torch.nn.utils.clip_grad_norm_(params, max_norm=1.0)
        assert abs(math.sqrt(S) - float(total)) <= 1e-6 * float(total)
        coef = oracle.clip_coef(S, 0.0, 1.0)
        torch_scaled = torch.cat([p.grad for p in params]).numpy()
        mine = flat * np.float32(coef)
        assert np.max(np.abs(mine - torch_scaled) / np.maximum(np.abs(torch_scaled), 1e-30)) <= 2e-7
        if target < 1.0:
            assert coef == 1.0


def test_clip_applies_at_equality_and_splits_over_ranks(orc):
    # norm exactly max_norm: coef = fl32(1/(1+1e-6)) < 1, as torch does
    assert oracle.clip_coef(1.0, 0.0, 1.0) == np.float32(1.0 / (1.0 + 1e-6))
    g = torch.zeros(4)
    g[0] = 1.0
    p = torch.nn.Parameter(torch.zeros(4))
    p.grad = g.clone()
    torch.nn.utils.clip_grad_norm_([p], max_norm=1.0)
    # torch forms 1 + 1e-6 in fp32, the oracle in fp64: the same factor to 1 ulp
    assert float(p.grad[0]) < 1.0
    assert abs(float(p.grad[0]) - oracle.clip_coef(1.0, 0.0, 1.0)) <= 2.0**-23
    # the global norm is the sum over ranks: 0.5 here + 3.5 elsewhere = 4 -> norm 2
    assert oracle.clip_coef(0.5, 3.5, 1.0) == np.float32(1.0 / (2.0 + 1e-6))
    assert oracle.clip_coef(123.0, 0.0, 0.0) == 1.0


# ---------------------------------------------------------------------------
# AdamW step
# ---------------------------------------------------------------------------

def test_fp32_scalars_golden(orc):
    s = oracle.adamw_scalars(hp(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, wd=0.1))
    want = {c["what"]: int(c["hex"], 16) for c in _golden("fp32_scalars.json")["cases"]}
    assert f32_bits(s.beta1) == want["(float)0.9"]
    assert f32_bits(s.one_minus_beta1) == want["(float)(1 - 0.9)"]
    assert f32_bits(s.beta2) == want["(float)0.95"]
    assert f32_bits(s.one_minus_beta2) == want["(float)(1 - 0.95)"]
    assert f32_bits(s.eps) == want["(float)1e-8"]
    assert f32_bits(s.decay) == want["(float)(1 - 3e-4*0.1)"]
    # bias corrections at t = 1: step_size = lr / (1 - beta1), sqrt(1 - beta2)
    assert s.step_size == np.float32(3e-4 / 0.1)
    assert s.bias_correction2_sqrt == np.float32(math.sqrt(1 - 0.95))


def _state(n, seed, p_scale=0.1):
    rng = np.random.default_rng(seed)
    p = (rng.uniform(-p_scale, p_scale, n)).astype(np.float32)
    return p, np.zeros(n, np.float32), np.zeros(n, np.float32)


def test_step1_closed_form(orc):
    """t = 1 from zero moments: m = (1-b1) g, v = (1-b2) g^2, so the update is
    lr * g / (|g| + eps) (eps after bias correction), and with decay the
    master becomes p (1 - lr wd) - lr g / (|g| + eps)."""
    rng = np.random.default_rng(8)
    n = 5000
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    g[:10] = np.float32(1e-8)            # |g| comparable to eps: eps placement matters
    g[10:20] = -np.float32(3e-9)
    for wd, lr in ((0.0, 1e-3), (0.1, 3e-4)):
        p0, m, v = _state(n, 9)
        p = p0.copy()
        assert oracle.adamw_step(hp(lr=lr, beta1=0.9, beta2=0.95, wd=wd), p, m, v, g) == 0
        gd = g.astype(np.float64)
        want = p0.astype(np.float64) * (1 - lr * wd) - lr * gd / (np.abs(gd) + 1e-8)
        kappa = np.abs(p0.astype(np.float64) * (1 - lr * wd)) + lr
        assert np.max(np.abs(p - want) / kappa) <= 1e-6
        assert np.max(np.abs(m - 0.1 * gd) / np.abs(0.1 * gd)) <= 2e-7
        assert np.max(np.abs(v - 0.05 * gd * gd) / (0.05 * gd * gd)) <= 4e-7


def test_step1_grad_scale_enters(orc):
    """With |g1| == eps the step is lr/2; a dropped grad_scale would give
    lr * 8/9 instead."""
    n = 64
    acc = np.full(n, 8e-8, np.float32)
    p, m, v = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)
    oracle.adamw_step(hp(lr=1e-3, eps=1e-8, scale=1.0 / 8), p, m, v, acc)
    assert np.allclose(p, -0.5e-3, rtol=1e-6, atol=0)


@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_constant_grad_k_steps_closed_form(orc, wd):
    """Constant g: m_hat = g and sqrt(v_hat) = |g| exactly in real arithmetic,
    so U = lr g / (|g| + eps) each step and
    p_k = d^k p0 - U (1 - d^k) / (1 - d)   (d = 1 - lr wd; p0 - k U for wd = 0)."""
    rng = np.random.default_rng(10)
    n, K, lr = 3000, 12, 2e-3
    g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    p0, m, v = _state(n, 11)
    p = p0.copy()
    for t in range(1, K + 1):
        oracle.adamw_step(hp(lr=lr, beta1=0.9, beta2=0.99, wd=wd, step=t), p, m, v, g)
        gd = g.astype(np.float64)
        U = lr * gd / (np.abs(gd) + 1e-8)
        d = 1 - lr * wd
        want = p0 * d**t - (U * t if wd == 0 else U * (1 - d**t) / (1 - d))
        kappa = np.abs(p0) * d**t + t * lr
        assert np.max(np.abs(p - want) / kappa) <= 1e-6 * t, t


def test_zero_grad_invariance_and_padding(orc):
    """wd = 0 and g = 0 from the zero state: nothing moves, bit for bit, for
    any number of steps.  Padding (p = 0, g = 0) stays exactly 0 for any wd."""
    p0, m, v = _state(4096, 12)
    p = p0.copy()
    g = np.zeros(4096, np.float32)
    for t in range(1, 8):
        oracle.adamw_step(hp(lr=1e-3, step=t), p, m, v, g)
    assert np.array_equal(p.view(np.uint32), p0.view(np.uint32))
    assert not m.any() and not v.any()
    z = np.zeros(16, np.float32)
    m2, v2, b = np.zeros(16, np.float32), np.zeros(16, np.float32), np.ones(16, np.uint16)
    for t in range(1, 4):
        oracle.adamw_step(hp(lr=1e-3, wd=0.3, step=t), z, m2, v2, np.zeros(16, np.float32), b)
    assert not z.view(np.uint32).any() and not b.any()


def test_sharding_invariance(orc):
    """The update is element-wise ([Memory page] §一: each parameter's Adam
    update is independent), so stepping the whole padded buffer and slicing
    equals stepping each rank's shard alone, bit for bit."""
    import workloads
    rng = np.random.default_rng(13)
    T, N = 1003, 8
    chunk, _, _, padded = oracle.shard_range(T, N, 0)
    p = np.zeros(padded, np.float32)
    p[:T] = rng.uniform(-0.1, 0.1, T)
    g = np.zeros(padded, np.float32)
    g[:T] = rng.standard_normal(T) * 1e-3
    m, v = np.zeros(padded, np.float32), np.zeros(padded, np.float32)
    pw, mw, vw = p.copy(), m.copy(), v.copy()
    H = hp(lr=1e-3, wd=0.1, beta2=0.95, scale=1 / 8)
    oracle.adamw_step(H, pw, mw, vw, g)
    for r in range(N):
        _, s, e, _ = oracle.shard_range(T, N, r)
        ps, ms, vs = p[s:e].copy(), m[s:e].copy(), v[s:e].copy()
        oracle.adamw_step(H, ps, ms, vs, g[s:e].copy())
        assert np.array_equal(ps.view(np.uint32), pw[s:e].view(np.uint32))
        assert np.array_equal(ms.view(np.uint32), mw[s:e].view(np.uint32))
    assert not pw[T:].any()


@pytest.mark.parametrize("seed", range(5))
def test_adamw_vs_torch_adamw(orc, seed):
    """Library pin: torch.optim.AdamW (CPU, foreach=False) with the same grads
    after the same scaling and clipping, random hyperparameters, t up to 10.
    torch associates some operations differently (lerp for the first
    moment), so this is a tolerance, not bit-exactness."""
    rng = np.random.default_rng(100 + seed)
    n = 4096
    lr = float(10 ** rng.uniform(-4, -2))
    b1, b2 = float(rng.uniform(0.8, 0.95)), float(rng.uniform(0.9, 0.999))
    eps = float(10 ** rng.uniform(-9, -6))
    wd = float(rng.uniform(0, 0.2))
    scale = 2.0 ** -int(rng.integers(0, 7))
    p0 = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([tp], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd, foreach=False)
    for t in range(1, 11):
        acc = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        S = oracle.grad_norm_sq(acc, scale)
        max_norm = 1.0 if t % 3 == 0 else 0.0
        if max_norm:
            max_norm = 0.5 * math.sqrt(S)          # force a clip
        H = hp(lr=lr, beta1=b1, beta2=b2, eps=eps, wd=wd, scale=scale, max_norm=max_norm, step=t)
        pb = np.empty(n, np.uint16)
        assert oracle.adamw_step(H, p, m, v, acc, pb, norm_sq=S) == 0
        tg = torch.from_numpy(acc) * np.float32(scale)
        tp.grad = tg.clone()
        if max_norm:
            torch.nn.utils.clip_grad_norm_([tp], max_norm=max_norm)
        opt.step()
        st = opt.state[tp]
        ref_p = tp.detach().numpy()
        kappa_p = np.abs(ref_p) + lr
        assert np.max(np.abs(p - ref_p) / kappa_p) <= 1e-6 * t, t
        ref_m = st["exp_avg"].numpy()
        assert np.max(np.abs(m - ref_m) / (np.abs(ref_m) + 1e-3 * scale * 1e-3)) <= 1e-5 * t
        ref_v = st["exp_avg_sq"].numpy()
        assert np.max(np.abs(v - ref_v) / np.abs(ref_v)) <= 1e-5 * t
        assert np.array_equal(pb, oracle.bf16_rne(p))


def test_adamw_float64_brute_force(orc):
    """A float64 evaluation of the same recurrence on a tiny buffer (the
    fp32 oracle must stay within a few fp32 ulps per step of it)."""
    rng = np.random.default_rng(14)
    n, lr, b1, b2, eps, wd, s = 257, 5e-3, 0.85, 0.97, 1e-7, 0.05, 0.25
    p = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    P, Mv, Vv = p.astype(np.float64), np.zeros(n), np.zeros(n)
    for t in range(1, 9):
        acc = (rng.standard_normal(n) * 1e-2).astype(np.float32)
        oracle.adamw_step(hp(lr=lr, beta1=b1, beta2=b2, eps=eps, wd=wd, scale=s, step=t), p, m, v, acc)
        G = acc.astype(np.float64) * s
        Mv = b1 * Mv + (1 - b1) * G
        Vv = b2 * Vv + (1 - b2) * G * G
        den = np.sqrt(Vv) / math.sqrt(1 - b2**t) + eps
        P = P * (1 - lr * wd) - (lr / (1 - b1**t)) * Mv / den
        assert np.max(np.abs(p - P) / (np.abs(P) + lr)) <= 1e-6 * t


def test_nonfinite_norm_skips_update(orc):
    p0, m, v = _state(100, 15)
    g = np.ones(100, np.float32)
    for S, extra in ((float("inf"), 0.0), (float("nan"), 0.0), (1.0, float("inf"))):
        p = p0.copy()
        assert oracle.adamw_step(hp(max_norm=1.0, extra=extra), p, m, v, g, norm_sq=S) == 1
        assert np.array_equal(p, p0) and not m.any() and not v.any()
    # without a norm there is no check, and the step proceeds
    p = p0.copy()
    assert oracle.adamw_step(hp(), p, m, v, g) == 0 and not np.array_equal(p, p0)


def test_adamw_rejects(orc):
    p, m, v = _state(4, 16)
    for bad in (dict(step=0), dict(beta1=1.0), dict(beta2=-0.1), dict(eps=0.0), dict(lr=-1.0),
                dict(wd=-0.1), dict(scale=0.0)):
        with pytest.raises(ValueError):
            oracle.adamw_step(hp(**bad), p, m, v, np.zeros(4, np.float32))


# ---------------------------------------------------------------------------
# the step with no fp32 master (the ZeRO page's ZeRO-3 listing)
# ---------------------------------------------------------------------------

def test_no_master_one_step_equals_master_recast(orc):
    """From master = widen(param) the two forms compute the same fp32 value;
    the no-master form's parameter is that value's bf16 re-cast.  The second
    case decays hard (lr*wd = 0.05) so a dropped or misplaced decay shows
    through the bf16 rounding; widen(param) is checked against a manual
    (1 - lr wd) p - u to a few bf16 ulps."""
    rng = np.random.default_rng(31)
    n = 4099
    b0 = oracle.bf16_rne(rng.uniform(-0.1, 0.1, n).astype(np.float32))
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    for lr, wd in ((3e-4, 0.1), (1e-2, 5.0)):
        H = hp(lr=lr, beta1=0.9, beta2=0.95, wd=wd, scale=1 / 8)
        master = oracle.bf16_widen(b0).copy()
        m1, v1, b1 = np.zeros(n, np.float32), np.zeros(n, np.float32), b0.copy()
        oracle.adamw_step(H, master, m1, v1, g, b1)
        b2, m2, v2 = b0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
        oracle.adamw_step_no_master(H, b2, m2, v2, g)
        assert np.array_equal(b1, b2) and np.array_equal(m1, m2) and np.array_equal(v1, v2)
        p0 = oracle.bf16_widen(b0).astype(np.float64)
        gd = g.astype(np.float64) / 8
        want = p0 * (1 - lr * wd) - lr * gd / (np.abs(gd) + 1e-8)
        ulp = np.abs(want) * 2.0**-7 + 1e-30
        assert np.all(np.abs(oracle.bf16_widen(b2) - want) <= ulp)


def test_no_master_stalls_below_half_an_ulp(orc):
    """Worked by hand: 0.1 rounds to bf16 0x3DCD; its ulp is 2^-11 =
    4.8828125e-4.  With constant g (wd = 0) every step moves by lr in real
    arithmetic.  lr = 1e-4 is under half an ulp: the bf16 parameter never
    moves (the fp32 master moves 10 lr in 10 steps).  lr = 3e-4 is over
    half an ulp: the parameter moves a whole ulp each step."""
    n = 64
    g = np.full(n, 2e-3, np.float32)
    for lr, want in ((1e-4, 0x3DCD), (3e-4, 0x3DCD - 10)):
        b = np.full(n, 0x3DCD, np.uint16)
        m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
        master = oracle.bf16_widen(b).copy()
        mm, vv = np.zeros(n, np.float32), np.zeros(n, np.float32)
        for t in range(1, 11):
            H = hp(lr=lr, beta1=0.9, beta2=0.999, step=t)
            oracle.adamw_step_no_master(H, b, m, v, g)
            oracle.adamw_step(H, master, mm, vv, g)
        assert np.all(b == want), (lr, hex(int(b[0])))
        assert np.allclose(master, oracle.bf16_widen(np.full(n, 0x3DCD, np.uint16)) - 10 * lr, rtol=0, atol=1e-6)


# ---------------------------------------------------------------------------
# ZeRO-1 form: the update vector, its gather and its apply
# ---------------------------------------------------------------------------

def _abits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def test_adam_update_added_to_param_equals_master_step(orc):
    """With no decay, p + update is the master path's new p, bit for bit
    (fl(p + fl(r * -s)) = fl(p - fl(r * s)) as IEEE rounding is symmetric),
    over steps with and without a clip; the moments agree too."""
    rng = np.random.default_rng(41)
    n = 5003
    p0 = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    p0[:3] = (0.0, -0.0, 1e-40)
    master, m1, v1 = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    p, m2, v2 = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    upd = np.empty(n, np.float32)
    for t in range(1, 7):
        acc = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        acc[:2] = 0.0
        S = oracle.grad_norm_sq(acc, 1 / 8)
        H = hp(lr=1e-4, beta1=0.9, beta2=0.999, scale=1 / 8, max_norm=0.6 * math.sqrt(S) if t % 2 else 0.0,
               extra=0.1 * S, step=t)
        assert oracle.adamw_step(H, master, m1, v1, acc, norm_sq=S) == 0
        assert oracle.adam_update(H, m2, v2, acc, upd, norm_sq=S) == 0
        p = p + upd   # numpy float32 addition, IEEE round to nearest
        assert np.array_equal(_abits(p), _abits(master)), t
        assert np.array_equal(m1, m2) and np.array_equal(v1, v2)


def _adam_update_float64(g, m, v, t, lr, b1, b2, eps):
    """Adam written from its equations in float64 (ZeRO page, §"ZeRO-1:
    切分优化器状态": exponential moving averages of g and g^2, both bias
    corrected, eps added to the corrected second moment's square root, the
    update is minus the learning rate times the corrected first moment over
    that denominator).  Returns the update and the new moments."""
    m = b1 * m + (1.0 - b1) * g
    v = b2 * v + (1.0 - b2) * g * g
    m_hat = m / (1.0 - b1 ** t)
    v_hat = v / (1.0 - b2 ** t)
    return -lr * m_hat / (np.sqrt(v_hat) + eps), m, v


def test_adam_update_vs_adam_equations_float64(orc):
    """The oracle's fp32 update and moments against Adam's equations
    evaluated in numpy float64 (the bias-corrected form m_hat / (sqrt(v_hat)
    + eps), not the oracle's op order): they agree to a few fp32 ulps per
    step."""
    rng = np.random.default_rng(43)
    n = 4096
    lr, b1, b2, eps = 1e-4, 0.9, 0.999, 1e-8
    m, v, upd = np.zeros(n, np.float32), np.zeros(n, np.float32), np.empty(n, np.float32)
    em, ev = np.zeros(n), np.zeros(n)
    for t in range(1, 9):
        acc = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        assert oracle.adam_update(hp(lr=lr, beta1=b1, beta2=b2, eps=eps, scale=1 / 8, step=t), m, v, acc, upd) == 0
        g = acc.astype(np.float64) / 8
        kappa_m = b1 * np.abs(em) + (1 - b1) * np.abs(g)   # guards a cancellation in m
        ref, em, ev = _adam_update_float64(g, em, ev, t, lr, b1, b2, eps)
        assert np.max(np.abs(upd - ref)) <= 4e-7 * t * lr, t
        assert np.max(np.abs(m - em) / kappa_m) <= 1e-6 * t
        assert np.max(np.abs(v - ev) / ev) <= 1e-6 * t


def test_adam_update_step1_closed_form(orc):
    """At t = 1 the bias corrections cancel the (1 - beta) factors:
    update = -lr g / (|g| + eps) up to a few roundings."""
    rng = np.random.default_rng(47)
    n = 3001
    g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    m, v, upd = np.zeros(n, np.float32), np.zeros(n, np.float32), np.empty(n, np.float32)
    assert oracle.adam_update(hp(lr=0.01, beta1=0.8, beta2=0.99, eps=1e-8), m, v, g, upd) == 0
    gd = g.astype(np.float64)
    want = -0.01 * gd / (np.abs(gd) + 1e-8)
    assert np.max(np.abs(upd - want)) <= 1e-8
    assert np.all(np.sign(upd) == -np.sign(g))


def test_adam_update_rejects_decay_and_skips_nonfinite(orc):
    n = 16
    m, v, g, u = (np.zeros(n, np.float32) for _ in range(4))
    with pytest.raises(ValueError):
        oracle.adam_update(hp(wd=0.1), m, v, g, u)
    u[:] = 7.0
    assert oracle.adam_update(hp(max_norm=1.0), m, v, g + 1, u, norm_sq=float("nan")) == 1
    # skipped: the moments stay, the update is -0.0 everywhere (what the
    # apply after the all-gather must add to change nothing)
    assert np.all(m == 0) and np.all(v == 0)
    assert np.all(u.view(np.uint32) == 0x80000000)
    assert oracle.adam_update(hp(), m, v, g + 1, u, norm_sq=float("inf")) == 1


def test_skipped_adam_update_applies_as_identity(orc):
    """A skipped ZeRO-1 step (non-finite norm) followed by the apply leaves
    every parameter bit for bit as it was: -0.0 is the identity of IEEE
    addition (numpy float32 addition agrees), so +-0.0, subnormals, +-inf,
    NaN and ordinary fp32 values all survive; bf16 parameters (finite, +-0,
    +-inf) too."""
    specials = np.array([0.0, -0.0, 1e-45, -1e-45, 1.17549435e-38, np.inf, -np.inf, np.nan, 1.0, -3.5e-7,
                         3.4028235e38], np.float32)
    rng = np.random.default_rng(7)
    p32 = np.concatenate([specials, rng.uniform(-1, 1, 1000).astype(np.float32)])
    n = p32.size
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    upd = np.full(n, 5.0, np.float32)   # a stale update from an earlier step
    g = rng.standard_normal(n).astype(np.float32)
    assert oracle.adam_update(hp(max_norm=1.0), m, v, g, upd, norm_sq=float("nan")) == 1
    numpy_sum = p32 + upd
    assert np.array_equal(numpy_sum.view(np.uint32), p32.view(np.uint32))
    before = p32.copy()
    oracle.flat_apply_update(upd, [p32], F32)
    assert np.array_equal(p32.view(np.uint32), before.view(np.uint32))
    b16 = np.concatenate([np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x0001, 0x3F80], np.uint16),
                          oracle.bf16_rne(rng.uniform(-1, 1, n - 6).astype(np.float32))])
    b_before = b16.copy()
    oracle.flat_apply_update(upd, [b16], BF16)
    assert np.array_equal(b16, b_before)


@pytest.mark.parametrize("seed", range(3))
def test_flat_apply_update_matches_slices(orc, seed):
    """fp32 tensors: numpy slicing of the update at the running offsets plus
    numpy float32 addition.  bf16 tensors: torch's in-place add of an fp32
    tensor into a bf16 one on the CPU.  Padding past the tensors is NaN and
    must never be read."""
    rng = np.random.default_rng(200 + seed)
    shapes = _rand_shapes(rng, int(rng.integers(1, 40)))
    numels = [int(np.prod(s)) for s in shapes]
    T = sum(numels)
    upd = np.full(T + 11, np.nan, np.float32)
    upd[:T] = (rng.standard_normal(T) * 1e-3).astype(np.float32)
    p32 = [rng.uniform(-1, 1, k).astype(np.float32) for k in numels]
    want32 = []
    off = 0
    for x, k in zip(p32, numels):
        want32.append(x + upd[off:off + k])
        off += k
    oracle.flat_apply_update(upd, p32, F32)
    for a, b in zip(p32, want32):
        assert np.array_equal(_abits(a), _abits(b))
    pb = [oracle.bf16_rne(rng.uniform(-1, 1, k).astype(np.float32)) for k in numels]
    wantb = []
    off = 0
    for x, k in zip(pb, numels):
        t = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16)
        t.add_(torch.from_numpy(upd[off:off + k].copy()))
        wantb.append(t.view(torch.int16).numpy().view(np.uint16))
        off += k
    oracle.flat_apply_update(upd, pb, BF16)
    for a, b in zip(pb, wantb):
        assert np.array_equal(a, b)


def test_flat_apply_update_zero_update_is_identity(orc):
    rng = np.random.default_rng(5)
    p = [rng.uniform(-1, 1, k).astype(np.float32) for k in (3, 1, 17)]
    before = [x.copy() for x in p]
    oracle.flat_apply_update(np.zeros(21, np.float32), p, F32)
    for a, b in zip(p, before):
        assert np.array_equal(a, b)


def test_zero1_flow_equals_one_buffer_step(orc):
    """The ZeRO page's ZeRO-1 flow on N ranks: flatten the model's grads
    (padded to N*chunk), each rank runs the update on its slice (a view at
    any element offset) with its own moments and writes its chunk of the
    gathered buffer, then every parameter adds its part.  The parameters
    equal one master step over the whole buffer followed by an unflatten:
    ranks are independent because the update is element-wise."""
    rng = np.random.default_rng(53)
    shapes = [(37, 11), (5,), (64, 3), (1,), (29, 7)]
    numels = [int(np.prod(s)) for s in shapes]
    T, N = sum(numels), 6
    chunk, _, _, padded = oracle.shard_range(T, N, 0)
    params = [rng.uniform(-0.1, 0.1, k).astype(np.float32) for k in numels]
    flat_master = oracle.flat_pack(params, F32, F32, padded)
    M, V = np.zeros(padded, np.float32), np.zeros(padded, np.float32)
    ms = [np.zeros(chunk, np.float32) for _ in range(N)]
    vs = [np.zeros(chunk, np.float32) for _ in range(N)]
    for t in range(1, 4):
        grads = [(rng.standard_normal(k) * 1e-3).astype(np.float32) for k in numels]
        flat_grad = oracle.flat_pack(grads, F32, F32, padded)
        H = hp(lr=1e-3, beta1=0.9, beta2=0.99, scale=1 / N, step=t)
        gathered = np.full(padded, np.nan, np.float32)
        for r in range(N):
            _, start, end, _ = oracle.shard_range(T, N, r)
            k = end - start
            u = np.empty(k, np.float32)
            m, v = ms[r][:k].copy(), vs[r][:k].copy()
            assert oracle.adam_update(H, m, v, np.ascontiguousarray(flat_grad[start:end]), u) == 0
            ms[r][:k], vs[r][:k] = m, v
            gathered[r * chunk:r * chunk + k] = u
        oracle.flat_apply_update(gathered, params, F32)
        oracle.adamw_step(H, flat_master, M, V, flat_grad)
        back = oracle.flat_unpack(flat_master, F32, numels, F32)
        for a, b in zip(params, back):
            assert np.array_equal(_abits(a), _abits(b)), t
        for r in range(N):
            _, start, end, _ = oracle.shard_range(T, N, r)
            assert np.array_equal(ms[r][:end - start], M[start:end])


# ---------------------------------------------------------------------------
# Tiled optimizer state (a storage layout: the three fp32 values of each
# element grouped per tile of `tile` elements)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,tile", [(0, 4), (1, 4), (3, 4), (4, 4), (5, 4), (17, 8), (64, 16), (8193, 8192),
                                    (3 * 8192 - 1, 8192)])
def test_state_tile_matches_numpy_reshape(orc, n, tile):
    """Against the layout's definition written with numpy: the buffer viewed
    as [tiles, 3, tile] holds master, exp_avg, exp_avg_sq of the tile's
    elements in rows 0, 1, 2; the end of the last tile is zero."""
    rng = np.random.default_rng(n + tile)
    p, m, v = (rng.standard_normal(n).astype(np.float32) for _ in range(3))
    state = oracle.state_tile(p, m, v, n, tile)
    tiles = -(-n // tile)
    assert state.size == oracle.state_tiled_numel(n, tile) == 3 * tile * tiles
    view = state.reshape(tiles, 3, tile)
    for k, src in enumerate((p, m, v)):
        stream = view[:, k, :].reshape(-1)
        assert np.array_equal(stream[:n].view(np.uint32), src.view(np.uint32))
        assert np.all(stream[n:].view(np.uint32) == 0)
    back = oracle.state_untile(state, n, tile)
    for a, b in zip(back, (p, m, v)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_state_tile_element_positions_brute_force(orc):
    """Each element's three values sit where the index arithmetic puts them,
    checked one element at a time on a small buffer with distinct values."""
    n, tile = 23, 4
    p = np.arange(n, dtype=np.float32)
    m = p + 1000
    v = p + 2000
    state = oracle.state_tile(p, m, v, n, tile)
    for e in range(n):
        t, j = divmod(e, tile)
        for k, base in enumerate((0, 1000, 2000)):
            assert state[(3 * t + k) * tile + j] == e + base


def test_state_tile_bits_and_missing_sources(orc):
    """Bit patterns (NaN payloads, -0.0, subnormals, inf) survive the
    round trip; a missing source tiles as zeros and a missing destination
    is left alone."""
    special = np.array([0x80000000, 0x7FC01234, 0xFF800000, 0x00000001, 0x7F7FFFFF, 0x3F800000, 0xFFFFFFFF],
                       dtype=np.uint32).view(np.float32)
    n, tile = special.size, 4
    state = oracle.state_tile(special, None, special[::-1].copy(), n, tile)
    p, m, v = oracle.state_untile(state, n, tile)
    assert np.array_equal(p.view(np.uint32), special.view(np.uint32))
    assert np.all(m.view(np.uint32) == 0)
    assert np.array_equal(v.view(np.uint32), special[::-1].view(np.uint32))
    assert oracle.state_tiled_numel(-1, 4) == -1 and oracle.state_tiled_numel(4, 0) == -1


def test_state_tile_then_step_equals_step(orc):
    """The layout changes no result: stepping the untiled arrays equals
    stepping the arrays read back out of a tiled buffer (the update is
    element-wise, so a permutation of storage commutes with it)."""
    rng = np.random.default_rng(9)
    n, tile = 1000, 64
    p = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    H = hp(lr=3e-4, beta1=0.9, beta2=0.95, wd=0.1, step=1)
    p2, m2, v2 = oracle.state_untile(oracle.state_tile(p, m, v, n, tile), n, tile)
    oracle.adamw_step(H, p, m, v, g)
    oracle.adamw_step(H, p2, m2, v2, g)
    for a, b in ((p, p2), (m, m2), (v, v2)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("n,tile", [(0, 4), (1, 4), (5, 4), (8, 4), (17, 8), (64, 16), (8193, 8192)])
def test_moments_tile_matches_numpy_reshape(orc, n, tile):
    """The moments-only layout against its numpy definition: the buffer as
    [tiles, 2, tile] holds exp_avg and exp_avg_sq of the tile's elements in
    rows 0 and 1, the end of the last tile zero; untile inverts it."""
    rng = np.random.default_rng(7 * n + tile)
    m, v = (rng.standard_normal(n).astype(np.float32) for _ in range(2))
    buf = oracle.moments_tile(m, v, n, tile)
    tiles = -(-n // tile)
    assert buf.size == oracle.moments_tiled_numel(n, tile) == 2 * tile * tiles
    view = buf.reshape(tiles, 2, tile)
    for k, src in enumerate((m, v)):
        run = view[:, k, :].reshape(-1)
        assert np.array_equal(run[:n].view(np.uint32), src.view(np.uint32))
        assert np.all(run[n:].view(np.uint32) == 0)
    for a, b in zip(oracle.moments_untile(buf, n, tile), (m, v)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert oracle.moments_tiled_numel(-1, 4) == -1


def test_moments_tile_then_update_equals_update(orc):
    """Tiling the moments, running the ZeRO-1 update and the no-master step
    on the arrays read back, equals running them on the split arrays."""
    rng = np.random.default_rng(11)
    n, tile = 777, 32
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = rng.uniform(0, 1e-7, n).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    H = hp(lr=3e-4, beta1=0.9, beta2=0.95, step=2)
    m2, v2 = oracle.moments_untile(oracle.moments_tile(m, v, n, tile), n, tile)
    u1, u2 = np.empty(n, np.float32), np.empty(n, np.float32)
    oracle.adam_update(H, m, v, g, u1)
    oracle.adam_update(H, m2, v2, g, u2)
    for a, b in ((m, m2), (v, v2), (u1, u2)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
