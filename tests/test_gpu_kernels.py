"""GPU parity of each library entry point against the oracle (small sizes).

Sizes span several workgroup tiles and ragged tails; every case runs
aligned (128-bit path) and as a misaligned view (scalar path).  Inputs are
seeded and drawn on the CPU, then copied to the GPU, so both sides consume
the same bits.  Every buffer carries a canary tail that must stay untouched.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import fsdp_sharded_optimizer_amd as zs
from tests.parity import (NORM_TOL, StateCheck, bits_equal, from_np, identical_fraction,
                          to_np)

pytestmark = pytest.mark.gpu

SIZES = [1, 7, 8, 9, 255, 2047, 2048, 2049, 8191, 100_003]
CANARY = 64


def dev_buf(a: np.ndarray, offset: int, bf16: bool = False):
    """Device copy of `a` placed `offset` elements into a larger buffer with
    a canary tail; returns (view, whole buffer)."""
    n = a.size
    fill = np.full(offset + n + CANARY, 0x7FBF if bf16 else 0, dtype=a.dtype)
    if not bf16:
        fill = fill.view(np.uint32)
        fill[:] = 0x7FBADBAD
        fill = fill.view(np.float32)
    fill[offset:offset + n] = a
    whole = from_np(fill, bf16=bf16)
    return whole[offset:offset + n], whole


def canary_ok(whole: torch.Tensor, offset: int, n: int) -> bool:
    w = to_np(whole)
    if w.dtype == np.uint16:
        return bool(np.all(w[offset + n:] == 0x7FBF) and np.all(w[:offset] == 0x7FBF))
    return bool(np.all(w.view(np.uint32)[offset + n:] == 0x7FBADBAD) and
                np.all(w.view(np.uint32)[:offset] == 0x7FBADBAD))


# ---------------------------------------------------------------------------
# grad_accum: bit-exact
# ---------------------------------------------------------------------------

# (acc offset, grad offset) in elements: both aligned; both misaligned (the
# scalar path); the read-only gradient alone off a 16-byte boundary (the
# vector path with dword-aligned gradient loads, except a bf16 gradient at an
# odd element, which is only 2-byte aligned)
OFFSETS = [(0, 0), (3, 4), (0, 1), (0, 2)]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("acc_off,grad_off", OFFSETS)
def test_grad_accum_bit_exact(n, dtype, acc_off, grad_off):
    print(f"grad_accum n={n} dtype={dtype} offsets={acc_off},{grad_off}", flush=True)
    rng = np.random.default_rng(n * 31 + acc_off * 7 + grad_off)
    M = 4
    mbs32 = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(M)]
    mbs = [oracle.bf16_rne(x) for x in mbs32] if dtype == "bf16" else mbs32
    code = oracle.BF16 if dtype == "bf16" else oracle.F32
    ref = np.empty(n, np.float32)
    acc, acc_whole = dev_buf(np.zeros(n, np.float32), acc_off)
    for k, g in enumerate(mbs):
        oracle.grad_accum(ref, g, code, overwrite=(k == 0))
        gd, g_whole = dev_buf(g, grad_off, bf16=(dtype == "bf16"))
        zs.grad_accum(acc, gd, overwrite=(k == 0))
        torch.cuda.synchronize()
        assert canary_ok(g_whole, grad_off, n)
        assert bits_equal(to_np(acc), ref), (k, identical_fraction(to_np(acc), ref))
    assert canary_ok(acc_whole, acc_off, n)


# ---------------------------------------------------------------------------
# grad_norm_sq
# ---------------------------------------------------------------------------

# the norm's 4096-element tiles and its partials' reduction: one workgroup up
# to 2048 partials (8,388,608 elements), chunks then one workgroup beyond
NORM_SIZES = SIZES + [4095, 4096, 4097, 3_000_001, 8_388_608, 8_388_609, 8_392_705]


@pytest.mark.parametrize("n", NORM_SIZES)
@pytest.mark.parametrize("offset", [0, 1])
def test_grad_norm_sq(n, offset):
    print(f"grad_norm_sq n={n} offset={offset}", flush=True)
    rng = np.random.default_rng(n + 17 * offset)
    acc = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    scale = 1.0 / 32
    want = oracle.grad_norm_sq(acc, scale)
    g, whole = dev_buf(acc, offset)
    out = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    zs.grad_norm_sq(g, scale, out)
    got = float(out.item())
    assert abs(math.sqrt(got) - math.sqrt(want)) <= NORM_TOL * math.sqrt(want)
    # a fixed association: the same bits run to run, and from the other alignment path
    out2 = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    zs.grad_norm_sq(g, scale, out2)
    g2, _ = dev_buf(acc, 0 if offset else 1)
    out3 = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    zs.grad_norm_sq(g2, scale, out3)
    assert out2.item() == got and out3.item() == got
    assert canary_ok(whole, offset, n)


@pytest.mark.parametrize("n", [1, 7, 4095, 4096, 4097, 100_003, 9_000_011])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("acc_off,grad_off", OFFSETS)
@pytest.mark.parametrize("overwrite", [False, True])
def test_grad_accum_norm_sq(n, dtype, acc_off, grad_off, overwrite):
    """The fused last micro-batch: the accumulator bit-exact, the squared
    norm of the scaled result within the bar and reproducible to the bit."""
    print(f"grad_accum_norm_sq n={n} dtype={dtype} offsets={acc_off},{grad_off} overwrite={overwrite}", flush=True)
    rng = np.random.default_rng(n * 13 + acc_off * 5 + grad_off + overwrite)
    code = oracle.BF16 if dtype == "bf16" else oracle.F32
    acc0 = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    g32 = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    g = oracle.bf16_rne(g32) if dtype == "bf16" else g32
    scale = 1.0 / 16
    ref = acc0.copy()
    oracle.grad_accum(ref, g, code, overwrite=overwrite)
    want = oracle.grad_norm_sq(ref, scale)
    outs = []
    for _ in range(2):
        acc, acc_whole = dev_buf(acc0, acc_off)
        gd, g_whole = dev_buf(g, grad_off, bf16=(dtype == "bf16"))
        out = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
        zs.grad_accum_norm_sq(acc, gd, overwrite, scale, out)
        assert bits_equal(to_np(acc), ref)
        assert canary_ok(acc_whole, acc_off, n) and canary_ok(g_whole, grad_off, n)
        outs.append(out.item())
    assert outs[0] == outs[1]
    assert abs(math.sqrt(outs[0]) - math.sqrt(want)) <= NORM_TOL * math.sqrt(want)


def test_grad_accum_norm_sq_empty_and_closed_form():
    out = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    e = torch.empty(0, dtype=torch.float32, device="cuda")
    zs.grad_accum_norm_sq(e, e.to(torch.bfloat16), True, 1.0, out)
    assert out.item() == 0.0
    # first micro-batch of 2^23 + 3 elements of 2^-7 at scale 1/8: exactly (2^23 + 3) * 2^-20
    n = (1 << 23) + 3
    acc = torch.empty(n, dtype=torch.float32, device="cuda")
    g = torch.full((n,), 2.0**-7, dtype=torch.bfloat16, device="cuda")
    zs.grad_accum_norm_sq(acc, g, True, 1.0 / 8, out)
    assert out.item() == n * 2.0**-20
    assert torch.all(acc == 2.0**-7)


def test_grad_norm_sq_empty_and_closed_form():
    out = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    zs.grad_norm_sq(torch.empty(0, dtype=torch.float32, device="cuda"), 1.0, out)
    assert out.item() == 0.0
    # 2^20 + 3 elements of 2^-7 at scale 1/8: exactly 1 + 3 * 2^-20
    g = torch.full(((1 << 20) + 3,), 2.0**-7, dtype=torch.float32, device="cuda")
    zs.grad_norm_sq(g, 1.0 / 8, out)
    assert out.item() == 1.0 + 3 * 2.0**-20


# ---------------------------------------------------------------------------
# adamw_step
# ---------------------------------------------------------------------------

def _hp(step, lr=3e-4, b1=0.9, b2=0.95, eps=1e-8, wd=0.1, scale=1 / 64, max_norm=0.0, extra=0.0):
    return (zs.AdamWConfig(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd, grad_scale=scale,
                           max_norm=max_norm, extra_norm_sq=extra, step=step),
            oracle.make_hp(lr, b1, b2, eps, wd, scale, max_norm, extra, step))


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("offset", [0, 3])
@pytest.mark.parametrize("mode", ["adam_f32", "adamw_bf16", "adamw_bf16_clip"])
def test_adamw_step_parity(n, offset, mode):
    """Three consecutive steps; each compared with the oracle to the bar,
    the GPU using its own norm and the oracle its own."""
    print(f"adamw n={n} offset={offset} mode={mode}", flush=True)
    rng = np.random.default_rng(n * 7 + offset + len(mode))
    p0 = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    wd = 0.0 if mode == "adam_f32" else 0.1
    bf16 = mode != "adam_f32"
    clip = mode.endswith("clip")
    p_ref, m_ref, v_ref = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    b_ref = np.zeros(n, np.uint16)
    p, pw = dev_buf(p0, offset)
    m, mw = dev_buf(np.zeros(n, np.float32), 0)
    v, vw = dev_buf(np.zeros(n, np.float32), 0)
    b, bw = dev_buf(np.zeros(n, np.uint16), offset, bf16=True) if bf16 else (None, None)
    norm = torch.zeros(1, dtype=torch.float64, device="cuda")
    for t in range(1, 4):
        acc = (rng.standard_normal(n) * 3e-3).astype(np.float32)
        g, gw = dev_buf(acc, offset)
        S_ref = oracle.grad_norm_sq(acc, 1 / 64)
        max_norm = 0.5 * math.sqrt(S_ref * 8) if clip else 0.0
        extra = 7 * S_ref if clip else 0.0          # the other ranks' share
        hp_gpu, hp_orc = _hp(t, wd=wd, max_norm=max_norm, extra=extra)
        prev = {"p": p_ref.copy(), "m": m_ref.copy()}
        oracle.adamw_step(hp_orc, p_ref, m_ref, v_ref, acc, b_ref if bf16 else None,
                          norm_sq=S_ref if clip else None)
        if clip:
            zs.grad_norm_sq(g, 1 / 64, norm)
        zs.adamw_step(hp_gpu, p, m, v, g, b, norm_sq=norm if clip else None)
        torch.cuda.synchronize()
        s = oracle.adamw_scalars(hp_orc)
        coef = oracle.clip_coef(S_ref, extra, max_norm) if clip else 1.0
        g2 = (acc * np.float32(1 / 64)) * np.float32(coef)
        gpu = {"p": to_np(p), "m": to_np(m), "v": to_np(v), "b": to_np(b) if bf16 else None}
        res = StateCheck(0.9, 3e-4, wd, s.step_size).check(
            gpu, {"p": p_ref, "m": m_ref, "v": v_ref, "b": b_ref}, prev, g2, f"t={t}")
        print(f"  t={t} {res}", flush=True)
        assert canary_ok(gw, offset, n)
    for whole, off in ((pw, offset), (mw, 0), (vw, 0)) + (((bw, offset),) if bf16 else ()):
        assert canary_ok(whole, off, n)


@pytest.mark.parametrize("n", [2049, 100_003])
@pytest.mark.parametrize("offset,grad_off", [(0, 0), (1, 1), (0, 1), (0, 3)])
def test_adamw_bit_exact_given_the_oracle_norm(n, offset, grad_off):
    """With the oracle's squared norm handed to the kernel, every output is
    bit-identical to the oracle: the element update is the same sequence of
    IEEE binary32 operations and the clip coefficient the same binary64 ones."""
    print(f"adamw bit-exact n={n} offset={offset} grad_off={grad_off}", flush=True)
    rng = np.random.default_rng(n + offset + 10 * grad_off)
    p_ref = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    m_ref, v_ref, b_ref = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
    p, _ = dev_buf(p_ref, offset)
    m, _ = dev_buf(m_ref, offset)
    v, _ = dev_buf(v_ref, offset)
    b, _ = dev_buf(b_ref, offset, bf16=True)
    for t in range(1, 6):
        acc = (rng.standard_normal(n) * 1e-2).astype(np.float32)
        S = oracle.grad_norm_sq(acc, 1 / 32)
        hp_gpu, hp_orc = _hp(t, scale=1 / 32, max_norm=math.sqrt(S) * 0.8 if t % 2 else 0.0,
                             extra=0.25 * S)
        oracle.adamw_step(hp_orc, p_ref, m_ref, v_ref, acc, b_ref, norm_sq=S)
        g, gw = dev_buf(acc, grad_off)
        norm = torch.tensor([S], dtype=torch.float64, device="cuda")
        zs.adamw_step(hp_gpu, p, m, v, g, b, norm_sq=norm)
        for name, gpu, ref in (("p", p, p_ref), ("m", m, m_ref), ("v", v, v_ref), ("b", b, b_ref)):
            assert bits_equal(to_np(gpu), ref), (t, name, identical_fraction(to_np(gpu), ref))
        assert canary_ok(gw, grad_off, n)


@pytest.mark.parametrize("n", [7, 2049, 100_003])
@pytest.mark.parametrize("b_off", [1, 2, 3])
@pytest.mark.parametrize("grad_off", [0, 1])
def test_adamw_bf16_output_at_any_offset(n, b_off, grad_off):
    """Master and moments 16-byte aligned, the bf16 output a view at element
    offset 1, 2 or 3 (the 128-bit path with element-wise bf16 stores): five
    clipped steps bit-identical to the oracle given its norm, the bf16
    buffer's canaries on both sides untouched."""
    print(f"adamw bf16 output offset n={n} b_off={b_off} grad_off={grad_off}", flush=True)
    rng = np.random.default_rng(n + 7 * b_off + grad_off)
    p_ref = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    m_ref, v_ref, b_ref = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
    p, _ = dev_buf(p_ref, 0)
    m, _ = dev_buf(m_ref, 0)
    v, _ = dev_buf(v_ref, 0)
    b, bw = dev_buf(b_ref, b_off, bf16=True)
    for t in range(1, 6):
        acc = (rng.standard_normal(n) * 1e-2).astype(np.float32)
        S = oracle.grad_norm_sq(acc, 1 / 32)
        hp_gpu, hp_orc = _hp(t, scale=1 / 32, max_norm=math.sqrt(S) * 0.8 if t % 2 else 0.0, extra=0.25 * S)
        oracle.adamw_step(hp_orc, p_ref, m_ref, v_ref, acc, b_ref, norm_sq=S)
        g, _ = dev_buf(acc, grad_off)
        zs.adamw_step(hp_gpu, p, m, v, g, b, norm_sq=torch.tensor([S], dtype=torch.float64, device="cuda"))
        for name, gpu, ref in (("p", p, p_ref), ("m", m, m_ref), ("v", v, v_ref), ("b", b, b_ref)):
            assert bits_equal(to_np(gpu), ref), (t, name, identical_fraction(to_np(gpu), ref))
        assert canary_ok(bw, b_off, n)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 7, 31, 32, 33, 2049, 100_003])
@pytest.mark.parametrize("off", [1, 2, 3, 4, 8, 31])
def test_shared_offset_views_peel_their_head(n, off):
    """Master and moments (adamw_step), or the moments (adam_update), as
    views sharing one element offset off a 128-byte boundary, with the bf16
    output, the update and the gradient at other offsets: the call runs its
    first 1-31 elements element by element and the rest on the vector path.
    Three clipped steps bit-identical to the oracle given its norm, every
    canary untouched (also when n is shorter than the head)."""
    print(f"shared offset n={n} off={off}", flush=True)
    rng = np.random.default_rng(100 * n + off)
    p_ref = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    m_ref, v_ref, b_ref = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
    m2_ref, v2_ref, u_ref = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)
    p, pw = dev_buf(p_ref, off)
    m, mw = dev_buf(m_ref, off)
    v, vw = dev_buf(v_ref, off)
    b, bw = dev_buf(b_ref, (off + 1) % 4, bf16=True)
    m2, m2w = dev_buf(m2_ref, off)
    v2, v2w = dev_buf(v2_ref, off)
    u, uw = dev_buf(u_ref, (off + 3) % 4)
    for t in range(1, 4):
        acc = (rng.standard_normal(n) * 1e-2).astype(np.float32)
        S = oracle.grad_norm_sq(acc, 1 / 16)
        norm = torch.tensor([S], dtype=torch.float64, device="cuda")
        g, gw = dev_buf(acc, (off + 2) % 4)
        hp_gpu, hp_orc = _hp(t, scale=1 / 16, max_norm=0.6 * math.sqrt(S), extra=0.1 * S)
        hu_gpu, hu_orc = _hp(t, wd=0.0, scale=1 / 16, max_norm=0.6 * math.sqrt(S), extra=0.1 * S)
        oracle.adamw_step(hp_orc, p_ref, m_ref, v_ref, acc, b_ref, norm_sq=S)
        oracle.adam_update(hu_orc, m2_ref, v2_ref, acc, u_ref, norm_sq=S)
        zs.adamw_step(hp_gpu, p, m, v, g, b, norm_sq=norm)
        zs.adam_update(hu_gpu, m2, v2, g, u, norm_sq=norm)
        for name, gpu, ref in (("p", p, p_ref), ("m", m, m_ref), ("v", v, v_ref), ("b", b, b_ref),
                               ("m2", m2, m2_ref), ("v2", v2, v2_ref), ("update", u, u_ref)):
            assert bits_equal(to_np(gpu), ref), (t, name, identical_fraction(to_np(gpu), ref))
        assert canary_ok(gw, (off + 2) % 4, n)
    for whole, o in ((pw, off), (mw, off), (vw, off), (bw, (off + 1) % 4), (m2w, off), (v2w, off),
                     (uw, (off + 3) % 4)):
        assert canary_ok(whole, o, n)


def test_adamw_skips_on_nonfinite_norm():
    n = 4099
    rng = np.random.default_rng(5)
    p0 = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    acc = rng.standard_normal(n).astype(np.float32)
    acc[1234] = np.inf
    p, m, v = from_np(p0), torch.ones(n, device="cuda"), torch.ones(n, device="cuda")
    b = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    g = from_np(acc)
    norm = torch.zeros(1, dtype=torch.float64, device="cuda")
    zs.grad_norm_sq(g, 1.0, norm)
    assert math.isinf(norm.item())
    hp_gpu, hp_orc = _hp(1, max_norm=1.0)
    zs.adamw_step(hp_gpu, p, m, v, g, b, norm_sq=norm)
    assert bits_equal(to_np(p), p0) and torch.all(m == 1) and torch.all(v == 1)
    assert not torch.any(b.view(torch.int16) != 0)
    # a finite local norm with a non-finite share from the other ranks
    good = from_np(np.ones(n, np.float32))
    zs.grad_norm_sq(good, 1.0, norm)
    hp_gpu, _ = _hp(1, max_norm=1.0, extra=float("inf"))
    zs.adamw_step(hp_gpu, p, m, v, good, b, norm_sq=norm)
    assert bits_equal(to_np(p), p0)
    # the oracle agrees
    pr, mr, vr = p0.copy(), np.ones(n, np.float32), np.ones(n, np.float32)
    assert oracle.adamw_step(hp_orc, pr, mr, vr, acc, norm_sq=float("inf")) == 1


def test_adamw_resume_is_bit_identical():
    """k steps straight vs j steps, a copy of the state through the host, and
    k - j more: the state is plain buffers plus the caller's step count."""
    n, k, j = 50_001, 6, 2
    rng = np.random.default_rng(9)
    p0 = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    grads = [from_np((rng.standard_normal(n) * 1e-3).astype(np.float32)) for _ in range(k)]

    def run(state, steps):
        p, m, v, b = state
        for t in steps:
            zs.adamw_step(_hp(t)[0], p, m, v, grads[t - 1], b)
        return state

    fresh = lambda: [from_np(p0), torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda"),
                     torch.zeros(n, dtype=torch.bfloat16, device="cuda")]
    a = run(fresh(), range(1, k + 1))
    half = run(fresh(), range(1, j + 1))
    host = [to_np(x) for x in half]
    reloaded = [from_np(host[0]), from_np(host[1]), from_np(host[2]), from_np(host[3], bf16=True)]
    b = run(reloaded, range(j + 1, k + 1))
    for x, y in zip(a, b):
        assert bits_equal(to_np(x), to_np(y))


# ---------------------------------------------------------------------------
# flat_pack / flat_unpack: bit-exact
# ---------------------------------------------------------------------------

def _shapes(rng, count, big=False):
    out = []
    for _ in range(count):
        nd = int(rng.integers(1, 3))
        hi = 300 if big else 40
        out.append(tuple(int(d) for d in rng.integers(1, hi, size=nd)))
    return out


@pytest.mark.parametrize("kind", ["f32", "bf16", "bf16_to_f32"])
@pytest.mark.parametrize("count,world,aligned_sizes", [(1, 8, True), (9, 64, True), (5, 3, False),
                                                       (40, 7, False), (70, 8, True)])
def test_flat_pack_unpack(kind, count, world, aligned_sizes):
    print(f"flat kind={kind} count={count} world={world}", flush=True)
    rng = np.random.default_rng(count * 101 + world)
    shapes = _shapes(rng, count, big=aligned_sizes)
    if aligned_sizes:   # numels multiple of 8: the 128-bit path
        shapes = [tuple(list(s[:-1]) + [s[-1] * 8]) for s in shapes]
    src_bf16 = kind != "f32"
    flat_bf16 = kind == "bf16"
    srcs_np = []
    for s in shapes:
        x = rng.uniform(-1, 1, s).astype(np.float32)
        srcs_np.append(oracle.bf16_rne(x).reshape(s) if src_bf16 else x)
    T = sum(x.size for x in srcs_np)
    _, _, _, padded = oracle.shard_range(T, world, 0)
    scode = oracle.BF16 if src_bf16 else oracle.F32
    fcode = oracle.BF16 if flat_bf16 else oracle.F32
    want = oracle.flat_pack(srcs_np, scode, fcode, padded)
    srcs = [from_np(x, bf16=src_bf16) for x in srcs_np]
    flat, flat_whole = dev_buf(np.zeros(padded, np.uint16 if flat_bf16 else np.float32), 0, bf16=flat_bf16)
    # poison the flat buffer so the zero padding must be written
    flat.fill_(float("nan"))
    zs.flat_pack(srcs, flat, padded)
    assert bits_equal(to_np(flat), want)
    assert canary_ok(flat_whole, 0, padded)
    # unflatten into fresh tensors of the flat dtype (or re-cast to bf16)
    dst_bf16 = flat_bf16 or kind == "bf16_to_f32"
    dsts = [torch.empty(s, dtype=torch.bfloat16 if dst_bf16 else torch.float32, device="cuda")
            for s in shapes]
    zs.flat_unpack(flat, dsts)
    back = oracle.flat_unpack(want, fcode, [x.size for x in srcs_np],
                              oracle.BF16 if dst_bf16 else oracle.F32)
    for d, r in zip(dsts, back):
        assert bits_equal(to_np(d).reshape(-1), r)


def test_flat_pack_misaligned_views():
    """Sources that are views at odd element offsets (2-byte aligned bf16)
    take the scalar path."""
    rng = np.random.default_rng(77)
    base = from_np(oracle.bf16_rne(rng.uniform(-1, 1, 10_000).astype(np.float32)), bf16=True)
    views = [base[1:2050], base[3000:3001], base[4001:9000]]
    T = sum(v.numel() for v in views)
    flat = torch.empty(T + 5, dtype=torch.float32, device="cuda")
    zs.flat_pack(views, flat, T + 5)
    want = oracle.flat_pack([to_np(v) for v in views], oracle.BF16, oracle.F32, T + 5)
    assert bits_equal(to_np(flat), want)


# ---------------------------------------------------------------------------
# grad_reduce_chunks (reduce-scatter arithmetic) and the all-gather placement
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N", [1, 2, 7, 16, 17, 64])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("overwrite", [True, False])
@pytest.mark.parametrize("acc_off,grad_off", [(0, 0), (1, 1), (0, 1), (0, 2)])
def test_grad_reduce_chunks_bit_exact(N, dtype, overwrite, acc_off, grad_off):
    """N rank chunks summed in rank order equal N sequential accumulations
    (the oracle's), bit for bit, with one chunk aliased twice."""
    n = 4097 if N > 16 else 100_003
    print(f"grad_reduce_chunks N={N} dtype={dtype} overwrite={overwrite} offsets={acc_off},{grad_off} n={n}",
          flush=True)
    rng = np.random.default_rng(N * 7 + acc_off * 11 + grad_off + 3 * overwrite)
    code = oracle.BF16 if dtype == "bf16" else oracle.F32
    chunks = []
    for _ in range(N):
        x = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        chunks.append(oracle.bf16_rne(x) if dtype == "bf16" else x)
    if N > 2:
        chunks[2] = chunks[0]                       # aliasing is allowed
    acc0 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    ref = acc0.copy()
    for k, c in enumerate(chunks):
        oracle.grad_accum(ref, c, code, overwrite=(overwrite and k == 0))
    acc, acc_whole = dev_buf(acc0, acc_off)
    dev_chunks = [dev_buf(c, grad_off + (k % 2) * 2, bf16=(dtype == "bf16"))[0] for k, c in enumerate(chunks)]
    if N > 2:
        dev_chunks[2] = dev_chunks[0]
    zs.grad_reduce_chunks(acc, dev_chunks, overwrite)
    assert bits_equal(to_np(acc), ref)
    assert canary_ok(acc_whole, acc_off, n)


def test_allgather_placement_roundtrip():
    """The all-gather's placement: the N ranks' bf16 chunks packed in rank
    order rebuild the FlatParameter bit for bit, and unflatten to the unit's
    tensors (a 70B-style block scaled down, world 64)."""
    import workloads
    shapes = workloads.block70b_tensor_shapes(hidden=512, ffn=1792, q_heads=64, kv_heads=8, head_dim=8)
    rng = np.random.default_rng(21)
    params = [oracle.bf16_rne(rng.uniform(-0.1, 0.1, s).astype(np.float32)).reshape(s) for _, s in shapes]
    total = sum(p.size for p in params)
    world = 64
    chunk, _, _, padded = zs.zero_shard_range(total, world, 0)
    flat_ref = oracle.flat_pack(params, oracle.BF16, oracle.BF16, padded)
    # each rank's chunk, as it would arrive from that rank
    chunks = [from_np(flat_ref[r * chunk:(r + 1) * chunk].copy(), bf16=True) for r in range(world)]
    flat = torch.empty(padded, dtype=torch.bfloat16, device="cuda")
    zs.flat_pack(chunks, flat, padded)
    assert bits_equal(to_np(flat), flat_ref)
    outs = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for _, s in shapes]
    zs.flat_unpack(flat, outs)
    for o, p in zip(outs, params):
        assert bits_equal(to_np(o).reshape(-1), p.reshape(-1))



# ---------------------------------------------------------------------------
# adamw_step_no_master (the ZeRO-3 listing's direct low-precision update)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 7, 4097, 100_003])
@pytest.mark.parametrize("offset,grad_off", [(0, 0), (1, 1), (0, 1)])
@pytest.mark.parametrize("clip", [False, True])
def test_adamw_no_master_bit_exact(n, offset, grad_off, clip):
    print(f"no-master n={n} offset={offset} grad_off={grad_off} clip={clip}", flush=True)
    rng = np.random.default_rng(n + offset + 3 * grad_off + clip)
    b_ref = oracle.bf16_rne(rng.uniform(-0.1, 0.1, n).astype(np.float32))
    m_ref, v_ref = np.zeros(n, np.float32), np.zeros(n, np.float32)
    b, _ = dev_buf(b_ref, offset, bf16=True)
    m, _ = dev_buf(m_ref, offset)
    v, _ = dev_buf(v_ref, offset)
    for t in range(1, 4):
        acc = (rng.standard_normal(n) * 1e-2).astype(np.float32)
        S = oracle.grad_norm_sq(acc, 1 / 32)
        hp_gpu, hp_orc = _hp(t, scale=1 / 32, max_norm=math.sqrt(S) * 0.7 if clip else 0.0, extra=0.1 * S)
        oracle.adamw_step_no_master(hp_orc, b_ref, m_ref, v_ref, acc, norm_sq=S if clip else None)
        g, _ = dev_buf(acc, grad_off)
        norm = torch.tensor([S], dtype=torch.float64, device="cuda") if clip else None
        zs.adamw_step_no_master(hp_gpu, b, m, v, g, norm_sq=norm)
        for name, gpu, ref in (("b", b, b_ref), ("m", m, m_ref), ("v", v, v_ref)):
            assert bits_equal(to_np(gpu), ref), (t, name, identical_fraction(to_np(gpu), ref))


def test_no_master_stalls_on_the_gpu():
    """The reading that keeps an fp32 master: with the 7B workload's
    hyperparameters (lr 3e-4, wd 0.1) and U(-0.1, 0.1) parameters, the
    direct bf16 update loses most small steps.  After 20 steps the share of
    elements whose bf16 parameter differs between the two forms is large,
    and the master form moves more elements per step."""
    n = 1 << 20
    rng = np.random.default_rng(5)
    b0 = oracle.bf16_rne(rng.uniform(-0.1, 0.1, n).astype(np.float32))
    master = from_np(oracle.bf16_widen(b0).copy())
    b_master = from_np(b0.copy(), bf16=True)
    b_direct = from_np(b0.copy(), bf16=True)
    m1, v1 = torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    m2, v2 = torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    moved_master = moved_direct = 0
    for t in range(1, 21):
        g = torch.from_numpy((rng.standard_normal(n) * 1e-3).astype(np.float32)).cuda()
        hp = zs.AdamWConfig(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_scale=1.0, step=t)
        before_m, before_d = b_master.clone(), b_direct.clone()
        zs.adamw_step(hp, master, m1, v1, g, b_master)
        zs.adamw_step_no_master(hp, b_direct, m2, v2, g)
        moved_master += int((b_master.view(torch.int16) != before_m.view(torch.int16)).sum())
        moved_direct += int((b_direct.view(torch.int16) != before_d.view(torch.int16)).sum())
    differ = float((b_master.view(torch.int16) != b_direct.view(torch.int16)).float().mean())
    print(f"moved per step: master {moved_master / 20 / n:.3f}, direct {moved_direct / 20 / n:.3f}; "
          f"differ after 20 steps: {differ:.3f}", flush=True)
    assert differ > 0.3
    assert moved_master > moved_direct


# ---------------------------------------------------------------------------
# adam_update and flat_apply_update (the ZeRO page's ZeRO-1 flow)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 7, 4097, 100_003])
@pytest.mark.parametrize("offset,upd_off", [(0, 0), (1, 1), (3, 3), (1, 0), (3, 0), (0, 1), (0, 2), (0, 3)])
@pytest.mark.parametrize("clip", [False, True])
def test_adam_update_bit_exact(n, offset, upd_off, clip):
    """The gradient (and the update) as views at any element offset, as a
    rank's slice of one resident flat buffer is; the moments are the rank's
    own allocations.  Given the oracle's squared norm every output is
    bit-identical, and nothing past the views is written."""
    print(f"adam_update n={n} grad offset={offset} update offset={upd_off} clip={clip}", flush=True)
    rng = np.random.default_rng(3 * n + offset + 5 * upd_off + 7 * clip)
    m_ref, v_ref, u_ref = np.zeros(n, np.float32), np.zeros(n, np.float32), np.empty(n, np.float32)
    m, mw = dev_buf(m_ref, 0)
    v, vw = dev_buf(v_ref, 0)
    u, uw = dev_buf(np.zeros(n, np.float32), upd_off)
    for t in range(1, 5):
        acc = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        S = oracle.grad_norm_sq(acc, 1 / 8)
        hp_gpu, hp_orc = _hp(t, lr=1e-4, b2=0.999, wd=0.0, scale=1 / 8,
                             max_norm=0.7 * math.sqrt(S * 8) if clip else 0.0, extra=7 * S)
        assert oracle.adam_update(hp_orc, m_ref, v_ref, acc, u_ref, norm_sq=S if clip else None) == 0
        g, gw = dev_buf(acc, offset)
        norm = torch.tensor([S], dtype=torch.float64, device="cuda") if clip else None
        zs.adam_update(hp_gpu, m, v, g, u, norm_sq=norm)
        torch.cuda.synchronize()
        for name, gpu, ref in (("update", u, u_ref), ("m", m, m_ref), ("v", v, v_ref)):
            assert bits_equal(to_np(gpu), ref), (t, name, identical_fraction(to_np(gpu), ref))
        assert canary_ok(gw, offset, n)
    for whole, off in ((uw, upd_off), (mw, 0), (vw, 0)):
        assert canary_ok(whole, off, n)


def test_adam_update_skips_on_nonfinite_norm():
    n = 4099
    g = from_np(np.ones(n, np.float32))
    m, v = torch.ones(n, device="cuda"), torch.ones(n, device="cuda")
    u = torch.full((n,), 7.0, device="cuda")
    norm = torch.tensor([float("nan")], dtype=torch.float64, device="cuda")
    zs.adam_update(_hp(1, wd=0.0, max_norm=1.0)[0], m, v, g, u, norm_sq=norm)
    torch.cuda.synchronize()
    assert torch.all(m == 1) and torch.all(v == 1)
    assert np.all(to_np(u).view(np.uint32) == 0x80000000)   # -0.0: the apply adds nothing
    with pytest.raises(zs.ZShardError):
        zs.adam_update(_hp(1, wd=0.1)[0], m, v, g, u)


@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("n,upd_off", [(1, 0), (4099, 0), (4099, 1), (70_001, 3)])
@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_skipped_zero1_step_leaves_parameters_unchanged(tiled, n, upd_off, bad):
    """A non-finite global norm in the ZeRO-1 flow: adam_update
    (adam_update_tiled) over a buffer holding a stale update, then
    flat_apply_update of that buffer into fp32 and bf16 parameters (with
    +-0.0, subnormals and +-inf among them).  Every parameter and moment is
    bit-identical afterwards and the update is -0.0, as in the oracle."""
    print(f"skipped zero-1 step tiled={tiled} n={n} update offset={upd_off} norm={bad}", flush=True)
    rng = np.random.default_rng(n + upd_off)
    g = from_np(rng.standard_normal(n).astype(np.float32))
    m0 = rng.standard_normal(n).astype(np.float32)
    v0 = np.abs(rng.standard_normal(n)).astype(np.float32)
    uw = torch.full((n + upd_off,), 5.0, device="cuda")   # stale values from an earlier step
    u = uw[upd_off:]
    norm = torch.tensor([bad], dtype=torch.float64, device="cuda")
    hp_gpu = _hp(3, wd=0.0, max_norm=1.0)[0]
    if tiled:
        mo = torch.empty(zs.moments_tiled_numel(n), device="cuda")
        zs.moments_tile(from_np(m0), from_np(v0), mo)
        zs.adam_update_tiled(hp_gpu, mo, g, u, norm_sq=norm)
        m, v = torch.empty(n, device="cuda"), torch.empty(n, device="cuda")
        zs.moments_untile(mo, m, v)
    else:
        m, v = from_np(m0), from_np(v0)
        zs.adam_update(hp_gpu, m, v, g, u, norm_sq=norm)
    u_ref = np.full(n, 5.0, np.float32)
    hp_orc = oracle.make_hp(hp_gpu.lr, hp_gpu.beta1, hp_gpu.beta2, hp_gpu.eps, 0.0, hp_gpu.grad_scale, 1.0,
                            0.0, 3)
    assert oracle.adam_update(hp_orc, m0.copy(), v0.copy(), to_np(g), u_ref, norm_sq=bad) == 1
    assert bits_equal(to_np(u), u_ref)
    assert bits_equal(to_np(m), m0) and bits_equal(to_np(v), v0)
    specials = np.array([0.0, -0.0, 1e-45, -1e-45, np.inf, -np.inf, 1.0, -2.5], np.float32)
    p32 = np.resize(specials, n) * np.float32(1.0)
    p32[len(specials):] = rng.uniform(-1, 1, max(n - len(specials), 0)).astype(np.float32)
    pb = oracle.bf16_rne(p32)
    dev32, devb = from_np(p32), from_np(pb, bf16=True)
    zs.flat_apply_update(u, [dev32])
    zs.flat_apply_update(u, [devb])
    assert bits_equal(to_np(dev32), p32)
    assert bits_equal(to_np(devb), pb)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("count,aligned_sizes,upd_offset", [(1, True, 0), (12, False, 0), (40, False, 0),
                                                            (70, True, 0), (9, True, 1)])
def test_flat_apply_update_bit_exact(dtype, count, aligned_sizes, upd_offset):
    """Every tensor adds its part of the gathered update; the update's
    padding is NaN and must never be read; batches of more than 32 tensors
    and tensors at unaligned offsets of the update are covered."""
    print(f"flat_apply_update dtype={dtype} count={count} upd_offset={upd_offset}", flush=True)
    rng = np.random.default_rng(count * 13 + len(dtype) + upd_offset)
    shapes = _shapes(rng, count, big=aligned_sizes)
    if aligned_sizes:
        shapes = [tuple(list(s[:-1]) + [s[-1] * 8]) for s in shapes]
    numels = [int(np.prod(s)) for s in shapes]
    T = sum(numels)
    upd_ref = np.full(T + 13, np.nan, np.float32)
    upd_ref[:T] = (rng.standard_normal(T) * 1e-2).astype(np.float32)
    bf16 = dtype == "bf16"
    if bf16:
        p_ref = [oracle.bf16_rne(rng.uniform(-1, 1, k).astype(np.float32)) for k in numels]
    else:
        p_ref = [rng.uniform(-1, 1, k).astype(np.float32) for k in numels]
    params = [from_np(x, bf16=bf16).reshape(s) for x, s in zip(p_ref, shapes)]
    upd, upd_whole = dev_buf(upd_ref, upd_offset)
    oracle.flat_apply_update(upd_ref, p_ref, oracle.BF16 if bf16 else oracle.F32)
    zs.flat_apply_update(upd, params)
    torch.cuda.synchronize()
    for d, r in zip(params, p_ref):
        assert bits_equal(to_np(d).reshape(-1), r)
    assert canary_ok(upd_whole, upd_offset, T + 13)


def test_binding_rejects_bad_norm_buffers():
    """The binding refuses a norm buffer that is not one float64, before any launch."""
    n = 1024
    p, m, v, g = (torch.zeros(n, device="cuda") for _ in range(4))
    hp = _hp(1)[0]
    for bad in (torch.zeros(1, device="cuda"), torch.zeros(0, dtype=torch.float64, device="cuda")):
        with pytest.raises(TypeError):
            zs.adamw_step(hp, p, m, v, g, norm_sq=bad)
    with pytest.raises(ValueError):
        zs.adamw_step(hp, p, m, v, g[:-1])



@pytest.mark.parametrize("src_off", [2, 4, 6])
def test_flat_dword_aligned_read_side(src_off):
    """Views 4 bytes past a 16-byte boundary on the read side (bf16 sources
    at even offsets for the pack, a flat view for the unpack) keep the vector
    path with dword-aligned loads; bit-exact, nothing written outside."""
    rng = np.random.default_rng(300 + src_off)
    base_np = oracle.bf16_rne(rng.uniform(-1, 1, 20_000).astype(np.float32))
    base = from_np(base_np, bf16=True)
    spans = [(src_off, src_off + 4096), (src_off + 5000, src_off + 5000 + 2051), (src_off + 8000, src_off + 16000)]
    views = [base[a:b] for a, b in spans]
    T = sum(b - a for a, b in spans)
    for flat_bf16 in (False, True):
        flat, flat_whole = dev_buf(np.zeros(T + 3, np.uint16 if flat_bf16 else np.float32), 0, bf16=flat_bf16)
        zs.flat_pack(views, flat, T + 3)
        code = oracle.BF16 if flat_bf16 else oracle.F32
        want = oracle.flat_pack([base_np[a:b] for a, b in spans], oracle.BF16, code, T + 3)
        assert bits_equal(to_np(flat), want)
        assert canary_ok(flat_whole, 0, T + 3)
    # unpack from a flat view that starts src_off elements into a bf16 buffer
    flat_np = oracle.bf16_rne(rng.uniform(-1, 1, T + 16).astype(np.float32))
    fv, _ = dev_buf(flat_np[src_off:src_off + T], src_off, bf16=True)
    outs = [torch.empty(b - a, dtype=torch.bfloat16, device="cuda") for a, b in spans]
    zs.flat_unpack(fv, outs)
    back = oracle.flat_unpack(np.ascontiguousarray(flat_np[src_off:src_off + T]), oracle.BF16,
                              [b - a for a, b in spans], oracle.BF16)
    for o, r in zip(outs, back):
        assert bits_equal(to_np(o), r)
    # apply: an fp32 update view 4 bytes past a boundary into aligned fp32 tensors
    upd_np = (rng.standard_normal(T + 8) * 1e-2).astype(np.float32)
    uv, _ = dev_buf(upd_np[1:1 + T], 1)
    ps_np = [rng.uniform(-1, 1, b - a).astype(np.float32) for a, b in spans]
    ps = [from_np(x) for x in ps_np]
    zs.flat_apply_update(uv, ps)
    oracle.flat_apply_update(np.ascontiguousarray(upd_np[1:1 + T]), ps_np, oracle.F32)
    for a_, r in zip(ps, ps_np):
        assert bits_equal(to_np(a_), r)


# sizes at and around the conversions' group (256 elements) and tile (512)
# boundaries: a lane's second group ragged, absent, or whole
CONVERSION_SIZES = [1, 3, 4, 5, 252, 255, 256, 257, 259, 260, 261, 508, 511, 512, 513, 516, 517, 767, 768,
                    769, 1023, 1024, 1025, 1029, 100_003]


def _fp32_with_specials(rng, n):
    """Random fp32 values whose low 16 bits are arbitrary, with exact halfway
    cases (both parities), values that round up to infinity, subnormals,
    signed zeros, infinities and NaNs mixed in."""
    x = rng.uniform(-2, 2, n).astype(np.float32)
    u = x.view(np.uint32)
    specials = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x7F7FFFFF, 0x7F7F8000, 0xFF7FFFFF,
                         0x00000001, 0x80008000, 0x00000000, 0x80000000, 0x7F800000, 0xFF800000,
                         0x7FC00001, 0xFFBFFFFF, 0x7F800001], dtype=np.uint32)
    k = min(n, len(specials))
    idx = rng.choice(n, size=k, replace=False)
    u[idx] = specials[:k]
    return u.view(np.float32)


@pytest.mark.parametrize("n", CONVERSION_SIZES)
@pytest.mark.parametrize("offset", [0, 1, 2])
def test_flat_conversions_at_tile_edges(n, offset):
    """The widening pack (bf16 -> fp32) and the re-casting unpack (fp32 ->
    bf16, round to nearest even) over tensors whose sizes sit at the edges of
    the conversion kernels' groups and tiles, at element offsets 0 (aligned),
    1 (scalar path) and 2 (bf16 side 4-byte aligned): bit-exact against the
    oracle, nothing written outside."""
    print(f"flat conversions n={n} offset={offset}", flush=True)
    rng = np.random.default_rng(n * 3 + offset)
    sizes = [n, n + 1, 7]
    T = sum(sizes)
    padded = T + 5
    # pack: bf16 tensors at `offset` into an fp32 flat buffer (poisoned, so
    # the zero padding must be written)
    srcs_np = [oracle.bf16_rne(rng.uniform(-1, 1, k).astype(np.float32)) for k in sizes]
    srcs = [dev_buf(x, offset, bf16=True)[0] for x in srcs_np]
    flat, flat_whole = dev_buf(np.full(padded, np.nan, np.float32), offset)
    zs.flat_pack(srcs, flat, padded)
    assert bits_equal(to_np(flat), oracle.flat_pack(srcs_np, oracle.BF16, oracle.F32, padded))
    assert canary_ok(flat_whole, offset, padded)
    # unpack: an fp32 flat buffer of arbitrary values into bf16 tensors at `offset`
    flat_np = _fp32_with_specials(rng, T)
    fv, _ = dev_buf(flat_np, offset)
    outs, wholes = zip(*[dev_buf(np.zeros(k, np.uint16), offset, bf16=True) for k in sizes])
    zs.flat_unpack(fv, list(outs))
    back = oracle.flat_unpack(flat_np, oracle.F32, sizes, oracle.BF16)
    for o, w_, r, k in zip(outs, wholes, back, sizes):
        assert bits_equal(to_np(o), r)
        assert canary_ok(w_, offset, k)


# ---------------------------------------------------------------------------
# degenerate hyperparameters and special gradient values
# ---------------------------------------------------------------------------

def _special_grads(n, rng):
    """Normal gradients with zeros of both signs, subnormals, values whose
    square overflows or underflows, the extremes of fp32, inf and NaN."""
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    specials = np.array([0.0, -0.0, 1e-45, -1e-45, 1e-40, 3e-39, 1e-20, 1e20, 3e38, -3.4e38,
                         np.inf, -np.inf, np.nan], dtype=np.float32)
    idx = rng.choice(n, size=len(specials) * 20, replace=False)
    g[idx] = np.tile(specials, 20)
    return g


def _same(gpu, ref):
    """Bit-identical, except that any NaN matches any NaN (payloads and signs
    of NaNs made by arithmetic differ between the CPU and the GPU)."""
    if gpu.dtype == np.uint16:
        nan_g = ((gpu & 0x7F80) == 0x7F80) & ((gpu & 0x7F) != 0)
        nan_r = ((ref & 0x7F80) == 0x7F80) & ((ref & 0x7F) != 0)
    else:
        nan_g, nan_r = np.isnan(gpu), np.isnan(ref)
    if not np.array_equal(nan_g, nan_r):
        return False
    return bits_equal(gpu[~nan_g], ref[~nan_r])


@pytest.mark.parametrize("case", ["betas_zero", "lr_zero", "eps_large", "wd_large", "beta_near_one"])
def test_adamw_degenerate_hyperparameters_and_special_values(case):
    """No norm pointer (nothing is skipped): inf and NaN gradients propagate
    element-wise, as in the oracle.  Three steps; every element identical to
    the oracle's, NaNs matched by position."""
    print(f"adamw degenerate case={case}", flush=True)
    hpk = dict(lr=3e-4, b1=0.9, b2=0.95, eps=1e-8, wd=0.1, scale=1 / 8)
    hpk.update({"betas_zero": dict(b1=0.0, b2=0.0), "lr_zero": dict(lr=0.0), "eps_large": dict(eps=1.0),
                "wd_large": dict(wd=1000.0, lr=1e-3), "beta_near_one": dict(b1=0.999999, b2=0.9999999)}[case])
    n = 8199
    rng = np.random.default_rng(len(case))
    p_ref = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    p_ref[:4] = (0.0, -0.0, 1e-40, 3e38)
    m_ref, v_ref, b_ref = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
    p, m, v = from_np(p_ref.copy()), from_np(m_ref.copy()), from_np(v_ref.copy())
    b = from_np(b_ref.copy(), bf16=True)
    for t in range(1, 4):
        acc = _special_grads(n, rng)
        hp_gpu, hp_orc = _hp(t, **hpk)
        assert oracle.adamw_step(hp_orc, p_ref, m_ref, v_ref, acc, b_ref) == 0
        zs.adamw_step(hp_gpu, p, m, v, from_np(acc), b)
        for name, gpu, ref in (("p", p, p_ref), ("m", m, m_ref), ("v", v, v_ref), ("b", b, b_ref)):
            assert _same(to_np(gpu), ref), (case, t, name)


def test_adam_update_and_no_master_special_values():
    n = 8199
    rng = np.random.default_rng(99)
    b0 = oracle.bf16_rne(rng.uniform(-0.1, 0.1, n).astype(np.float32))
    m_ref, v_ref = np.zeros(n, np.float32), np.zeros(n, np.float32)
    m2_ref, v2_ref, u_ref, b_ref = m_ref.copy(), v_ref.copy(), np.empty(n, np.float32), b0.copy()
    m, v, m2, v2 = (from_np(x.copy()) for x in (m_ref, v_ref, m2_ref, v2_ref))
    u = torch.empty(n, device="cuda")
    b = from_np(b0.copy(), bf16=True)
    for t in range(1, 4):
        acc = _special_grads(n, rng)
        hp_gpu, hp_orc = _hp(t, wd=0.0, scale=1 / 8)
        oracle.adam_update(hp_orc, m_ref, v_ref, acc, u_ref)
        oracle.adamw_step_no_master(hp_orc, b_ref, m2_ref, v2_ref, acc)
        g = from_np(acc)
        zs.adam_update(hp_gpu, m, v, g, u)
        zs.adamw_step_no_master(hp_gpu, b, m2, v2, g)
        for name, gpu, ref in (("update", u, u_ref), ("m", m, m_ref), ("v", v, v_ref), ("b", b, b_ref),
                               ("m2", m2, m2_ref), ("v2", v2, v2_ref)):
            assert _same(to_np(gpu), ref), (t, name)


# ---------------------------------------------------------------------------
# every size from 0 to 257, aligned and as misaligned views
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("offset,out_off", [(0, 0), (1, 1), (0, 1), (0, 2), (0, 3)])
def test_every_small_size(offset, out_off):
    """Each entry point at every n in [0, 257] (all tails of the 4- and
    8-element vectors and of the first workgroup tiles), against the oracle:
    accumulations, reductions and the step forms (split and tiled state)
    bit-exact, the norm within the bar, flatten and unflatten of a random
    3-way split bit-exact.  out_off places the write-only outputs (the bf16
    re-cast, the ZeRO-1 update) at their own element offset: with every
    other buffer aligned that is the 128-bit path with element-wise output
    stores."""
    rng = np.random.default_rng(1234 + offset + 10 * out_off)
    norm = torch.zeros(1, dtype=torch.float64, device="cuda")
    for n in range(0, 258):
        g32 = (rng.standard_normal(n) * 1e-2).astype(np.float32)
        g16 = oracle.bf16_rne((rng.standard_normal(n) * 1e-2).astype(np.float32))
        acc0 = (rng.standard_normal(n) * 1e-2).astype(np.float32)
        # grad_accum (bf16, add) and grad_accum_norm_sq (fp32, overwrite)
        ref = acc0.copy()
        oracle.grad_accum(ref, g16, oracle.BF16, overwrite=False)
        acc, aw = dev_buf(acc0, offset)
        zs.grad_accum(acc, dev_buf(g16, offset, bf16=True)[0], overwrite=False)
        assert bits_equal(to_np(acc), ref), ("grad_accum", n)
        ref2 = acc0.copy()
        oracle.grad_accum(ref2, g32, oracle.F32, overwrite=True)
        acc2, _ = dev_buf(acc0, offset)
        zs.grad_accum_norm_sq(acc2, dev_buf(g32, offset)[0], True, 0.5, norm)
        assert bits_equal(to_np(acc2), ref2), ("grad_accum_norm_sq", n)
        want = oracle.grad_norm_sq(ref2, 0.5)
        got = norm.item()
        assert (got == 0.0 and want == 0.0) or abs(math.sqrt(got) - math.sqrt(want)) <= NORM_TOL * math.sqrt(want), n
        zs.grad_norm_sq(dev_buf(ref2, offset)[0], 0.5, norm)
        got = norm.item()
        assert (got == 0.0 and want == 0.0) or abs(math.sqrt(got) - math.sqrt(want)) <= NORM_TOL * math.sqrt(want), n
        # grad_reduce_chunks: three bf16 chunks into acc
        chunks = [oracle.bf16_rne((rng.standard_normal(n) * 1e-2).astype(np.float32)) for _ in range(3)]
        ref3 = acc0.copy()
        for c in chunks:
            oracle.grad_accum(ref3, c, oracle.BF16, overwrite=False)
        acc3, _ = dev_buf(acc0, offset)
        zs.grad_reduce_chunks(acc3, [dev_buf(c, offset, bf16=True)[0] for c in chunks], False)
        assert bits_equal(to_np(acc3), ref3), ("grad_reduce_chunks", n)
        # the three step forms, clipped with the oracle's norm
        S = oracle.grad_norm_sq(g32, 1 / 8) + 1e-3
        nrm = torch.tensor([S], dtype=torch.float64, device="cuda")
        hp_gpu, hp_orc = _hp(3, scale=1 / 8, max_norm=0.5 * math.sqrt(S), extra=0.0)
        hp0_gpu, hp0_orc = _hp(3, wd=0.0, scale=1 / 8, max_norm=0.5 * math.sqrt(S), extra=0.0)
        p0 = rng.uniform(-0.1, 0.1, n).astype(np.float32)
        m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
        v0 = (rng.uniform(0, 1e-7, n)).astype(np.float32)
        pr, mr, vr, br = p0.copy(), m0.copy(), v0.copy(), np.zeros(n, np.uint16)
        oracle.adamw_step(hp_orc, pr, mr, vr, g32, br, norm_sq=S)
        p, m, v = dev_buf(p0, offset)[0], dev_buf(m0, offset)[0], dev_buf(v0, offset)[0]
        b, bw = dev_buf(np.zeros(n, np.uint16), out_off, bf16=True)
        zs.adamw_step(hp_gpu, p, m, v, dev_buf(g32, offset)[0], b, norm_sq=nrm)
        for name, x, r in (("p", p, pr), ("m", m, mr), ("v", v, vr), ("b", b, br)):
            assert bits_equal(to_np(x), r), ("adamw_step", n, name)
        assert canary_ok(bw, out_off, n), ("adamw_step bf16 canary", n)
        st, stw = dev_buf(oracle.state_tile(p0, m0, v0, n, 8192), 0)
        bt, btw = dev_buf(np.zeros(n, np.uint16), out_off, bf16=True)
        zs.adamw_step_tiled(hp_gpu, st, dev_buf(g32, offset)[0], bt, norm_sq=nrm)
        assert bits_equal(to_np(st), oracle.state_tile(pr, mr, vr, n, 8192)), ("adamw_step_tiled", n)
        assert bits_equal(to_np(bt), br) and canary_ok(btw, out_off, n) and canary_ok(stw, 0, st.numel()), \
            ("adamw_step_tiled bf16", n)
        mu, vu, uu = m0.copy(), v0.copy(), np.empty(n, np.float32)
        oracle.adam_update(hp0_orc, mu, vu, g32, uu, norm_sq=S)
        m, v = dev_buf(m0, offset)[0], dev_buf(v0, offset)[0]
        u, uw = dev_buf(np.zeros(n, np.float32), out_off)
        zs.adam_update(hp0_gpu, m, v, dev_buf(g32, offset)[0], u, norm_sq=nrm)
        for name, x, r in (("update", u, uu), ("m", m, mu), ("v", v, vu)):
            assert bits_equal(to_np(x), r), ("adam_update", n, name)
        assert canary_ok(uw, out_off, n), ("adam_update canary", n)
        b0 = oracle.bf16_rne(p0)
        bn, mn, vn = b0.copy(), m0.copy(), v0.copy()
        oracle.adamw_step_no_master(hp_orc, bn, mn, vn, g32, norm_sq=S)
        b, m, v = dev_buf(b0, offset, bf16=True)[0], dev_buf(m0, offset)[0], dev_buf(v0, offset)[0]
        zs.adamw_step_no_master(hp_gpu, b, m, v, dev_buf(g32, offset)[0], norm_sq=nrm)
        for name, x, r in (("b", b, bn), ("m", m, mn), ("v", v, vn)):
            assert bits_equal(to_np(x), r), ("adamw_step_no_master", n, name)
        # flatten a random 3-way split of n bf16 elements (padded by 0..3) and unflatten it
        cuts = np.sort(rng.integers(0, n + 1, size=2))
        parts = [g16[:cuts[0]], g16[cuts[0]:cuts[1]], g16[cuts[1]:]]
        pad = n + int(rng.integers(0, 4))
        want_flat = oracle.flat_pack([np.ascontiguousarray(x) for x in parts], oracle.BF16, oracle.F32, pad)
        flat, _ = dev_buf(np.zeros(pad, np.float32), offset)
        if pad > 0:
            flat.fill_(float("nan"))
        zs.flat_pack([dev_buf(np.ascontiguousarray(x), offset, bf16=True)[0] for x in parts], flat, pad)
        assert bits_equal(to_np(flat), want_flat), ("flat_pack", n)
        outs = [dev_buf(np.zeros(x.size, np.uint16), offset, bf16=True)[0] for x in parts]
        zs.flat_unpack(flat, outs)
        for o, x in zip(outs, parts):
            assert bits_equal(to_np(o), oracle.bf16_rne(oracle.bf16_widen(x))), ("flat_unpack", n)
    torch.cuda.synchronize()
