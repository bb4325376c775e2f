"""GPU parity of the tiled optimizer-state entry points against the oracle.

The tiled layout keeps a shard's fp32 master, exp_avg and exp_avg_sq in one
buffer, three runs of ZS_STATE_TILE floats per tile of elements.  The
conversions must match the oracle's layout bit for bit (padding included);
the tiled AdamW step, read back through the oracle's untile, must meet the
same bar as adamw_step and, handed the oracle's norm, be bit-identical to the
oracle.  Sizes span several tiles and ragged ends, with the bf16 output at
every element offset modulo 4.  Every buffer carries a canary tail.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import fsdp_sharded_optimizer_amd as zs
from tests.parity import StateCheck, bits_equal, from_np, identical_fraction, to_np
from tests.test_gpu_kernels import _hp, canary_ok, dev_buf

pytestmark = pytest.mark.gpu

T = 8192   # ZS_STATE_TILE (test_abi checks the header against this value)
SIZES = [1, 3, 4, 5, 255, 8191, 8192, 8193, 3 * 8192 + 7, 100_003]
CANARY = 64


def state_dev(state_np: np.ndarray):
    """A device copy of a tiled state with a canary tail; (view, whole)."""
    return dev_buf(state_np, 0)


def random_state(rng, n):
    p = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = (rng.uniform(0, 1e-7, n)).astype(np.float32)
    return p, m, v


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("offset", [0, 1])
def test_state_tile_untile_bit_exact(n, offset):
    """Tile from (possibly misaligned) split views, with one source missing,
    equals the oracle's tiled buffer bit for bit, padding zeros included;
    untile into views back to the inputs, a missing destination untouched."""
    print(f"state tile/untile n={n} offset={offset}", flush=True)
    rng = np.random.default_rng(n + 13 * offset)
    p, m, v = random_state(rng, n)
    want = oracle.state_tile(p, None, v, n, T)
    assert zs.state_tiled_numel(n) == want.size
    pd, pw = dev_buf(p, offset)
    vd, vw = dev_buf(v, offset)
    st, stw = state_dev(np.full(want.size, np.nan, np.float32))
    zs.state_tile(pd, None, vd, st)
    torch.cuda.synchronize()
    assert bits_equal(to_np(st), want), identical_fraction(to_np(st), want)
    assert canary_ok(stw, 0, want.size) and canary_ok(pw, offset, n) and canary_ok(vw, offset, n)
    # untile the oracle's full state (moments present) into views
    full = oracle.state_tile(p, m, v, n, T)
    st2, _ = state_dev(full)
    outs = [dev_buf(np.zeros(n, np.float32), offset) for _ in range(3)]
    zs.state_untile(st2, outs[0][0], None, outs[2][0])
    torch.cuda.synchronize()
    assert bits_equal(to_np(outs[0][0]), p) and bits_equal(to_np(outs[2][0]), v)
    assert np.all(to_np(outs[1][0]).view(np.uint32) == 0)          # skipped: left as it was
    for view, whole in outs:
        assert canary_ok(whole, offset, n)


def test_state_tile_all_sources_missing_and_empty():
    n = 3 * T + 5
    st, stw = state_dev(np.full(zs.state_tiled_numel(n), np.nan, np.float32))
    zs.state_tile(None, None, None, st, n=n)
    torch.cuda.synchronize()
    assert np.all(to_np(st).view(np.uint32) == 0) and canary_ok(stw, 0, st.numel())
    empty = torch.empty(0, dtype=torch.float32, device="cuda")
    zs.state_tile(empty, empty, empty, empty)
    zs.state_untile(empty, empty, empty, empty)
    with pytest.raises(ValueError):
        zs.state_tile(torch.zeros(n, device="cuda"), None, None, torch.zeros(10, device="cuda"))


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("b_off", [0, 1, 2, 3])
@pytest.mark.parametrize("mode", ["adam_f32", "adamw_bf16", "adamw_bf16_clip"])
def test_adamw_step_tiled_parity(n, b_off, mode):
    """Three steps on a tiled state; after each, the state read back through
    the oracle's untile meets the bar against the oracle on split arrays,
    and the padding of the last tile is untouched.  b_off = 1..3 puts the
    bf16 output off a 16-byte boundary (element-wise bf16 stores inside the
    128-bit path)."""
    print(f"adamw tiled n={n} b_off={b_off} mode={mode}", flush=True)
    rng = np.random.default_rng(n * 5 + b_off + len(mode))
    p_ref = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    m_ref, v_ref = np.zeros(n, np.float32), np.zeros(n, np.float32)
    wd = 0.0 if mode == "adam_f32" else 0.1
    bf16 = mode != "adam_f32"
    clip = mode.endswith("clip")
    b_ref = np.zeros(n, np.uint16)
    st, stw = state_dev(oracle.state_tile(p_ref, m_ref, v_ref, n, T))
    b, bw = dev_buf(np.zeros(n, np.uint16), b_off, bf16=True) if bf16 else (None, None)
    norm = torch.zeros(1, dtype=torch.float64, device="cuda")
    for t in range(1, 4):
        acc = (rng.standard_normal(n) * 3e-3).astype(np.float32)
        g, gw = dev_buf(acc, 0)
        S_ref = oracle.grad_norm_sq(acc, 1 / 64)
        max_norm = 0.5 * math.sqrt(S_ref * 8) if clip else 0.0
        extra = 7 * S_ref if clip else 0.0
        hp_gpu, hp_orc = _hp(t, wd=wd, max_norm=max_norm, extra=extra)
        prev = {"p": p_ref.copy(), "m": m_ref.copy()}
        oracle.adamw_step(hp_orc, p_ref, m_ref, v_ref, acc, b_ref if bf16 else None,
                          norm_sq=S_ref if clip else None)
        if clip:
            zs.grad_norm_sq(g, 1 / 64, norm)
        zs.adamw_step_tiled(hp_gpu, st, g, b, norm_sq=norm if clip else None)
        torch.cuda.synchronize()
        state = to_np(st)
        gp, gm, gv = oracle.state_untile(state, n, T)
        s = oracle.adamw_scalars(hp_orc)
        coef = oracle.clip_coef(S_ref, extra, max_norm) if clip else 1.0
        g2 = (acc * np.float32(1 / 64)) * np.float32(coef)
        res = StateCheck(0.9, 3e-4, wd, s.step_size).check(
            {"p": gp, "m": gm, "v": gv, "b": to_np(b) if bf16 else None},
            {"p": p_ref, "m": m_ref, "v": v_ref, "b": b_ref}, prev, g2, f"t={t}")
        print(f"  t={t} {res}", flush=True)
        # padding of the last tile: still the zeros the oracle's tile wrote
        idx = np.arange(state.size)
        in_range = (idx // (3 * T)) * T + idx % T < n
        assert np.all(state.view(np.uint32)[~in_range] == 0), "padding written"
        assert canary_ok(gw, 0, n)
    assert canary_ok(stw, 0, st.numel())
    if bf16:
        assert canary_ok(bw, b_off, n)


@pytest.mark.parametrize("n", [8193, 100_003])
@pytest.mark.parametrize("b_off", [0, 1])
def test_adamw_step_tiled_bit_exact_given_the_oracle_norm(n, b_off):
    """Handed the oracle's squared norm, the tiled step's state and bf16
    output are bit-identical to the oracle's split-array step."""
    print(f"adamw tiled bit-exact n={n} b_off={b_off}", flush=True)
    rng = np.random.default_rng(n + b_off)
    p_ref = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    m_ref, v_ref, b_ref = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
    st, _ = state_dev(oracle.state_tile(p_ref, m_ref, v_ref, n, T))
    b, _ = dev_buf(b_ref, b_off, bf16=True)
    for t in range(1, 6):
        acc = (rng.standard_normal(n) * 1e-2).astype(np.float32)
        S = oracle.grad_norm_sq(acc, 1 / 32)
        hp_gpu, hp_orc = _hp(t, scale=1 / 32, max_norm=math.sqrt(S) * 0.8 if t % 2 else 0.0, extra=0.25 * S)
        oracle.adamw_step(hp_orc, p_ref, m_ref, v_ref, acc, b_ref, norm_sq=S)
        g, _ = dev_buf(acc, 1)
        norm = torch.tensor([S], dtype=torch.float64, device="cuda")
        zs.adamw_step_tiled(hp_gpu, st, g, b, norm_sq=norm)
        want = oracle.state_tile(p_ref, m_ref, v_ref, n, T)
        got = to_np(st)
        assert bits_equal(got, want), (t, identical_fraction(got, want))
        assert bits_equal(to_np(b), b_ref), t


def test_tiled_step_equals_split_step_and_dev_scalars():
    """On the GPU: the tiled step (host scalars and device scalars) and the
    split-array step give identical bits, over five steps with a clip."""
    n = 5 * T + 333
    rng = np.random.default_rng(77)
    p0 = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    p = from_np(p0)
    m = torch.zeros(n, dtype=torch.float32, device="cuda")
    v = torch.zeros(n, dtype=torch.float32, device="cuda")
    b = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    st = torch.empty(zs.state_tiled_numel(n), dtype=torch.float32, device="cuda")
    st2 = torch.empty_like(st)
    zs.state_tile(p, None, None, st)
    zs.state_tile(p, None, None, st2)
    b1, b2 = torch.zeros_like(b), torch.zeros_like(b)
    norm = torch.zeros(1, dtype=torch.float64, device="cuda")
    sc = torch.empty(64, dtype=torch.uint8, device="cuda")
    for t in range(1, 6):
        g = from_np((rng.standard_normal(n) * 1e-2).astype(np.float32))
        zs.grad_norm_sq(g, 1 / 32, norm)
        hp = zs.AdamWConfig(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_scale=1 / 32,
                            max_norm=0.5, extra_norm_sq=0.1, step=t)
        zs.adamw_step(hp, p, m, v, g, b, norm_sq=norm)
        zs.adamw_step_tiled(hp, st, g, b1, norm_sq=norm)
        sc[:56].copy_(torch.frombuffer(bytearray(zs.scalars_bytes(hp)), dtype=torch.uint8))
        zs.adamw_step_tiled_dev(sc, st2, g, b2, norm_sq=norm)
        torch.cuda.synchronize()
        split = oracle.state_tile(to_np(p), to_np(m), to_np(v), n, T)
        assert bits_equal(to_np(st), split), t
        assert bits_equal(to_np(st2), split), t
        assert bits_equal(to_np(b1), to_np(b)) and bits_equal(to_np(b2), to_np(b)), t
    back = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(3)]
    zs.state_untile(st, *back)
    torch.cuda.synchronize()
    for x, y in zip(back, (p, m, v)):
        assert bits_equal(to_np(x), to_np(y))


def test_adamw_step_tiled_skips_on_nonfinite_norm():
    n = 4 * T + 9
    rng = np.random.default_rng(3)
    p0, m0, v0 = random_state(rng, n)
    state0 = oracle.state_tile(p0, m0, v0, n, T)
    st, _ = state_dev(state0)
    b0 = oracle.bf16_rne(p0)
    b, _ = dev_buf(b0, 0, bf16=True)
    g = from_np((rng.standard_normal(n) * 1e-3).astype(np.float32))
    for bad in (float("inf"), float("nan")):
        norm = torch.tensor([bad], dtype=torch.float64, device="cuda")
        hp = zs.AdamWConfig(lr=1e-3, weight_decay=0.1, max_norm=1.0, step=1)
        zs.adamw_step_tiled(hp, st, g, b, norm_sq=norm)
        torch.cuda.synchronize()
        assert bits_equal(to_np(st), state0) and bits_equal(to_np(b), b0)
    # extra_norm_sq non-finite (the other ranks' share) skips too
    norm = torch.tensor([1.0], dtype=torch.float64, device="cuda")
    zs.adamw_step_tiled(zs.AdamWConfig(lr=1e-3, extra_norm_sq=float("inf"), step=1), st, g, b, norm_sq=norm)
    torch.cuda.synchronize()
    assert bits_equal(to_np(st), state0)


# ---------------------------------------------------------------------------
# tiled moments (exp_avg, exp_avg_sq): the no-master and ZeRO-1 update forms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 5, 8192, 8193, 3 * 8192 + 7, 100_003])
@pytest.mark.parametrize("offset", [0, 1])
def test_moments_tile_untile_bit_exact(n, offset):
    """moments_tile from (possibly misaligned) views, one source missing,
    equals the oracle's layout bit for bit, padding zeros included;
    moments_untile inverts it into views."""
    print(f"moments tile/untile n={n} offset={offset}", flush=True)
    rng = np.random.default_rng(3 * n + offset)
    _, m, v = random_state(rng, n)
    want = oracle.moments_tile(None, v, n, T)
    assert zs.moments_tiled_numel(n) == want.size
    vd, vw = dev_buf(v, offset)
    mo, mow = state_dev(np.full(want.size, np.nan, np.float32))
    zs.moments_tile(None, vd, mo, n=n)
    torch.cuda.synchronize()
    assert bits_equal(to_np(mo), want) and canary_ok(mow, 0, want.size) and canary_ok(vw, offset, n)
    full, _ = state_dev(oracle.moments_tile(m, v, n, T))
    outs = [dev_buf(np.zeros(n, np.float32), offset) for _ in range(2)]
    zs.moments_untile(full, outs[0][0], outs[1][0])
    torch.cuda.synchronize()
    assert bits_equal(to_np(outs[0][0]), m) and bits_equal(to_np(outs[1][0]), v)
    for view, whole in outs:
        assert canary_ok(whole, offset, n)


@pytest.mark.parametrize("n", [1, 7, 8193, 100_003])
@pytest.mark.parametrize("upd_off", [0, 1, 2, 3])
@pytest.mark.parametrize("clip", [False, True])
def test_adam_update_tiled_bit_exact(n, upd_off, clip):
    """Four steps of the ZeRO-1 update on tiled moments, the update a view
    at any element offset, handed the oracle's norm: moments and update
    bit-identical to the oracle's split-array adam_update."""
    print(f"adam_update tiled n={n} upd_off={upd_off} clip={clip}", flush=True)
    rng = np.random.default_rng(11 * n + upd_off + 5 * clip)
    m_ref, v_ref, u_ref = np.zeros(n, np.float32), np.zeros(n, np.float32), np.empty(n, np.float32)
    mo, mow = state_dev(oracle.moments_tile(m_ref, v_ref, n, T))
    u, uw = dev_buf(np.zeros(n, np.float32), upd_off)
    for t in range(1, 5):
        acc = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        S = oracle.grad_norm_sq(acc, 1 / 8)
        hp_gpu, hp_orc = _hp(t, lr=1e-4, b2=0.999, wd=0.0, scale=1 / 8,
                             max_norm=0.7 * math.sqrt(S * 8) if clip else 0.0, extra=7 * S)
        assert oracle.adam_update(hp_orc, m_ref, v_ref, acc, u_ref, norm_sq=S if clip else None) == 0
        g, gw = dev_buf(acc, 1)
        norm = torch.tensor([S], dtype=torch.float64, device="cuda") if clip else None
        zs.adam_update_tiled(hp_gpu, mo, g, u, norm_sq=norm)
        torch.cuda.synchronize()
        assert bits_equal(to_np(mo), oracle.moments_tile(m_ref, v_ref, n, T)), t
        assert bits_equal(to_np(u), u_ref), (t, identical_fraction(to_np(u), u_ref))
        assert canary_ok(gw, 1, n)
    assert canary_ok(mow, 0, mo.numel()) and canary_ok(uw, upd_off, n)


@pytest.mark.parametrize("n", [1, 7, 8193, 100_003])
@pytest.mark.parametrize("p_off", [0, 1, 3])
@pytest.mark.parametrize("clip", [False, True])
def test_adamw_no_master_tiled_bit_exact(n, p_off, clip):
    """Four steps of the no-master update on tiled moments, the bf16
    parameter aligned (vector path) or at an odd element offset (the
    element-wise path), handed the oracle's norm: bit-identical."""
    print(f"no-master tiled n={n} p_off={p_off} clip={clip}", flush=True)
    rng = np.random.default_rng(13 * n + p_off + 7 * clip)
    b_ref = oracle.bf16_rne(rng.uniform(-0.1, 0.1, n).astype(np.float32))
    m_ref, v_ref = np.zeros(n, np.float32), np.zeros(n, np.float32)
    mo, mow = state_dev(oracle.moments_tile(m_ref, v_ref, n, T))
    b, bw = dev_buf(b_ref, p_off, bf16=True)
    for t in range(1, 5):
        acc = (rng.standard_normal(n) * 1e-2).astype(np.float32)
        S = oracle.grad_norm_sq(acc, 1 / 16)
        hp_gpu, hp_orc = _hp(t, lr=2e-3, scale=1 / 16, max_norm=0.5 * math.sqrt(S) if clip else 0.0, extra=0.1 * S)
        assert oracle.adamw_step_no_master(hp_orc, b_ref, m_ref, v_ref, acc, norm_sq=S if clip else None) == 0
        g, _ = dev_buf(acc, 0)
        norm = torch.tensor([S], dtype=torch.float64, device="cuda") if clip else None
        zs.adamw_step_no_master_tiled(hp_gpu, b, mo, g, norm_sq=norm)
        torch.cuda.synchronize()
        assert bits_equal(to_np(mo), oracle.moments_tile(m_ref, v_ref, n, T)), t
        assert bits_equal(to_np(b), b_ref), (t, identical_fraction(to_np(b), b_ref))
    assert canary_ok(mow, 0, mo.numel()) and canary_ok(bw, p_off, n)
