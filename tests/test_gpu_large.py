"""GPU parity for calls longer than one launch.

A HIP launch must stay below 2^32 work-items, so the library runs a call of
more than 2^31 elements as several launches over consecutive pieces of the
buffers (and several table entries per tensor for the flat copies).  Every
case here crosses at least one piece boundary, aligned (vector path) and as
a view one element off (scalar path), and the last one runs the scalar
AdamW path past 2^32 elements.  Inputs are drawn on the GPU with seeded
generators and copied to the host for the oracle.  The steps are
element-wise, so the oracle runs the sampled elements alone (both sides of
every piece boundary, the head, the tail and random elements) and carries
its own state from step to step; the norm it forms over the whole buffer.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import fsdp_sharded_optimizer_amd as zs
from tests.parity import NORM_TOL, bits_equal, identical_fraction, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = "cuda"
PIECE = 1 << 31            # elements per launch
N = PIECE + 4099           # one piece boundary, a ragged last piece
FILL = 1 << 27             # elements per generator call when filling


def log(msg):
    print(msg, flush=True)


def host(t: torch.Tensor) -> np.ndarray:
    return to_np(t)


def sample_indices(n: int, seed: int, k: int = 1 << 16) -> torch.Tensor:
    rng = np.random.default_rng(seed)
    parts = [np.arange(min(n, 2048)), np.arange(max(0, n - 2048), n), rng.integers(0, n, size=k)]
    for b in range(PIECE, n, PIECE):
        parts.append(np.arange(b - 2048, min(n, b + 2048)))
    return torch.from_numpy(np.unique(np.concatenate(parts)).astype(np.int64)).to(DEV)


def gen(seed: int) -> torch.Generator:
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def buffer(n: int, offset: int, dtype=torch.float32):
    """A length-n view `offset` elements into a fresh allocation."""
    whole = torch.empty(n + offset + 8, dtype=dtype, device=DEV)
    return whole[offset:offset + n]


def fill_normal(t: torch.Tensor, std: float, seed: int) -> torch.Tensor:
    g = gen(seed)
    for a in range(0, t.numel(), FILL):
        t[a:a + FILL].normal_(0.0, std, generator=g)
    return t


def fill_uniform(t: torch.Tensor, lo: float, hi: float, seed: int) -> torch.Tensor:
    g = gen(seed)
    for a in range(0, t.numel(), FILL):
        t[a:a + FILL].uniform_(lo, hi, generator=g)
    return t


def bf16_normal(n: int, offset: int, std: float, seed: int) -> torch.Tensor:
    out = buffer(n, offset, torch.bfloat16)
    tmp = torch.empty(min(n, FILL), dtype=torch.float32, device=DEV)
    g = gen(seed)
    for a in range(0, n, FILL):
        b = min(n, a + FILL)
        tmp[:b - a].normal_(0.0, std, generator=g)
        out[a:b].copy_(tmp[:b - a])   # round to nearest even
    return out


def need_gib(gib: float):
    """Skip (on a smaller GPU) when the device has less free memory than a
    case needs."""
    free = torch.cuda.mem_get_info()[0] / 2**30
    if free < gib:
        pytest.skip(f"needs {gib:.0f} GiB of free device memory, {free:.0f} GiB free")


def release():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def check(name, gpu: torch.Tensor, idx: torch.Tensor, ref: np.ndarray):
    got = host(gpu[idx])
    assert bits_equal(got, ref), (name, identical_fraction(got, ref))


@pytest.mark.parametrize("offset", [0, 1])
def test_adamw_forms_across_pieces(offset):
    """adamw_step (clipped, bf16 re-cast), then adamw_step_no_master and
    adam_update on the same state, over N elements: bit-exact on the
    sample."""
    need_gib(45)
    log(f"adamw forms across pieces n={N} offset={offset}")
    idx = sample_indices(N, seed=11 + offset)
    master = fill_uniform(buffer(N, offset), -0.1, 0.1, 101)
    m = fill_normal(buffer(N, offset), 1e-4, 102)
    v = fill_uniform(buffer(N, offset), 0.0, 1e-8, 103)
    grad = fill_normal(buffer(N, offset), 1e-3, 104)
    bf16 = buffer(N, offset, torch.bfloat16)
    scale, extra, max_norm = 1.0 / 64, 2.0, 1.0
    S = oracle.grad_norm_sq(host(grad), scale)   # the oracle's norm over the whole buffer feeds both sides
    gpu_norm = torch.zeros(1, dtype=torch.float64, device=DEV)
    zs.grad_norm_sq(grad, scale, gpu_norm)
    assert abs(math.sqrt(gpu_norm.item()) - math.sqrt(S)) <= NORM_TOL * math.sqrt(S)
    assert oracle.clip_coef(S, extra, max_norm) < 1.0
    norm = torch.tensor([S], dtype=torch.float64, device=DEV)
    p_ref, m_ref, v_ref, g_s = host(master[idx]), host(m[idx]), host(v[idx]), host(grad[idx])
    b_ref = np.empty(idx.numel(), np.uint16)

    log("  adamw_step")
    hp = zs.AdamWConfig(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_scale=scale,
                        max_norm=max_norm, extra_norm_sq=extra, step=3)
    zs.adamw_step(hp, master, m, v, grad, bf16, norm_sq=norm)
    H = oracle.make_hp(3e-4, 0.9, 0.95, 1e-8, 0.1, scale, max_norm, extra, 3)
    assert oracle.adamw_step(H, p_ref, m_ref, v_ref, g_s, b_ref, norm_sq=S) == 0
    for name, gpu, ref in (("master", master, p_ref), ("m", m, m_ref), ("v", v, v_ref), ("bf16", bf16, b_ref)):
        check(name, gpu, idx, ref)

    log("  adamw_step_no_master")
    hp.step = 4
    zs.adamw_step_no_master(hp, bf16, m, v, grad, norm_sq=norm)
    H = oracle.make_hp(3e-4, 0.9, 0.95, 1e-8, 0.1, scale, max_norm, extra, 4)
    assert oracle.adamw_step_no_master(H, b_ref, m_ref, v_ref, g_s, norm_sq=S) == 0
    for name, gpu, ref in (("bf16", bf16, b_ref), ("m", m, m_ref), ("v", v, v_ref)):
        check(name, gpu, idx, ref)

    log("  adam_update")
    hu = zs.AdamWConfig(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0, grad_scale=scale,
                        max_norm=max_norm, extra_norm_sq=extra, step=5)
    zs.adam_update(hu, m, v, grad, master, norm_sq=norm)   # the update into the master's buffer
    H = oracle.make_hp(3e-4, 0.9, 0.95, 1e-8, 0.0, scale, max_norm, extra, 5)
    u_ref = np.empty(idx.numel(), np.float32)
    assert oracle.adam_update(H, m_ref, v_ref, g_s, u_ref, norm_sq=S) == 0
    for name, gpu, ref in (("update", master, u_ref), ("m", m, m_ref), ("v", v, v_ref)):
        check(name, gpu, idx, ref)
    del master, m, v, grad, bf16
    release()


STATE_TILE = 8192   # ZS_STATE_TILE (test_abi checks the header against this value)


@pytest.mark.parametrize("b_off", [0, 1])
def test_tiled_state_across_pieces(b_off):
    """state_tile, a clipped adamw_step_tiled and state_untile over N
    elements (a launch piece starts the tiled state 3 * 2^31 floats in):
    the state read at the layout's positions and the untiled arrays
    bit-exact on the sample.  b_off = 1 puts the bf16 output off a 16-byte
    boundary (element-wise bf16 stores inside the 128-bit path)."""
    need_gib(72)
    log(f"tiled state across pieces n={N} bf16 offset={b_off}")
    idx = sample_indices(N, seed=61 + b_off)
    master = fill_uniform(buffer(N, 0), -0.1, 0.1, 601)
    m = fill_normal(buffer(N, 0), 1e-4, 602)
    v = fill_uniform(buffer(N, 0), 0.0, 1e-8, 603)
    grad = fill_normal(buffer(N, 0), 1e-3, 604)
    bf16 = buffer(N, b_off, torch.bfloat16)
    state = torch.empty(zs.state_tiled_numel(N), dtype=torch.float32, device=DEV)
    where = (idx // STATE_TILE) * (3 * STATE_TILE) + idx % STATE_TILE
    p_ref, m_ref, v_ref, g_s = host(master[idx]), host(m[idx]), host(v[idx]), host(grad[idx])

    log("  state_tile")
    zs.state_tile(master, m, v, state)
    for k, (name, ref) in enumerate((("master", p_ref), ("m", m_ref), ("v", v_ref))):
        check(f"tile {name}", state, where + k * STATE_TILE, ref)
    tail = torch.arange(N, zs.state_tiled_numel(N) // 3, device=DEV)      # the last tile's unused ends
    tail_at = (tail // STATE_TILE) * (3 * STATE_TILE) + tail % STATE_TILE
    for k in range(3):
        assert not host(state[tail_at + k * STATE_TILE]).view(np.uint32).any()

    log("  adamw_step_tiled")
    scale, extra, max_norm = 1.0 / 64, 2.0, 1.0
    S = oracle.grad_norm_sq(host(grad), scale)
    assert oracle.clip_coef(S, extra, max_norm) < 1.0
    norm = torch.tensor([S], dtype=torch.float64, device=DEV)
    hp = zs.AdamWConfig(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_scale=scale,
                        max_norm=max_norm, extra_norm_sq=extra, step=3)
    zs.adamw_step_tiled(hp, state, grad, bf16, norm_sq=norm)
    H = oracle.make_hp(3e-4, 0.9, 0.95, 1e-8, 0.1, scale, max_norm, extra, 3)
    b_ref = np.empty(idx.numel(), np.uint16)
    assert oracle.adamw_step(H, p_ref, m_ref, v_ref, g_s, b_ref, norm_sq=S) == 0
    for k, (name, ref) in enumerate((("master", p_ref), ("m", m_ref), ("v", v_ref))):
        check(f"step {name}", state, where + k * STATE_TILE, ref)
    check("bf16", bf16, idx, b_ref)

    log("  state_untile")
    zs.state_untile(state, master, m, v)
    for name, gpu, ref in (("master", master, p_ref), ("m", m, m_ref), ("v", v, v_ref)):
        check(f"untile {name}", gpu, idx, ref)
    del master, m, v, grad, bf16, state
    release()


@pytest.mark.parametrize("out_off", [0, 1])
def test_tiled_moments_across_pieces(out_off):
    """moments_tile, a clipped adam_update_tiled (the update a view
    out_off elements into its buffer), adamw_step_no_master_tiled and
    moments_untile over N elements (a launch piece starts the tiled moments
    2 * 2^31 floats in): bit-exact on the sample."""
    need_gib(62)
    log(f"tiled moments across pieces n={N} out_off={out_off}")
    idx = sample_indices(N, seed=71 + out_off)
    m = fill_normal(buffer(N, 0), 1e-4, 701)
    v = fill_uniform(buffer(N, 0), 0.0, 1e-8, 702)
    grad = fill_normal(buffer(N, 0), 1e-3, 703)
    upd = buffer(N, out_off)
    param = bf16_normal(N, out_off, 0.05, 704)
    mo = torch.empty(zs.moments_tiled_numel(N), dtype=torch.float32, device=DEV)
    where = (idx // STATE_TILE) * (2 * STATE_TILE) + idx % STATE_TILE
    m_ref, v_ref, g_s, b_ref = host(m[idx]), host(v[idx]), host(grad[idx]), host(param[idx])

    log("  moments_tile")
    zs.moments_tile(m, v, mo)
    check("tile m", mo, where, m_ref)
    check("tile v", mo, where + STATE_TILE, v_ref)

    scale, extra, max_norm = 1.0 / 64, 2.0, 1.0
    S = oracle.grad_norm_sq(host(grad), scale)
    assert oracle.clip_coef(S, extra, max_norm) < 1.0
    norm = torch.tensor([S], dtype=torch.float64, device=DEV)
    log("  adam_update_tiled")
    hu = zs.AdamWConfig(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0, grad_scale=scale,
                        max_norm=max_norm, extra_norm_sq=extra, step=3)
    zs.adam_update_tiled(hu, mo, grad, upd, norm_sq=norm)
    u_ref = np.empty(idx.numel(), np.float32)
    H = oracle.make_hp(3e-4, 0.9, 0.95, 1e-8, 0.0, scale, max_norm, extra, 3)
    assert oracle.adam_update(H, m_ref, v_ref, g_s, u_ref, norm_sq=S) == 0
    check("update", upd, idx, u_ref)
    check("m", mo, where, m_ref)
    check("v", mo, where + STATE_TILE, v_ref)

    log("  adamw_step_no_master_tiled")
    hp = zs.AdamWConfig(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_scale=scale,
                        max_norm=max_norm, extra_norm_sq=extra, step=4)
    zs.adamw_step_no_master_tiled(hp, param, mo, grad, norm_sq=norm)
    H = oracle.make_hp(3e-4, 0.9, 0.95, 1e-8, 0.1, scale, max_norm, extra, 4)
    assert oracle.adamw_step_no_master(H, b_ref, m_ref, v_ref, g_s, norm_sq=S) == 0
    check("bf16", param, idx, b_ref)

    log("  moments_untile")
    zs.moments_untile(mo, m, v)
    check("untile m", m, idx, m_ref)
    check("untile v", v, idx, v_ref)
    del m, v, grad, upd, param, mo
    release()


@pytest.mark.parametrize("offset", [0, 1])
def test_accumulations_across_pieces(offset):
    """grad_accum (overwrite, add) and grad_accum_norm_sq (the accumulating
    Q = 1 form; the overwriting bf16 Q = 4 form; the overwriting fp32 form)
    over N elements: acc bit-exact on the sample, the norm within the bar of
    the oracle's over the whole buffer."""
    need_gib(40)
    log(f"accumulations across pieces n={N} offset={offset}")
    idx = sample_indices(N, seed=21 + offset)
    scale = 1.0 / 32
    acc = buffer(N, offset)
    gs = [bf16_normal(N, offset, 1e-3, 201 + k) for k in range(3)]
    ws = torch.empty(zs.grad_accum_norm_sq_workspace_bytes(N), dtype=torch.uint8, device=DEV)
    norm = torch.zeros(1, dtype=torch.float64, device=DEV)

    log("  overwrite, add, add + norm")
    zs.grad_accum(acc, gs[0], overwrite=True)
    zs.grad_accum(acc, gs[1], overwrite=False)
    zs.grad_accum_norm_sq(acc, gs[2], False, scale, norm, ws)
    full = np.empty(N, np.float32)
    for k, g in enumerate(gs):
        oracle.grad_accum(full, host(g), oracle.BF16, overwrite=(k == 0))
    S = oracle.grad_norm_sq(full, scale)
    assert abs(math.sqrt(norm.item()) - math.sqrt(S)) <= NORM_TOL * math.sqrt(S)
    check("acc", acc, idx, full[host(idx)])

    log("  overwrite + norm (bf16)")
    zs.grad_accum_norm_sq(acc, gs[1], True, scale, norm, ws)
    ref = oracle.bf16_widen(host(gs[1]))
    S = oracle.grad_norm_sq(ref, scale)
    assert abs(math.sqrt(norm.item()) - math.sqrt(S)) <= NORM_TOL * math.sqrt(S)
    check("acc", acc, idx, ref[host(idx)])
    del gs, ref, full

    log("  overwrite + norm (fp32)")
    g32 = fill_normal(buffer(N, offset), 1e-3, 210)
    zs.grad_accum_norm_sq(acc, g32, True, scale, norm, ws)
    ref = host(g32)
    S = oracle.grad_norm_sq(ref, scale)
    assert abs(math.sqrt(norm.item()) - math.sqrt(S)) <= NORM_TOL * math.sqrt(S)
    check("acc", acc, idx, ref[host(idx)])
    del acc, g32, ws
    release()


@pytest.mark.parametrize("offset", [0, 1])
def test_one_pass_last_micro_batch_across_pieces(offset):
    """grad_sum_norm_sq and a clipped adamw_step_tiled_sum over N elements,
    on accumulator + bf16 gradient and on the gradient alone (offset 1: the
    gradient 2 bytes off a 4-byte boundary, the element-wise paths): the
    norm bit for bit grad_accum_norm_sq's and within the bar of the
    oracle's over the whole buffer, the state and bf16 output bit-exact on
    the sample, the accumulator unchanged."""
    need_gib(80)
    log(f"one-pass last micro-batch across pieces n={N} offset={offset}")
    idx = sample_indices(N, seed=81 + offset)
    where = (idx // STATE_TILE) * (3 * STATE_TILE) + idx % STATE_TILE
    master = fill_uniform(buffer(N, 0), -0.1, 0.1, 801)
    state = torch.empty(zs.state_tiled_numel(N), dtype=torch.float32, device=DEV)
    zs.state_tile(master, None, None, state)
    p_ref = host(master[idx])
    del master
    m_ref, v_ref = np.zeros(idx.numel(), np.float32), np.zeros(idx.numel(), np.float32)
    b_ref = np.empty(idx.numel(), np.uint16)
    bf16 = buffer(N, offset, torch.bfloat16)
    acc = fill_normal(buffer(N, 0), 1e-3, 802)
    g = bf16_normal(N, offset, 1e-3, 803)
    scale, extra, max_norm = 1.0 / 64, 2.0, 1.0
    ws = torch.empty(zs.grad_accum_norm_sq_workspace_bytes(N), dtype=torch.uint8, device=DEV)
    acc_s, g_s = host(acc[idx]), host(g[idx])
    for step, with_acc in ((3, True), (4, False)):
        log(f"  step {step}: {'accumulator + gradient' if with_acc else 'the gradient alone'}")
        a = acc if with_acc else None
        norm = torch.zeros(1, dtype=torch.float64, device=DEV)
        zs.grad_sum_norm_sq(a, g, not with_acc, scale, norm, ws)
        full = host(acc) if with_acc else np.empty(N, np.float32)
        oracle.grad_accum(full, host(g), oracle.BF16, overwrite=not with_acc)
        S = oracle.grad_norm_sq(full, scale)
        del full
        assert abs(math.sqrt(norm.item()) - math.sqrt(S)) <= NORM_TOL * math.sqrt(S)
        stored = buffer(N, 0)
        stored.copy_(acc)
        norm2 = torch.zeros(1, dtype=torch.float64, device=DEV)
        zs.grad_accum_norm_sq(stored, g, not with_acc, scale, norm2, ws)
        assert norm.item() == norm2.item()
        del stored
        assert oracle.clip_coef(S, extra, max_norm) < 1.0
        norm.fill_(S)
        hp = zs.AdamWConfig(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_scale=scale,
                            max_norm=max_norm, extra_norm_sq=extra, step=step)
        zs.adamw_step_tiled_sum(hp, state, a, g, bf16, norm_sq=norm)
        gsum = acc_s.copy() if with_acc else np.empty(idx.numel(), np.float32)
        oracle.grad_accum(gsum, g_s, oracle.BF16, overwrite=not with_acc)
        H = oracle.make_hp(3e-4, 0.9, 0.95, 1e-8, 0.1, scale, max_norm, extra, step)
        assert oracle.adamw_step(H, p_ref, m_ref, v_ref, gsum, b_ref, norm_sq=S) == 0
        for k, (name, ref) in enumerate((("master", p_ref), ("m", m_ref), ("v", v_ref))):
            check(f"step {name}", state, where + k * STATE_TILE, ref)
        check("bf16", bf16, idx, b_ref)
        check("acc unchanged", acc, idx, acc_s)
    del state, bf16, acc, g, ws
    release()


@pytest.mark.parametrize("offset", [0, 1])
def test_reduce_chunks_across_pieces(offset):
    """Three bf16 rank chunks (the third the first again) summed into acc
    over N elements, overwriting: bit-exact on the sample."""
    need_gib(25)
    log(f"grad_reduce_chunks across pieces n={N} offset={offset}")
    idx = sample_indices(N, seed=31 + offset)
    acc = buffer(N, offset)
    c0 = bf16_normal(N, offset, 1e-3, 301)
    c1 = bf16_normal(N, 1 - offset, 1e-3, 302)
    zs.grad_reduce_chunks(acc, [c0, c1, c0], True)
    ref = np.empty(idx.numel(), np.float32)
    s0, s1 = host(c0[idx]), host(c1[idx])
    for k, c in enumerate((s0, s1, s0)):
        oracle.grad_accum(ref, c, oracle.BF16, overwrite=(k == 0))
    check("acc", acc, idx, ref)
    del acc, c0, c1
    release()


@pytest.mark.parametrize("offset", [0, 1])
def test_flat_across_pieces(offset):
    """flat_pack (bf16 copy with padding; bf16 -> fp32 widening),
    flat_unpack (fp32 -> bf16 re-cast) and flat_apply_update (bf16
    tensors) with a tensor of N elements between two small ones: bit-exact
    on the sample, the padding zero."""
    need_gib(35)
    log(f"flat across pieces n={N} offset={offset}")
    sizes = [5, N, 7]
    T = sum(sizes)
    padded = T + 3
    idx = sample_indices(N, seed=41 + offset)
    ts = [bf16_normal(k, offset, 0.1, 401 + i) for i, k in enumerate(sizes)]
    fidx = idx + sizes[0]   # the big tensor's elements in the flat buffer

    log("  pack, bf16 copy")
    flat = buffer(padded, offset, torch.bfloat16)
    flat[-3:].fill_(1.0)
    zs.flat_pack(ts, flat, padded)
    check("pack", flat, fidx, host(ts[1][idx]))
    assert bits_equal(host(flat[:5]), host(ts[0])) and bits_equal(host(flat[T - 7:T]), host(ts[2]))
    assert not host(flat[T:]).any()
    del flat

    log("  pack, widening")
    flat32 = buffer(padded, offset)
    flat32[-3:].fill_(float("nan"))
    zs.flat_pack(ts, flat32, padded)
    check("widen", flat32, fidx, oracle.bf16_widen(host(ts[1][idx])))
    assert not host(flat32[T:]).view(np.uint32).any()

    log("  unpack, re-cast")
    fill_normal(flat32, 1.0, 402)
    outs = [buffer(k, 1 - offset, torch.bfloat16) for k in sizes]
    zs.flat_unpack(flat32[:T], outs)
    check("recast", outs[1], idx, oracle.bf16_rne(host(flat32[fidx])))
    assert bits_equal(host(outs[2]), oracle.bf16_rne(host(flat32[T - 7:T])))

    log("  apply, bf16 tensors")
    fill_normal(flat32, 1e-2, 403)
    before = host(ts[1][idx])
    upd = host(flat32[fidx])
    zs.flat_apply_update(flat32[:T], ts)
    ref = [before]
    oracle.flat_apply_update(upd, ref, oracle.BF16)
    check("apply", ts[1], idx, ref[0])
    del ts, flat32, outs
    release()


def test_adamw_scalar_path_past_2_to_32():
    """The scalar AdamW path (a view one element off: 256-thread workgroups,
    one element per work-item) over 2^32 + 5 elements, four piece boundaries
    and a ragged tail: bit-exact on the sample (about 77 GB of buffers)."""
    need_gib(85)
    n = (1 << 32) + 5
    log(f"adamw scalar path n={n} offset=1")
    idx = sample_indices(n, seed=51)
    master = fill_uniform(buffer(n, 1), -0.1, 0.1, 501)
    m = torch.zeros(n + 9, device=DEV)[1:n + 1]
    v = torch.zeros(n + 9, device=DEV)[1:n + 1]
    grad = fill_normal(buffer(n, 1), 1e-3, 502)
    bf16 = buffer(n, 1, torch.bfloat16)
    p_ref, g_s = host(master[idx]), host(grad[idx])
    m_ref, v_ref = np.zeros(idx.numel(), np.float32), np.zeros(idx.numel(), np.float32)
    b_ref = np.empty(idx.numel(), np.uint16)
    hp = zs.AdamWConfig(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_scale=1.0 / 64, step=1)
    zs.adamw_step(hp, master, m, v, grad, bf16)
    H = oracle.make_hp(3e-4, 0.9, 0.95, 1e-8, 0.1, 1.0 / 64, 0.0, 0.0, 1)
    assert oracle.adamw_step(H, p_ref, m_ref, v_ref, g_s, b_ref) == 0
    for name, gpu, ref in (("master", master, p_ref), ("m", m, m_ref), ("v", v, v_ref), ("bf16", bf16, b_ref)):
        check(name, gpu, idx, ref)
    del master, m, v, grad, bf16
    release()
