"""GPU parity of whole per-rank steps on the five workloads.

Each workload runs end to end through the library (accumulate every
micro-batch, form the norm, clip, AdamW with the bf16 re-cast; pack and
unpack for the FSDP unit) next to the oracle, step by step.  Inputs are
drawn on the GPU with seeded generators and copied to the host for the
oracle, so both sides consume the same bits; no oracle input comes from
the library's outputs.

Small cases compare every element.  At the real shard lengths, the bench's
launch configuration is compared element by element over the whole shard
(or fixed 1 GiB slices when the host lacks the memory; the test names the
mode), and longer or other configurations compare the squared norm over
the whole shard and the optimizer state on a sample of elements (the update
is element-wise, so the oracle steps the sampled elements alone), plus
every element of the FSDP unit.
"""
import math
import time

import numpy as np
import pytest
import torch

import oracle
import workloads
import fsdp_sharded_optimizer_amd as zs
from tests.parity import NORM_TOL, StateCheck, bits_equal, identical_fraction, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def log(msg):
    print(msg, flush=True)


def sample_indices(n: int, k: int = 1 << 20, seed: int = 0) -> torch.Tensor:
    """First and last 4096 elements, the neighbourhoods of a few workgroup
    tile edges, and k uniform random indices; sorted, unique."""
    rng = np.random.default_rng(seed)
    parts = [np.arange(min(n, 4096)), np.arange(max(0, n - 4096), n),
             rng.integers(0, n, size=min(k, n))]
    for edge in (2048, 4096, 8192 * 7, 1 << 20, (n // 2048) * 2048):
        parts.append(np.arange(max(0, edge - 9), min(n, edge + 9)))
    idx = np.unique(np.concatenate(parts))
    return torch.from_numpy(idx.astype(np.int64)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return to_np(t)


STATE_TILE = 8192   # ZS_STATE_TILE (test_abi checks the header against this value)


def run_shard(w: workloads.Workload, n: int, sampled: bool, full_norm: bool, fused=True,
              layout: str = "split"):
    """Drive the library and the oracle through w.steps steps of one shard.
    fused True: the last micro-batch forms the norm in the same pass
    (grad_accum_norm_sq); False: grad_accum for every micro-batch, then
    grad_norm_sq; "sum": the last micro-batch is not stored, its norm pass
    and AdamW read the accumulator and its gradient (grad_sum_norm_sq, then
    adamw_step_tiled_sum, bench.py's step, or adamw_step_sum on split
    state).  layout "tiled": the optimizer state in one tiled buffer and
    adamw_step_tiled; the compared elements are read at the positions the
    header's layout gives them."""
    one_pass = fused == "sum"
    master = workloads.master_init(w, n, DEV)
    param = master.to(torch.bfloat16) if w.bf16_param else None
    if layout == "tiled":
        state = torch.empty(zs.state_tiled_numel(n), dtype=torch.float32, device=DEV)
        zs.state_tile(master, None, None, state)
    else:
        exp_avg = torch.zeros(n, dtype=torch.float32, device=DEV)
        exp_avg_sq = torch.zeros(n, dtype=torch.float32, device=DEV)
    acc = torch.empty(n, dtype=torch.float32, device=DEV)
    norm = torch.zeros(1, dtype=torch.float64, device=DEV)
    ws = torch.empty(max(zs.grad_norm_sq_workspace_bytes(n), zs.grad_accum_norm_sq_workspace_bytes(n), 8),
                     dtype=torch.uint8, device=DEV)

    idx = sample_indices(n, seed=w.cfg) if sampled else None
    pick = (lambda t: t[idx]) if sampled else (lambda t: t)
    p_ref = host(pick(master))
    if layout == "tiled":
        e = idx if sampled else torch.arange(n, device=DEV)
        where = (e // STATE_TILE) * (3 * STATE_TILE) + e % STATE_TILE   # each element's master in the state
        state_at = lambda k: state[where + k * STATE_TILE]              # k = 0 master, 1 exp_avg, 2 exp_avg_sq
        del master
    else:
        state_at = lambda k: pick((master, exp_avg, exp_avg_sq)[k])
    m_ref = np.zeros(p_ref.size, np.float32)
    v_ref = np.zeros(p_ref.size, np.float32)
    b_ref = host(pick(param)) if param is not None else None
    acc_ref = np.empty(p_ref.size, np.float32)
    acc_full = np.empty(n, np.float32) if full_norm else None
    code = oracle.BF16 if w.grad_dtype == "bf16" else oracle.F32
    report = []
    last = w.micro_batches - 1
    for t in range(1, w.steps + 1):
        t0 = time.perf_counter()
        for mb in range(w.micro_batches):
            g = workloads.grad_draw(w, n, t, mb, DEV)
            if one_pass and mb == last:
                zs.grad_sum_norm_sq(acc if mb > 0 else None, g, mb == 0, w.grad_scale, norm, ws)
                g_last = g
                if mb > 0:   # the accumulator holds the earlier micro-batches' sum, bit for bit
                    assert bits_equal(host(pick(acc)), acc_ref), (t, "acc before the last")
            elif fused and mb == last:
                zs.grad_accum_norm_sq(acc, g, mb == 0, w.grad_scale, norm, ws)
            else:
                zs.grad_accum(acc, g, overwrite=(mb == 0))
            oracle.grad_accum(acc_ref, host(pick(g)), code, overwrite=(mb == 0))
            if full_norm:
                oracle.grad_accum(acc_full, host(g), code, overwrite=(mb == 0))
            del g
        if not fused:
            zs.grad_norm_sq(acc, w.grad_scale, norm, ws)
        s_gpu = float(norm.item())
        s_ref = oracle.grad_norm_sq(acc_full if full_norm else acc_ref, w.grad_scale) \
            if (full_norm or not sampled) else None
        if s_ref is not None:
            assert abs(math.sqrt(s_gpu) - math.sqrt(s_ref)) <= NORM_TOL * math.sqrt(s_ref), (t, s_gpu, s_ref)
        # the accumulated gradient itself is bit-exact (the one-pass step never stores it)
        if not one_pass:
            assert bits_equal(host(pick(acc)), acc_ref), (t, "acc")
        extra = workloads.other_ranks_norm_sq(w, t, n)
        hp = zs.AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                            weight_decay=w.weight_decay, grad_scale=w.grad_scale, max_norm=w.max_norm,
                            extra_norm_sq=extra, step=t)
        if one_pass and layout == "tiled":
            zs.adamw_step_tiled_sum(hp, state, acc if last > 0 else None, g_last, param, norm_sq=norm)
            del g_last
        elif one_pass:
            zs.adamw_step_sum(hp, master, exp_avg, exp_avg_sq, acc if last > 0 else None, g_last, param, norm_sq=norm)
            del g_last
        elif layout == "tiled":
            zs.adamw_step_tiled(hp, state, acc, param, norm_sq=norm)
        else:
            zs.adamw_step(hp, master, exp_avg, exp_avg_sq, acc, param, norm_sq=norm)
        ohp = oracle.make_hp(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, w.grad_scale, w.max_norm,
                             extra, t)
        prev = {"p": p_ref.copy(), "m": m_ref.copy()}
        clip_norm = s_ref if s_ref is not None else None
        if w.max_norm > 0:
            assert clip_norm is not None, "a clipped workload needs the oracle's own norm"
        assert oracle.adamw_step(ohp, p_ref, m_ref, v_ref, acc_ref, b_ref, norm_sq=clip_norm) == 0
        coef = oracle.clip_coef(clip_norm, extra, w.max_norm) if clip_norm is not None else 1.0
        g2 = (acc_ref * np.float32(w.grad_scale)) * np.float32(coef)
        gpu = {"p": host(state_at(0)), "m": host(state_at(1)), "v": host(state_at(2)),
               "b": host(pick(param)) if param is not None else None}
        s = oracle.adamw_scalars(ohp)
        res = StateCheck(w.beta1, w.lr, w.weight_decay, s.step_size).check(
            gpu, {"p": p_ref, "m": m_ref, "v": v_ref, "b": b_ref}, prev, g2, f"{w.name} t={t}")
        # the two sides run the same IEEE operations: with the same fp32 clip
        # coefficient (the norms differ only in their last bits), every
        # compared element is bit-identical, beyond the tolerance above
        coef_gpu = oracle.clip_coef(s_gpu, extra, w.max_norm) if clip_norm is not None else 1.0
        if np.float32(coef_gpu) == np.float32(coef):
            for k, ref_arr in (("p", p_ref), ("m", m_ref), ("v", v_ref), ("b", b_ref)):
                if ref_arr is not None:
                    assert bits_equal(gpu[k], ref_arr), (w.name, t, k, identical_fraction(gpu[k], ref_arr))
        res.update(step=t, coef=coef, norm=math.sqrt(s_gpu + extra), secs=round(time.perf_counter() - t0, 1))
        log(f"  {w.name} n={n} {layout} {res}")
        report.append(res)
    return report


# ---------------------------------------------------------------------------
# small sizes: every element
# ---------------------------------------------------------------------------

SMALL = [("llama7b_shard", 1_000_037), ("llama13b_shard_clip", 600_011), ("zero3_70b_shard", 2_000_003)]


@pytest.mark.parametrize("name,n,fused,layout",
                         [(w, n, f, lay) for w, n in SMALL for f in (True, False, "sum") for lay in ("split", "tiled")])
def test_workload_small(name, n, fused, layout):
    """Every element, at a reduced shard length.  The gradient std is scaled
    by sqrt(full/n) so the global norm, and with it the clipping pattern of
    the 13B workload, is the one of the full shard."""
    from dataclasses import replace
    w = workloads.WORKLOADS[name]
    _, start, end, _ = zs.zero_shard_range(w.total, w.world, w.rank)
    w = replace(w, grad_std=w.grad_std * math.sqrt((end - start) / n))
    log(f"workload {name} small n={n} {layout}")
    rep = run_shard(w, n, sampled=False, full_norm=False, fused=fused, layout=layout)
    if name == "llama13b_shard_clip":
        clipped = [r["step"] for r in rep if r["coef"] < 1.0]
        assert clipped == [2, 5, 8], clipped
    if name == "zero3_70b_shard":
        assert all(r["coef"] < 1.0 for r in rep)


def test_tiny_zero1_rank3_view():
    """The ZeRO-1 workload: rank 3's shard is a view into the flat fp32
    parameter and gradient buffers (element offset 375,003: not 16-byte
    aligned), moments are this rank's own buffers; 5 steps of Adam.
    Everything outside the shard must stay bit-identical."""
    w = workloads.WORKLOADS["tiny_zero1"]
    chunk, start, end, padded = zs.zero_shard_range(w.total, w.world, w.rank)
    assert (chunk, start, end, padded) == oracle.shard_range(w.total, w.world, w.rank)
    n = end - start
    flat_p = torch.zeros(padded, dtype=torch.float32, device=DEV)
    flat_p[:w.total] = workloads.master_init(w, w.total, DEV)
    flat_g = torch.zeros(padded, dtype=torch.float32, device=DEV)
    p_all0 = host(flat_p)
    p_ref = p_all0[start:end].copy()
    m = torch.zeros(n, dtype=torch.float32, device=DEV)
    v = torch.zeros(n, dtype=torch.float32, device=DEV)
    m_ref, v_ref = np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in range(1, w.steps + 1):
        flat_g[:w.total] = workloads.grad_draw(w, w.total, t, 0, DEV)
        g_ref = host(flat_g)[start:end]
        hp = zs.AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=0.0,
                            grad_scale=w.grad_scale, step=t)
        zs.adamw_step(hp, flat_p[start:end], m, v, flat_g[start:end])
        ohp = oracle.make_hp(w.lr, w.beta1, w.beta2, w.eps, 0.0, w.grad_scale, 0.0, 0.0, t)
        prev = {"p": p_ref.copy(), "m": m_ref.copy()}
        oracle.adamw_step(ohp, p_ref, m_ref, v_ref, g_ref)
        p_all = host(flat_p)
        res = StateCheck(w.beta1, w.lr, 0.0, 0.0).check(
            {"p": p_all[start:end], "m": host(m), "v": host(v)}, {"p": p_ref, "m": m_ref, "v": v_ref},
            prev, g_ref * np.float32(w.grad_scale), f"tiny t={t}")
        log(f"  tiny_zero1 {res}")
        assert bits_equal(p_all[start:end], p_ref) and bits_equal(host(m), m_ref) and bits_equal(host(v), v_ref)
        assert bits_equal(p_all[:start], p_all0[:start]) and bits_equal(p_all[end:], p_all0[end:])
    assert not host(flat_p)[w.total:].any()


def _unit(w, shapes):
    """The FSDP unit flow for one rank: pack the unit, widen the rank's
    range into the fp32 master, accumulate its bf16 gradient, AdamW with the
    bf16 re-cast written back into the flat buffer, unpack.  Returns the
    GPU results and the oracle's."""
    total = sum(workloads.numel_of(s) for _, s in shapes)
    chunk, start, end, padded = zs.zero_shard_range(total, w.world, w.rank)
    assert (chunk, start, end, padded) == oracle.shard_range(total, w.world, w.rank)
    n = end - start
    wu = workloads.replace_unit(w, shapes)
    params = workloads.unit_tensors(wu, DEV)
    params_ref = [host(p) for p in params]
    flat = torch.empty(padded, dtype=torch.bfloat16, device=DEV)
    zs.flat_pack(params, flat, padded)
    flat_ref = oracle.flat_pack(params_ref, oracle.BF16, oracle.BF16, padded)
    assert bits_equal(host(flat), flat_ref), "flat_pack"
    master = torch.empty(n, dtype=torch.float32, device=DEV)
    zs.flat_pack([flat[start:end]], master, n)
    master_ref = oracle.flat_pack([flat_ref[start:end]], oracle.BF16, oracle.F32, n)
    assert bits_equal(host(master), master_ref), "widen"
    g = workloads.grad_draw(w, n, 1, 0, DEV)
    acc = torch.empty(n, dtype=torch.float32, device=DEV)
    zs.grad_accum(acc, g, overwrite=True)
    acc_ref = np.empty(n, np.float32)
    oracle.grad_accum(acc_ref, host(g), oracle.BF16, overwrite=True)
    m = torch.zeros(n, dtype=torch.float32, device=DEV)
    v = torch.zeros(n, dtype=torch.float32, device=DEV)
    m_ref, v_ref = np.zeros(n, np.float32), np.zeros(n, np.float32)
    hp = zs.AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                        grad_scale=w.grad_scale, step=1)
    zs.adamw_step(hp, master, m, v, acc, flat[start:end])
    ohp = oracle.make_hp(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, w.grad_scale, 0.0, 0.0, 1)
    prev = {"p": master_ref.copy(), "m": m_ref.copy()}
    b_ref = flat_ref[start:end]            # a view: the oracle writes its bf16 into its flat buffer
    oracle.adamw_step(ohp, master_ref, m_ref, v_ref, acc_ref, b_ref)
    res = StateCheck(w.beta1, w.lr, w.weight_decay, 0.0).check(
        {"p": host(master), "m": host(m), "v": host(v), "b": host(flat[start:end])},
        {"p": master_ref, "m": m_ref, "v": v_ref, "b": b_ref}, prev, acc_ref * np.float32(w.grad_scale),
        "unit")
    for got, want in ((master, master_ref), (m, m_ref), (v, v_ref), (flat[start:end], b_ref)):
        assert bits_equal(host(got), want), "unit step not bit-identical"
    outs = [torch.empty_like(p) for p in params]
    zs.flat_unpack(flat, outs)
    outs_ref = oracle.flat_unpack(flat_ref, oracle.BF16, [p.size for p in params_ref], oracle.BF16)
    return params_ref, outs, outs_ref, (start, end), res


def _check_unit(shapes, params_ref, outs, outs_ref, rng):
    """Outside the rank's range every element is bit-identical to the input;
    inside it is the oracle's re-cast (<= 1 bf16 ulp; bit-identical
    fraction reported)."""
    start, end = rng
    off = 0
    same = 0
    for s, p0, o, r in zip(shapes, params_ref, outs, outs_ref):
        o = host(o).reshape(-1)
        k = o.size
        lo, hi = max(start - off, 0), min(end - off, k)
        inside = np.zeros(k, bool)
        if lo < hi:
            inside[lo:hi] = True
        assert np.array_equal(o[~inside], p0.reshape(-1)[~inside]), f"outside the shard changed in {s}"
        if inside.any():
            d = np.abs(o[inside].astype(np.int32) - r[inside].astype(np.int32))
            assert d.max() <= 1
            same += int((d == 0).sum())
        off += k
    return same / max(end - start, 1)


def test_fsdp_unit_scaled_block():
    """The 70B-style block with every dimension divided by 16 (same tensor
    order, world 64, rank 17), every element compared."""
    w = workloads.WORKLOADS["fsdp_unit_70b_block"]
    shapes = workloads.block70b_tensor_shapes(hidden=512, ffn=1792, q_heads=64, kv_heads=8, head_dim=8)
    params_ref, outs, outs_ref, rng, res = _unit(w, shapes)
    frac = _check_unit(shapes, params_ref, outs, outs_ref, rng)
    log(f"  unit (scaled) {res} bf16 identical {frac:.6f}")


# ---------------------------------------------------------------------------
# full sizes (the real shard lengths)
# ---------------------------------------------------------------------------

def test_full_fsdp_unit_70b_block():
    w = workloads.WORKLOADS["fsdp_unit_70b_block"]
    log("full fsdp unit 70b block: 855,654,400 elements, world 64, rank 17")
    params_ref, outs, outs_ref, rng, res = _unit(w, list(w.unit_shapes))
    assert rng == (227_283_200, 240_652_800)
    frac = _check_unit(list(w.unit_shapes), params_ref, outs, outs_ref, rng)
    log(f"  unit {res} bf16 identical {frac:.6f}")


@pytest.mark.parametrize("name,full_norm,fused,layout", [
    ("llama7b_shard", True, True, "split"), ("zero3_70b_shard", True, False, "tiled"),
    ("llama13b_shard_clip", True, True, "tiled")])
def test_full_shard(name, full_norm, fused, layout):
    """The real shard lengths in the configurations the every-element test
    below does not run: the 7B shard on split buffers, the 70B shard with
    the norm as its own pass, and all ten steps of the 13B workload (its
    clip pattern, steps 2, 5 and 8); the norm over the whole shard, the
    optimizer state on sampled elements."""
    w = workloads.WORKLOADS[name]
    _, start, end, _ = zs.zero_shard_range(w.total, w.world, w.rank)
    n = end - start
    log(f"full {name} ({layout}): shard of {n} elements, {w.steps} steps x {w.micro_batches} micro-batches")
    rep = run_shard(w, n, sampled=True, full_norm=full_norm, fused=fused, layout=layout)
    if name == "llama13b_shard_clip":
        assert [r["step"] for r in rep if r["coef"] < 1.0] == [2, 5, 8]
    if name == "zero3_70b_shard":
        assert all(0.70 < r["coef"] < 0.76 for r in rep), rep
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# full sizes, every element (or fixed 1 GiB slices when the host is short of
# memory): the bench's launch configuration against the oracle holding the
# same state
# ---------------------------------------------------------------------------

CMP_CHUNK = 1 << 26         # elements per comparison chunk: 256 MiB of fp32
SLICE = 1 << 28             # a 1 GiB slice of fp32 state


def _host_mem_available() -> int:
    with open("/proc/meminfo") as f:
        for line in f:
            if line.startswith("MemAvailable:"):
                return int(line.split()[1]) * 1024
    return 0


def _tiled_chunk(state: torch.Tensor, c0: int, c1: int, k: int) -> np.ndarray:
    """Elements [c0, c1) (c0 a multiple of the tile) of run k (0 master, 1
    exp_avg, 2 exp_avg_sq) of a tiled state, copied to the host."""
    t0, t1 = c0 // STATE_TILE, (c1 + STATE_TILE - 1) // STATE_TILE
    blk = state[3 * STATE_TILE * t0:3 * STATE_TILE * t1].view(t1 - t0, 3, STATE_TILE)
    return host(blk[:, k, :].reshape(-1)[:c1 - c0])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,steps", [("llama7b_shard", 3), ("zero3_70b_shard", 2), ("llama13b_shard_clip", 2)])
def test_full_shard_every_element(name, steps):
    """The real shard lengths through the bench's launch configuration
    (grad_accum per micro-batch but the last; for the last, grad_sum_norm_sq
    and adamw_step_tiled_sum with the bf16 re-cast, clipped where the
    workload clips, the sum never stored) next to the oracle stepping the
    same state from the same inputs (accumulating every micro-batch, then
    its norm and AdamW).  Every step compares, element by element: the
    accumulator before the last micro-batch (bit-exact, whole shard), the
    squared norm over the whole shard (1e-5), and the
    master, exp_avg, exp_avg_sq and bf16 parameter of the compared ranges,
    read back in 256 MiB chunks.  Mode "full": the compared range is the
    whole shard; mode "slices" (when the host lacks the memory for the
    oracle's full state): the first, middle and last 1 GiB of state, exact
    by the update's element-wise independence (Memory page, 一、显存账本).
    Where the GPU's fp32 clip coefficient equals the oracle's (always, unless
    the two norms straddle a rounding boundary of it), every compared element
    must be bit-identical; otherwise the 2e-6 / 1-ulp bar applies."""
    w = workloads.WORKLOADS[name]
    _, start, end, _ = zs.zero_shard_range(w.total, w.world, w.rank)
    n = end - start
    # the oracle's accumulator, master, exp_avg, exp_avg_sq and bf16 parameter,
    # one gradient draw, and room for the chunks in flight
    need = n * (4 * 4 + 2 + (2 if w.grad_dtype == "bf16" else 4)) + (4 << 30)
    mode = "full" if _host_mem_available() > 1.5 * need else "slices"
    if mode == "full":
        ranges = [(0, n)]
    else:
        mid = (n // 2 // STATE_TILE) * STATE_TILE
        ranges = [(0, SLICE), (mid, mid + SLICE), (n - n % STATE_TILE - SLICE, n)]
    log(f"full {name} every element: n={n}, {steps} steps x {w.micro_batches} micro-batches, mode={mode}, "
        f"compared elements per step {sum(b - a for a, b in ranges)}")

    master = workloads.master_init(w, n, DEV)
    param = master.to(torch.bfloat16)
    state = torch.empty(zs.state_tiled_numel(n), dtype=torch.float32, device=DEV)
    zs.state_tile(master, None, None, state)
    ref = []
    for a, b in ranges:
        ref.append({"p": host(master[a:b]), "m": np.zeros(b - a, np.float32), "v": np.zeros(b - a, np.float32),
                    "b": host(param[a:b])})
    del master
    acc = torch.empty(n, dtype=torch.float32, device=DEV)
    norm = torch.zeros(1, dtype=torch.float64, device=DEV)
    ws = torch.empty(max(zs.grad_accum_norm_sq_workspace_bytes(n), 8), dtype=torch.uint8, device=DEV)
    acc_ref = np.empty(n, np.float32)
    code = oracle.BF16 if w.grad_dtype == "bf16" else oracle.F32
    last = w.micro_batches - 1
    for t in range(1, steps + 1):
        t0 = time.perf_counter()
        for mb in range(w.micro_batches):
            g = workloads.grad_draw(w, n, t, mb, DEV)
            if mb == last:
                if mb > 0:   # the accumulator before the last micro-batch, bit-exact
                    for c0 in range(0, n, CMP_CHUNK):
                        c1 = min(c0 + CMP_CHUNK, n)
                        assert bits_equal(host(acc[c0:c1]), acc_ref[c0:c1]), (t, "acc", c0)
                zs.grad_sum_norm_sq(acc if mb > 0 else None, g, mb == 0, w.grad_scale, norm, ws)
                g_last = g
            else:
                zs.grad_accum(acc, g, overwrite=(mb == 0))
            oracle.grad_accum(acc_ref, host(g), code, overwrite=(mb == 0))
            del g
        s_gpu = float(norm.item())
        s_ref = oracle.grad_norm_sq(acc_ref, w.grad_scale)
        assert abs(math.sqrt(s_gpu) - math.sqrt(s_ref)) <= NORM_TOL * math.sqrt(s_ref), (t, s_gpu, s_ref)
        extra = workloads.other_ranks_norm_sq(w, t, n)
        hp = zs.AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                            grad_scale=w.grad_scale, max_norm=w.max_norm, extra_norm_sq=extra, step=t)
        zs.adamw_step_tiled_sum(hp, state, acc if last > 0 else None, g_last, param, norm_sq=norm)
        del g_last
        ohp = oracle.make_hp(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, w.grad_scale, w.max_norm, extra, t)
        coef_gpu = oracle.clip_coef(s_gpu, extra, w.max_norm)
        coef = oracle.clip_coef(s_ref, extra, w.max_norm)
        same_coef = np.float32(coef_gpu) == np.float32(coef)
        checker = StateCheck(w.beta1, w.lr, w.weight_decay, 0.0)
        compared = identical = 0
        for (a, b), r in zip(ranges, ref):
            # the state before the step: only the tolerance path needs it
            prev = None if same_coef else {"p": r["p"].copy(), "m": r["m"].copy()}
            assert oracle.adamw_step(ohp, r["p"], r["m"], r["v"], np.ascontiguousarray(acc_ref[a:b]), r["b"],
                                     norm_sq=s_ref) == 0
            for c0 in range(a, b, CMP_CHUNK):
                c1 = min(c0 + CMP_CHUNK, b)
                lo, hi = c0 - a, c1 - a
                gpu = {"p": _tiled_chunk(state, c0, c1, 0), "m": _tiled_chunk(state, c0, c1, 1),
                       "v": _tiled_chunk(state, c0, c1, 2), "b": host(param[c0:c1])}
                orc = {k: r[k][lo:hi] for k in ("p", "m", "v", "b")}
                same = all(bits_equal(gpu[k], orc[k]) for k in ("p", "m", "v", "b"))
                if not same:
                    assert not same_coef, (t, c0, "not bit-identical although the clip coefficients agree")
                    g2 = (acc_ref[c0:c1] * np.float32(w.grad_scale)) * np.float32(coef)
                    checker.check(gpu, orc, {"p": prev["p"][lo:hi], "m": prev["m"][lo:hi]}, g2, f"{name} t={t}")
                compared += c1 - c0
                identical += (c1 - c0) if same else 0
        log(f"  {name} t={t} mode={mode} compared={compared} bit-identical={identical} coef={coef:.6f} "
            f"norm={math.sqrt(s_gpu + extra):.6f} secs={time.perf_counter() - t0:.1f}")
    del state, acc, param, acc_ref, ref
    torch.cuda.empty_cache()


def test_tiny_zero1_full_flow():
    """The ZeRO page's ZeRO-1 flow for the 1,000,003-parameter model over 8
    ranks, every rank's share run on this GPU: flatten the model's fp32
    grads (padded to 8 x 125,001), each rank's Adam update on its slice of
    the resident flat gradient (odd ranks' slices and chunks start at
    misaligned offsets) written into its chunk of the gathered buffer, then
    the apply into the 12 parameter tensors.  Five steps, bit-identical to
    the oracle running the same flow; the gathered buffer's padding is NaN
    and never reaches a parameter."""
    w = workloads.WORKLOADS["tiny_zero1"]
    T, N = w.total, w.world
    chunk, _, _, padded = zs.zero_shard_range(T, N, 0)
    ranges = [zs.zero_shard_range(T, N, r)[1:3] for r in range(N)]
    params = [p.cuda() for p in workloads.param_tensors(w)]
    p_ref = [p.numpy().reshape(-1).copy() for p in workloads.param_tensors(w)]
    m = [torch.zeros(chunk, device="cuda") for _ in range(N)]
    v = [torch.zeros(chunk, device="cuda") for _ in range(N)]
    m_ref = [np.zeros(chunk, np.float32) for _ in range(N)]
    v_ref = [np.zeros(chunk, np.float32) for _ in range(N)]
    flat = torch.empty(padded, device="cuda")
    gathered = torch.empty(padded, device="cuda")
    for t in range(1, w.steps + 1):
        log(f"  tiny_zero1 flow step {t}")
        grads = workloads.grad_tensors(w, t)
        hp = zs.AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=0.0,
                            grad_scale=w.grad_scale, step=t)
        hp_orc = oracle.make_hp(w.lr, w.beta1, w.beta2, w.eps, 0.0, w.grad_scale, 0.0, 0.0, t)
        zs.flat_pack([g.cuda() for g in grads], flat, padded)
        gathered.fill_(float("nan"))
        for r, (s, e) in enumerate(ranges):
            k = e - s
            zs.adam_update(hp, m[r][:k], v[r][:k], flat[s:e], gathered[r * chunk:r * chunk + k])
        zs.flat_apply_update(gathered, params)
        # the oracle runs the same flow
        flat_ref = oracle.flat_pack([g.numpy().reshape(-1) for g in grads], oracle.F32, oracle.F32, padded)
        g_ref = np.full(padded, np.nan, np.float32)
        for r, (s, e) in enumerate(ranges):
            k = e - s
            mm, vv, uu = m_ref[r][:k].copy(), v_ref[r][:k].copy(), np.empty(k, np.float32)
            oracle.adam_update(hp_orc, mm, vv, np.ascontiguousarray(flat_ref[s:e]), uu)
            m_ref[r][:k], v_ref[r][:k] = mm, vv
            g_ref[r * chunk:r * chunk + k] = uu
        oracle.flat_apply_update(g_ref, p_ref, oracle.F32)
        torch.cuda.synchronize()
        assert bits_equal(to_np(flat)[:T], flat_ref[:T])
        assert bits_equal(to_np(gathered), g_ref)
        for i, (a, b) in enumerate(zip(params, p_ref)):
            assert bits_equal(to_np(a).reshape(-1), b), (t, i)
        for r in range(N):
            assert bits_equal(to_np(m[r]), m_ref[r]) and bits_equal(to_np(v[r]), v_ref[r]), (t, r)
    assert all(bool(torch.isfinite(p).all()) for p in params)


def test_zero1_flow_llama7b_sampled():
    """The ZeRO-1 flow at the Llama-7B size in bench.py's launch configuration:
    adam_update on rank 0's 842,301,952-element slice (two steps, the second
    clipped) and flat_apply_update of a 6,738,415,616-element update into the
    291 bf16 parameter tensors.  Both are element-wise, so the oracle runs the
    sampled elements alone (first and last 4096, tile edges, 2^20 random)."""
    w = workloads.WORKLOADS["llama7b_shard"]
    chunk, start, end, padded = zs.zero_shard_range(w.total, w.world, w.rank)
    n = end - start
    gen = torch.Generator(device=DEV)
    gen.manual_seed(workloads.seed_of(w.cfg, workloads.PURPOSE_GRAD, 9, 0))
    idx = sample_indices(n, seed=1)
    grad = torch.randn(n, generator=gen, device=DEV).mul_(1e-3 / 8)
    m = torch.zeros(n, device=DEV)
    v = torch.zeros(n, device=DEV)
    upd = torch.empty(n, device=DEV)
    m_ref, v_ref = np.zeros(idx.numel(), np.float32), np.zeros(idx.numel(), np.float32)
    for t in (1, 2):
        clip = t == 2
        norm = None
        hp = zs.AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=0.0,
                            grad_scale=1.0 / w.world, max_norm=1.0 if clip else 0.0, extra_norm_sq=3.0, step=t)
        S = 0.0
        if clip:   # the oracle's norm over the whole slice feeds both sides; the GPU's is checked against it
            S = oracle.grad_norm_sq(host(grad), 1.0 / w.world)
            gpu_norm = torch.zeros(1, dtype=torch.float64, device=DEV)
            zs.grad_norm_sq(grad, 1.0 / w.world, gpu_norm)
            assert abs(math.sqrt(gpu_norm.item()) - math.sqrt(S)) <= NORM_TOL * math.sqrt(S)
            norm = torch.tensor([S], dtype=torch.float64, device=DEV)
        log(f"  zero1 7B adam_update step {t} clip={clip}")
        zs.adam_update(hp, m, v, grad, upd, norm_sq=norm)
        g_s = host(grad[idx])
        u_ref = np.empty(idx.numel(), np.float32)
        H = oracle.make_hp(w.lr, w.beta1, w.beta2, w.eps, 0.0, 1.0 / w.world, hp.max_norm, 3.0, t)
        if clip:
            assert oracle.clip_coef(S, 3.0, 1.0) < 0.9   # the second step clips
        assert oracle.adam_update(H, m_ref, v_ref, g_s, u_ref, norm_sq=S if clip else None) == 0
        for name, gpu, ref in (("update", upd, u_ref), ("m", m, m_ref), ("v", v, v_ref)):
            got = host(gpu[idx])
            assert bits_equal(got, ref), (t, name, identical_fraction(got, ref))
    del grad, m, v, upd
    torch.cuda.empty_cache()

    log("  zero1 7B flat_apply_update over 291 tensors")
    gathered = torch.randn(padded, generator=gen, device=DEV).mul_(1e-4)
    buf = torch.rand(w.total, generator=gen, device=DEV).mul_(0.2).sub_(0.1).to(torch.bfloat16)
    params, off = [], 0
    for _, shp in workloads.LLAMA7B:
        k = workloads.numel_of(shp)
        params.append(buf[off:off + k].view(shp))
        off += k
    pidx = sample_indices(w.total, seed=2)
    before = host(buf[pidx]).copy()
    u_s = host(gathered[pidx])
    zs.flat_apply_update(gathered, params)
    torch.cuda.synchronize()
    oracle.flat_apply_update(u_s, [before], oracle.BF16)   # element-wise: the samples as one tensor
    got = host(buf[pidx])
    assert bits_equal(got, before), identical_fraction(got, before)


def test_reduce_chunks_and_no_master_full_size_sampled():
    """The two entry points bench.py times after the step, at the Llama-7B
    shard size in the same launch configuration: grad_reduce_chunks over the
    8 bf16 micro-batch draws (overwrite), then adamw_step_no_master on the
    bf16 shard with that sum as its gradient, two steps.  Element-wise, so
    the oracle runs the sampled elements alone."""
    w = workloads.WORKLOADS["llama7b_shard"]
    _, start, end, _ = zs.zero_shard_range(w.total, w.world, w.rank)
    n = end - start
    idx = sample_indices(n, seed=3)
    grads = [workloads.grad_draw(w, n, 1, mb, DEV) for mb in range(w.micro_batches)]
    acc = torch.empty(n, device=DEV)
    log("  7B grad_reduce_chunks, 8 bf16 chunks")
    zs.grad_reduce_chunks(acc, grads, True)
    acc_ref = np.empty(idx.numel(), np.float32)
    for k, g in enumerate(grads):
        oracle.grad_accum(acc_ref, host(g[idx]), oracle.BF16, overwrite=(k == 0))
    got = host(acc[idx])
    assert bits_equal(got, acc_ref), identical_fraction(got, acc_ref)
    del grads
    torch.cuda.empty_cache()

    param = workloads.master_init(w, n, DEV).to(torch.bfloat16)
    m = torch.zeros(n, device=DEV)
    v = torch.zeros(n, device=DEV)
    b_ref = host(param[idx])
    m_ref, v_ref = np.zeros(idx.numel(), np.float32), np.zeros(idx.numel(), np.float32)
    for t in (1, 2):
        log(f"  7B adamw_step_no_master step {t}")
        hp = zs.AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                            grad_scale=w.grad_scale, step=t)
        zs.adamw_step_no_master(hp, param, m, v, acc)
        H = oracle.make_hp(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, w.grad_scale, 0.0, 0.0, t)
        assert oracle.adamw_step_no_master(H, b_ref, m_ref, v_ref, acc_ref) == 0
        for name, gpu, ref in (("b", param, b_ref), ("m", m, m_ref), ("v", v, v_ref)):
            got = host(gpu[idx])
            assert bits_equal(got, ref), (t, name, identical_fraction(got, ref))


def test_full_unit_conversions_every_element():
    """The two conversions bench.py times on the 70B block unit, at full
    size and in the same launch configuration: the widening pack of the 9
    bf16 tensors (855,654,400 elements) into an fp32 flat buffer, and the
    re-casting unpack of an fp32 flat buffer of arbitrary values back into
    bf16 tensors; every element against the oracle."""
    w = workloads.WORKLOADS["fsdp_unit_70b_block"]
    params = workloads.unit_tensors(w, DEV)
    sizes = [p.numel() for p in params]
    total = sum(sizes)
    log(f"  unit widening pack: {total} elements")
    flat32 = torch.full((total,), float("nan"), device=DEV)
    zs.flat_pack(params, flat32, total)
    params_ref = [host(p).reshape(-1) for p in params]
    want = oracle.flat_pack(params_ref, oracle.BF16, oracle.F32, total)
    assert bits_equal(host(flat32), want)
    del want
    log("  unit re-casting unpack")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(workloads.seed_of(w.cfg, workloads.PURPOSE_GRAD, 7, 0))
    flat32.normal_(0.0, 0.05, generator=gen)      # arbitrary fp32 values: the re-cast must round
    outs = [torch.empty_like(p) for p in params]
    zs.flat_unpack(flat32, outs)
    back = oracle.flat_unpack(host(flat32), oracle.F32, sizes, oracle.BF16)
    for i, (o, r) in enumerate(zip(outs, back)):
        assert bits_equal(host(o).reshape(-1), r), i
    del params, outs, flat32, back
    torch.cuda.empty_cache()


def test_full_size_fp32_gradient_paths():
    """fp32 gradients (a reduce-scatter's fp32 output) at the Llama-7B shard
    size: the overwriting fused accumulation with the norm (one group per
    lane, uncapped) and the two-chunk fp32 reduction (its own residency
    cap); the accumulator on a sample, the norm over the whole shard."""
    w = workloads.WORKLOADS["llama7b_shard"]
    _, start, end, _ = zs.zero_shard_range(w.total, w.world, w.rank)
    n = end - start
    idx = sample_indices(n, seed=5)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(workloads.seed_of(w.cfg, workloads.PURPOSE_GRAD, 8, 0))
    c0 = torch.randn(n, generator=gen, device=DEV).mul_(1e-3)
    c1 = torch.randn(n, generator=gen, device=DEV).mul_(1e-3)
    acc = torch.empty(n, device=DEV)
    norm = torch.zeros(1, dtype=torch.float64, device=DEV)
    log("  7B fp32 overwrite + norm")
    zs.grad_accum_norm_sq(acc, c0, True, w.grad_scale, norm)
    c0_host = host(c0)
    S = oracle.grad_norm_sq(c0_host, w.grad_scale)
    assert abs(math.sqrt(norm.item()) - math.sqrt(S)) <= NORM_TOL * math.sqrt(S)
    assert bits_equal(host(acc[idx]), c0_host[host(idx)])
    del c0_host
    log("  7B fp32 reduce, two chunks")
    zs.grad_reduce_chunks(acc, [c0, c1], True)
    ref = np.empty(idx.numel(), np.float32)
    oracle.grad_accum(ref, host(c0[idx]), oracle.F32, overwrite=True)
    oracle.grad_accum(ref, host(c1[idx]), oracle.F32, overwrite=False)
    got = host(acc[idx])
    assert bits_equal(got, ref), identical_fraction(got, ref)
    del c0, c1, acc
    torch.cuda.empty_cache()
