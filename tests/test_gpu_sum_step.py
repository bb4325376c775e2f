"""GPU parity of the step that folds the last micro-batch into AdamW.

grad_sum_norm_sq forms the squared norm of the last micro-batch's sum
without storing it, and adamw_step_tiled_sum steps the tiled state on that
sum, formed again as it is read.  Against the oracle: the norm within the bar
of the oracle's norm of its accumulated gradient; handed the oracle's norm,
the state and bf16 output bit-identical to the oracle's accumulate-then-step.
Against the library's own two-call path: the norm bit for bit that of
grad_accum_norm_sq (same association), the state and output bit for bit
those of grad_accum then adamw_step_tiled, and the accumulator untouched.
Sizes span several tiles and the norm's partial blocks with ragged ends;
offsets put the gradient off 4-byte (bf16, the element-wise path) and
16-byte boundaries and the bf16 output off 16 bytes.  Every buffer carries a
canary tail.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import fsdp_sharded_optimizer_amd as zs
from tests.parity import bits_equal, identical_fraction, to_np
from tests.test_gpu_kernels import NORM_TOL, _hp, canary_ok, dev_buf

pytestmark = pytest.mark.gpu

T = 8192   # ZS_STATE_TILE
SIZES = [1, 3, 255, 256, 257, 1023, 1024, 1025, 8193, 100_003, 1_000_037]


def _grad(rng, n, dtype):
    g32 = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    return oracle.bf16_rne(g32) if dtype == "bf16" else g32


def _code(dtype):
    return oracle.BF16 if dtype == "bf16" else oracle.F32


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("overwrite", [False, True])
@pytest.mark.parametrize("acc_off,grad_off", [(0, 0), (1, 1), (3, 2)])
def test_grad_sum_norm_sq(n, dtype, overwrite, acc_off, grad_off):
    """The norm of the last micro-batch's sum: within the bar of the
    oracle's, bit for bit grad_accum_norm_sq's, and the accumulator (and the
    gradient) left as they were."""
    print(f"grad_sum_norm_sq n={n} dtype={dtype} overwrite={overwrite} offsets={acc_off},{grad_off}", flush=True)
    rng = np.random.default_rng(n * 11 + acc_off * 3 + grad_off + 7 * overwrite)
    acc0 = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    g = _grad(rng, n, dtype)
    scale = 1.0 / 16
    ref = acc0.copy()
    oracle.grad_accum(ref, g, _code(dtype), overwrite=overwrite)
    want = oracle.grad_norm_sq(ref, scale)
    acc, acc_whole = dev_buf(acc0, acc_off)
    gd, g_whole = dev_buf(g, grad_off, bf16=(dtype == "bf16"))
    out = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    zs.grad_sum_norm_sq(acc, gd, overwrite, scale, out)
    got = out.item()
    assert abs(math.sqrt(got) - math.sqrt(want)) <= NORM_TOL * math.sqrt(want)
    assert bits_equal(to_np(acc), acc0), "the accumulator was written"
    assert canary_ok(acc_whole, acc_off, n) and canary_ok(g_whole, grad_off, n)
    # the fused pass that stores the sum forms the same bits
    acc2, _ = dev_buf(acc0, 0)
    out2 = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    zs.grad_accum_norm_sq(acc2, gd, overwrite, scale, out2)
    assert out2.item() == got
    assert bits_equal(to_np(acc2), ref)


def test_grad_sum_norm_sq_overwrite_reads_no_accumulator_and_empty():
    n = 70_001
    rng = np.random.default_rng(5)
    g = _grad(rng, n, "bf16")
    gd, _ = dev_buf(g, 0, bf16=True)
    out = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    zs.grad_sum_norm_sq(None, gd, True, 1.0 / 8, out)
    ref = np.empty(n, np.float32)
    oracle.grad_accum(ref, g, oracle.BF16, overwrite=True)
    want = oracle.grad_norm_sq(ref, 1.0 / 8)
    assert abs(math.sqrt(out.item()) - math.sqrt(want)) <= NORM_TOL * math.sqrt(want)
    e = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    zs.grad_sum_norm_sq(None, e, True, 1.0, out)
    assert out.item() == 0.0
    # closed form: 2^23 + 3 elements of 2^-7 onto an accumulator of 2^-7, at
    # scale 1/8: every sum is 2^-6, the norm exactly (2^23 + 3) * 2^-18
    n = (1 << 23) + 3
    acc = torch.full((n,), 2.0**-7, dtype=torch.float32, device="cuda")
    gb = torch.full((n,), 2.0**-7, dtype=torch.bfloat16, device="cuda")
    zs.grad_sum_norm_sq(acc, gb, False, 1.0 / 8, out)
    assert out.item() == n * 2.0**-18
    assert torch.all(acc == 2.0**-7)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("with_acc", [True, False])
@pytest.mark.parametrize("grad_off,b_off", [(0, 0), (1, 1), (2, 3)])
def test_adamw_step_tiled_sum_bit_exact(n, dtype, with_acc, grad_off, b_off):
    """Three steps, each on the sum of an accumulator and a last
    micro-batch (or the micro-batch alone).  Handed the oracle's norm, the
    tiled state and the bf16 output equal the oracle's accumulate-then-step
    bit for bit.  With the GPU's own norms, the one-pass path
    (grad_sum_norm_sq, adamw_step_tiled_sum) equals the two-call path
    (grad_accum_norm_sq, adamw_step_tiled) bit for bit, norm included, and
    never writes the accumulator."""
    print(f"adamw_step_tiled_sum n={n} dtype={dtype} acc={with_acc} offsets={grad_off},{b_off}", flush=True)
    rng = np.random.default_rng(n * 3 + grad_off * 5 + b_off + 11 * with_acc + len(dtype))
    p_ref = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    m_ref, v_ref, b_ref = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
    start = oracle.state_tile(p_ref, m_ref, v_ref, n, T)
    st, stw = dev_buf(start, 0)             # one-pass path, oracle's norm
    st_one, st_one_w = dev_buf(start, 0)    # one-pass path, its own norm
    st_two, _ = dev_buf(start, 0)           # two-call path, its own norm
    b, bw = dev_buf(b_ref, b_off, bf16=True)
    b_one, b_one_w = dev_buf(b_ref, b_off, bf16=True)
    b_two, _ = dev_buf(b_ref, b_off, bf16=True)
    norm = torch.zeros(1, dtype=torch.float64, device="cuda")
    norm_one = torch.zeros(1, dtype=torch.float64, device="cuda")
    norm_two = torch.zeros(1, dtype=torch.float64, device="cuda")
    scale = 1.0 / 32
    for t in range(1, 4):
        acc0 = (rng.standard_normal(n) * 1e-2).astype(np.float32)
        g = _grad(rng, n, dtype)
        ref = acc0.copy()
        oracle.grad_accum(ref, g, _code(dtype), overwrite=not with_acc)
        S = oracle.grad_norm_sq(ref, scale)
        hp_gpu, hp_orc = _hp(t, scale=scale, max_norm=math.sqrt(S) * 0.8 if t != 2 else 0.0, extra=0.25 * S)
        oracle.adamw_step(hp_orc, p_ref, m_ref, v_ref, ref, b_ref, norm_sq=S)
        acc, acc_whole = dev_buf(acc0, 0)
        acc_arg = acc if with_acc else None
        gd, g_whole = dev_buf(g, grad_off, bf16=(dtype == "bf16"))
        norm.fill_(S)
        zs.adamw_step_tiled_sum(hp_gpu, st, acc_arg, gd, b, norm_sq=norm)
        zs.grad_sum_norm_sq(acc_arg, gd, not with_acc, scale, norm_one)
        zs.adamw_step_tiled_sum(hp_gpu, st_one, acc_arg, gd, b_one, norm_sq=norm_one)
        acc2, _ = dev_buf(acc0, 0)
        zs.grad_accum_norm_sq(acc2, gd, not with_acc, scale, norm_two)
        zs.adamw_step_tiled(hp_gpu, st_two, acc2, b_two, norm_sq=norm_two)
        torch.cuda.synchronize()
        want = oracle.state_tile(p_ref, m_ref, v_ref, n, T)
        got = to_np(st)
        assert bits_equal(got, want), (t, identical_fraction(got, want))
        assert bits_equal(to_np(b), b_ref), t
        assert norm_one.item() == norm_two.item(), t
        assert abs(math.sqrt(norm_one.item()) - math.sqrt(S)) <= NORM_TOL * math.sqrt(S)
        assert bits_equal(to_np(st_one), to_np(st_two)), t
        assert bits_equal(to_np(b_one), to_np(b_two)), t
        assert bits_equal(to_np(acc), acc0), "the accumulator was written"
        assert canary_ok(acc_whole, 0, n) and canary_ok(g_whole, grad_off, n)
    assert canary_ok(stw, 0, st.numel()) and canary_ok(bw, b_off, n)
    assert canary_ok(st_one_w, 0, st.numel()) and canary_ok(b_one_w, b_off, n)


@pytest.mark.parametrize("with_acc", [True, False])
def test_adamw_step_tiled_sum_dev_scalars_and_no_output(with_acc):
    """Scalars from device memory give the host-scalar step's bits; without
    a bf16 output the state is the same as with one."""
    n = 3 * T + 77
    rng = np.random.default_rng(41 + with_acc)
    p0 = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    start = oracle.state_tile(p0, None, None, n, T)
    st_h, _ = dev_buf(start, 0)
    st_d, _ = dev_buf(start, 0)
    st_n, _ = dev_buf(start, 0)
    b_h = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    b_d = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    norm = torch.zeros(1, dtype=torch.float64, device="cuda")
    sc = torch.empty(64, dtype=torch.uint8, device="cuda")
    for t in range(1, 5):
        acc, _ = dev_buf((rng.standard_normal(n) * 1e-2).astype(np.float32), 0)
        gd, _ = dev_buf(_grad(rng, n, "bf16"), 0, bf16=True)
        acc_arg = acc if with_acc else None
        zs.grad_sum_norm_sq(acc_arg, gd, not with_acc, 1 / 32, norm)
        hp = zs.AdamWConfig(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_scale=1 / 32,
                            max_norm=0.3, extra_norm_sq=0.01, step=t)
        zs.adamw_step_tiled_sum(hp, st_h, acc_arg, gd, b_h, norm_sq=norm)
        zs.adamw_step_tiled_sum(hp, st_n, acc_arg, gd, None, norm_sq=norm)
        sc[:56].copy_(torch.frombuffer(bytearray(zs.scalars_bytes(hp)), dtype=torch.uint8))
        zs.adamw_step_tiled_sum_dev(sc, st_d, acc_arg, gd, b_d, norm_sq=norm)
        torch.cuda.synchronize()
        assert bits_equal(to_np(st_d), to_np(st_h)), t
        assert bits_equal(to_np(st_n), to_np(st_h)), t
        assert bits_equal(to_np(b_d), to_np(b_h)), t


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_adamw_step_tiled_sum_skips_on_nonfinite_norm(bad):
    """A non-finite global norm leaves the state and the output as they were."""
    n = 2 * T + 5
    rng = np.random.default_rng(3)
    start = oracle.state_tile(rng.uniform(-0.1, 0.1, n).astype(np.float32), None, None, n, T)
    st, _ = dev_buf(start, 0)
    b = torch.full((n,), 1.5, dtype=torch.bfloat16, device="cuda")
    acc, _ = dev_buf((rng.standard_normal(n) * 1e-2).astype(np.float32), 0)
    gd, _ = dev_buf(_grad(rng, n, "bf16"), 0, bf16=True)
    norm = torch.tensor([bad], dtype=torch.float64, device="cuda")
    hp, _ = _hp(1, max_norm=1.0)
    zs.adamw_step_tiled_sum(hp, st, acc, gd, b, norm_sq=norm)
    torch.cuda.synchronize()
    assert bits_equal(to_np(st), start)
    assert torch.all(b == 1.5)


def test_adamw_step_tiled_sum_rejects():
    n = 1000
    st = torch.zeros(zs.state_tiled_numel(n), dtype=torch.float32, device="cuda")
    acc = torch.zeros(n, dtype=torch.float32, device="cuda")
    g = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    hp, _ = _hp(1)
    with pytest.raises(ValueError):   # size mismatch, caught in the binding
        zs.adamw_step_tiled_sum(hp, st, acc[:10], g)
    with pytest.raises(zs.ZShardError):   # the gradient overlapping the state
        zs.adamw_step_tiled_sum(hp, st, acc, st[:n].view(torch.bfloat16)[:n])
    with pytest.raises(zs.ZShardError):   # the accumulator overlapping the state
        zs.adamw_step_tiled_sum(hp, st, st[8:8 + n], g)
    with pytest.raises(zs.ZShardError):   # workspace too small
        out = torch.zeros(1, dtype=torch.float64, device="cuda")
        zs.grad_sum_norm_sq(acc, g, False, 1.0, out, torch.empty(8, dtype=torch.uint8, device="cuda"))


# split state: (master, exp_avg, exp_avg_sq) offsets, the gradient's offset
SPLIT_OFFSETS = [((0, 0, 0), 0), ((3, 3, 3), 1), ((1, 2, 0), 0), ((8, 8, 8), 2)]


@pytest.mark.parametrize("n", [1, 255, 257, 8193, 100_003])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("with_acc", [True, False])
@pytest.mark.parametrize("offs,grad_off", SPLIT_OFFSETS)
def test_adamw_step_sum_split_bit_exact(n, dtype, with_acc, offs, grad_off):
    """The split-buffer form, two steps: handed the oracle's norm, master,
    moments and bf16 output equal the oracle's accumulate-then-step bit for
    bit; with the GPU's own norm, equal grad_accum_norm_sq then adamw_step.
    Offsets: all aligned; the state sharing one offset off a 128-byte
    boundary (peeled) with the gradient 2 bytes off 4 (bf16: element-wise);
    the state at different offsets (element-wise); a shared 32-byte offset."""
    print(f"adamw_step_sum n={n} dtype={dtype} acc={with_acc} offs={offs} grad_off={grad_off}", flush=True)
    rng = np.random.default_rng(n + 17 * grad_off + 5 * sum(offs) + with_acc + len(dtype))
    p_ref = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    m_ref, v_ref, b_ref = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
    bufs = [dev_buf(x, o) for x, o in zip((p_ref, m_ref, v_ref), offs)]
    two = [dev_buf(x, o) for x, o in zip((p_ref, m_ref, v_ref), offs)]
    b, bw = dev_buf(b_ref, 1, bf16=True)
    b_two, _ = dev_buf(b_ref, 1, bf16=True)
    scale = 1.0 / 16
    for t in range(1, 3):
        acc0 = (rng.standard_normal(n) * 1e-2).astype(np.float32)
        g = _grad(rng, n, dtype)
        ref = acc0.copy()
        oracle.grad_accum(ref, g, _code(dtype), overwrite=not with_acc)
        S = oracle.grad_norm_sq(ref, scale)
        hp_gpu, hp_orc = _hp(t, scale=scale, max_norm=math.sqrt(S) * 0.7, extra=0.1 * S)
        oracle.adamw_step(hp_orc, p_ref, m_ref, v_ref, ref, b_ref, norm_sq=S)
        acc, acc_whole = dev_buf(acc0, 0)
        gd, g_whole = dev_buf(g, grad_off, bf16=(dtype == "bf16"))
        norm = torch.tensor([S], dtype=torch.float64, device="cuda")
        zs.adamw_step_sum(hp_gpu, *(x for x, _ in bufs), acc if with_acc else None, gd, b, norm_sq=norm)
        # the two-call path with its own norm, and the one-pass norm next to it
        own = torch.zeros(1, dtype=torch.float64, device="cuda")
        zs.grad_sum_norm_sq(acc if with_acc else None, gd, not with_acc, scale, own)
        acc2, _ = dev_buf(acc0, 0)
        own2 = torch.zeros(1, dtype=torch.float64, device="cuda")
        zs.grad_accum_norm_sq(acc2, gd, not with_acc, scale, own2)
        torch.cuda.synchronize()
        assert own.item() == own2.item()
        for (x, _), want in zip(bufs, (p_ref, m_ref, v_ref)):
            assert bits_equal(to_np(x), want), (t, identical_fraction(to_np(x), want))
        assert bits_equal(to_np(b), b_ref), t
        assert bits_equal(to_np(acc), acc0), "the accumulator was written"
        # the two-call path from the same start, with the oracle's norm: the same bits
        zs.adamw_step(hp_gpu, *(x for x, _ in two), acc2, b_two, norm_sq=norm)
        torch.cuda.synchronize()
        for (x, _), (y, _) in zip(two, bufs):
            assert bits_equal(to_np(x), to_np(y)), t
        assert canary_ok(acc_whole, 0, n) and canary_ok(g_whole, grad_off, n)
    for (x, whole), o in zip(bufs, offs):
        assert canary_ok(whole, o, n)
    assert canary_ok(bw, 1, n)


def test_adamw_step_sum_dev_scalars():
    """Split state, scalars from device memory: the host-scalar step's bits."""
    n = 50_003
    rng = np.random.default_rng(12)
    p0 = rng.uniform(-0.1, 0.1, n).astype(np.float32)
    h = [dev_buf(x, 0)[0] for x in (p0, np.zeros(n, np.float32), np.zeros(n, np.float32))]
    d = [dev_buf(x, 0)[0] for x in (p0, np.zeros(n, np.float32), np.zeros(n, np.float32))]
    b_h = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    b_d = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    norm = torch.zeros(1, dtype=torch.float64, device="cuda")
    sc = torch.empty(64, dtype=torch.uint8, device="cuda")
    for t in range(1, 4):
        acc, _ = dev_buf((rng.standard_normal(n) * 1e-2).astype(np.float32), 0)
        gd, _ = dev_buf(_grad(rng, n, "bf16"), 0, bf16=True)
        zs.grad_sum_norm_sq(acc, gd, False, 1 / 32, norm)
        hp = zs.AdamWConfig(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_scale=1 / 32,
                            max_norm=0.3, extra_norm_sq=0.01, step=t)
        zs.adamw_step_sum(hp, *h, acc, gd, b_h, norm_sq=norm)
        sc[:56].copy_(torch.frombuffer(bytearray(zs.scalars_bytes(hp)), dtype=torch.uint8))
        zs.adamw_step_sum_dev(sc, *d, acc, gd, b_d, norm_sq=norm)
        torch.cuda.synchronize()
        for x, y in zip(h, d):
            assert bits_equal(to_np(x), to_np(y)), t
        assert bits_equal(to_np(b_h), to_np(b_d)), t


def test_one_pass_random_configurations():
    """160 seeded random cases (length up to 70,000 across tile and block
    edges; bf16 or fp32 gradient, with or without an accumulator; tiled or
    split state at random element offsets; bf16 output present or not, at
    random offsets; clip on or off): the one-pass norm is grad_accum_norm_sq's
    bits, and the one-pass step, handed the oracle's norm, the oracle's
    accumulate-then-step bits."""
    rng = np.random.default_rng(2027)
    for case in range(160):
        n = int(rng.choice([int(rng.integers(1, 600)), int(rng.integers(1, 70_000)),
                            int(rng.choice([255, 256, 257, 1023, 1024, 1025, 8191, 8192, 8193, 16384]))]))
        dtype = str(rng.choice(["bf16", "f32"]))
        with_acc = bool(rng.integers(0, 2))
        tiled = bool(rng.integers(0, 2))
        offs = [int(x) for x in rng.integers(0, 4, size=3)] if not tiled else [0, 0, 0]
        if rng.integers(0, 2):
            offs = [offs[0]] * 3   # a shared offset: the peeled form
        g_off, b_off = int(rng.integers(0, 3)), int(rng.integers(0, 4))
        with_b = bool(rng.integers(0, 4))
        clip = bool(rng.integers(0, 2))
        scale = float(rng.choice([1 / 8, 1 / 64]))
        tag = (case, n, dtype, with_acc, tiled, offs, g_off, b_off, with_b, clip)
        p = rng.uniform(-0.1, 0.1, n).astype(np.float32)
        m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        v = rng.uniform(0, 1e-6, n).astype(np.float32)
        acc0 = (rng.standard_normal(n) * 1e-2).astype(np.float32)
        g = _grad(rng, n, dtype)
        ref = acc0.copy()
        oracle.grad_accum(ref, g, _code(dtype), overwrite=not with_acc)
        S = oracle.grad_norm_sq(ref, scale)
        hp_gpu, hp_orc = _hp(int(rng.integers(1, 9)), scale=scale, max_norm=math.sqrt(S) * 0.6 if clip else 0.0,
                             extra=0.3 * S)
        b_ref = np.zeros(n, np.uint16)
        p_ref, m_ref, v_ref = p.copy(), m.copy(), v.copy()
        oracle.adamw_step(hp_orc, p_ref, m_ref, v_ref, ref, b_ref if with_b else None, norm_sq=S)
        acc, _ = dev_buf(acc0, 0)
        acc_arg = acc if with_acc else None
        gd, _ = dev_buf(g, g_off, bf16=(dtype == "bf16"))
        b = dev_buf(np.zeros(n, np.uint16), b_off, bf16=True)[0] if with_b else None
        # the norm: bit for bit the fused pass's
        one = torch.zeros(1, dtype=torch.float64, device="cuda")
        zs.grad_sum_norm_sq(acc_arg, gd, not with_acc, scale, one)
        acc2, _ = dev_buf(acc0, 0)
        two = torch.zeros(1, dtype=torch.float64, device="cuda")
        zs.grad_accum_norm_sq(acc2, gd, not with_acc, scale, two)
        norm = torch.tensor([S], dtype=torch.float64, device="cuda")
        if tiled:
            st, _ = dev_buf(oracle.state_tile(p, m, v, n, T), 0)
            zs.adamw_step_tiled_sum(hp_gpu, st, acc_arg, gd, b, norm_sq=norm)
            got = oracle.state_untile(to_np(st), n, T)
        else:
            bufs = [dev_buf(x, o)[0] for x, o in zip((p, m, v), offs)]
            zs.adamw_step_sum(hp_gpu, *bufs, acc_arg, gd, b, norm_sq=norm)
            got = [to_np(x) for x in bufs]
        torch.cuda.synchronize()
        assert one.item() == two.item(), tag
        for x, want in zip(got, (p_ref, m_ref, v_ref)):
            assert bits_equal(x, want), (tag, identical_fraction(x, want))
        if with_b:
            assert bits_equal(to_np(b), b_ref), tag
