"""The C-ABI library on the host: it loads, exports every declared symbol,
and its argument checks return the documented codes before any launch.

No test here reaches a kernel launch (there is no GPU in this container):
every call either is host-only (zero_shard_range, the workspace size) or
fails validation, or is an n == 0 no-op that returns before launching.
Pointers passed to failing calls are never dereferenced.
"""
import ctypes
import json
import os
import re

import pytest

import oracle
import fsdp_sharded_optimizer_amd as zs
from fsdp_sharded_optimizer_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zshard.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*ZS_API\s+(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(autouse=True)
def no_launch_reached():
    """Every call here must stop before a launch: on a host without a GPU a
    launch attempt leaves a HIP error behind, and that fails the test."""
    yield
    assert zs.lib().zs_last_hip_error() == 0, "a call got past validation to a kernel launch"


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) == 35 and set(names) == set(B.EXPORTS), names
    L = zs.lib()
    for name in names:
        assert getattr(L, name) is not None


def test_library_exports_nothing_else():
    """The dynamic symbol table holds the declared functions and no internal
    (launcher, kernel stub) symbol of the library's own code."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True, check=True).stdout
    defined = {line.split()[-1] for line in out.splitlines() if line.split() and line.split()[-2] in ("T", "W")}
    ours = {s for s in defined if s.startswith("_ZN2zs") or s in B.EXPORTS}
    assert ours == set(B.EXPORTS), sorted(ours - set(B.EXPORTS))


def test_shard_range_matches_oracle_brute_force(orc):
    for T in list(range(0, 130)) + [1_000_003, 6_738_415_616, 13_015_864_320, 855_654_400, 70_000_000_000]:
        for N in (1, 2, 3, 7, 8, 13, 64, 129):
            for r in sorted({0, 1, N // 2, N - 1} & set(range(N))):
                assert zs.zero_shard_range(T, N, r) == oracle.shard_range(T, N, r), (T, N, r)


def test_shard_range_golden():
    with open(os.path.join(ROOT, "tests", "golden", "shard_ranges.json")) as f:
        for c in json.load(f)["cases"]:
            got = zs.zero_shard_range(c["total"], c["world"], c["rank"])
            assert got == (c["chunk"], c["start"], c["end"], c["padded_total"]), c["name"]


def test_shard_range_errors():
    L = zs.lib()
    out = B.Shard()
    for args in [(10, 0, 0), (10, 4, 4), (10, 4, -1), (-1, 4, 0)]:
        assert L.zero_shard_range(*args, ctypes.byref(out)) == B.ZS_EINVAL
    assert L.zero_shard_range(10, 4, 0, None) == B.ZS_EINVAL
    # world*chunk would overflow int64
    assert L.zero_shard_range(2**63 - 1, 3, 0, ctypes.byref(out)) == B.ZS_EINVAL
    with pytest.raises(zs.ZShardError):
        zs.zero_shard_range(10, 0, 0)


def test_workspace_bytes():
    assert zs.grad_norm_sq_workspace_bytes(0) == 0
    assert zs.grad_norm_sq_workspace_bytes(-1) == -1
    assert zs.grad_norm_sq_workspace_bytes(1) == 8
    # one partial per 4096-element tile; beyond 2048 partials, a 2048-entry chunk stage too
    assert zs.grad_norm_sq_workspace_bytes(4096 * 2048) == 2048 * 8
    assert zs.grad_norm_sq_workspace_bytes(4096 * 2048 + 1) == (2049 + 2048) * 8
    assert zs.grad_norm_sq_workspace_bytes(10**10) == (-(-10**10 // 4096) + 2048) * 8
    # beyond the per-call element limit: -1
    assert zs.grad_norm_sq_workspace_bytes(2**63 - 1) == -1 and zs.grad_accum_norm_sq_workspace_bytes(2**39 + 1) == -1


FAKE = 0x7F0000000000   # never dereferenced: every call below fails validation


def _hp(**kw):
    base = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, grad_scale=1.0,
                max_norm=0.0, extra_norm_sq=0.0, step=1)
    base.update(kw)
    return B.AdamW(**base)


def _adamw(hp, master=FAKE, m=FAKE + 2**20, v=FAKE + 2**21, g=FAKE + 2**22, b=0, n=1024, norm=0):
    return zs.lib().adamw_step(ctypes.byref(hp) if hp is not None else None, master, m, v, g, b, n,
                               norm, None)


def test_adamw_rejects_hyperparameters():
    for bad in (dict(step=0), dict(beta1=1.0), dict(beta1=-0.5), dict(beta2=1.0), dict(eps=0.0),
                dict(eps=float("nan")), dict(lr=-1e-3), dict(weight_decay=-0.1), dict(grad_scale=0.0),
                dict(grad_scale=float("inf")), dict(max_norm=float("nan")), dict(extra_norm_sq=-1.0)):
        assert _adamw(_hp(**bad)) == B.ZS_EINVAL, bad
    assert _adamw(None) == B.ZS_EINVAL


def test_adamw_rejects_pointers():
    assert _adamw(_hp(), master=0) == B.ZS_EINVAL
    assert _adamw(_hp(), g=0) == B.ZS_EINVAL
    assert _adamw(_hp(), master=FAKE + 2) == B.ZS_EINVAL          # fp32 must be 4-byte aligned
    assert _adamw(_hp(), b=FAKE + 2**23 + 1) == B.ZS_EINVAL       # bf16 must be 2-byte aligned
    assert _adamw(_hp(), norm=FAKE + 2**24 + 4) == B.ZS_EINVAL    # fp64 must be 8-byte aligned
    assert _adamw(_hp(), n=-1) == B.ZS_EINVAL
    # overlaps: exp_avg inside master, bf16 over grad, norm inside exp_avg_sq
    assert _adamw(_hp(), m=FAKE + 4) == B.ZS_EOVERLAP
    assert _adamw(_hp(), b=FAKE + 2**22 + 64) == B.ZS_EOVERLAP
    assert _adamw(_hp(), norm=FAKE + 2**21 + 8) == B.ZS_EOVERLAP
    # adjacent, not overlapping buffers pass the overlap check (n = 0 no-op)
    assert _adamw(_hp(), n=0) == B.ZS_OK
    assert _adamw(_hp(), master=0, m=0, v=0, g=0, n=0) == B.ZS_OK


def test_adamw_no_master_rejects():
    L = zs.lib()
    call = lambda hp=None, b=FAKE, m=FAKE + 2**20, v=FAKE + 2**21, g=FAKE + 2**22, n=1024, norm=0: \
        L.adamw_step_no_master(ctypes.byref(hp or _hp()), b, m, v, g, n, norm, None)
    assert call(hp=_hp(step=0)) == B.ZS_EINVAL
    assert call(b=0) == B.ZS_EINVAL
    assert call(b=FAKE + 1) == B.ZS_EINVAL
    assert call(m=FAKE + 1024) == B.ZS_EOVERLAP                   # exp_avg inside the bf16 parameter
    assert call(norm=FAKE + 2**21 + 64) == B.ZS_EOVERLAP          # norm inside exp_avg_sq
    assert call(n=0) == B.ZS_OK


def test_adamw_scalars_match_the_oracle_bit_for_bit(orc):
    """The library's host scalars and the oracle's are formed independently
    (both binary64, one rounding each): identical bits over random
    hyperparameters and steps, and the hand-worked golden patterns."""
    import random
    import struct
    rnd = random.Random(5)
    names = ("beta1", "beta2", "one_minus_beta1", "one_minus_beta2", "step_size", "bias_correction2_sqrt", "eps",
             "decay", "grad_scale")
    bits = lambda x: struct.unpack("<I", struct.pack("<f", x))[0]
    for _ in range(300):
        kw = dict(lr=10 ** rnd.uniform(-6, -1), beta1=rnd.choice([0.0, 0.5, 0.9, rnd.uniform(0, 0.999999)]),
                  beta2=rnd.choice([0.0, 0.95, 0.999, rnd.uniform(0, 0.9999999)]), eps=10 ** rnd.uniform(-12, 0),
                  weight_decay=rnd.choice([0.0, 0.1, rnd.uniform(0, 10)]), grad_scale=2.0 ** -rnd.randint(0, 12),
                  max_norm=rnd.choice([0.0, 1.0]), extra_norm_sq=rnd.uniform(0, 3), step=rnd.randint(1, 100000))
        got = zs.adamw_scalars(zs.AdamWConfig(**kw))
        want = oracle.adamw_scalars(oracle.make_hp(kw["lr"], kw["beta1"], kw["beta2"], kw["eps"],
                                                   kw["weight_decay"], kw["grad_scale"], kw["max_norm"],
                                                   kw["extra_norm_sq"], kw["step"]))
        for nm in names:
            assert bits(getattr(got, nm)) == bits(getattr(want, nm)), (nm, kw)
        assert got.clip == (1 if kw["max_norm"] > 0 else 0)
        assert got.max_norm == kw["max_norm"] and got.extra_norm_sq == kw["extra_norm_sq"]
    assert len(zs.scalars_bytes(zs.AdamWConfig(lr=1e-3))) == 56


def test_adamw_scalars_and_step_dev_reject():
    L = zs.lib()
    out = B.AdamWScalars()
    assert L.adamw_scalars(ctypes.byref(_hp(step=0)), ctypes.byref(out)) == B.ZS_EINVAL
    assert L.adamw_scalars(ctypes.byref(_hp()), None) == B.ZS_EINVAL
    assert L.adamw_scalars(None, ctypes.byref(out)) == B.ZS_EINVAL
    sc = FAKE + 2**30
    call = lambda s=sc, master=FAKE, n=1024, norm=0: L.adamw_step_dev(
        s, master, FAKE + 2**20, FAKE + 2**21, FAKE + 2**22, 0, n, norm, None)
    assert call(s=0) == B.ZS_EINVAL
    assert call(s=sc + 4) == B.ZS_EINVAL                     # scalars must be 8-byte aligned
    assert call(s=FAKE + 64) == B.ZS_EOVERLAP                # scalars inside the master being written
    assert call(norm=FAKE + 2**21 + 8) == B.ZS_EOVERLAP      # norm inside exp_avg_sq
    assert call(n=(1 << 39) + 1) == B.ZS_EINVAL
    assert call(n=0) == B.ZS_OK


def test_state_tile_constant_matches_the_header():
    """ZS_STATE_TILE in the header, the binding's constant and the tests'
    layout definition (test_oracle_pins: 8192) agree."""
    text = open(HEADER).read()
    assert int(re.search(r"#define ZS_STATE_TILE (\d+)", text).group(1)) == B.STATE_TILE == 8192


def test_state_tiled_numel():
    L = zs.lib()
    T = B.STATE_TILE
    for n in (0, 1, T - 1, T, T + 1, 5 * T, 842301952, 1 << 39):
        assert L.state_tiled_numel(n) == oracle.state_tiled_numel(n, T) == 3 * T * (-(-n // T)), n
    assert L.state_tiled_numel(-1) == -1 and L.state_tiled_numel((1 << 39) + 1) == -1


def test_state_tile_and_untile_reject():
    L = zs.lib()
    n = 1024
    st = FAKE + 2**30
    sb = 3 * B.STATE_TILE * 4                                   # tiled bytes of 1024 elements
    tile = lambda p=FAKE, m=FAKE + 2**20, v=FAKE + 2**21, s=st, k=n: L.state_tile(p, m, v, s, k, None)
    untile = lambda p=FAKE, m=FAKE + 2**20, v=FAKE + 2**21, s=st, k=n: L.state_untile(s, p, m, v, k, None)
    for call in (tile, untile):
        assert call(s=0) == B.ZS_EINVAL
        assert call(s=st + 4) == B.ZS_EINVAL                      # the state must be 16-byte aligned
        assert call(p=FAKE + 2) == B.ZS_EINVAL                    # fp32 must be 4-byte aligned
        assert call(k=-1) == B.ZS_EINVAL
        assert call(k=(1 << 39) + 1) == B.ZS_EINVAL
        assert call(v=st + sb - 4) == B.ZS_EOVERLAP               # a split array over the state's end
        assert call(k=0) == B.ZS_OK
        assert call(s=0, k=0) == B.ZS_OK
    assert untile(m=FAKE + 64) == B.ZS_EOVERLAP                   # two destinations overlap
    assert tile(p=FAKE + 2, m=0, v=0) == B.ZS_EINVAL


def test_adamw_step_tiled_rejects():
    L = zs.lib()
    n = 1024
    st = FAKE
    sb = 3 * B.STATE_TILE * 4
    call = lambda hp=None, s=st, g=FAKE + 2**20, b=0, k=n, norm=0: L.adamw_step_tiled(
        ctypes.byref(hp or _hp()), s, g, b, k, norm, None)
    for bad in (dict(step=0), dict(beta1=1.0), dict(eps=0.0), dict(lr=-1.0), dict(grad_scale=0.0)):
        assert call(hp=_hp(**bad)) == B.ZS_EINVAL, bad
    assert L.adamw_step_tiled(None, st, FAKE + 2**20, 0, n, 0, None) == B.ZS_EINVAL
    assert call(s=0) == B.ZS_EINVAL
    assert call(g=0) == B.ZS_EINVAL
    assert call(s=st + 4) == B.ZS_EINVAL                            # the state must be 16-byte aligned
    assert call(g=FAKE + 2**20 + 2) == B.ZS_EINVAL
    assert call(b=FAKE + 2**21 + 1) == B.ZS_EINVAL
    assert call(norm=FAKE + 2**22 + 4) == B.ZS_EINVAL
    assert call(g=st + sb - 8) == B.ZS_EOVERLAP                     # grad over the end of the state
    assert call(b=FAKE + 2**20 + 64) == B.ZS_EOVERLAP               # bf16 output over the grad
    assert call(norm=st + 1024) == B.ZS_EOVERLAP                    # norm inside the written state
    assert call(k=(1 << 39) + 1) == B.ZS_EINVAL
    assert call(k=0) == B.ZS_OK
    sc = FAKE + 2**30
    dev = lambda s=sc, k=n, norm=0: L.adamw_step_tiled_dev(s, st, FAKE + 2**20, 0, k, norm, None)
    assert dev(s=0) == B.ZS_EINVAL
    assert dev(s=sc + 4) == B.ZS_EINVAL
    assert dev(s=st + 64) == B.ZS_EOVERLAP                          # scalars inside the written state
    assert dev(k=0) == B.ZS_OK


def test_moments_calls_reject():
    L = zs.lib()
    T = B.STATE_TILE
    n = 1024
    mo = FAKE + 2**30
    mb = 2 * T * 4                                                # tiled bytes of 1024 elements
    assert L.moments_tiled_numel(1) == 2 * T and L.moments_tiled_numel(-1) == -1
    assert L.moments_tiled_numel(5 * T + 1) == oracle.moments_tiled_numel(5 * T + 1, T) == 12 * T
    assert L.moments_tile(FAKE, FAKE + 2**20, mo + 4, n, None) == B.ZS_EINVAL             # off 16 bytes
    assert L.moments_tile(FAKE, mo + mb - 4, mo, n, None) == B.ZS_EOVERLAP
    assert L.moments_untile(mo, FAKE, FAKE + 8, n, None) == B.ZS_EOVERLAP                  # two destinations
    assert L.moments_untile(mo, FAKE + 2, None, n, None) == B.ZS_EINVAL
    assert L.moments_tile(None, None, None, 0, None) == B.ZS_OK
    upd = lambda hp=None, m=mo, g=FAKE, u=FAKE + 2**20, k=n, norm=0: L.adam_update_tiled(
        ctypes.byref(hp or _hp()), m, g, u, k, norm, None)
    assert upd(hp=_hp(weight_decay=0.1)) == B.ZS_EINVAL                                      # no decay
    assert upd(hp=_hp(step=0)) == B.ZS_EINVAL
    assert upd(m=mo + 4) == B.ZS_EINVAL
    assert upd(u=FAKE + 2**20 + 2) == B.ZS_EINVAL                                            # fp32: 4 bytes
    assert upd(g=mo + 16) == B.ZS_EOVERLAP
    assert upd(norm=mo + 64) == B.ZS_EOVERLAP                                                # norm in the moments
    assert upd(k=0) == B.ZS_OK
    nm = lambda hp=None, p=FAKE, m=mo, g=FAKE + 2**20, k=n, norm=0: L.adamw_step_no_master_tiled(
        ctypes.byref(hp or _hp()), p, m, g, k, norm, None)
    assert nm(hp=_hp(eps=0.0)) == B.ZS_EINVAL
    assert nm(p=FAKE + 1) == B.ZS_EINVAL                                                     # bf16: 2 bytes
    assert nm(m=mo + 8) == B.ZS_EINVAL
    assert nm(p=mo + mb - 2) == B.ZS_EOVERLAP
    assert nm(k=(1 << 39) + 1) == B.ZS_EINVAL
    assert nm(k=0) == B.ZS_OK


def test_adam_update_rejects():
    L = zs.lib()
    call = lambda hp=None, m=FAKE, v=FAKE + 2**20, g=FAKE + 2**21, u=FAKE + 2**22, n=1024, norm=0: \
        L.adam_update(ctypes.byref(hp or _hp()), m, v, g, u, n, norm, None)
    assert call(hp=_hp(weight_decay=0.1)) == B.ZS_EINVAL            # the ZeRO-1 form has no decay
    assert call(hp=_hp(weight_decay=0.1), n=0) == B.ZS_EINVAL
    assert call(hp=_hp(step=0)) == B.ZS_EINVAL
    assert call(u=0) == B.ZS_EINVAL
    assert call(g=FAKE + 2**21 + 2) == B.ZS_EINVAL                  # fp32 must be 4-byte aligned
    assert call(u=FAKE + 2**21 + 4) == B.ZS_EOVERLAP                # update over grad
    assert call(norm=FAKE + 2**22 + 8) == B.ZS_EOVERLAP             # norm inside the update
    assert call(n=0) == B.ZS_OK


def test_flat_apply_update_rejects():
    L = zs.lib()
    upd = FAKE + 2**30
    two = _tensors((FAKE, 10), (FAKE + 2**20, 6))
    assert L.flat_apply_update(upd, two, 2, 7, None) == B.ZS_EINVAL                   # dtype
    assert L.flat_apply_update(upd, two, -1, B.ZS_F32, None) == B.ZS_EINVAL
    assert L.flat_apply_update(0, two, 2, B.ZS_F32, None) == B.ZS_EINVAL
    assert L.flat_apply_update(upd + 2, two, 2, B.ZS_F32, None) == B.ZS_EINVAL        # misaligned update
    assert L.flat_apply_update(upd, _tensors((FAKE + 1, 4)), 1, B.ZS_BF16, None) == B.ZS_EINVAL
    assert L.flat_apply_update(upd, _tensors((upd + 8, 4)), 1, B.ZS_F32, None) == B.ZS_EOVERLAP   # [upd+8, upd+24) over [upd, upd+16)
    assert L.flat_apply_update(upd, _tensors((FAKE, 8), (FAKE + 16, 8)), 2, B.ZS_F32, None) == B.ZS_EOVERLAP
    assert L.flat_apply_update(upd, _tensors((0, 0)), 1, B.ZS_BF16, None) == B.ZS_OK


def test_grad_accum_rejects():
    L = zs.lib()
    assert L.grad_accum(FAKE, FAKE + 2**20, 7, 16, 0, None) == B.ZS_EINVAL       # dtype
    assert L.grad_accum(0, FAKE, B.ZS_BF16, 16, 0, None) == B.ZS_EINVAL
    assert L.grad_accum(FAKE + 1, FAKE + 2**20, B.ZS_F32, 16, 0, None) == B.ZS_EINVAL
    assert L.grad_accum(FAKE, FAKE + 2**20 + 1, B.ZS_BF16, 16, 0, None) == B.ZS_EINVAL
    assert L.grad_accum(FAKE, FAKE + 32, B.ZS_BF16, 16, 0, None) == B.ZS_EOVERLAP
    assert L.grad_accum(FAKE, FAKE, B.ZS_F32, -1, 0, None) == B.ZS_EINVAL
    assert L.grad_accum(0, 0, B.ZS_F32, 0, 1, None) == B.ZS_OK                    # n = 0 no-op


def test_grad_norm_sq_rejects():
    L = zs.lib()
    n = 1 << 20
    need = zs.grad_norm_sq_workspace_bytes(n)
    ws, out = FAKE + 2**30, FAKE + 2**31
    assert L.grad_norm_sq(FAKE, n, 1.0, out, ws, need - 8, None) == B.ZS_EWORKSPACE
    assert L.grad_norm_sq(FAKE, n, 1.0, 0, ws, need, None) == B.ZS_EINVAL
    assert L.grad_norm_sq(FAKE, n, 1.0, out + 4, ws, need, None) == B.ZS_EINVAL
    assert L.grad_norm_sq(FAKE, n, 0.0, out, ws, need, None) == B.ZS_EINVAL
    assert L.grad_norm_sq(0, n, 1.0, out, ws, need, None) == B.ZS_EINVAL
    assert L.grad_norm_sq(FAKE, n, 1.0, out, 0, need, None) == B.ZS_EINVAL
    assert L.grad_norm_sq(FAKE, n, 1.0, FAKE + 8, ws, need, None) == B.ZS_EOVERLAP
    assert L.grad_norm_sq(FAKE, n, 1.0, out, FAKE + 64, need, None) == B.ZS_EOVERLAP


def test_grad_reduce_chunks_rejects():
    L = zs.lib()
    n = 1 << 16
    acc = FAKE
    chunks = (ctypes.c_void_p * 3)(FAKE + 2**30, FAKE + 2**31, FAKE + 2**32)
    call = lambda **k: L.grad_reduce_chunks(k.get("acc", acc), k.get("chunks", chunks), k.get("count", 3),
                                            k.get("dt", B.ZS_BF16), k.get("n", n), k.get("ow", 1), None)
    assert call(count=-1) == B.ZS_EINVAL
    assert call(count=0, ow=1) == B.ZS_EINVAL
    assert call(count=0, ow=0) == B.ZS_OK                  # nothing to add
    assert call(n=0) == B.ZS_OK
    assert call(dt=9) == B.ZS_EINVAL
    assert call(acc=0) == B.ZS_EINVAL
    assert call(chunks=None) == B.ZS_EINVAL
    bad = (ctypes.c_void_p * 3)(FAKE + 2**30, 0, FAKE + 2**32)
    assert call(chunks=bad) == B.ZS_EINVAL
    odd = (ctypes.c_void_p * 3)(FAKE + 2**30, FAKE + 2**31 + 1, FAKE + 2**32)
    assert call(chunks=odd) == B.ZS_EINVAL                  # bf16 must be 2-byte aligned
    over = (ctypes.c_void_p * 3)(FAKE + 2**30, FAKE + 1024, FAKE + 2**32)
    assert call(chunks=over) == B.ZS_EOVERLAP               # a chunk inside acc
    same = (ctypes.c_void_p * 3)(FAKE + 2**30, FAKE + 2**30, FAKE + 2**30)
    assert call(chunks=same, n=-1) == B.ZS_EINVAL


def test_grad_accum_norm_sq_rejects():
    L = zs.lib()
    n = 1 << 20
    need = zs.grad_accum_norm_sq_workspace_bytes(n)
    assert need == (n // 256 + 2048) * 8         # one partial per 256 elements + the chunk stage
    assert zs.grad_accum_norm_sq_workspace_bytes(0) == 0 and zs.grad_accum_norm_sq_workspace_bytes(-3) == -1
    acc, g, ws, out = FAKE, FAKE + 2**30, FAKE + 2**31, FAKE + 2**32
    call = lambda **k: L.grad_accum_norm_sq(k.get("acc", acc), k.get("g", g), k.get("dt", B.ZS_BF16), k.get("n", n),
                                            0, k.get("s", 1.0), k.get("out", out), k.get("ws", ws),
                                            k.get("wsb", need), None)
    assert call(wsb=need - 8) == B.ZS_EWORKSPACE
    assert call(dt=5) == B.ZS_EINVAL
    assert call(out=0) == B.ZS_EINVAL
    assert call(out=out + 4) == B.ZS_EINVAL
    assert call(s=-1.0) == B.ZS_EINVAL
    assert call(acc=0) == B.ZS_EINVAL
    assert call(ws=0) == B.ZS_EINVAL
    assert call(g=FAKE + 64) == B.ZS_EOVERLAP                      # grad inside acc
    assert call(out=FAKE + 16) == B.ZS_EOVERLAP                    # norm inside acc
    assert call(ws=g + 1024) == B.ZS_EOVERLAP                      # workspace inside grad
    assert call(n=-1) == B.ZS_EINVAL


def test_grad_sum_norm_sq_rejects():
    L = zs.lib()
    n = 1 << 20
    need = zs.grad_accum_norm_sq_workspace_bytes(n)
    acc, g, ws, out = FAKE, FAKE + 2**30, FAKE + 2**31, FAKE + 2**32
    call = lambda **k: L.grad_sum_norm_sq(k.get("acc", acc), k.get("g", g), k.get("dt", B.ZS_BF16), k.get("n", n),
                                          k.get("ovr", 0), k.get("s", 1.0), k.get("out", out), k.get("ws", ws),
                                          k.get("wsb", need), None)
    assert call(wsb=need - 8) == B.ZS_EWORKSPACE
    assert call(dt=5) == B.ZS_EINVAL
    assert call(out=0) == B.ZS_EINVAL
    assert call(out=out + 4) == B.ZS_EINVAL
    assert call(s=float("inf")) == B.ZS_EINVAL
    assert call(acc=0) == B.ZS_EINVAL                              # an accumulator is read unless overwrite
    assert call(acc=acc + 2) == B.ZS_EINVAL
    assert call(g=g + 1) == B.ZS_EINVAL                            # bf16 at an odd address
    assert call(ws=0) == B.ZS_EINVAL
    assert call(out=FAKE + 16) == B.ZS_EOVERLAP                    # norm inside acc
    assert call(ws=g + 1024) == B.ZS_EOVERLAP                      # workspace inside grad
    assert call(ws=FAKE + 64) == B.ZS_EOVERLAP                     # workspace inside acc
    assert call(n=-1) == B.ZS_EINVAL
    # overwrite: the accumulator is not read, so none is needed and none can overlap
    assert call(ovr=1, acc=0, wsb=need - 8) == B.ZS_EWORKSPACE
    assert call(ovr=1, acc=ws + 64, g=0) == B.ZS_EINVAL           # a gradient is still needed


def test_adamw_step_tiled_sum_rejects():
    L = zs.lib()
    n = 1024
    st = FAKE
    sb = 3 * B.STATE_TILE * 4
    acc0, g0 = FAKE + 2**20, FAKE + 2**21
    call = lambda hp=None, s=st, a=acc0, g=g0, dt=B.ZS_BF16, b=0, k=n, norm=0: L.adamw_step_tiled_sum(
        ctypes.byref(hp or _hp()), s, a, g, dt, b, k, norm, None)
    for bad in (dict(step=0), dict(beta2=-0.1), dict(eps=float("nan")), dict(grad_scale=0.0)):
        assert call(hp=_hp(**bad)) == B.ZS_EINVAL, bad
    assert L.adamw_step_tiled_sum(None, st, acc0, g0, B.ZS_BF16, 0, n, 0, None) == B.ZS_EINVAL
    assert call(dt=7) == B.ZS_EINVAL
    assert call(s=0) == B.ZS_EINVAL
    assert call(g=0) == B.ZS_EINVAL
    assert call(s=st + 4) == B.ZS_EINVAL                            # the state must be 16-byte aligned
    assert call(a=acc0 + 2) == B.ZS_EINVAL                          # fp32 accumulator off 4 bytes
    assert call(g=g0 + 1) == B.ZS_EINVAL                            # bf16 gradient at an odd address
    assert call(g=g0 + 2, dt=B.ZS_F32) == B.ZS_EINVAL               # fp32 gradient off 4 bytes
    assert call(b=FAKE + 2**22 + 1) == B.ZS_EINVAL
    assert call(norm=FAKE + 2**23 + 4) == B.ZS_EINVAL
    assert call(a=st + sb - 8) == B.ZS_EOVERLAP                     # accumulator over the end of the state
    assert call(g=st + 64) == B.ZS_EOVERLAP                         # gradient inside the state
    assert call(g=acc0 + 64) == B.ZS_EOVERLAP                       # gradient inside the accumulator
    assert call(b=g0 + 64) == B.ZS_EOVERLAP                         # bf16 output over the gradient
    assert call(norm=st + 1024) == B.ZS_EOVERLAP                    # norm inside the written state
    assert call(k=(1 << 39) + 1) == B.ZS_EINVAL
    assert call(k=0) == B.ZS_OK
    assert call(k=0, s=0, a=0, g=0) == B.ZS_OK                      # nothing to step: no buffer needed
    sc = FAKE + 2**30
    dev = lambda s=sc, k=n, norm=0, dt=B.ZS_BF16: L.adamw_step_tiled_sum_dev(s, st, acc0, g0, dt, 0, k, norm, None)
    assert L.adamw_step_tiled_sum_dev(0, st, acc0, g0, B.ZS_BF16, 0, n, 0, None) == B.ZS_EINVAL
    assert dev(s=sc + 4) == B.ZS_EINVAL
    assert dev(dt=3) == B.ZS_EINVAL
    assert dev(s=st + 64) == B.ZS_EOVERLAP                          # scalars inside the written state
    assert dev(k=0) == B.ZS_OK


def test_adamw_step_sum_rejects():
    L = zs.lib()
    n = 1024
    p, m, v = FAKE, FAKE + 2**16, FAKE + 2**17
    acc0, g0 = FAKE + 2**20, FAKE + 2**21
    call = lambda hp=None, a=acc0, g=g0, dt=B.ZS_BF16, b=0, k=n, norm=0, pp=p: L.adamw_step_sum(
        ctypes.byref(hp or _hp()), pp, m, v, a, g, dt, b, k, norm, None)
    for bad in (dict(step=0), dict(beta1=1.5), dict(eps=0.0), dict(max_norm=float("nan"))):
        assert call(hp=_hp(**bad)) == B.ZS_EINVAL, bad
    assert L.adamw_step_sum(None, p, m, v, acc0, g0, B.ZS_BF16, 0, n, 0, None) == B.ZS_EINVAL
    assert call(dt=2) == B.ZS_EINVAL
    assert call(pp=0) == B.ZS_EINVAL
    assert call(g=0) == B.ZS_EINVAL
    assert call(pp=p + 2) == B.ZS_EINVAL                            # master off 4 bytes
    assert call(a=acc0 + 2) == B.ZS_EINVAL                          # accumulator off 4 bytes
    assert call(g=g0 + 1) == B.ZS_EINVAL                            # bf16 gradient at an odd address
    assert call(b=FAKE + 2**22 + 1) == B.ZS_EINVAL
    assert call(a=m + 64) == B.ZS_EOVERLAP                          # accumulator inside exp_avg
    assert call(g=acc0 + 64) == B.ZS_EOVERLAP                       # gradient inside the accumulator
    assert call(b=p + 64) == B.ZS_EOVERLAP                          # bf16 output inside the master
    assert call(norm=v + 64) == B.ZS_EOVERLAP                       # norm inside a written buffer
    assert call(k=(1 << 39) + 1) == B.ZS_EINVAL
    assert call(k=0) == B.ZS_OK
    sc = FAKE + 2**30
    dev = lambda s=sc, k=n: L.adamw_step_sum_dev(s, p, m, v, acc0, g0, B.ZS_BF16, 0, k, 0, None)
    assert dev(s=0) == B.ZS_EINVAL
    assert dev(s=sc + 4) == B.ZS_EINVAL
    assert dev(s=m + 8) == B.ZS_EOVERLAP                            # scalars inside exp_avg
    assert dev(k=0) == B.ZS_OK


def test_grad_reduce_chunks_norm_sq_rejects():
    L = zs.lib()
    n = 1 << 20
    need = zs.grad_reduce_chunks_norm_sq_workspace_bytes(n)
    assert need == (n // 512 + 2048) * 8         # one partial per 512 elements + the chunk stage
    assert zs.grad_reduce_chunks_norm_sq_workspace_bytes(0) == 0
    assert zs.grad_reduce_chunks_norm_sq_workspace_bytes(2**39 + 1) == -1
    acc, ws, out = FAKE, FAKE + 2**31, FAKE + 2**32
    chunks = (ctypes.c_void_p * 2)(FAKE + 2**30, FAKE + 2**30 + 2**22)
    call = lambda **k: L.grad_reduce_chunks_norm_sq(
        k.get("acc", acc), k.get("chunks", chunks), k.get("count", 2), k.get("dt", B.ZS_BF16), k.get("n", n), 1,
        k.get("s", 1.0), k.get("out", out), k.get("ws", ws), k.get("wsb", need), None)
    assert call(count=0) == B.ZS_EINVAL and call(count=-1) == B.ZS_EINVAL
    assert call(wsb=need - 8) == B.ZS_EWORKSPACE
    assert call(dt=5) == B.ZS_EINVAL
    assert call(chunks=None) == B.ZS_EINVAL
    assert call(out=0) == B.ZS_EINVAL and call(out=out + 4) == B.ZS_EINVAL
    assert call(s=float("inf")) == B.ZS_EINVAL and call(s=0.0) == B.ZS_EINVAL
    assert call(acc=0) == B.ZS_EINVAL and call(acc=acc + 2) == B.ZS_EINVAL
    assert call(ws=0) == B.ZS_EINVAL
    assert call(chunks=(ctypes.c_void_p * 2)(FAKE + 2**30, FAKE + 64)) == B.ZS_EOVERLAP   # a chunk inside acc
    assert call(chunks=(ctypes.c_void_p * 2)(FAKE + 2**30, FAKE + 2**30 + 1)) == B.ZS_EINVAL  # odd bf16 address
    assert call(out=FAKE + 16) == B.ZS_EOVERLAP                    # norm inside acc
    assert call(ws=FAKE + 2**30 + 1024) == B.ZS_EOVERLAP           # workspace inside a chunk
    assert call(n=-1) == B.ZS_EINVAL


def _tensors(*pairs):
    arr = (B.Tensor * len(pairs))()
    for i, (p, k) in enumerate(pairs):
        arr[i].ptr, arr[i].numel = p, k
    return arr


def test_flat_rejects():
    L = zs.lib()
    flat = FAKE + 2**30
    two = _tensors((FAKE, 10), (FAKE + 2**20, 6))
    assert L.flat_pack(two, 2, B.ZS_F32, flat, B.ZS_F32, 15, None) == B.ZS_EINVAL      # padded < total
    assert L.flat_pack(two, 2, B.ZS_F32, flat, B.ZS_BF16, 16, None) == B.ZS_EINVAL     # narrowing pack
    assert L.flat_unpack(flat, B.ZS_BF16, two, 2, B.ZS_F32, None) == B.ZS_EINVAL       # widening unpack
    assert L.flat_pack(two, -1, B.ZS_F32, flat, B.ZS_F32, 16, None) == B.ZS_EINVAL
    assert L.flat_pack(_tensors((0, 4)), 1, B.ZS_F32, flat, B.ZS_F32, 4, None) == B.ZS_EINVAL
    assert L.flat_pack(_tensors((FAKE + 2, 4)), 1, B.ZS_F32, flat, B.ZS_F32, 4, None) == B.ZS_EINVAL
    assert L.flat_pack(_tensors((FAKE, -4)), 1, B.ZS_F32, flat, B.ZS_F32, 4, None) == B.ZS_EINVAL
    assert L.flat_pack(two, 2, B.ZS_F32, 0, B.ZS_F32, 16, None) == B.ZS_EINVAL
    assert L.flat_pack(_tensors((flat + 8, 4)), 1, B.ZS_F32, flat, B.ZS_F32, 8, None) == B.ZS_EOVERLAP
    # unpack destinations must not overlap each other
    assert L.flat_unpack(flat, B.ZS_F32, _tensors((FAKE, 8), (FAKE + 16, 8)), 2, B.ZS_F32,
                         None) == B.ZS_EOVERLAP
    # nothing to do
    assert L.flat_pack(None, 0, B.ZS_F32, 0, B.ZS_F32, 0, None) == B.ZS_OK
    assert L.flat_unpack(flat, B.ZS_F32, _tensors((0, 0)), 1, B.ZS_F32, None) == B.ZS_OK


def test_strerror():
    L = zs.lib()
    for code in (B.ZS_OK, B.ZS_EINVAL, B.ZS_EOVERLAP, B.ZS_EWORKSPACE, B.ZS_EHIP, 12345):
        assert isinstance(L.zs_strerror(code), bytes)
    assert L.zs_last_hip_error() == 0


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        zs.grad_accum(torch.zeros(4), torch.zeros(4), overwrite=True)


def test_element_count_limit():
    """More than 2^39 elements in one call is refused before any launch
    (every launch grid then fits 32 bits); far-apart fake buffers so that only
    the count is wrong."""
    L = zs.lib()
    big = (1 << 39) + 1
    step = 1 << 42
    a, g = FAKE, FAKE + step
    assert L.grad_accum(a, g, B.ZS_BF16, big, 1, None) == B.ZS_EINVAL
    assert L.grad_reduce_chunks(a, (ctypes.c_void_p * 1)(g), 1, B.ZS_BF16, big, 1, None) == B.ZS_EINVAL
    assert L.grad_norm_sq(a, big, 1.0, g, FAKE + 2 * step, 1 << 40, None) == B.ZS_EINVAL
    assert _adamw(_hp(), master=FAKE, m=FAKE + step, v=FAKE + 2 * step, g=FAKE + 3 * step, n=big) == B.ZS_EINVAL
    assert L.flat_unpack(a, B.ZS_F32, _tensors((g, big)), 1, B.ZS_F32, None) == B.ZS_EINVAL
    half = (1 << 38) + 1   # each tensor allowed, their sum not
    assert L.flat_unpack(a, B.ZS_F32, _tensors((g, half), (g + step, half)), 2, B.ZS_F32, None) == B.ZS_EINVAL


def test_ceiling_library_rejects_before_launch():
    """The benchmark's bandwidth-ceiling kernels (libzsceiling.so: the split
    and the tiled state layout) reject bad arguments, or return for n == 0,
    without a launch (a launch attempt here would return a HIP error, not -1
    or 0)."""
    from fsdp_sharded_optimizer_amd import build as zbuild
    if not os.path.exists(zbuild.CEILING_LIB):
        pytest.skip("libzsceiling.so not built")
    L = ctypes.CDLL(zbuild.CEILING_LIB)
    f = L.zsc_adamw_traffic
    f.restype = ctypes.c_int32
    f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]
    a = 1 << 20   # 16-byte aligned, never dereferenced: every call below fails validation or is a no-op
    assert f(a, a + 64, a + 128, a + 192, None, 0, 0, None) == 0           # empty: nothing to do
    assert f(a, a + 64, a + 128, a + 192, None, -1, 0, None) == -1         # negative n
    assert f(a, a + 64, a + 128, a + 192, None, (1 << 39) + 1, 0, None) == -1
    assert f(None, a + 64, a + 128, a + 192, None, 16, 0, None) == -1      # null buffer
    assert f(a + 4, a + 64, a + 128, a + 192, None, 16, 0, None) == -1     # written buffer off 16 bytes
    assert f(a, a + 64, a + 128, a + 194, None, 16, 0, None) == -1         # grad off 4 bytes
    assert f(a, a + 64, a + 128, a + 192, a + 258, 16, 0, None) == -1      # bf16 output off 16 bytes
    assert f(a, a + 64, a + 128, a + 192, None, 16, -1, None) == -1        # LDS reservation out of range
    assert f(a, a + 64, a + 128, a + 192, None, 16, 65537, None) == -1
    t = L.zsc_adamw_traffic_tiled
    t.restype = ctypes.c_int32
    t.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]
    assert t(a, a + 64, None, 0, 0, None) == 0
    assert t(a, a + 64, None, -1, 0, None) == -1
    assert t(a, a + 64, None, (1 << 31) + 1, 0, None) == -1               # one launch at most
    assert t(None, a + 64, None, 16, 0, None) == -1
    assert t(a + 4, a + 64, None, 16, 0, None) == -1                       # state off 16 bytes
    assert t(a, a + 66, None, 16, 0, None) == -1                           # grad off 4 bytes
    assert t(a, a + 64, a + 130, 16, 0, None) == -1                        # bf16 output off 16 bytes
    assert t(a, a + 64, None, 16, 70000, None) == -1
    u = L.zsc_adamw_traffic_tiled_sum
    u.restype = ctypes.c_int32
    u.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]
    assert u(a, a + 64, a + 128, None, 0, 0, None) == 0
    assert u(a, a + 64, a + 128, None, (1 << 31) + 1, 0, None) == -1
    assert u(a, a + 64, None, None, 16, 0, None) == -1                     # no gradient
    assert u(a + 8, None, a + 128, None, 16, 0, None) == -1                # state off 16 bytes
    assert u(a, a + 66, a + 128, None, 16, 0, None) == -1                  # accumulator off 4 bytes
    assert u(a, a + 64, a + 130, None, 16, 0, None) == -1                  # bf16 gradient off 4 bytes
    assert u(a, None, a + 128, a + 136, 16, 0, None) == -1                 # bf16 output off 16 bytes
    assert u(a, None, a + 128, None, 16, -5, None) == -1


def test_plain_c_consumer(tmp_path):
    """include/zshard.h compiles as strict C11 and libzshard.so links from C:
    tests/c_consumer.c (host-only calls and rejecting paths) builds with gcc
    -Wall -Wextra -Wpedantic -Werror and runs clean."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "c_consumer")
    libdir = os.path.dirname(B.LIB_PATH)
    subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Wpedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
                    "-o", exe, os.path.join(ROOT, "tests", "c_consumer.c"), B.LIB_PATH,
                    f"-Wl,-rpath,{libdir}"], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, (out.returncode, out.stderr)
    assert out.stdout.strip() == "c consumer: ok"


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    """No fallback path: with the library absent every call raises."""
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "libzshard.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        B.lib()
    with pytest.raises(RuntimeError):
        zs.zero_shard_range(10, 2, 0)


def test_product_code_does_not_use_the_oracle():
    """The package (binding, call ordering, ledger, HIP sources) neither
    imports nor loads anything under oracle/."""
    pkg = os.path.join(ROOT, "fsdp_sharded_optimizer_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".c", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, flags=re.M), f
                assert "orc_" not in text and "liboracle" not in text and "oracle/" not in text, f


def test_noalloc_rejects_before_any_device_call():
    """grad_accum_norm_sq_noalloc validates on the host first: a size beyond
    its scratch, a bad dtype or scale, null or misaligned pointers come back
    ZS_EINVAL without a HIP call (no GPU here; the fixture checks that no
    launch was attempted)."""
    L = zs.lib()
    f = L.grad_accum_norm_sq_noalloc
    acc, g, out = FAKE, FAKE + 2**32, FAKE + 2**33
    assert B.NOALLOC_MAX_ELEMS == 2_146_959_360
    assert zs.grad_accum_norm_sq_workspace_bytes(B.NOALLOC_MAX_ELEMS) == 64 << 20
    for n in (B.NOALLOC_MAX_ELEMS + 1, 1 << 39, -1):
        assert f(acc, g, B.ZS_BF16, n, 0, 1.0, out, None) == B.ZS_EINVAL, n
    assert f(acc, g, 7, 16, 0, 1.0, out, None) == B.ZS_EINVAL
    assert f(acc, g, B.ZS_BF16, 16, 0, 0.0, out, None) == B.ZS_EINVAL
    assert f(acc, g, B.ZS_BF16, 16, 0, float("nan"), out, None) == B.ZS_EINVAL
    assert f(acc, g, B.ZS_BF16, 16, 0, 1.0, None, None) == B.ZS_EINVAL
    assert f(acc, g, B.ZS_BF16, 16, 0, 1.0, out + 4, None) == B.ZS_EINVAL
    assert f(None, g, B.ZS_BF16, 16, 0, 1.0, out, None) == B.ZS_EINVAL
    assert f(acc + 2, g, B.ZS_BF16, 16, 0, 1.0, out, None) == B.ZS_EINVAL
    assert f(acc, g + 1, B.ZS_BF16, 16, 0, 1.0, out, None) == B.ZS_EINVAL
