"""Property tests of the C ABI's host-side validation (CPU only).

Random argument sets for adamw_step, flat_pack and flat_unpack, for the
tiled-state calls (adamw_step_tiled, state_tile, state_untile), and for
the one-pass last micro-batch (adamw_step_tiled_sum, adamw_step_sum,
grad_sum_norm_sq): sizes, alignments, null pointers, overlapping buffers
and hyperparameters.  A
Python model of the rules include/zshard.h documents (and of the order in
which they are checked) predicts each return code.  Only argument sets the
model says must fail, or are no-ops, are passed to the library, so no call
reaches a kernel launch; the autouse fixture also checks that no HIP error
was left behind.  Pointers are never dereferenced.
"""
import ctypes
import math

import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import fsdp_sharded_optimizer_amd as zs
from fsdp_sharded_optimizer_amd import _binding as B

BASE = 0x7F0000000000      # fake device addresses, never dereferenced
MAX_ELEMS = 1 << 39
EINVAL, EOVERLAP, OK = B.ZS_EINVAL, B.ZS_EOVERLAP, B.ZS_OK

SETTINGS = settings(max_examples=1500, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@pytest.fixture(autouse=True)
def no_launch_reached():
    yield
    assert zs.lib().zs_last_hip_error() == 0, "a call got past validation to a kernel launch"


def overlap(p, nbytes, q, qbytes):
    if nbytes <= 0 or qbytes <= 0:
        return False
    return p < q + qbytes and q < p + nbytes


# A pointer: rarely null, else one of a few slots 4 KiB apart (so that
# buffers of a few thousand bytes often overlap) plus a byte offset (mostly
# aligned, sometimes 1 or 2 bytes off).
pointers = st.sampled_from([0] + [None] * 9).flatmap(
    lambda z: st.just(0) if z == 0 else st.builds(lambda slot, off: BASE + slot * 4096 + off, st.integers(0, 7),
                                                    st.sampled_from([0, 0, 0, 4, 8, 16, 64, 1, 2, 6])))
odd_values = st.sampled_from([0.0, -0.0, -1e-3, 1.0, 1.5, math.inf, -math.inf, math.nan, 1e-300])
VALID_HP = (3e-4, 0.9, 0.95, 1e-8, 0.1, 1.0 / 64, 1.0, 0.5, 3)


@st.composite
def hyperparameters(draw):
    """A valid set, or (half the time) one field replaced by an odd value."""
    hp = list(VALID_HP)
    if draw(st.booleans()):
        i = draw(st.integers(0, 8))
        hp[i] = draw(st.integers(-2, 1)) if i == 8 else draw(odd_values)
    return tuple(hp)


# ---------------------------------------------------------------------------
# adamw_step
# ---------------------------------------------------------------------------

def adamw_model(hp, ptrs, n, norm):
    lr, b1, b2, eps, wd, scale, max_norm, extra, step = hp
    if not (0 <= n <= MAX_ELEMS) or step < 1:
        return EINVAL
    if not (0.0 <= b1 < 1.0) or not (0.0 <= b2 < 1.0):
        return EINVAL
    if not (eps > 0.0 and math.isfinite(eps)) or not (lr >= 0.0 and math.isfinite(lr)):
        return EINVAL
    if not (wd >= 0.0 and math.isfinite(wd)) or not (scale > 0.0 and math.isfinite(scale)):
        return EINVAL
    if math.isnan(max_norm) or extra < 0.0:
        return EINVAL
    if norm and norm % 8:
        return EINVAL
    if n == 0:
        return OK
    master, m, v, g, b = ptrs
    if not (master and m and v and g):
        return EINVAL
    if master % 4 or m % 4 or v % 4 or g % 4 or (b and b % 2):
        return EINVAL
    bufs = [(master, 4 * n, True), (m, 4 * n, True), (v, 4 * n, True), (g, 4 * n, False), (b, 2 * n if b else 0, True)]
    for i in range(5):
        for j in range(i + 1, 5):
            if overlap(bufs[i][0], bufs[i][1], bufs[j][0], bufs[j][1]):
                return EOVERLAP
        if norm and bufs[i][2] and overlap(bufs[i][0], bufs[i][1], norm, 8):
            return EOVERLAP
    return None   # valid: would launch


@SETTINGS
@given(hp=hyperparameters(),
       ptrs=st.tuples(pointers, pointers, pointers, pointers, pointers),
       n=st.sampled_from([-1, 0, 1, 3, 64, 1000, 1000, 1500, 5000, MAX_ELEMS + 1]),
       norm=st.one_of(st.just(0), st.builds(lambda slot, off: BASE + slot * 4096 + off,
                                            st.integers(0, 7), st.sampled_from([0, 8, 4000, 4]))))
def test_adamw_step_validation_matches_the_documented_rules(hp, ptrs, n, norm):
    want = adamw_model(hp, ptrs, n, norm)
    if want is None:
        return   # a valid call would launch a kernel: not made here
    c = B.AdamW(*hp[:8], hp[8])
    got = zs.lib().adamw_step(ctypes.byref(c), *[p or None for p in ptrs], n, norm or None, None)
    assert got == want, (hp, [hex(p) for p in ptrs], n, hex(norm))


# ---------------------------------------------------------------------------
# flat_pack / flat_unpack
# ---------------------------------------------------------------------------

def flat_model(tensors, count, flat, flat_dt, t_dt, padded, unpack):
    if count < 0:
        return EINVAL
    if flat_dt not in (0, 1) or t_dt not in (0, 1):
        return EINVAL
    if flat_dt != t_dt and not ((not unpack and t_dt == 1 and flat_dt == 0) or (unpack and flat_dt == 0 and t_dt == 1)):
        return EINVAL
    fsz, tsz = (4 if flat_dt == 0 else 2), (4 if t_dt == 0 else 2)
    total = 0
    for p, k in tensors[:count]:
        if not (0 <= k <= MAX_ELEMS) or total > MAX_ELEMS - k:
            return EINVAL
        if k > 0 and (not p or p % tsz):
            return EINVAL
        total += k
    if unpack:
        padded = total
    if not (0 <= padded <= MAX_ELEMS) or total > padded:
        return EINVAL
    if padded == 0:
        return OK
    if not flat or flat % fsz:
        return EINVAL
    for i, (p, k) in enumerate(tensors[:count]):
        if overlap(p, k * tsz, flat, padded * fsz):
            return EOVERLAP
        if unpack:
            for q, kk in tensors[i + 1:count]:
                if overlap(p, k * tsz, q, kk * tsz):
                    return EOVERLAP
    return None


numels = st.sampled_from([0, 1, 5, 300, 1000, 2000, 1000, 300, -1, MAX_ELEMS])
tensor_lists = st.lists(st.tuples(pointers, numels), min_size=0, max_size=4)
dtype_pairs = st.sampled_from([(0, 0), (1, 1), (0, 1), (1, 0), (0, 0), (1, 1), (0, 1), (2, 0), (0, -1)])


@SETTINGS
@given(tensors=tensor_lists, flat=pointers, dts=dtype_pairs,
       pad=st.sampled_from([0, 0, 3, 700, -1, MAX_ELEMS + 1]), unpack=st.booleans(),
       count_delta=st.sampled_from([0, 0, 0, 0, 0, -1]))
def test_flat_validation_matches_the_documented_rules(tensors, flat, dts, pad, unpack, count_delta):
    """dts = (flat dtype, tensor dtype); the pack's padded_total is the
    tensors' total plus pad (or pad itself when it is out of range)."""
    flat_dt, t_dt = dts
    count = len(tensors) if count_delta == 0 else -1
    total = sum(max(k, 0) for _, k in tensors)
    padded = pad if pad < 0 or pad > MAX_ELEMS else total + pad
    want = flat_model(tensors, count, flat, flat_dt, t_dt, padded, unpack)
    if want is None:
        return
    arr = (B.Tensor * max(len(tensors), 1))()
    for i, (p, k) in enumerate(tensors):
        arr[i].ptr, arr[i].numel = p or None, k
    L = zs.lib()
    if unpack:
        got = L.flat_unpack(flat or None, flat_dt, arr, count, t_dt, None)
    else:
        got = L.flat_pack(arr, count, t_dt, flat or None, flat_dt, padded, None)
    assert got == want, (tensors, count, hex(flat), flat_dt, t_dt, padded, unpack)


# ---------------------------------------------------------------------------
# tiled state: adamw_step_tiled, state_tile, state_untile
# ---------------------------------------------------------------------------

TILE = 8192   # ZS_STATE_TILE (test_abi checks the header against this value)


def tiled_bytes(n):
    return 4 * 3 * TILE * (-(-n // TILE))


# slots 64 KiB apart: a tiled state of up to one tile (96 KiB) overlaps the next slot or two
big_pointers = st.sampled_from([0] + [None] * 9).flatmap(
    lambda z: st.just(0) if z == 0 else st.builds(lambda slot, off: BASE + slot * 65536 + off, st.integers(0, 7),
                                                    st.sampled_from([0, 0, 0, 4, 8, 16, 64, 1, 2, 6])))
tiled_sizes = st.sampled_from([-1, 0, 1, 3, 1000, 5000, 8192, 9000, MAX_ELEMS + 1])


def hp_model(hp, n, norm):
    """adamw_step's shared hyperparameter, size and norm-alignment checks."""
    lr, b1, b2, eps, wd, scale, max_norm, extra, step = hp
    if not (0 <= n <= MAX_ELEMS) or step < 1:
        return EINVAL
    if not (0.0 <= b1 < 1.0) or not (0.0 <= b2 < 1.0):
        return EINVAL
    if not (eps > 0.0 and math.isfinite(eps)) or not (lr >= 0.0 and math.isfinite(lr)):
        return EINVAL
    if not (wd >= 0.0 and math.isfinite(wd)) or not (scale > 0.0 and math.isfinite(scale)):
        return EINVAL
    if math.isnan(max_norm) or extra < 0.0:
        return EINVAL
    if norm and norm % 8:
        return EINVAL
    return None


def tiled_step_model(hp, state, g, b, n, norm):
    rc = hp_model(hp, n, norm)
    if rc is not None:
        return rc
    if n == 0:
        return OK
    if not (state and g):
        return EINVAL
    if state % 16 or g % 4 or (b and b % 2):
        return EINVAL
    bufs = [(state, tiled_bytes(n), True), (g, 4 * n, False), (b, 2 * n if b else 0, True)]
    for i in range(3):
        for j in range(i + 1, 3):
            if overlap(bufs[i][0], bufs[i][1], bufs[j][0], bufs[j][1]):
                return EOVERLAP
        if norm and bufs[i][2] and overlap(bufs[i][0], bufs[i][1], norm, 8):
            return EOVERLAP
    return None


@SETTINGS
@given(hp=hyperparameters(), ptrs=st.tuples(big_pointers, big_pointers, big_pointers), n=tiled_sizes,
       norm=st.one_of(st.just(0), st.builds(lambda slot, off: BASE + slot * 65536 + off,
                                            st.integers(0, 7), st.sampled_from([0, 8, 40000, 4]))))
def test_adamw_step_tiled_validation_matches_the_documented_rules(hp, ptrs, n, norm):
    state, g, b = ptrs
    want = tiled_step_model(hp, state, g, b, n, norm)
    if want is None:
        return   # a valid call would launch a kernel: not made here
    c = B.AdamW(*hp[:8], hp[8])
    got = zs.lib().adamw_step_tiled(ctypes.byref(c), state or None, g or None, b or None, n, norm or None, None)
    assert got == want, (hp, [hex(p) for p in ptrs], n, hex(norm))


def tile_model(srcs, state, n):
    if not (0 <= n <= MAX_ELEMS):
        return EINVAL
    if n == 0:
        return OK
    if not state or state % 16:
        return EINVAL
    for src in srcs:
        if src and src % 4:
            return EINVAL
        if src and overlap(src, 4 * n, state, tiled_bytes(n)):
            return EOVERLAP
    return None


def untile_model(state, dsts, n):
    if not (0 <= n <= MAX_ELEMS):
        return EINVAL
    if n == 0:
        return OK
    if not state or state % 16:
        return EINVAL
    for k, d in enumerate(dsts):
        if not d:
            continue
        if d % 4:
            return EINVAL
        if overlap(d, 4 * n, state, tiled_bytes(n)):
            return EOVERLAP
        for e in dsts[k + 1:]:
            if e and overlap(d, 4 * n, e, 4 * n):
                return EOVERLAP
    return None


@SETTINGS
@given(ptrs=st.tuples(big_pointers, big_pointers, big_pointers, big_pointers), n=tiled_sizes, untile=st.booleans())
def test_state_tile_validation_matches_the_documented_rules(ptrs, n, untile):
    a, b, c, state = ptrs
    L = zs.lib()
    if untile:
        want = untile_model(state, (a, b, c), n)
        if want is None:
            return
        got = L.state_untile(state or None, a or None, b or None, c or None, n, None)
    else:
        want = tile_model((a, b, c), state, n)
        if want is None:
            return
        got = L.state_tile(a or None, b or None, c or None, state or None, n, None)
    assert got == want, (untile, [hex(p) for p in ptrs], n)


def moments_update_model(hp, moments, g, u, n, norm):
    rc = hp_model(hp, n, norm)
    if rc is not None:
        return rc
    if hp[4] != 0.0:   # weight decay
        return EINVAL
    if n == 0:
        return OK
    if not (moments and g and u):
        return EINVAL
    if moments % 16 or g % 4 or u % 4:
        return EINVAL
    bufs = [(moments, 4 * 2 * TILE * (-(-n // TILE)), True), (g, 4 * n, False), (u, 4 * n, True)]
    for i in range(3):
        for j in range(i + 1, 3):
            if overlap(bufs[i][0], bufs[i][1], bufs[j][0], bufs[j][1]):
                return EOVERLAP
        if norm and bufs[i][2] and overlap(bufs[i][0], bufs[i][1], norm, 8):
            return EOVERLAP
    return None


@SETTINGS
@given(hp=hyperparameters(), ptrs=st.tuples(big_pointers, big_pointers, big_pointers), n=tiled_sizes,
       wd0=st.booleans(),
       norm=st.one_of(st.just(0), st.builds(lambda slot, off: BASE + slot * 65536 + off,
                                            st.integers(0, 7), st.sampled_from([0, 8, 40000, 4]))))
def test_adam_update_tiled_validation_matches_the_documented_rules(hp, ptrs, n, wd0, norm):
    if wd0:
        hp = hp[:4] + (0.0,) + hp[5:]
    mo, g, u = ptrs
    want = moments_update_model(hp, mo, g, u, n, norm)
    if want is None:
        return
    c = B.AdamW(*hp[:8], hp[8])
    got = zs.lib().adam_update_tiled(ctypes.byref(c), mo or None, g or None, u or None, n, norm or None, None)
    assert got == want, (hp, [hex(p) for p in ptrs], n, hex(norm))


# ---------------------------------------------------------------------------
# the one-pass last micro-batch: adamw_step_tiled_sum, grad_sum_norm_sq
# ---------------------------------------------------------------------------

F32, BF16 = B.ZS_F32, B.ZS_BF16
dtypes = st.sampled_from([F32, BF16, BF16, 7])


def tiled_sum_model(hp, state, acc, g, dt, b, n, norm):
    rc = hp_model(hp, n, norm)
    if rc is not None:
        return rc
    if dt not in (F32, BF16):
        return EINVAL
    if n == 0:
        return OK
    gsz = 4 if dt == F32 else 2
    if not (state and g):
        return EINVAL
    if state % 16 or g % gsz or (acc and acc % 4) or (b and b % 2):
        return EINVAL
    bufs = [(state, tiled_bytes(n), True), (acc, 4 * n if acc else 0, False), (g, gsz * n, False),
            (b, 2 * n if b else 0, True)]
    for i in range(4):
        for j in range(i + 1, 4):
            if overlap(bufs[i][0], bufs[i][1], bufs[j][0], bufs[j][1]):
                return EOVERLAP
        if norm and bufs[i][2] and overlap(bufs[i][0], bufs[i][1], norm, 8):
            return EOVERLAP
    return None


@SETTINGS
@given(hp=hyperparameters(), ptrs=st.tuples(big_pointers, big_pointers, big_pointers, big_pointers),
       dt=dtypes, n=tiled_sizes,
       norm=st.one_of(st.just(0), st.builds(lambda slot, off: BASE + slot * 65536 + off,
                                            st.integers(0, 7), st.sampled_from([0, 8, 40000, 4]))))
def test_adamw_step_tiled_sum_validation_matches_the_documented_rules(hp, ptrs, dt, n, norm):
    state, acc, g, b = ptrs
    want = tiled_sum_model(hp, state, acc, g, dt, b, n, norm)
    if want is None:
        return   # a valid call would launch a kernel: not made here
    c = B.AdamW(*hp[:8], hp[8])
    got = zs.lib().adamw_step_tiled_sum(ctypes.byref(c), state or None, acc or None, g or None, dt, b or None, n,
                                        norm or None, None)
    assert got == want, (hp, [hex(p) for p in ptrs], dt, n, hex(norm))


def sum_norm_workspace(n):
    return 0 if n <= 0 else ((n + 255) // 256 + 2048) * 8


def sum_norm_model(acc, g, dt, n, overwrite, scale, out, ws, wsb):
    if dt not in (F32, BF16) or not (0 <= n <= MAX_ELEMS):
        return EINVAL
    if not out or out % 8:
        return EINVAL
    if not (scale > 0.0 and math.isfinite(scale)):
        return EINVAL
    gsz = 4 if dt == F32 else 2
    if overwrite:
        acc = 0   # not read
    if n > 0 and (not g or g % gsz):
        return EINVAL
    if n > 0 and not overwrite and (not acc or acc % 4):
        return EINVAL
    need = sum_norm_workspace(n)
    if need > 0 and (not ws or ws % 8):
        return EINVAL
    if wsb < need:
        return B.ZS_EWORKSPACE
    acc_bytes = 4 * n if acc else 0
    if (overlap(acc, acc_bytes, out, 8) or overlap(g, gsz * n, out, 8) or overlap(ws, need, out, 8)
            or overlap(ws, need, acc, acc_bytes) or overlap(ws, need, g, gsz * n)):
        return EOVERLAP
    return None


@SETTINGS
@given(ptrs=st.tuples(pointers, pointers, pointers, pointers), dt=dtypes,
       n=st.sampled_from([-1, 0, 1, 3, 255, 1000, 5000, MAX_ELEMS + 1]), overwrite=st.booleans(),
       scale=st.sampled_from([1.0 / 64, 1.0 / 64, 0.0, -1.0, math.inf, math.nan]),
       ws_short=st.sampled_from([0, 0, 0, 8]))
def test_grad_sum_norm_sq_validation_matches_the_documented_rules(ptrs, dt, n, overwrite, scale, ws_short):
    acc, g, out, ws = ptrs
    need = sum_norm_workspace(n)
    wsb = max(need - ws_short, 0)
    want = sum_norm_model(acc, g, dt, n, overwrite, scale, out, ws, wsb)
    if want is None:
        return   # a valid call would launch a kernel (n == 0 too: it writes the norm 0)
    got = zs.lib().grad_sum_norm_sq(acc or None, g or None, dt, n, 1 if overwrite else 0, scale, out or None,
                                    ws or None, wsb, None)
    assert got == want, ([hex(p) for p in ptrs], dt, n, overwrite, scale, wsb)


def split_sum_model(hp, p, m, v, acc, g, dt, b, n, norm):
    rc = hp_model(hp, n, norm)
    if rc is not None:
        return rc
    if dt not in (F32, BF16):
        return EINVAL
    if n == 0:
        return OK
    gsz = 4 if dt == F32 else 2
    if not (p and m and v and g):
        return EINVAL
    if p % 4 or m % 4 or v % 4 or g % gsz or (acc and acc % 4) or (b and b % 2):
        return EINVAL
    bufs = [(p, 4 * n, True), (m, 4 * n, True), (v, 4 * n, True), (acc, 4 * n if acc else 0, False),
            (g, gsz * n, False), (b, 2 * n if b else 0, True)]
    for i in range(6):
        for j in range(i + 1, 6):
            if overlap(bufs[i][0], bufs[i][1], bufs[j][0], bufs[j][1]):
                return EOVERLAP
        if norm and bufs[i][2] and overlap(bufs[i][0], bufs[i][1], norm, 8):
            return EOVERLAP
    return None


@SETTINGS
@given(hp=hyperparameters(), ptrs=st.tuples(pointers, pointers, pointers, pointers, pointers, pointers),
       dt=dtypes, n=st.sampled_from([-1, 0, 1, 3, 255, 1000, MAX_ELEMS + 1]),
       norm=st.one_of(st.just(0), st.builds(lambda slot, off: BASE + slot * 4096 + off,
                                            st.integers(0, 7), st.sampled_from([0, 8, 2000, 4]))))
def test_adamw_step_sum_validation_matches_the_documented_rules(hp, ptrs, dt, n, norm):
    p, m, v, acc, g, b = ptrs
    want = split_sum_model(hp, p, m, v, acc, g, dt, b, n, norm)
    if want is None:
        return   # a valid call would launch a kernel: not made here
    c = B.AdamW(*hp[:8], hp[8])
    got = zs.lib().adamw_step_sum(ctypes.byref(c), p or None, m or None, v or None, acc or None, g or None, dt,
                                  b or None, n, norm or None, None)
    assert got == want, (hp, [hex(x) for x in ptrs], dt, n, hex(norm))
