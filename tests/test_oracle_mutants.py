"""The oracle's pins catch plausible mistakes (CPU only).

Each mutant is a copy of oracle/oracle.c with one deliberate slip — a
swapped beta, a dropped factor, eps on the wrong side of the division, an
off-by-one in the step counter or an index, a truncating cast, a floor
instead of a ceiling.  The copy is compiled to a temporary library, the
oracle is routed to it, and the fast pins of test_oracle_pins.py run
against it: every mutant must fail at least one of them, and the
unmutated source must pass them all.  Every slip keeps memory accesses in
bounds, so a mutant can only compute wrong values.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
import tests.test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "oracle.c")

# (name, text in oracle.c, replacement); every occurrence is replaced (a slip
# in arithmetic the two AdamW forms share is made in both)
MUTANTS = [
    ("bf16: ties always round down",
     "if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1u;", "if (lo > 0x8000u) hi += 1u;"),
    ("bf16: ties always round up",
     "if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1u;", "if (lo >= 0x8000u) hi += 1u;"),
    ("bf16: NaN not canonicalised", "if (isnan(x)) return (uint16_t)0x7FC0;", ""),
    ("widen: wrong shift", "return bits_f32((uint32_t)b << 16);", "return bits_f32((uint32_t)b << 15);"),
    ("shard: floor instead of ceiling", "int64_t chunk = (total + world - 1) / world;",
     "int64_t chunk = total / world;"),
    ("shard: start not clamped to total", "if (start > total) start = total;", ""),
    ("shard: end not clipped", "if (end > total) end = total;", ""),
    ("pack: first padding element left unwritten", "for (int64_t k = total; k < padded_total; ++k) {",
     "for (int64_t k = total + 1; k < padded_total; ++k) {"),
    ("pack: offsets lag by one after the first tensor",
     "            convert_one(src[t], src_dtype, j, flat, flat_dtype, offset + j);\n        offset += numel[t];",
     "            convert_one(src[t], src_dtype, j, flat, flat_dtype, offset + j - (offset > 0 && j > 0));\n"
     "        offset += numel[t];"),
    ("unpack: reads the previous element",
     "convert_one(flat, flat_dtype, offset + j, dst[t], dst_dtype, j);",
     "convert_one(flat, flat_dtype, offset + j - (j > 0), dst[t], dst_dtype, j);"),
    ("accum: overwrite ignored", "if (overwrite) acc[i] = g;", "if (0) acc[i] = g;"),
    ("accum: adds twice", "else acc[i] = acc[i] + g;", "else acc[i] = acc[i] + g + g;"),
    ("norm: scale dropped", "float g1 = acc[i] * s32;", "float g1 = acc[i];"),
    ("norm: last element of each block dropped",
     "int64_t hi = lo + ORC_NORM_BLOCK < n ? lo + ORC_NORM_BLOCK : n;",
     "int64_t hi = lo + ORC_NORM_BLOCK < n ? lo + ORC_NORM_BLOCK - 1 : n - 1;"),
    ("clip: no 1e-6 in the denominator", "double coef = max_norm / (total + 1e-6);",
     "double coef = max_norm / total;"),
    ("clip: not clamped to 1", "if (coef > 1.0) coef = 1.0;", ""),
    ("clip: other ranks ignored", "double total = sqrt(norm_sq_local + extra_norm_sq);",
     "double total = sqrt(norm_sq_local);"),
    ("scalars: step counter off by one", "double bc1 = 1.0 - pow(hp->beta1, (double)hp->step);",
     "double bc1 = 1.0 - pow(hp->beta1, (double)hp->step + 1.0);"),
    ("scalars: second correction uses beta1", "double bc2 = 1.0 - pow(hp->beta2, (double)hp->step);",
     "double bc2 = 1.0 - pow(hp->beta1, (double)hp->step);"),
    ("scalars: sqrt of the second correction dropped", "s->bias_correction2_sqrt = (float)sqrt(bc2);",
     "s->bias_correction2_sqrt = (float)bc2;"),
    ("scalars: step size multiplies by the correction", "s->step_size = (float)(hp->lr / bc1);",
     "s->step_size = (float)(hp->lr * bc1);"),
    ("scalars: decay without lr", "s->decay = (float)(1.0 - hp->lr * hp->weight_decay);",
     "s->decay = (float)(1.0 - hp->weight_decay);"),
    ("adamw: grad scale dropped", "float g = grad[i] * s.grad_scale;", "float g = grad[i];"),
    ("adamw: clip coefficient not applied", "        g = g * coef;\n", ""),
    ("adamw: first moment decays with beta2", "float m_a = s.beta1 * m;", "float m_a = s.beta2 * m;"),
    ("adamw: (1 - beta2) dropped", "float v_b = s.one_minus_beta2 * gg;", "float v_b = gg;"),
    ("adamw: eps before the bias correction",
     "float den = root / s.bias_correction2_sqrt;\n        den = den + s.eps;",
     "float den = root + s.eps;\n        den = den / s.bias_correction2_sqrt;"),
    ("adamw: decay not applied", "float pd = p * s.decay;", "float pd = p;"),
    ("adamw: update added instead of subtracted", "p = pd - u;", "p = pd + u;"),
    ("adamw: bf16 cast of the old master", "param_bf16[i] = orc_bf16_rne(p);",
     "param_bf16[i] = orc_bf16_rne(pd);"),
    ("adamw: non-finite norm not skipped", "if (!isfinite(S)) return 1;", ""),
    ("no master: decay skipped", "param_bf16[i] = orc_bf16_rne(pd - u);", "param_bf16[i] = orc_bf16_rne(p - u);"),
    ("no master: update dropped", "param_bf16[i] = orc_bf16_rne(pd - u);", "param_bf16[i] = orc_bf16_rne(pd);"),
    ("zero-1 update: sign not flipped", "const float neg_step_size = -s.step_size;",
     "const float neg_step_size = s.step_size;"),
    ("zero-1 update: first moment not stored",
     "        exp_avg[i] = m;\n        exp_avg_sq[i] = v;\n        update[i]",
     "        exp_avg_sq[i] = v;\n        update[i]"),
    ("zero-1 update: bias correction of v dropped", "float denom = sqrtf(v) / s.bias_correction2_sqrt + s.eps;",
     "float denom = sqrtf(v) + s.eps;"),
    ("zero-1 update: a skipped step leaves the stale update",
     "for (int64_t i = 0; i < n; ++i) update[i] = -0.0f;", ""),
    ("zero-1 update: a skipped step writes +0.0 (turns -0.0 parameters into +0.0)",
     "update[i] = -0.0f;", "update[i] = 0.0f;"),
    ("apply: offset ignored", "float u = update[offset + j];", "float u = update[j];"),
    ("apply: bf16 truncated instead of rounded", "p[j] = orc_bf16_rne(orc_bf16_widen(p[j]) + u);",
     "p[j] = (uint16_t)(f32_bits(orc_bf16_widen(p[j]) + u) >> 16);"),
    ("apply: fp32 update subtracted", "p[j] = p[j] + u;", "p[j] = p[j] - u;"),
    ("tiled state: streams laid out tile-major instead of per tile",
     "buf[((int64_t)runs * t + k) * tile + j] = x;", "buf[((int64_t)k * tiles + t) * tile + j] = x;"),
    ("tiled state: one tile too many when n is a multiple of the tile", "if (n % tile != 0) tiles += 1;",
     "tiles += 1;"),
    ("tiled state: the end of the last tile left unwritten", "float x = 0.0f;\n                if (e < n",
     "float x = buf[((int64_t)runs * t + k) * tile + j];\n                if (e < n"),
    ("tiled state: untile reads the previous run",
     "dst[k][e] = buf[((int64_t)runs * t + k) * tile + j];",
     "dst[k][e] = buf[((int64_t)runs * t + (k > 0 ? k - 1 : 0)) * tile + j];"),
    ("tiled moments: untile swaps the two runs", "float* dst[2] = {exp_avg, exp_avg_sq};",
     "float* dst[2] = {exp_avg_sq, exp_avg};"),
]


def pin_suite():
    """The fast pins (the exhaustive bf16 sweep is left to test_oracle_pins)."""
    orc = oracle
    suite = [
        lambda: pins.test_bf16_rne_ties_and_overflow(orc),
        lambda: pins.test_shard_range_golden(orc),
        lambda: pins.test_shard_range_brute_force_small(orc),
        lambda: pins.test_shard_range_rejects(orc),
        lambda: pins.test_flat_pack_bf16_and_widen(orc),
        lambda: pins.test_fsdp_unit_rank17_maps_into_gate_proj(orc),
        lambda: pins.test_grad_accum_closed_form_power_of_two(orc),
        lambda: pins.test_grad_accum_overwrite_keeps_negative_zero(orc),
        lambda: pins.test_grad_accum_matches_torch_add(orc),
        lambda: pins.test_grad_accum_error_bound_vs_exact_sum(orc),
        lambda: pins.test_norm_sq_closed_forms(orc),
        lambda: pins.test_norm_sq_vs_exact_sum(orc),
        lambda: pins.test_clip_coef_vs_torch_clip_grad_norm(orc),
        lambda: pins.test_clip_applies_at_equality_and_splits_over_ranks(orc),
        lambda: pins.test_fp32_scalars_golden(orc),
        lambda: pins.test_step1_closed_form(orc),
        lambda: pins.test_step1_grad_scale_enters(orc),
        lambda: pins.test_constant_grad_k_steps_closed_form(orc, 0.0),
        lambda: pins.test_constant_grad_k_steps_closed_form(orc, 0.1),
        lambda: pins.test_zero_grad_invariance_and_padding(orc),
        lambda: pins.test_sharding_invariance(orc),
        lambda: pins.test_adamw_float64_brute_force(orc),
        lambda: pins.test_nonfinite_norm_skips_update(orc),
        lambda: pins.test_adamw_rejects(orc),
        lambda: pins.test_no_master_one_step_equals_master_recast(orc),
        lambda: pins.test_no_master_stalls_below_half_an_ulp(orc),
        lambda: pins.test_adam_update_added_to_param_equals_master_step(orc),
        lambda: pins.test_adam_update_vs_adam_equations_float64(orc),
        lambda: pins.test_adam_update_step1_closed_form(orc),
        lambda: pins.test_adam_update_rejects_decay_and_skips_nonfinite(orc),
        lambda: pins.test_skipped_adam_update_applies_as_identity(orc),
        lambda: pins.test_flat_apply_update_zero_update_is_identity(orc),
        lambda: pins.test_zero1_flow_equals_one_buffer_step(orc),
        lambda: pins.test_state_tile_element_positions_brute_force(orc),
        lambda: pins.test_state_tile_bits_and_missing_sources(orc),
        lambda: pins.test_state_tile_then_step_equals_step(orc),
        lambda: pins.test_moments_tile_then_update_equals_update(orc),
    ]
    for n, tile in ((5, 4), (64, 16), (8193, 8192)):
        suite.append(lambda n=n, tile=tile: pins.test_moments_tile_matches_numpy_reshape(orc, n, tile))
    for n, tile in ((5, 4), (17, 8), (64, 16), (8193, 8192)):
        suite.append(lambda n=n, tile=tile: pins.test_state_tile_matches_numpy_reshape(orc, n, tile))
    for seed in range(3):
        suite.append(lambda seed=seed: pins.test_flat_pack_matches_concatenate(orc, seed))
    for seed in range(2):
        suite.append(lambda seed=seed: pins.test_adamw_vs_torch_adamw(orc, seed))
        suite.append(lambda seed=seed: pins.test_flat_apply_update_matches_slices(orc, seed))
    return suite


def failures(path):
    failed = 0
    with oracle.use_library(path):
        for check in pin_suite():
            try:
                check()
            except (AssertionError, ValueError, OverflowError, FloatingPointError):
                failed += 1
    return failed


def compile_variant(source: str, tmpdir: str, tag: str) -> str:
    c = os.path.join(tmpdir, f"m_{tag}.c")
    so = os.path.join(tmpdir, f"m_{tag}.so")
    with open(c, "w") as f:
        f.write(source)
    subprocess.run(["gcc", "-O1", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
                    "-shared", "-w", "-o", so, c, "-lm"], check=True)
    return so


@pytest.fixture(scope="module")
def workdir():
    with tempfile.TemporaryDirectory() as d:
        yield d


def test_unmutated_oracle_passes_every_fast_pin(workdir):
    source = open(SRC).read()
    assert failures(compile_variant(source, workdir, "clean")) == 0


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(workdir, name, old, new):
    source = open(SRC).read()
    assert source.count(old) >= 1, f"mutation site missing: {name}"
    so = compile_variant(source.replace(old, new), workdir, str(abs(hash(name))))
    assert failures(so) > 0, f"no pin catches: {name}"
