"""The memory ledger against the figures the pages print (CPU only)."""
import json
import os

import pytest

from fsdp_sharded_optimizer_amd import ledger

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "memory_ledger.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def computed():
    return {
        "70B model state at 16 B/param (bytes)": ledger.per_rank(70e9, 1, 0).total,
        "70B ZeRO-3 per card, N = 64 (bytes)": ledger.per_rank(70e9, 64, 3).total,
        "80 GB cards to hold the 70B state": ledger.cards_to_hold(70e9, 80e9),
        "redundant share of the 16 bytes": ledger.redundant_fraction(),
        "70B fp16 parameters (bytes)": ledger.per_rank(70e9, 1, 0).params,
        "Llama-7B FP16 weights (bytes, 7e9 parameters)": ledger.per_rank(7e9, 8, 1).params,
    }


def test_ledger_matches_the_pages():
    got = computed()
    for case in golden()["consistent"]:
        v = got[case["what"]]
        assert abs(v - case["value"]) <= case["rel_tol"] * case["value"], (case["what"], v)


def test_ledger_flags_the_inconsistent_figures():
    """The ZeRO page's ZeRO-1/2 per-card figures do not follow from its own
    terms (14 GB of FP16 weights, 28 GB of states); the ledger, fed those
    terms, gives 17.5 GB for both, as the page's own sums do."""
    # ZeRO-1 on the page: FP16 weights (2 B) whole, the 4 B of optimizer
    # states per parameter sharded; ZeRO-2 on the page: FP16 weights whole,
    # gradients (2 B) and its optimizer term (2 B) sharded
    z1 = ledger.per_rank(7e9, 8, 1, param_bytes=2, grad_bytes=0, optim_bytes=4).total / 1e9
    z2 = ledger.per_rank(7e9, 8, 2, param_bytes=2, grad_bytes=2, optim_bytes=2).total / 1e9
    printed = {c["what"]: c["printed"] for c in golden()["inconsistent"]}
    assert abs(printed["Llama-7B ZeRO-1 per card, N = 8 (GB)"] - z1) > 20
    assert abs(printed["Llama-7B ZeRO-2 per card, N = 8 (GB)"] - z2) > 3


def test_stage_monotone_and_sixteen_over_n():
    for n in (1, 8, 64):
        totals = [ledger.per_rank(1e9, n, s).total for s in range(4)]
        assert all(a >= b for a, b in zip(totals, totals[1:]))
        assert totals[3] == pytest.approx(16e9 / n)


def test_library_shard_bytes_of_the_workloads():
    """What this library's buffers take per rank, for the sizes bench.py
    prints: the 70B ZeRO-3 shard (1,093,750,000 elements) with one bf16
    gradient in flight fits 288 GB many times over, and each staged bf16
    micro-batch gradient adds 2 B per element.  (The bytes themselves are
    pinned against the device allocator in tests/test_gpu_shard_optimizer.py.)"""
    b70 = ledger.library_shard_bytes(1_093_750_000)
    assert 20e9 < b70 < 25e9
    one, eight = (ledger.library_shard_bytes(842_301_952, grad_buffers=k) for k in (1, 8))
    assert eight - one == 7 * 2 * 842_301_952


def test_rejects():
    with pytest.raises(ValueError):
        ledger.per_rank(1e9, 0, 1)
    with pytest.raises(ValueError):
        ledger.per_rank(1e9, 8, 4)
