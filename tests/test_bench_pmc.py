"""The traffic records bench.py reports (bench_pmc.py), on the host: the
gfx950 code objects read out of the built library, the digest that keys a
record, and the recording arithmetic on synthetic counter files."""
import csv
import json
import os

import pytest

import bench_pmc
from fsdp_sharded_optimizer_amd import build as zbuild

ADAMW = "zs::(anonymous namespace)::adamw_kernel<4, 1, 64, false, true, true, 0>"


@pytest.fixture(scope="module")
def digests():
    if not os.path.exists(zbuild.LIB):
        pytest.skip("libzshard.so not built")
    return bench_pmc.kernel_digests()


def test_code_objects_are_the_gfx950_device_elfs(digests):
    objs = bench_pmc.code_objects()
    assert objs and all(o[:4] == b"\x7fELF" for o in objs)
    # every kernel of the library is in one of them, each file's kernels share its digest
    adamw = {d for k, d in digests.items() if "adamw_kernel" in k}
    accum = {d for k, d in digests.items() if "accum_kernel" in k or "reduce_chunks_kernel" in k}
    assert len(adamw) == 1 and len(accum) == 1 and adamw != accum
    assert all(len(d) == 64 for d in digests.values())
    assert bench_pmc.kernel_digests() == digests          # stable


def _rec(label, n, symbol, digest, fetch=10.0, write=20.0):
    return {"label": label, "shard_elems": n, "kernel": ADAMW, "symbol": symbol, "code_object_sha256": digest,
            "grid": 64, "fetch_kib": fetch, "fetch_scale": 2.0, "write_kib": write, "write_scale": 1.0,
            "dispatches": [1, 1], "algorithmic_bytes": 40 * 1024}


def test_traffic_only_for_the_recorded_code_object(tmp_path, digests):
    sym = next(k for k in digests if "adamw_kernelILi4ELi1ELi64ELb0ELb1ELb1E" in k)
    path = str(tmp_path / "rec.json")
    with open(path, "w") as f:
        json.dump({"records": [_rec("adamw_step_tiled", 100, sym, digests[sym]),
                               _rec("adamw_step_tiled", 200, sym, "0" * 64)]}, f)
    assert bench_pmc.traffic("adamw_step_tiled", 100, digests, path) == (10.0 * 2.0 + 20.0) * 1024
    assert bench_pmc.traffic("adamw_step_tiled", 200, digests, path) is None      # another build's counters
    assert bench_pmc.traffic("adamw_step_tiled", 300, digests, path) is None      # no record
    assert bench_pmc.traffic("grad_accum_add", 100, digests, path) is None
    changed = dict(digests, **{sym: "f" * 64})
    assert bench_pmc.traffic("adamw_step_tiled", 100, changed, path) is None      # the kernel changed


def _counter_csv(path, counter, rows):
    fields = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"]
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for i, (kernel, grid, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Grid_Size": grid, "Kernel_Name": kernel, "Counter_Name": counter,
                        "Counter_Value": value})


def test_record_calibrates_on_the_device_copy_and_selects_the_grid(tmp_path, digests):
    """Counters of two passes: the runtime copy kernel's largest dispatches
    (the 4 GiB copy) set the scales, smaller copies are ignored (also those
    on the same grid, the step rigs' set-up copies), and the kernel's
    dispatches at the listed grid are averaged (another grid of the same
    kernel, another shard, is not)."""
    copy = bench_pmc.COPY_KERNEL
    k = "void " + ADAMW + "(zs::AdamwArgs)"
    _counter_csv(str(tmp_path / "f" / "x_counter_collection.csv"), "FETCH_SIZE",
                 [(copy, 131072, 900000.0), (copy, 131072, 2097150.0), (copy, 131072, 2097154.0), (copy, 512, 3.0),
                  (k, 640, 100.0), (k, 640, 110.0), (k, 960, 999.0)])
    _counter_csv(str(tmp_path / "w" / "x_counter_collection.csv"), "WRITE_SIZE",
                 [(copy, 131072, 1800000.0), (copy, 131072, 4194304.0), (copy, 512, 1.0), (k, 640, 300.0),
                  (k, 640, 300.0), (k, 960, 7.0)])
    log = tmp_path / "bench.log"
    bench = {"code_objects_sha256": sorted(set(digests.values())),
             "pmc_kernels": [{"label": "adamw_step_tiled", "kernel": ADAMW, "shard_elems": 2560, "grid": 640,
                              "algorithmic_bytes": 30 * 2560}]}
    log.write_text("noise\n" + json.dumps(bench) + "\n")
    path = str(tmp_path / "rec.json")
    (rec,) = bench_pmc.record(str(tmp_path / "f"), str(tmp_path / "w"), str(log), path)
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["fetch_kib"] == 105.0 and rec["write_kib"] == 300.0 and rec["dispatches"] == [2, 2]
    assert bench_pmc.traffic("adamw_step_tiled", 2560, digests, path) == (105.0 * 2 + 300.0) * 1024
    # a bench log from another build is refused
    bench["code_objects_sha256"] = ["0" * 64]
    log.write_text(json.dumps(bench) + "\n")
    with pytest.raises(RuntimeError):
        bench_pmc.record(str(tmp_path / "f"), str(tmp_path / "w"), str(log), path)
