"""HBM traffic records for bench.py's roofline, keyed to the built code.

bench.py reports `traffic` for a kernel only from a record taken on the
code object that is running: the record holds the sha256 of the gfx950 code
object (the device ELF of the source file that defines the kernel, read out
of libzshard.so's offload bundles) and the kernel's symbol; any change to
the device code of that file changes the digest and the record no longer
applies (traffic null).  Records are written only by `record` below, from
two rocprofv3 counter passes of bench.py (FETCH_SIZE, then WRITE_SIZE),
each scaled by what the same counter reads for the 4 GiB device copy that
bench.py runs in the same process.

    python bench_pmc.py digest                      # digests of the current build
    python bench_pmc.py record FETCH_DIR WRITE_DIR  # add records from two passes
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import struct
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(ROOT, "fsdp_sharded_optimizer_amd", "libzshard.so")
RECORDS = os.path.join(ROOT, "bench_pmc.json")
ARCH = "gfx950"
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 4 << 30   # bench.py's device copy: 4 GiB read and 4 GiB written


def _elf_sections(data: bytes):
    """(name, type, addr, offset, size, link, entsize) of a little-endian ELF64."""
    shoff = struct.unpack_from("<Q", data, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)
    raw = [struct.unpack_from("<IIQQQQIIQQ", data, shoff + i * shentsize) for i in range(shnum)]
    strtab_off = raw[shstrndx][4]

    def name(o):
        s = strtab_off + o
        return data[s:data.index(b"\0", s)].decode()
    return [(name(r[0]), r[1], r[3], r[4], r[5], r[6], r[9]) for r in raw]


def code_objects(lib_path: str = LIB) -> list:
    """The gfx950 device ELFs in the library's .hip_fatbin (one per source file with kernels)."""
    with open(lib_path, "rb") as f:
        data = f.read()
    secs = {s[0]: s for s in _elf_sections(data)}
    if ".hip_fatbin" not in secs:
        raise RuntimeError(f"{lib_path}: no .hip_fatbin section")
    _, _, _, off, size, _, _ = secs[".hip_fatbin"]
    blob = data[off:off + size]
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    out = []
    pos = blob.find(magic)
    while pos >= 0:
        count = struct.unpack_from("<Q", blob, pos + len(magic))[0]
        p = pos + len(magic) + 8
        for _ in range(count):
            eoff, esize, tlen = struct.unpack_from("<QQQ", blob, p)
            p += 24
            triple = blob[p:p + tlen].decode()
            p += tlen
            if triple.endswith("-" + ARCH) and esize > 0:
                obj = blob[pos + eoff:pos + eoff + esize]
                if obj[:4] != b"\x7fELF":
                    raise RuntimeError("compressed or unknown code object format")
                out.append(obj)
        pos = blob.find(magic, pos + 1)
    return out


def _symbols(obj: bytes) -> set:
    """Names in a device ELF's symbol tables."""
    names = set()
    secs = _elf_sections(obj)
    for name, typ, _, off, size, link, entsize in secs:
        if typ not in (2, 11) or entsize == 0:   # SHT_SYMTAB, SHT_DYNSYM
            continue
        stroff = secs[link][3]
        for k in range(size // entsize):
            st_name = struct.unpack_from("<I", obj, off + k * entsize)[0]
            if st_name:
                s = stroff + st_name
                names.add(obj[s:obj.index(b"\0", s)].decode())
    return names


def kernel_digests(lib_path: str = LIB) -> dict:
    """{kernel symbol: sha256 of the code object that defines it}."""
    out = {}
    for obj in code_objects(lib_path):
        digest = hashlib.sha256(obj).hexdigest()
        for s in _symbols(obj):
            if s.endswith(".kd"):
                out[s[:-3]] = digest
    return out


def load_records(path: str = RECORDS) -> list:
    if not os.path.exists(path):
        return []
    with open(path) as f:
        return json.load(f)["records"]


def traffic(label: str, n: int, digests: dict = None, path: str = RECORDS):
    """Calibrated HBM bytes per launch of the kernel bench.py labels
    `label` at shard length n, or None: no record for it, or the code object
    that defines its kernel is not the one the record was taken on."""
    digests = kernel_digests() if digests is None else digests
    for r in load_records(path):
        if r["label"] == label and r["shard_elems"] == n:
            if digests.get(r["symbol"]) != r["code_object_sha256"]:
                return None
            return r["fetch_kib"] * 1024 * r["fetch_scale"] + r["write_kib"] * 1024 * r["write_scale"]
    return None


# --------------------------------------------------------------------------
# recording (run locally on the counter passes' output)
# --------------------------------------------------------------------------

def _bare(name: str) -> str:
    """A demangled kernel name without its return type and parameter list."""
    return name.strip().removeprefix("void ").rsplit("(", 1)[0].strip()


def _demangle(names):
    p = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True, check=True)
    return p.stdout.splitlines()


def _counter_rows(pass_dir: str, counter: str) -> dict:
    """{kernel name: [(grid size in work-items, counter value), ...]} from
    a rocprofv3 --pmc csv (one row per dispatch)."""
    files = glob.glob(os.path.join(pass_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise RuntimeError(f"no counter_collection.csv under {pass_dir}")
    per = {}
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] == counter:
                    per.setdefault(row["Kernel_Name"], []).append((int(row["Grid_Size"]),
                                                                   float(row["Counter_Value"])))
    return per


def _copy_reading(rows) -> float:
    """The counter per dispatch of bench.py's 4 GiB device copy: the
    runtime's copy kernel also runs the small device-to-host reads and the
    step rigs' set-up copies (gradients of up to 2.2 GB), on the same grid
    size, so take the dispatches that read within 10 % of the largest."""
    top = max(v for _, v in rows)
    vals = [v for _, v in rows if v >= 0.9 * top]
    return sum(vals) / len(vals)


def _mean_for_grid(rows, grid):
    """Mean counter value over the dispatches of one grid size (None: all)."""
    vals = [v for g, v in rows if grid is None or g == grid]
    if not vals:
        raise RuntimeError(f"no dispatch with grid size {grid}")
    return sum(vals) / len(vals), len(vals)


def record(fetch_dir: str, write_dir: str, bench_log: str, path: str = RECORDS, lib_path: str = LIB) -> list:
    """Records for the kernels bench.py lists in its `pmc_kernels` (label,
    kernel name as rocprofv3 prints it, shard length, grid size of the
    launch, algorithmic bytes), from the JSON line the counter passes'
    bench run printed (bench_log)."""
    with open(bench_log) as f:
        line = [l for l in f if l.startswith("{")][-1]
    bench = json.loads(line)
    fetch = _counter_rows(fetch_dir, "FETCH_SIZE")
    write = _counter_rows(write_dir, "WRITE_SIZE")
    fscale = COPY_BYTES / 1024 / _copy_reading(fetch[COPY_KERNEL])
    wscale = COPY_BYTES / 1024 / _copy_reading(write[COPY_KERNEL])
    digests = kernel_digests(lib_path)
    if sorted(set(digests.values())) != bench["code_objects_sha256"]:
        raise RuntimeError("the library here is not the build the counter passes ran")
    symbols = list(digests)
    pretty = {_bare(dem): sym for sym, dem in zip(symbols, _demangle(symbols))}

    def prof_name(table, name):
        hits = [k for k in table if _bare(k) == name]
        if len(hits) != 1:
            raise RuntimeError(f"{name}: {len(hits)} matches among the profiled kernels")
        return hits[0]

    recs = load_records(path)
    new = []
    for info in bench["pmc_kernels"]:
        label, name, n, grid = info["label"], info["kernel"], info["shard_elems"], info["grid"]
        sym = pretty.get(name)
        if sym is None:
            raise RuntimeError(f"{name} not found in the library's code objects")
        fv = _mean_for_grid(fetch[prof_name(fetch, name)], grid)
        wv = _mean_for_grid(write[prof_name(write, name)], grid)
        rec = {"label": label, "shard_elems": n, "kernel": name, "symbol": sym,
               "code_object_sha256": digests[sym], "grid": grid,
               "fetch_kib": fv[0], "fetch_scale": round(fscale, 4),
               "write_kib": wv[0], "write_scale": round(wscale, 4),
               "dispatches": [fv[1], wv[1]],
               "algorithmic_bytes": info["algorithmic_bytes"]}
        recs = [r for r in recs if not (r["label"] == label and r["shard_elems"] == n)]
        recs.append(rec)
        new.append(rec)
    with open(path, "w") as f:
        json.dump({"about": "rocprofv3 FETCH_SIZE / WRITE_SIZE per dispatch (KiB) of bench.py's kernels, "
                            "written by bench_pmc.py record; scales from the 4 GiB device copy",
                   "records": recs}, f, indent=1)
        f.write("\n")
    return new


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "digest":
        for k, v in sorted(kernel_digests().items()):
            print(v[:16], k)
    elif len(sys.argv) == 5 and sys.argv[1] == "record":
        for r in record(sys.argv[2], sys.argv[3], sys.argv[4]):
            meas = r["fetch_kib"] * 1024 * r["fetch_scale"] + r["write_kib"] * 1024 * r["write_scale"]
            print(f"{r['label']} n={r['shard_elems']}: {meas / r['algorithmic_bytes']:.4f} x algorithmic")
    else:
        sys.exit(__doc__)
