"""Turn rocprofv3 byte counters into HBM traffic per launch.

    python -m dynamic_shape_gemm_amd.pmc --config 2 \
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \
        --copy-bytes BYTES --out profiles/traffic.json

Each DIR holds the *_counter_collection.csv of one `rocprofv3 --pmc` run:
FETCH_SIZE (then WRITE_SIZE) of the benchmark, and the same counter for a
plain copy of COPY_BYTES (bench.py --copy-reference).  The copy calibrates
each counter: scale = bytes the copy moved / bytes the counter reports.  For
every library micro-kernel the record holds the scaled fetch + write bytes
averaged per dispatch, tagged with the hash of the kernel source it was
measured on (bench.py reports it only while that source is unchanged).
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
# Tile<uM, uN, uK, waves_m, waves_n, stages, preread, N x K B[, convolution]>
TILE = re.compile(r"Tile<(\d+), (\d+), (\d+), \d+, \d+, \d+, (?:true|false), (true|false)(?:, (true|false))?>")


def read_counter(d: str, counter: str):
    """{kernel name: [per-dispatch value]} for one counter."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for f in files:
        for row in csv.DictReader(open(f)):
            if row["Counter_Name"] != counter:
                continue
            per[row["Kernel_Name"]][row["Dispatch_Id"]] += float(row["Counter_Value"])
    return {k: list(v.values()) for k, v in per.items()}


def lib_name(kernel_name: str):
    m = TILE.search(kernel_name)
    if not m or "gemm_tile_kernel" not in kernel_name:
        return None
    # the N x K flag marks the kernels that take B as N x K; the convolution
    # forms of those count apart
    name = f"m{m.group(1)}n{m.group(2)}k{m.group(3)}" + ("_nk" if m.group(4) == "true" else "")
    return name + ("_conv" if m.group(5) == "true" else "")


def copy_scale(d: str, counter: str, nbytes: float) -> float:
    vals = read_counter(d, counter)
    # the copy kernel is the one whose dispatches report the most bytes
    name = max(vals, key=lambda k: sum(vals[k]) / len(vals[k]))
    per_dispatch_kib = sum(vals[name]) / len(vals[name])
    return nbytes / (per_dispatch_kib * 1024.0), name, per_dispatch_kib


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--copy-bytes", type=float, required=True)
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    sf, cname, cf = copy_scale(a.copy_fetch, "FETCH_SIZE", a.copy_bytes)
    sw, _, cw = copy_scale(a.copy_write, "WRITE_SIZE", a.copy_bytes)
    fetch = read_counter(a.fetch, "FETCH_SIZE")
    write = read_counter(a.write, "WRITE_SIZE")
    kernels = {}
    for kname, vals in fetch.items():
        ln = lib_name(kname)
        if ln is None or kname not in write:
            continue
        f_kib = sum(vals) / len(vals)
        w_kib = sum(write[kname]) / len(write[kname])
        kernels[ln] = {
            "dispatches": len(vals),
            "fetch_kib_per_launch": round(f_kib, 1),
            "write_kib_per_launch": round(w_kib, 1),
            "hbm_bytes_per_launch": round(f_kib * 1024.0 * sf + w_kib * 1024.0 * sw),
        }
    src = os.path.join(HERE, "csrc", "kernels.hip")
    rec = {
        "config": a.config,
        "kernel_source_sha256_16": hashlib.sha256(open(src, "rb").read()).hexdigest()[:16],
        "copy_reference": {"kernel": cname[:80], "bytes": a.copy_bytes, "fetch_kib": round(cf, 1),
                           "write_kib": round(cw, 1), "fetch_scale": round(sf, 4), "write_scale": round(sw, 4)},
        "kernels": kernels,
    }
    os.makedirs(os.path.dirname(a.out) or ".", exist_ok=True)
    json.dump(rec, open(a.out, "w"), indent=1)
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
