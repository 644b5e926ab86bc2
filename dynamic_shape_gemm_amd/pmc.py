"""Turn rocprofv3 counters into per-kernel figures.

HBM traffic per launch (the default mode):

    python -m dynamic_shape_gemm_amd.pmc --config all \
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \
        --copy-bytes BYTES --out profiles/traffic.json

Each DIR holds the *_counter_collection.csv of one `rocprofv3 --pmc` run:
FETCH_SIZE (then WRITE_SIZE) of the benchmark, and the same counter for a
plain copy of COPY_BYTES (bench.py --copy-reference).  The copy calibrates
each counter: scale = bytes the copy moved / bytes the counter reports.  For
every library micro-kernel the record holds the scaled fetch + write bytes
averaged per dispatch, tagged with the hash of the kernel source it was
measured on (bench.py reports it only while that source is unchanged).

Counter summary (`python -m dynamic_shape_gemm_amd.pmc counters --dirs D1 D2
--out FILE`): per library kernel, MFMA busy cycles over the SIMD cycles of
the dispatch (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs x CUs x 4)), LDS
bank-conflict cycles per LDS-active cycle, the share of wave cycles waiting
on any dependency and waiting to issue LDS instructions, and the L2 hit
rate.
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
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
# Tile<uM, uN, uK, waves_m, waves_n, stages, preread, N x K B[, convolution]>
TILE = re.compile(r"Tile<(\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (?:true|false), (true|false)(?:, (true|false))?>")
# skinny-M tiles whose waves split K: WSplit<uM, uN, waves, stages, N x K B>,
# named m<uM>n<uN>k<64 * waves>
WSPLIT = re.compile(r"WSplit<(\d+), (\d+), (\d+), (\d+), (true|false)>")
# tiles the library also has with another stage count, named with "x<stages>"
DEEP = {(128, 128, 4), (64, 64, 2), (64, 128, 2), (128, 64, 2)}
# tiles the library also has on fewer, larger waves, named with "w<waves>"
WIDE = {(256, 256, 4)}


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
    w = WSPLIT.search(kernel_name)
    if w and "gemm_wsplit_kernel" in kernel_name:
        name = f"m{w.group(1)}n{w.group(2)}k{64 * int(w.group(3))}"
        return name + ("_nk" if w.group(5) == "true" else "")
    m = TILE.search(kernel_name)
    if not m or "gemm_tile_kernel" not in kernel_name:
        return None
    # the N x K flag marks the kernels that take B as N x K; the convolution
    # forms of those count apart
    bm, bn, stages = int(m.group(1)), int(m.group(2)), int(m.group(6))
    waves = int(m.group(4)) * int(m.group(5))
    name = f"m{bm}n{bn}k{m.group(3)}" + (f"x{stages}" if (bm, bn, stages) in DEEP else "")
    name += f"w{waves}" if (bm, bn, waves) in WIDE else ""
    name += "_nk" if m.group(7) == "true" else ""
    return name + ("_conv" if m.group(8) == "true" else "")


def copy_scale(d: str, counter: str, nbytes: float) -> float:
    vals = read_counter(d, counter)
    # the copy kernel is the one whose dispatches report the most bytes
    name = max(vals, key=lambda k: sum(vals[k]) / len(vals[k]))
    per_dispatch_kib = sum(vals[name]) / len(vals[name])
    return nbytes / (per_dispatch_kib * 1024.0), name, per_dispatch_kib


def read_all(dirs):
    """{library kernel: {counter: per-dispatch mean}} over every counter of
    the given rocprofv3 --pmc output directories."""
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for d in dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        for f in files:
            for row in csv.DictReader(open(f)):
                ln = lib_name(row["Kernel_Name"])
                if ln is None:
                    continue
                per[(ln, row["Counter_Name"])][row["Dispatch_Id"]] += float(row["Counter_Value"])
        for (ln, cn), vals in per.items():
            acc[ln][cn].extend(vals.values())
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}, \
        {k: max(len(v) for v in cs.values()) for k, cs in acc.items()}


def counters_markdown(dirs, cus: int, command: str, xcds: int = 8) -> str:
    """Per-kernel counter summary: MFMA busy share of the SIMD cycles while
    the GPU is active (GRBM_GUI_ACTIVE counts the active cycles of every XCD,
    so one XCD's are GRBM_GUI_ACTIVE / xcds), LDS bank-conflict cycles per
    LDS-active cycle, share of wave time waiting on LDS, and the L2 hit
    rate."""
    vals, n = read_all(dirs)
    out = ["| kernel | dispatches | MFMA busy | LDS bank conflicts / LDS active | waves waiting (any) | "
           "waves waiting to issue LDS | L2 hit rate |",
           "|---|---:|---:|---:|---:|---:|---:|"]

    def ratio(a, b):
        return f"{100.0 * a / b:.1f}%" if b else "n/a"

    for k in sorted(vals, key=lambda k: -n[k]):
        v = vals[k]
        gui = v.get("GRBM_GUI_ACTIVE", 0.0) / xcds
        mfma = ratio(v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0), gui * cus * 4)
        bank = ratio(v.get("SQ_LDS_BANK_CONFLICT", 0.0), v.get("SQ_LDS_IDX_ACTIVE", 0.0))
        wait = ratio(v.get("SQ_WAIT_INST_LDS", 0.0), v.get("SQ_WAVE_CYCLES", 0.0))
        wany = ratio(v.get("SQ_WAIT_ANY", 0.0), v.get("SQ_WAVE_CYCLES", 0.0))
        hit, miss = v.get("TCC_HIT_sum", 0.0), v.get("TCC_MISS_sum", 0.0)
        out.append(f"| `{k}` | {n[k]} | {mfma} | {bank} | {wany} | {wait} | {ratio(hit, hit + miss)} |")
    return "\n".join(out) + "\n"


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "counters":
        ap = argparse.ArgumentParser(prog="pmc counters")
        ap.add_argument("counters")
        ap.add_argument("--dirs", nargs="+", required=True)
        ap.add_argument("--cus", type=int, default=256)
        ap.add_argument("--xcds", type=int, default=8)
        ap.add_argument("--out", required=True)
        ap.add_argument("--command", default="")
        a = ap.parse_args()
        text = counters_markdown(a.dirs, a.cus, a.command, a.xcds)
        os.makedirs(os.path.dirname(a.out) or ".", exist_ok=True)
        open(a.out, "w").write(text)
        print(text)
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", required=True, help="all (the default benchmark) or a sweep number")
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
        "config": a.config if a.config == "all" else int(a.config),
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
