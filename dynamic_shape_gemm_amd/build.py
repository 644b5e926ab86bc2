"""Build libmkp.so (HIP micro-kernels + polymerizer + C-ABI) for gfx950.

Run as `python dynamic_shape_gemm_amd/build.py` (not -m: importing the package loads the library); `__graft_entry__.build()`
calls `build_library()`.  The library is built in-tree, next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmkp.so")
ROOT = os.path.dirname(HERE)

SOURCES = ["kernels.hip", "planner.cpp", "api.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    # packed fp32 VALU forms stay off: only plain fp32 instructions are emitted
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


RESOURCE_REPORT = os.path.join(HERE, "_build", "resource_usage.txt")


def parse_resource_usage(remarks: str) -> dict:
    """Per-kernel register, scratch and occupancy figures from the
    compiler's kernel-resource-usage remarks."""
    out, name = {}, None
    for line in remarks.splitlines():
        if "Function Name:" in line:
            name = line.split("Function Name:", 1)[1].split()[0]
            out[name] = {}
            continue
        if name is None:
            continue
        for key, field in (("VGPRs:", "vgpr"), ("AGPRs:", "agpr"), ("ScratchSize [bytes/lane]:", "scratch"),
                           ("Occupancy [waves/SIMD]:", "occupancy"), ("LDS Size [bytes/block]:", "lds")):
            if key in line:
                try:
                    out[name][field] = int(line.split(key, 1)[1].split()[0])
                except ValueError:
                    pass
    return out


def build_library(verbose: bool = False) -> str:
    objs = []
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(obj_dir, src.rsplit(".", 1)[0] + ".o")
        cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".hip"):
            cmd += ["-Rpass-analysis=kernel-resource-usage", "-fno-caret-diagnostics"]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, stderr=subprocess.PIPE, text=True)
        usage = parse_resource_usage(res.stderr) if src.endswith(".hip") else {}
        other = "\n".join(l for l in res.stderr.splitlines()
                          if "kernel-resource-usage" not in l and "packed-fp32-ops" not in l)
        if other.strip():
            print(other, file=sys.stderr, flush=True)
        if res.returncode != 0:
            raise subprocess.CalledProcessError(res.returncode, cmd)
        if usage:
            with open(RESOURCE_REPORT, "w") as f:
                for k in sorted(usage):
                    u = usage[k]
                    f.write(f"{k} vgpr={u.get('vgpr')} agpr={u.get('agpr')} scratch={u.get('scratch')} "
                            f"lds={u.get('lds')} occupancy={u.get('occupancy')}\n")
            # a GEMM micro-kernel that spills to scratch has lost its register
            # tiling; refuse to ship it
            spills = [k for k, u in usage.items() if "gemm_tile_kernel" in k and u.get("scratch", 0) > 0]
            if spills:
                raise RuntimeError("GEMM micro-kernels use scratch memory: " + ", ".join(spills))
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs, "-ldl"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
