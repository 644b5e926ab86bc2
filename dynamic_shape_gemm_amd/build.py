"""Build libmkp.so (HIP micro-kernels + polymerizer + C-ABI) for gfx950.

Run as `python dynamic_shape_gemm_amd/build.py` (not -m: importing the package loads the library); `__graft_entry__.build()`
calls `build_library()`.  The library is built in-tree, next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
import sysconfig

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmkp.so")
ROOT = os.path.dirname(HERE)

# (source, object, extra flags): the kernel file builds as four translation
# units (single-tile kernels; two-tile kernels per B layout; convolution
# kernels), compiled side by side
UNITS = [
    ("kernels.hip", "kernels_p1.o", ["-DMKP_PART=1"]),
    ("kernels.hip", "kernels_p2.o", ["-DMKP_PART=2"]),
    ("kernels.hip", "kernels_p3.o", ["-DMKP_PART=3"]),
    ("kernels.hip", "kernels_p4.o", ["-DMKP_PART=4"]),
    ("planner.cpp", "planner.o", []),
    ("api.cpp", "api.o", []),
]
SOURCES = sorted({u[0] for u in UNITS})

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
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    jobs = []
    for src, obj_name, extra in UNITS:
        obj = os.path.join(obj_dir, obj_name)
        cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src),
               "-o", obj]
        if src.endswith(".hip"):
            cmd += ["-Rpass-analysis=kernel-resource-usage", "-fno-caret-diagnostics"]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((src, obj, cmd, subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True)))
    usage, objs, failed = {}, [], None
    for src, obj, cmd, proc in jobs:
        _, err = proc.communicate()
        if src.endswith(".hip"):
            usage.update(parse_resource_usage(err))
        other = "\n".join(l for l in err.splitlines()
                          if "kernel-resource-usage" not in l and "packed-fp32-ops" not in l)
        if other.strip():
            print(other, file=sys.stderr, flush=True)
        if proc.returncode != 0 and failed is None:
            failed = subprocess.CalledProcessError(proc.returncode, cmd)
        objs.append(obj)
    if failed is not None:
        raise failed
    with open(RESOURCE_REPORT, "w") as f:
        for k in sorted(usage):
            u = usage[k]
            f.write(f"{k} vgpr={u.get('vgpr')} agpr={u.get('agpr')} scratch={u.get('scratch')} "
                    f"lds={u.get('lds')} occupancy={u.get('occupancy')}\n")
    # a GEMM micro-kernel that spills to scratch has lost its register
    # tiling; refuse to ship it
    spills = [k for k, u in usage.items()
              if ("gemm_tile_kernel" in k or "gemm_dual_kernel" in k) and u.get("scratch", 0) > 0]
    if spills:
        raise RuntimeError("GEMM micro-kernels use scratch memory: " + ", ".join(spills))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs, "-ldl"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    build_fast_binding(verbose)
    return LIB


FAST = os.path.join(HERE, "_mkpfast" + (sysconfig.get_config_var("EXT_SUFFIX") or ".so"))


def build_fast_binding(verbose: bool = False) -> str:
    """The CPython marshalling module for the GEMM entry points (host C,
    linked against libmkp.so next to it)."""
    tmp = FAST + ".tmp"
    cmd = [os.environ.get("CC", "gcc"), "-O2", "-shared", "-fPIC", "-Wall", "-I", sysconfig.get_paths()["include"],
           "-I", os.path.join(ROOT, "include"), os.path.join(CSRC, "pymkp.c"), "-o", tmp, "-L", HERE, "-lmkp",
           "-Wl,-rpath,$ORIGIN"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, FAST)
    return FAST


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
