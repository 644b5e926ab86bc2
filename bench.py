"""Throughput of the polymerized dynamic-shape GEMM on one MI355X.

One step = one pass over the whole workload through the C-ABI (plan-cache
lookup, polymerization on a miss, every region's micro-kernel).  Default
workload: all five synthetic sweeps back to back in one process --
the single (105,256,512) GEMM; the encoder linears (64 GEMMs, M = 16 L,
L ~ U{1..512}); the irregular/square pair (105,1024,12544) and 4096^3; the
skinny-M decoder projections (128 GEMMs, M ~ U{1..256}); the batched
per-head scores (32 calls of 48 x (S,S,64)).  `--config C` times one sweep.

Prints ONE JSON line (rank 0, N=1):
  value = total algorithmic FLOPs of the step / step time, in TFLOP/s;
  roofline = the dominant kernel's achieved rate over its launches (HIP
    events on the launch stream, via the library's launch trace) against the
    MI355X peak of its bound;
  config.per_config = each sweep timed on its own (TFLOP/s, per-shape
    fractions of their rooflines, its own dominant kernel);
  config.gates = the 4096^3 GEMM's fraction of the bf16 MFMA peak and the
    skinny-M sweep's fraction of the HBM peak;
  cpu_baseline = the CPU oracle on a bounded sample of the same workload.
Inputs are resident in HBM before timing; every GEMM of a sweep has its own
buffers (the decoder weights rotate over four copies), so the working set
(GBs) is far beyond the 256 MB MALL.
"""
from __future__ import annotations

import argparse
import gc
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)

METRIC = "TFLOP/s and % of bf16 MFMA / HBM roofline over dynamic-shape GEMM sweeps"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Workload:
    """Device-resident operands for one sweep of a config."""

    def __init__(self, cfg: int, copies: int = 1, b_layout: str = "kn", qkv: str = "merged",
                 epilogue: str = "none"):
        import torch
        import workloads

        self.cfg = cfg
        # epilogue: none; bias = every GEMM adds a bias vector; bias_gelu = and
        # the FFN-up GEMMs (N = 3072) apply GELU, fused into the GEMM;
        # bias_gelu_unfused = the same done by separate elementwise passes
        # after the GEMM (torch), for comparison
        self.epilogue = epilogue
        self.biases = {}
        # the query/key/value projection (N = 3 x 768 of the encoder linears):
        # merged = one call over the side-by-side weights; grouped = one
        # grouped call over three 768-wide weights; separate = three calls
        self.qkv = qkv if cfg == 2 else "merged"
        # kn: B is K x N (mkp_gemm); nk: B is kept as N x K, a linear layer's
        # weight layout (mkp_gemm_bt) -- the same products either way
        self.bt = b_layout == "nk"
        self.cases = workloads.config_cases(cfg)
        self.calls = []  # (case, A ptr, B ptr, C tensor)
        self.host = []   # (a bits, b bits) kept for the CPU baseline
        self.keep = []
        weights = {}
        for i, case in enumerate(self.cases):
            a = workloads.make_a(case)
            if cfg == 4:
                # decoder weights are shared by every decode step; keep
                # `copies` distinct device copies and rotate through them
                if case.seed_b not in weights:
                    b = workloads.make_b(case)
                    tb = self._dev_b(torch, b)
                    weights[case.seed_b] = (b, [tb] + [tb.clone() for _ in range(copies - 1)])
                b, tbs = weights[case.seed_b]
                tb = tbs[i % len(tbs)]
            else:
                b = workloads.make_b(case)
                tb = self._dev_b(torch, b)
            ta = torch.from_numpy(a.view(np.int16)).cuda()
            tc = torch.empty((case.batch, case.M, case.N), dtype=torch.float32, device="cuda")
            self.keep += [ta, tb]
            self.calls.append((case, ta.data_ptr(), tb.data_ptr(), tc))
            self.host.append((case, a, b))
        self.flops = sum(c.flops for c in self.cases)
        self.bytes = sum(c.bytes for c in self.cases)
        if epilogue != "none":
            if cfg != 2:
                raise SystemExit("--epilogue applies to the encoder linears (config 2)")
            rng = np.random.default_rng(202)
            for case in self.cases:
                if case.N not in self.biases:
                    self.biases[case.N] = torch.from_numpy(rng.uniform(-1, 1, case.N).astype(np.float32)).cuda()

    def _dev_b(self, torch, b):
        t = torch.from_numpy(b.view(np.int16)).cuda()
        return t.transpose(-1, -2).contiguous() if self.bt else t

    def is_qkv(self, case) -> bool:
        return self.qkv != "merged" and case.N == 2304 and case.batch == 1

    def calls_per_case(self):
        return [3 if self.qkv == "separate" and self.is_qkv(c) else 1 for c in self.cases]

    def _qkv_step(self, mkp, case, pa, pb, tc, stream):
        """The 2304-wide product as three 768-wide ones: B_g and C_g are
        the g-th column blocks (or, for N x K weights, row blocks of B)."""
        M, K, n = case.M, case.K, 768
        pc = tc.data_ptr()
        pbs = [pb + 2 * g * (n * K if self.bt else n) for g in range(3)]
        ldb = K if self.bt else case.N
        pcs = [pc + 4 * g * n for g in range(3)]
        if self.qkv == "grouped":
            fn = mkp.mkp_gemm_grouped_bt if self.bt else mkp.mkp_gemm_grouped
            fn(M, K, pa, K, [n] * 3, pbs, [ldb] * 3, pcs, [case.N] * 3, stream)
        else:
            fn = mkp.mkp_gemm_bt if self.bt else mkp.mkp_gemm
            for g in range(3):
                fn(M, n, K, pa, K, pbs[g], ldb, pcs[g], case.N, stream)

    def _epilogue_step(self, mkp, case, pa, pb, tc, stream):
        import torch

        act = "gelu" if self.epilogue.startswith("bias_gelu") and case.N == 3072 else "none"
        bias = self.biases[case.N]
        if self.epilogue.endswith("_unfused"):
            if self.bt:
                mkp.mkp_gemm_bt(case.M, case.N, case.K, pa, case.K, pb, case.K, tc, case.N, stream)
            else:
                mkp.mkp_gemm(case.M, case.N, case.K, pa, case.K, pb, case.N, tc, case.N, stream)
            tc.add_(bias)
            if act == "gelu":
                tc.copy_(torch.nn.functional.gelu(tc))
            return
        mkp.mkp_gemm_ex(1, case.M, case.N, case.K, pa, case.K, 0, pb, case.K if self.bt else case.N, 0,
                        mkp.MKP_B_NK if self.bt else mkp.MKP_B_KN, tc, case.N, 0, 1.0, 0.0, bias, act, stream)

    def step(self, mkp, stream):
        for case, pa, pb, tc in self.calls:
            if self.epilogue != "none":
                self._epilogue_step(mkp, case, pa, pb, tc, stream)
            elif self.is_qkv(case):
                self._qkv_step(mkp, case, pa, pb, tc, stream)
            elif self.bt:
                mkp.mkp_gemm_batched_bt(case.batch, case.M, case.N, case.K, pa, case.K, case.M * case.K, pb, case.K,
                                        case.N * case.K, tc, case.N, case.M * case.N, stream)
            elif case.batch == 1:
                mkp.mkp_gemm(case.M, case.N, case.K, pa, case.K, pb, case.N, tc, case.N, stream)
            else:
                mkp.mkp_gemm_batched(case.batch, case.M, case.N, case.K, pa, case.K, case.M * case.K, pb, case.N,
                                     case.K * case.N, tc, case.N, case.M * case.N, stream)


class MultiWorkload:
    """Several sweeps run back to back as one step (the default benchmark:
    all five configs in order)."""

    def __init__(self, parts):
        self.parts = parts
        self.cfg = "all"
        self.bt = parts[0].bt
        self.qkv = parts[0].qkv if any(p.cfg == 2 for p in parts) else "merged"
        self.epilogue = next((p.epilogue for p in parts if p.cfg == 2), "none")
        self.cases = [c for p in parts for c in p.cases]
        self.host = [h for p in parts for h in p.host]
        self.flops = sum(p.flops for p in parts)
        self.bytes = sum(p.bytes for p in parts)
        self._owner = {c.tag: p for p in parts for c in p.cases}

    def is_qkv(self, case) -> bool:
        return self._owner[case.tag].is_qkv(case)

    def calls_per_case(self):
        return [n for p in self.parts for n in p.calls_per_case()]

    def config_of_case(self):
        """Config number of every case, in step order."""
        return [p.cfg for p in self.parts for _ in p.cases]

    def step(self, mkp, stream):
        for p in self.parts:
            p.step(mkp, stream)


class ConvWorkload:
    """Device-resident operands for the convolution sweep (NHWC inputs, KRSC
    filters, NPQK fp32 outputs), each call through mkp_conv2d."""

    bt = True
    qkv = "merged"
    epilogue = "none"

    def __init__(self):
        import torch
        import workloads

        self.cfg = "conv"
        self.cases = workloads.conv_cases()
        self.calls, self.host, self.keep = [], [], []
        for case in self.cases:
            x, w = workloads.make_conv_operands(case)
            tx = torch.from_numpy(x.view(np.int16)).cuda()
            tw = torch.from_numpy(w.view(np.int16)).cuda()
            ty = torch.empty((case.N, case.P, case.Q, case.K), dtype=torch.float32, device="cuda")
            self.keep += [tx, tw]
            self.calls.append((case, tx.data_ptr(), tw.data_ptr(), ty))
            self.host.append((case, x, w))
        self.flops = sum(c.flops for c in self.cases)
        self.bytes = sum(c.bytes for c in self.cases)

    def is_qkv(self, case) -> bool:
        return False

    def calls_per_case(self):
        return [1] * len(self.cases)

    def step(self, mkp, stream):
        for c, px, pw, ty in self.calls:
            mkp.mkp_conv2d(c.N, c.H, c.W, c.C, c.K, c.R, c.S, c.stride, c.stride, c.pad, c.pad, 1, 1, px, pw, ty,
                           None, 0, stream)


def conv_vs_gemm(wl, mkp, stream):
    """Each convolution against a plain N x K GEMM of the same M = N P Q,
    N = K, K = R S C (A a zero-filled M x K buffer), both through the
    library: mean of 50 back-to-back calls after 20 warm-up, between two HIP
    events on the launch stream.  Returns [(tag, M, N, K, conv us, GEMM us)]."""
    import torch

    cur = torch.cuda.current_stream()

    def timeit(fn):
        for _ in range(20):
            fn()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        gc.disable()   # as in timed_steps
        try:
            s.record(cur)
            for _ in range(50):
                fn()
            e.record(cur)
            torch.cuda.synchronize()
        finally:
            gc.enable()
        return s.elapsed_time(e) * 1e3 / 50

    rows = []
    for c, px, pw, ty in wl.calls:
        M, N, K = c.M, c.K, c.Kg
        ta = torch.zeros((M, K), dtype=torch.int16, device="cuda")
        tc = torch.empty((M, N), dtype=torch.float32, device="cuda")
        t_conv = timeit(lambda: mkp.mkp_conv2d(c.N, c.H, c.W, c.C, c.K, c.R, c.S, c.stride, c.stride, c.pad, c.pad,
                                               1, 1, px, pw, ty, None, 0, stream))
        t_gemm = timeit(lambda: mkp.mkp_gemm_bt(M, N, K, ta, K, pw, K, tc, N, stream))
        rows.append((c.tag, M, N, K, round(t_conv, 3), round(t_gemm, 3)))
        del ta, tc
    return rows


def conv_cpu_baseline(wl, budget_s: float):
    """The convolution oracle as it stands on the first image of each call in
    order, until `budget_s` seconds have elapsed."""
    from oracle import conv as ocv

    t0 = time.perf_counter()
    flops, n = 0, 0
    img = 0
    while time.perf_counter() - t0 < budget_s:
        done = False
        for case, x, w in wl.host:
            if time.perf_counter() - t0 >= budget_s:
                break
            if img >= case.N:
                continue
            ocv.conv2d(x[img:img + 1], w, (case.stride, case.stride), (case.pad, case.pad))
            flops += case.flops // case.N
            n += 1
            done = True
        img += 1
        if not done:
            break
    dt = time.perf_counter() - t0
    import os as _os
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": len(_os.sched_getaffinity(0)),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"binary64 convolution oracle (numpy), one image at a time over the calls in order, {n} images, "
                      f"{flops / 1e9:.1f} GFLOP in {dt:.1f} s"}


def timed_steps(wl, mkp, steps, stream):
    """Milliseconds for `steps` steps between two events on the stream.  The
    Python collector is run before and paused inside (as timeit does): a
    full collection stalls the host for tens of ms and the GPU then idles,
    which would be charged to whichever call it interrupted."""
    import torch
    torch.cuda.synchronize()
    gc.collect()
    was = gc.isenabled()
    gc.disable()
    try:
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        cur = torch.cuda.current_stream()
        s.record(cur)
        for _ in range(steps):
            wl.step(mkp, stream)
        e.record(cur)
        torch.cuda.synchronize()
    finally:
        if was:
            gc.enable()
    return s.elapsed_time(e)  # ms


def roofline_from_trace(recs):
    """Per-kernel aggregates of one traced step; the dominant kernel is the
    one with the largest total time.  Its bound follows from the algorithmic
    intensity of its launches (FLOPs / bytes against the MFMA/HBM ridge)."""
    agg = {}
    for r in recs:
        a = agg.setdefault(r["kernel"], {"us": 0.0, "flops": 0.0, "bytes": 0.0, "n": 0})
        a["us"] += r["us"]
        a["flops"] += r["flops"]
        a["bytes"] += r["bytes"]
        a["n"] += 1
    gemm = {k: v for k, v in agg.items() if v["flops"] > 0}
    dom = max(gemm, key=lambda k: gemm[k]["us"])
    d = gemm[dom]
    intensity = d["flops"] / max(d["bytes"], 1.0)
    if intensity >= RIDGE:
        achieved = d["flops"] / (d["us"] * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        achieved = d["bytes"] / (d["us"] * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(achieved / roof["peak"], 4)
    roof["traffic"] = None
    roof["kernel"] = dom
    roof["launches"] = d["n"]
    roof["avg_launch_us"] = round(d["us"] / d["n"], 3)
    roof["algorithmic_per_launch"] = {"flops": d["flops"] / d["n"], "bytes": d["bytes"] / d["n"]}
    per_kernel = {k: {"launches": v["n"], "avg_us": round(v["us"] / v["n"], 3)} for k, v in agg.items()}
    return roof, per_kernel


def sweep_fraction(recs_by_call, wl):
    """Per-GEMM fraction of its own roofline R = min(P, I*BW)."""
    fr = []
    for case, us in zip(wl.cases, recs_by_call):
        I = case.flops / case.bytes
        R = min(PEAK_BF16_TFLOPS * 1e12, I * PEAK_HBM_GBS * 1e9)
        fr.append(case.flops / (us * 1e-6) / R)
    return fr


def cpu_baseline(wl, budget_s: float):
    """The oracle as it stands, on the first rows of the workload's GEMMs in
    order, 64 rows at a time, until `budget_s` seconds have elapsed."""
    import oracle
    t0 = time.perf_counter()
    flops = 0
    rows_done = []
    while time.perf_counter() - t0 < budget_s:
        progressed = False
        for idx, (case, a, b) in enumerate(wl.host):
            if time.perf_counter() - t0 >= budget_s:
                break
            start = len([r for r in rows_done if r[0] == idx]) * 64
            if start >= case.M:
                continue
            rows = min(64, case.M - start)
            oracle.gemm(a[0, start:start + rows], b[0])
            flops += 2 * rows * case.N * case.K
            rows_done.append((idx, rows))
            progressed = True
        if not progressed:
            break
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"fp64 oracle on the first rows of the workload's {len(wl.host)} GEMMs in order (batch entry 0), "
                      f"64-row blocks, {sum(r for _, r in rows_done)} rows, {flops / 1e9:.1f} GFLOP in {dt:.1f} s"}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def kernel_source_hash() -> str:
    import hashlib
    src = os.path.join(ROOT, "dynamic_shape_gemm_amd", "csrc", "kernels.hip")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def measured_ceilings(table_path: str):
    """Sustained MFMA rate and copy bandwidth the offline stage measured."""
    try:
        for line in open(table_path):
            tok = line.split("#", 1)[0].split()
            if tok and tok[0] == "measured":
                out = {"mfma_tflops": round(float(tok[1]), 1), "hbm_gbps": round(float(tok[2]), 1)}
                if len(tok) > 3:
                    out["hbm_read_gbps"] = round(float(tok[3]), 1)
                return out
    except OSError:
        pass
    return None


def recorded_traffic(kernel: str, config):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    record (profiles/traffic.json), valid only for the kernel source it was
    taken from; None otherwise."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash() or rec.get("config") != config:
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def copy_reference(mib: int, reps: int):
    """A plain device copy of known size, for scaling rocprofv3 byte counters."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_reference_bytes_read": 4 * n, "copy_reference_bytes_written": 4 * n, "reps": reps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="all", choices=["all", "1", "2", "3", "4", "5"],
                    help="all five sweeps back to back (default) or one of them")
    ap.add_argument("--workload", choices=["gemm", "conv"], default="gemm",
                    help="the GEMM sweep of --config (default) or the ResNet-50 convolution sweep")
    ap.add_argument("--vs-gemm", action="store_true",
                    help="with --workload conv: also time each convolution against the plain GEMM of its shape "
                         "(reported under config.conv_vs_gemm)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--detail", action="store_true", help="per-GEMM timings to stderr")
    ap.add_argument("--b-layout", choices=["kn", "nk"], default="kn",
                    help="B as K x N (default) or kept N x K, a linear layer's weight layout")
    ap.add_argument("--qkv", choices=["merged", "grouped", "separate"], default="merged",
                    help="encoder linears: run the query/key/value projection as one call (default), "
                         "one grouped call over three weights, or three calls")
    ap.add_argument("--epilogue", choices=["none", "bias", "bias_gelu", "bias_gelu_unfused"], default="none",
                    help="encoder linears with a bias on every GEMM (and GELU on the FFN-up GEMMs), fused into the "
                         "GEMM epilogue or, for comparison, as separate passes")
    ap.add_argument("--fused-reduce", type=int, choices=[0, 1], default=None,
                    help="split-K partials summed by a second pass (0) or by the last split of each tile after "
                         "agent-scope fences (1); default: the library's setting")
    ap.add_argument("--fuse-regions", type=int, choices=[0, 1], default=0,
                    help="one-launch Pattern II plans over kernel pairs when the model prefers them (1) or never (0)")
    ap.add_argument("--copy-reference", type=int, default=0, metavar="MiB",
                    help="only run a plain copy of MiB (to scale rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_reference:
        torch.cuda.set_device(0)
        copy_reference(args.copy_reference, 5)
        return
    import dynamic_shape_gemm_amd as mkp
    import workloads

    torch.cuda.set_device(0)
    every = args.workload == "gemm" and args.config == "all"
    log(f"[bench] generating {'convolution sweep' if args.workload == 'conv' else f'config {args.config}'} inputs")
    if args.epilogue != "none" and args.qkv != "merged":
        raise SystemExit("--epilogue and --qkv are separate experiments")
    if args.workload == "conv":
        wl = ConvWorkload()
    elif every:
        wl = MultiWorkload([Workload(c, copies=4, b_layout=args.b_layout, qkv=args.qkv,
                                     epilogue=args.epilogue if c == 2 else "none")
                            for c in (1, 2, 3, 4, 5)])
    else:
        wl = Workload(int(args.config), copies=4, b_layout=args.b_layout, qkv=args.qkv, epilogue=args.epilogue)
    stream = torch.cuda.current_stream().cuda_stream
    mkp.mkp_set_option("fuse_regions", args.fuse_regions)
    if args.fused_reduce is not None:
        mkp.mkp_set_option("fused_reduce", args.fused_reduce)
    mkp.mkp_cache_clear()

    # first step: plan misses (polymerization) + launches, timed on its own
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    wl.step(mkp, stream)
    torch.cuda.synchronize()
    first_ms = (time.perf_counter() - t0) * 1e3
    stats0 = mkp.mkp_stats()
    log(f"[bench] first step {first_ms:.2f} ms, {stats0['misses']} plans in {stats0['plan_us_total']:.1f} us")
    for _ in range(max(args.warmup - 1, 0)):
        wl.step(mkp, stream)
    torch.cuda.synchronize()
    log(f"[bench] warmup done, timing {args.steps} steps")
    ms = timed_steps(wl, mkp, args.steps, stream)
    ms_per_step = ms / args.steps
    value = wl.flops / (ms_per_step * 1e-3) / 1e12
    log(f"[bench] {ms_per_step:.3f} ms/step, {value:.1f} TFLOP/s")
    # each sweep of the pass timed on its own (same step count)
    part_ms = {}
    if every:
        for part in wl.parts:
            part_ms[part.cfg] = timed_steps(part, mkp, args.steps, stream) / args.steps
            log(f"[bench]   config {part.cfg}: {part_ms[part.cfg]:.3f} ms/step, "
                f"{part.flops / (part_ms[part.cfg] * 1e-3) / 1e12:.1f} TFLOP/s")

    # traced steps: per-launch HIP events on the launch stream
    ntr = 3
    mkp.mkp_set_option("trace", 1)
    recs_all = []
    for _ in range(ntr):
        wl.step(mkp, stream)
        torch.cuda.synchronize()
        recs_all.append(mkp.mkp_trace_dump())
    mkp.mkp_set_option("trace", 0)
    roof, per_kernel = roofline_from_trace([r for recs in recs_all for r in recs])
    traffic_key = "all" if every else (int(args.config) if args.workload == "gemm" else None)
    roof["traffic"] = recorded_traffic(roof["kernel"], traffic_key) if traffic_key is not None else None
    # per-call durations (a call may hold several launches), median of the
    # traced steps; each record also learns which case it belongs to
    counts = wl.calls_per_case()
    per_step = []
    case_recs = [[] for _ in wl.cases]
    for recs in recs_all:
        by_call = {}
        for r in recs:
            by_call.setdefault(r["call"], []).append(r)
        calls = sorted(by_call)
        assert len(calls) == sum(counts), (len(calls), sum(counts))
        per_case, i = [], 0
        for ci, c in enumerate(counts):   # a case made of several library calls sums them
            rs = [r for k in calls[i:i + c] for r in by_call[k]]
            per_case.append(sum(r["us"] for r in rs))
            case_recs[ci] += rs
            i += c
        per_step.append(per_case)
    per_call = [float(np.median(v)) for v in zip(*per_step)]
    fr = sweep_fraction(per_call, wl)
    if args.detail:
        for ci, (case, us, f) in enumerate(zip(wl.cases, per_call, fr)):
            # the GEMM view of the call (a convolution: N P Q x K x R S C)
            gm, gn, gk = (case.M, case.K, case.Kg) if wl.cfg == "conv" else (case.M, case.N, case.K)
            if wl.cfg == "conv":
                # a convolution is planned on the kernels with a convolution
                # form: name the ones its traced calls launched
                names = list(dict.fromkeys(r["kernel"] for r in case_recs[ci]))
                log(f"  {case.tag:>14} {gm:5d}x{gn:5d}x{gk:5d} b{case.batch:<3d} {us:9.2f} us "
                    f"{case.flops / us / 1e6:8.1f} TF/s  {100 * f:5.1f}% of R  conv {'+'.join(names)}")
                continue
            if wl.is_qkv(case):
                plan = mkp.mkp_plan_describe_grouped(case.M, case.K, [768] * 3, bt=wl.bt)
                if wl.qkv == "separate":
                    plan = dict(mkp.mkp_plan_describe(1, case.M, 768, case.K, bt=wl.bt), pattern="3x")
            else:
                plan = mkp.mkp_plan_describe(case.batch, gm, gn, gk, bt=wl.bt)
            ks = "+".join(f"{r['kernel']}/s{r['s']}" for r in plan["regions"]) + (" (1 launch)" if plan.get("fused")
                                                                                    else "")
            log(f"  {case.tag:>14} {gm:5d}x{gn:5d}x{gk:5d} b{case.batch:<3d} {us:9.2f} us "
                f"{case.flops / us / 1e6:8.1f} TF/s  {100 * f:5.1f}% of R  {plan['pattern']:4s} {ks}")

    per_config, gates = None, None
    if every:
        cfg_of = wl.config_of_case()
        per_config = {}
        for part in wl.parts:
            idx = [i for i, c in enumerate(cfg_of) if c == part.cfg]
            sub_recs = [r for i in idx for r in case_recs[i]]
            sub_roof, _ = roofline_from_trace(sub_recs)
            sub_roof["traffic"] = recorded_traffic(sub_roof["kernel"], part.cfg)
            kern_us = sum(per_call[i] for i in idx)
            per_config[str(part.cfg)] = {
                "workload": workloads.CONFIG_NAMES[part.cfg],
                "gemm_calls": len(part.cases),
                "ms_per_step": round(part_ms[part.cfg], 4),
                "tflops": round(part.flops / (part_ms[part.cfg] * 1e-3) / 1e12, 2),
                "flops_per_step": part.flops,
                "bytes_per_step": part.bytes,
                # algorithmic bytes over the sweep's kernel time (traced)
                "hbm_gbps_kernel_time": round(part.bytes / (kern_us * 1e-6) / 1e9, 1),
                "roofline_frac_median": round(float(np.median([fr[i] for i in idx])), 4),
                "roofline_frac_min": round(float(np.min([fr[i] for i in idx])), 4),
                "dominant": sub_roof,
            }
        sq = next(i for i, c in enumerate(wl.cases) if c.tag == "c3[square]")
        dec = [i for i, c in enumerate(cfg_of) if c == 4]
        gates = {
            "square_4096_tflops": round(wl.cases[sq].flops / (per_call[sq] * 1e-6) / 1e12, 1),
            "square_4096_frac_of_bf16_peak": round(wl.cases[sq].flops / (per_call[sq] * 1e-6) / 1e12 /
                                                   PEAK_BF16_TFLOPS, 4),
            "decoder_sweep_frac_of_hbm_peak": round(sum(wl.cases[i].bytes for i in dec) /
                                                    (sum(per_call[i] for i in dec) * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "decoder_dominant_kernel_frac": per_config["4"]["dominant"]["frac"],
            "decoder_dominant_kernel_bound": per_config["4"]["dominant"]["bound"],
        }

    workload_name = (workloads.CONV_NAME if args.workload == "conv" else
                     "all five sweeps: " + "; ".join(workloads.CONFIG_NAMES[c] for c in (1, 2, 3, 4, 5)) if every
                     else workloads.CONFIG_NAMES[int(args.config)])
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": workload_name,
            "config_index": None if args.workload == "conv" else ("all" if every else int(args.config)),
            "b_layout": "nk" if args.workload == "conv" else args.b_layout,
            "qkv": wl.qkv,
            "epilogue": wl.epilogue,
            "fuse_regions": args.fuse_regions,
            "fused_reduce": args.fused_reduce,
            "gemms_per_step": len(wl.cases),
            "flops_per_step": wl.flops,
            "bytes_per_step": wl.bytes,
            "first_step_ms": round(first_ms, 3),
            "plans_built": stats0["misses"],
            "plan_us_total": round(stats0["plan_us_total"], 1),
            "roofline_frac_median": round(float(np.median(fr)), 4),
            "roofline_frac_min": round(float(np.min(fr)), 4),
            "kernels": per_kernel,
            "table": os.path.relpath(mkp.mkp_stats()["table"], ROOT) if os.path.isabs(mkp.mkp_stats()["table"])
            else mkp.mkp_stats()["table"],
            "measured_ceiling": measured_ceilings(mkp.mkp_stats()["table"]),
            "kernel_source_sha256_16": kernel_source_hash(),
        },
        "roofline": roof,
    }
    if per_config is not None:
        out["config"]["per_config"] = per_config
        out["config"]["gates"] = gates
    if args.vs_gemm and args.workload == "conv":
        log("[bench] each convolution against the GEMM of its shape")
        out["config"]["conv_vs_gemm"] = conv_vs_gemm(wl, mkp, stream)
    if not args.no_cpu:
        log(f"[bench] CPU oracle baseline ({args.cpu_seconds:.0f} s budget)")
        out["cpu_baseline"] = (conv_cpu_baseline(wl, args.cpu_seconds) if args.workload == "conv"
                               else cpu_baseline(wl, args.cpu_seconds))
    print(json.dumps(out), flush=True)

if __name__ == "__main__":
    main()
