"""Measured evaluation of the polymerizer on one GPU.

    python -m dynamic_shape_gemm_amd.planner_eval --config 2 --json out.json --md out.md

For every distinct GEMM shape of a sweep it times, through the C ABI:

* MikPoly: the plan the cost model picks (the default options);
* MikPoly-WAVE and MikPoly-PIPE: the plans picked when the cost keeps only
  f_wave or only f_pipe (MikPoly page, section 5 "cost-model effectiveness");
* every micro-kernel forced alone over the whole output (Pattern I) with
  every split-K factor up to the K-step count: the best of these per shape
  is the "best fixed tile", and the best at one split the "fixed tile, no
  split-K";
* the R cheapest candidates of the whole modelled space (plan_rank 1..R).

ORACLE (the page's exhaustive measured search) is read as the fastest
measured plan of all of the above: every Pattern I plan and the R best
modelled plans of Patterns I and II, MikPoly's own plan included.  Each
variant is timed as `reps` back-to-back calls after `warmup` calls.  The
calls rotate over enough copies of the operands (at least 768 MB in all,
beyond the 256 MB last-level cache) that each one streams them from HBM, as
the sweeps' GEMMs do in the benchmark; MikPoly's plan is timed first and
again last (the faster counts), so a clock still ramping up at the start of
a shape does not count against it.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def table_splits(path):
    for raw in open(path):
        tok = raw.split("#", 1)[0].split()
        if tok and tok[0] == "splitk":
            return [int(x) for x in tok[1:]]
    return [1]


def geomean(xs):
    xs = [x for x in xs if x > 0]
    return math.exp(sum(math.log(x) for x in xs) / len(xs)) if xs else float("nan")


ROTATE_BYTES = 768 << 20


class Shape:
    def __init__(self, case, torch, mkp):
        self.case = case
        self.b, self.M, self.N, self.K = case.batch, case.M, case.N, case.K
        g = torch.Generator(device="cpu").manual_seed(1234)
        # values do not change the time of a GEMM: uniform bf16 in [-1, 1)
        A = (torch.rand((self.b, self.M, self.K), generator=g) * 2 - 1).to(torch.bfloat16).cuda()
        B = (torch.rand((self.b, self.K, self.N), generator=g) * 2 - 1).to(torch.bfloat16).cuda()
        per = self.b * (2 * self.M * self.K + 2 * self.K * self.N + 4 * self.M * self.N)
        n = max(1, min(64, -(-ROTATE_BYTES // max(per, 1))))
        self.copies = [(A, B, torch.empty((self.b, self.M, self.N), dtype=torch.float32, device="cuda"))]
        for _ in range(n - 1):
            self.copies.append((A.clone(), B.clone(),
                                torch.empty((self.b, self.M, self.N), dtype=torch.float32, device="cuda")))
        self.i = 0
        self.mkp = mkp
        self.stream = torch.cuda.current_stream().cuda_stream

    @property
    def flops(self):
        return 2.0 * self.b * self.M * self.N * self.K

    def call(self):
        m = self.mkp
        A, B, C = self.copies[self.i % len(self.copies)]
        self.i += 1
        if self.b == 1:
            return m.mkp_gemm_raw(self.M, self.N, self.K, A, self.K, B, self.N, C, self.N, self.stream)
        return m.mkp_gemm_batched_raw(self.b, self.M, self.N, self.K, A, self.K, self.M * self.K, B,
                                      self.N, self.K * self.N, C, self.N, self.M * self.N, self.stream)

    def free(self):
        del self.copies


def time_variant(torch, shp, warmup, reps):
    """Microseconds per call, or None if the library has no such plan."""
    rc = shp.call()
    if rc != 0:
        msg = shp.mkp.last_error()
        if "plan_rank" not in msg:   # a rank beyond the candidate list is expected
            log(f"[eval] {shp.b}x{shp.M}x{shp.N}x{shp.K}: error {rc}: {msg}")
        return None
    for _ in range(warmup):
        shp.call()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream()
    s.record(cur)
    for _ in range(reps):
        shp.call()
    e.record(cur)
    torch.cuda.synchronize()
    return s.elapsed_time(e) * 1e3 / reps


def evaluate_shape(torch, mkp, shp, kernels, splits, ranks, warmup, reps):
    t0 = time.perf_counter()
    rec = {"shape": [shp.b, shp.M, shp.N, shp.K], "flops": shp.flops}
    measured = []   # (us, label)

    def run(label, opts):
        for k, v in opts:
            mkp.mkp_set_option(k, v)
        try:
            us = time_variant(torch, shp, warmup, reps)
        finally:
            for k, v in reversed(opts):
                mkp.mkp_set_option(k, {"force_kernel": "", "force_splitk": 0, "cost_model": "full",
                                       "plan_rank": 0}[k])
        if us is not None:
            measured.append((us, label))
        return us

    plan = mkp.mkp_plan_describe(shp.b, shp.M, shp.N, shp.K)
    rec["plan"] = {"pattern": plan["pattern"],
                   "regions": [(r["kernel"], r["m"], r["n"], r["s"]) for r in plan["regions"]],
                   "plan_us": plan["plan_us"]}
    rec["mikpoly_us"] = run("mikpoly", [])
    rec["wave_us"] = run("wave", [("cost_model", "wave")])
    rec["pipe_us"] = run("pipe", [("cost_model", "pipe")])
    t3 = -(-shp.K // 64)
    fixed = {}
    for kn in kernels:
        per = {}
        for s in splits:
            if s > max(t3, 1):
                continue
            us = run(f"{kn}/s{s}", [("force_kernel", kn), ("force_splitk", s)])
            if us is not None:
                per[s] = us
        if per:
            bs = min(per, key=per.get)
            fixed[kn] = {"s1_us": per.get(1), "best_us": per[bs], "best_s": bs}
    rec["fixed"] = fixed
    rank_us = []
    for r in range(1, ranks + 1):
        us = run(f"rank{r}", [("plan_rank", r)])
        if us is None:
            break
        rank_us.append(us)
    rec["rank_us"] = rank_us
    again = run("mikpoly", [])
    if again is not None and (rec["mikpoly_us"] is None or again < rec["mikpoly_us"]):
        rec["mikpoly_us"] = again
    if not measured:
        raise RuntimeError(f"no variant of {rec['shape']} ran")
    best = min(measured)
    rec["oracle_us"], rec["oracle_from"] = best
    bf = min(fixed.items(), key=lambda kv: kv[1]["best_us"])
    rec["best_fixed_us"], rec["best_fixed"] = bf[1]["best_us"], f"{bf[0]}/s{bf[1]['best_s']}"
    s1 = [(v["s1_us"], k) for k, v in fixed.items() if v["s1_us"] is not None]
    rec["fixed_s1_us"], rec["fixed_s1"] = min(s1) if s1 else (None, None)
    rec["variants_measured"] = len(measured)
    rec["search_s"] = time.perf_counter() - t0
    return rec


def summarize(recs):
    out = {"shapes": len(recs)}
    tot_flops = sum(r["flops"] for r in recs)

    def agg(key):
        us = [r[key] for r in recs]
        if any(u is None for u in us):
            return None
        return round(tot_flops / sum(us) / 1e6, 2)   # TFLOP/s over the sweep (us -> 1e6)

    for name, key in (("oracle", "oracle_us"), ("mikpoly", "mikpoly_us"), ("wave", "wave_us"),
                      ("pipe", "pipe_us"), ("best_fixed", "best_fixed_us"), ("fixed_s1", "fixed_s1_us")):
        rel = [r["oracle_us"] / r[key] for r in recs if r[key]]
        out[name] = {"tflops_sweep": agg(key), "geomean_vs_oracle": round(geomean(rel), 4),
                     "min_vs_oracle": round(min(rel), 4) if rel else None}
    gate = [r["best_fixed_us"] / r["mikpoly_us"] for r in recs]
    out["gate_vs_best_fixed"] = {"min": round(min(gate), 4), "geomean": round(geomean(gate), 4),
                                 "below_0.5": sum(1 for g in gate if g < 0.5)}
    out["plan_us_median"] = round(statistics.median(r["plan"]["plan_us"] for r in recs), 2)
    out["oracle_search_s_median"] = round(statistics.median(r["search_s"] for r in recs), 3)
    out["variants_per_shape_median"] = statistics.median(r["variants_measured"] for r in recs)
    return out


def markdown(cfg, name, summary, recs, cmd):
    lines = [f"# Polymerizer, measured: config {cfg} ({name})", "",
             "Command (from the repository root, on one MI355X):", "", "```", cmd, "```", "",
             f"{summary['shapes']} distinct shapes; per shape about {summary['variants_per_shape_median']:.0f} "
             "measured plans (every micro-kernel forced alone with every split-K factor, the ablated cost "
             "models, the best modelled candidates by rank). ORACLE = the fastest of them.", "",
             "| variant | TFLOP/s over the sweep | geomean vs ORACLE | worst shape vs ORACLE |",
             "|---|---:|---:|---:|"]
    label = {"oracle": "ORACLE (measured search)", "mikpoly": "MikPoly (cost model)",
             "wave": "MikPoly-WAVE (f_wave only)", "pipe": "MikPoly-PIPE (f_pipe only)",
             "best_fixed": "best fixed tile (per shape, best split)", "fixed_s1": "best fixed tile, no split-K"}
    for k, lab in label.items():
        v = summary[k]
        lines.append(f"| {lab} | {v['tflops_sweep']} | {v['geomean_vs_oracle']} | {v['min_vs_oracle']} |")
    g = summary["gate_vs_best_fixed"]
    lines += ["", f"MikPoly vs the best fixed tile of each shape: min {g['min']}, geomean {g['geomean']}, "
              f"shapes below 0.5: {g['below_0.5']}.", "",
              f"Search time per shape: cost model {summary['plan_us_median']} us (median); "
              f"measuring the candidates {summary['oracle_search_s_median']} s (median).", "",
              "Shapes where MikPoly is furthest from ORACLE:", "",
              "| batch, M, N, K | MikPoly us | plan | ORACLE us | ORACLE plan | best fixed us |",
              "|---|---:|---|---:|---|---:|"]
    worst = sorted(recs, key=lambda r: r["oracle_us"] / r["mikpoly_us"])[:10]
    for r in worst:
        plan = " + ".join(f"{k}[{m}x{n}]/s{s}" for k, m, n, s in r["plan"]["regions"])
        lines.append(f"| {r['shape']} | {r['mikpoly_us']:.2f} | {r['plan']['pattern']} {plan} | "
                     f"{r['oracle_us']:.2f} | {r['oracle_from']} | {r['best_fixed_us']:.2f} ({r['best_fixed']}) |")
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--ranks", type=int, default=16)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--max-shapes", type=int, default=0, help="0 = every distinct shape")
    ap.add_argument("--json", default="")
    ap.add_argument("--md", default="")
    a = ap.parse_args()

    import torch
    sys.path.insert(0, ROOT)
    import dynamic_shape_gemm_amd as mkp
    import workloads

    if not torch.cuda.is_available():
        raise SystemExit("planner_eval needs a GPU")
    torch.cuda.init()
    # the calls give B as K x N: the fixed-kernel baselines are the K x N kernels
    kernels = [k for k in mkp.mkp_kernel_names() if not k.endswith("_nk")]
    splits = table_splits(os.environ.get("MKP_CALIB", os.path.join(HERE, "calib", "gfx950.tbl")))
    seen, cases = set(), []
    for c in workloads.config_cases(a.config):
        key = (c.batch, c.M, c.N, c.K)
        if key not in seen:
            seen.add(key)
            cases.append(c)
    if a.max_shapes:
        cases = cases[:a.max_shapes]
    log(f"[eval] config {a.config}: {len(cases)} shapes, {len(kernels)} kernels, splits {splits}")
    recs = []
    for i, c in enumerate(cases):
        shp = Shape(c, torch, mkp)
        rec = evaluate_shape(torch, mkp, shp, kernels, splits, a.ranks, a.warmup, a.reps)
        shp.free()
        recs.append(rec)
        log(f"[eval] {i + 1}/{len(cases)} {rec['shape']} mikpoly {rec['mikpoly_us']:.2f} us, oracle "
            f"{rec['oracle_us']:.2f} us ({rec['oracle_from']}), best fixed {rec['best_fixed_us']:.2f} us")
    summary = summarize(recs)
    summary["config"] = a.config
    summary["workload"] = workloads.CONFIG_NAMES.get(a.config, str(a.config))
    print(json.dumps(summary))
    if a.json:
        json.dump({"summary": summary, "shapes": recs}, open(a.json, "w"), indent=1)
    if a.md:
        cmd = ("python3 -m dynamic_shape_gemm_amd.planner_eval " + " ".join(
            f"--{k.replace('_', '-')} {v}" for k, v in (("config", a.config), ("ranks", a.ranks),
                                                        ("warmup", a.warmup), ("reps", a.reps)))
               + f" --md {os.path.relpath(a.md, ROOT) if os.path.isabs(a.md) else a.md}")
        open(a.md, "w").write(markdown(a.config, summary["workload"], summary, recs, cmd))


if __name__ == "__main__":
    main()
