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

ORACLE (the page's exhaustive measured search) is, with `--space full`
(the default), the fastest plan of the whole candidate space: every Pattern
I plan measured, and every Pattern II plan -- each tile-aligned cut of either
dimension, each pair of distinct kernels, each split of each region --
priced as the sum of its two regions' measured times.  A region is timed on
its own as the forced kernel and split over a sub-matrix of the region's
extent; its time does not depend on where the sub-matrix starts (the cuts
keep every alignment), so each (kernel, split, extent) is timed once and
serves as a first region at one cut and as a second region at others.  The
two launches of a Pattern II plan run back to back on one stream, so their
sum is the plan's time; the report checks this on the Pattern II plans the
cost model picks, measured whole.  With `--space ranked` ORACLE is the
fastest of the Pattern I plans and the R best modelled plans.  Each
variant is timed as `reps` back-to-back calls after `warmup` calls.  The
calls rotate over enough copies of the operands (at least 768 MB in all,
beyond the 256 MB last-level cache) that each one streams them from HBM, as
the sweeps' GEMMs do in the benchmark; MikPoly's plan is timed first and
again last (the faster counts), so a clock still ramping up at the start of
a shape does not count against it.
"""
from __future__ import annotations

import argparse
import gc
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

    def call(self, m_ext=None, n_ext=None):
        """One call over the whole output, or over its first m_ext rows (or
        n_ext columns) with the operands' strides unchanged."""
        m = self.mkp
        A, B, C = self.copies[self.i % len(self.copies)]
        self.i += 1
        M = self.M if m_ext is None else m_ext
        N = self.N if n_ext is None else n_ext
        if self.b == 1:
            return m.mkp_gemm_raw(M, N, self.K, A, self.K, B, self.N, C, self.N, self.stream)
        return m.mkp_gemm_batched_raw(self.b, M, N, self.K, A, self.K, self.M * self.K, B,
                                      self.N, self.K * self.N, C, self.N, self.M * self.N, self.stream)

    def free(self):
        del self.copies


def time_variant(torch, shp, warmup, reps, m_ext=None, n_ext=None):
    """Microseconds per call, or None if the library has no such plan."""
    rc = shp.call(m_ext, n_ext)
    if rc != 0:
        msg = shp.mkp.last_error()
        if "plan_rank" not in msg:   # a rank beyond the candidate list is expected
            log(f"[eval] {shp.b}x{shp.M}x{shp.N}x{shp.K}: error {rc}: {msg}")
        return None
    for _ in range(warmup):
        shp.call(m_ext, n_ext)
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream()
    # no collector pass inside the timed calls (it stalls the host, and the
    # GPU idles, for tens of ms)
    gc.disable()
    try:
        s.record(cur)
        for _ in range(reps):
            shp.call(m_ext, n_ext)
        e.record(cur)
        torch.cuda.synchronize()
    finally:
        gc.enable()
    return s.elapsed_time(e) * 1e3 / reps


def tile_dims(name):
    """(uM, uN) from a kernel name m<uM>n<uN>k<uK>..."""
    i, j = name.index("n"), name.index("k")
    return int(name[1:i]), int(name[i + 1:j])


def full_space_pattern_II(torch, mkp, shp, kernels, splits, warmup, reps):
    """The cheapest measured Pattern II plan over every tile-aligned cut of
    M and of N, every ordered pair of distinct kernels and every split of
    each region: (us, label, regions timed).  Each (kernel, split, extent)
    region is timed once, over the first rows (columns) of the output."""
    t3 = max(-(-shp.K // 64), 1)
    usable = [s for s in splits if s <= t3]
    timed = {}
    t0 = time.perf_counter()

    def region(k, s, dim, ext):
        key = (k, s, dim, ext)
        if key not in timed:
            mkp.mkp_set_option("force_kernel", k)
            mkp.mkp_set_option("force_splitk", s)
            timed[key] = time_variant(torch, shp, warmup, reps, *((ext, None) if dim == 0 else (None, ext)))
            if len(timed) % 2000 == 0:
                log(f"[eval]   {len(timed)} regions timed ({time.perf_counter() - t0:.0f} s)")
        return timed[key]

    best = (math.inf, None)
    try:
        for dim, ext in ((0, shp.M), (1, shp.N)):
            dims = {k: tile_dims(k)[dim] for k in kernels}
            # the best split of each kernel over each extent it serves
            best_of = {}
            for k in kernels:
                exts = {c for c in range(dims[k], ext, dims[k])}
                exts |= {ext - c for a in kernels for c in range(dims[a], ext, dims[a])}
                for e in sorted(exts):
                    vals = [(region(k, s, dim, e), s) for s in usable]
                    vals = [v for v in vals if v[0] is not None]
                    if vals:
                        best_of[(k, e)] = min(vals)
            for a in kernels:
                for cut in range(dims[a], ext, dims[a]):
                    r1 = best_of.get((a, cut))
                    if r1 is None:
                        continue
                    for b in kernels:
                        r2 = best_of.get((b, ext - cut))
                        if b == a or r2 is None:
                            continue
                        if r1[0] + r2[0] < best[0]:
                            tag = "M" if dim == 0 else "N"
                            best = (r1[0] + r2[0], f"II-{tag} {a}/s{r1[1]}[{cut}] + {b}/s{r2[1]}[{ext - cut}]")
    finally:
        mkp.mkp_set_option("force_kernel", "")
        mkp.mkp_set_option("force_splitk", 0)
    return best[0], best[1], len(timed), timed


def evaluate_shape(torch, mkp, shp, kernels, splits, ranks, warmup, reps, space="full", region_reps=3):
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
    if space == "full":
        us, label, n, timed = full_space_pattern_II(torch, mkp, shp, kernels, splits, 1, region_reps)
        rec["regions_timed"] = n
        if label is not None:
            measured.append((us, label))
            rec["best_II_us"], rec["best_II"] = us, label
        # the composition checked on the cost model's own Pattern II plan
        if plan["pattern"] in ("II-M", "II-N") and not plan.get("fused") and not plan.get("transpose_b"):
            dim = 0 if plan["pattern"] == "II-M" else 1
            parts = []
            for r in plan["regions"]:
                ext = r["m"] if dim == 0 else r["n"]
                parts.append(timed.get((r["kernel"], r["s"], dim, ext)))
            if all(p is not None for p in parts) and rec["mikpoly_us"]:
                rec["II_sum_vs_whole"] = round(sum(parts) / rec["mikpoly_us"], 4)
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
    if any("regions_timed" in r for r in recs):
        out["regions_timed_median"] = statistics.median(r.get("regions_timed", 0) for r in recs)
        chk = [r["II_sum_vs_whole"] for r in recs if "II_sum_vs_whole" in r]
        out["II_sum_vs_whole"] = {"plans": len(chk), "geomean": round(geomean(chk), 4) if chk else None,
                                  "min": min(chk) if chk else None, "max": max(chk) if chk else None}
    return out


def markdown(cfg, name, summary, recs, cmd, space="full", sample=""):
    if space == "full":
        what = (f"{summary['shapes']} distinct shapes{sample}. ORACLE = the fastest plan of the whole candidate "
                "space: every micro-kernel forced alone over the output with every split-K factor (Pattern I, "
                "measured), and every Pattern II plan -- each tile-aligned cut of M and of N, each pair of "
                "distinct kernels, each split of each region -- priced as the sum of its two regions, each "
                f"region timed on its own (median {summary['regions_timed_median']:.0f} regions timed per "
                "shape). The ablated cost models and the best modelled candidates by rank are measured as "
                "well.")
        chk = summary["II_sum_vs_whole"]
        if chk["plans"]:
            what += (f" Check of the sum: on the {chk['plans']} Pattern II plans the cost model picked, the "
                     f"sum of the two regions' times over the plan measured whole is {chk['geomean']} "
                     f"(geomean; {chk['min']} to {chk['max']}).")
    else:
        what = (f"{summary['shapes']} distinct shapes{sample}; per shape about "
                f"{summary['variants_per_shape_median']:.0f} measured plans (every micro-kernel forced alone "
                "with every split-K factor, the ablated cost models, the best modelled candidates by rank). "
                "ORACLE = the fastest of them.")
    lines = [f"# Polymerizer, measured: config {cfg} ({name})", "",
             "Command (from the repository root, on one MI355X):", "", "```", cmd, "```", "", what, "",
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
    ap.add_argument("--sample", type=int, default=0,
                    help="time this many distinct shapes drawn at random (seeded), 0 = all")
    ap.add_argument("--seed", type=int, default=7)
    ap.add_argument("--space", choices=["full", "ranked"], default="full")
    ap.add_argument("--region-reps", type=int, default=3)
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
    sample = ""
    if a.sample and a.sample < len(cases):
        pick = sorted(np.random.default_rng(a.seed).choice(len(cases), size=a.sample, replace=False))
        sample = f" (a seeded sample, seed {a.seed}, of the sweep's {len(cases)})"
        cases = [cases[i] for i in pick]
    if a.max_shapes:
        cases = cases[:a.max_shapes]
    log(f"[eval] config {a.config}: {len(cases)} shapes, {len(kernels)} kernels, splits {splits}")
    recs = []
    for i, c in enumerate(cases):
        shp = Shape(c, torch, mkp)
        rec = evaluate_shape(torch, mkp, shp, kernels, splits, a.ranks, a.warmup, a.reps, a.space, a.region_reps)
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
        opts = [("config", a.config), ("ranks", a.ranks), ("warmup", a.warmup), ("reps", a.reps),
                ("space", a.space), ("region-reps", a.region_reps)]
        if a.sample:
            opts += [("sample", a.sample), ("seed", a.seed)]
        cmd = ("python3 -m dynamic_shape_gemm_amd.planner_eval " + " ".join(f"--{k} {v}" for k, v in opts)
               + f" --md {os.path.relpath(a.md, ROOT) if os.path.isabs(a.md) else a.md}")
        open(a.md, "w").write(markdown(a.config, summary["workload"], summary, recs, cmd, a.space, sample))


if __name__ == "__main__":
    main()
