"""The library's polymerizer (through the C-ABI, no GPU) against the
cost-model oracle: the MikPoly page's case study, exact search (the pruned
search reaches the exhaustive minimum over the same space), recomputed plan
costs, and coverage of the output by the chosen regions."""
import json
import os

import numpy as np
import pytest

from oracle import cost_model as cm

GOLD = os.path.join(os.path.dirname(__file__), "golden", "mikpoly_case_study.json")


@pytest.fixture(scope="module")
def mkp():
    import dynamic_shape_gemm_amd as m
    return m


def to_regions(plan):
    return [cm.Region(r["m0"], r["n0"], r["m"], r["n"], r["kernel"], r["s"]) for r in plan["regions"]]


def case_table_text(Ta, Tb):
    g = json.load(open(GOLD))
    A, B = g["kernel_A"], g["kernel_B"]
    fa = g["shape"][2] // A["tile"][2]
    fb = g["shape"][2] // B["tile"][2]
    wa = g["resident_warps_per_sm"] // A["warps"]
    wb = g["resident_warps_per_sm"] // B["warps"]
    return g, f"""device {g['sms']}
launch_us 0
splitk 1
kernel A {A['tile'][0]} {A['tile'][1]} {A['tile'][2]} {wa}
kernel B {B['tile'][0]} {B['tile'][1]} {B['tile'][2]} {wb}
g A 1:{Ta / fa} {fa}:{Ta}
g B 1:{Tb / fb} {fb}:{Tb}
"""


@pytest.mark.parametrize("Ta,Tb", [(10.0, 3.0), (10.0, 4.9), (10.0, 6.0), (10.0, 12.0)])
def test_case_study_through_library(mkp, Ta, Tb):
    g, text = case_table_text(Ta, Tb)
    M, N, K = g["shape"]
    tab = cm.parse_table(text)
    plan = mkp.mkp_plan_with_table(text, 1, M, N, K)
    ex = mkp.mkp_plan_with_table(text, 1, M, N, K, exhaustive=True)
    best = cm.exhaustive_best(tab, M, N, K)
    assert plan["cost_us"] == pytest.approx(best[0], rel=1e-12)
    assert ex["cost_us"] == pytest.approx(best[0], rel=1e-12)
    assert cm.plan_cost(tab, to_regions(plan), K, 1) == pytest.approx(plan["cost_us"], rel=1e-12)
    # never worse than the page's two strategies (2 Ta and Ta + 2 Tb)
    assert plan["cost_us"] <= min(2 * Ta, Ta + 2 * Tb) + 1e-9
    if Ta > 2 * Tb:
        assert plan["pattern"] in ("II-M", "II-N")
    if Tb >= Ta:  # B is never cheaper per task: one wave of A per region pair cannot win
        assert plan["cost_us"] == pytest.approx(2 * Ta)


def random_table(rng, nk, tails=False, skinny=False):
    cus = int(rng.integers(2, 12))
    lines = [f"device {cus}", f"launch_us {rng.uniform(0, 3):.3f}", "splitk 1 2 3 4 8",
             f"reduce {rng.uniform(0, 2):.3f} {rng.uniform(100, 2000):.1f}"]
    names = []
    for i in range(nk):
        uM = int(rng.choice([16, 32, 48, 64]))
        uN = int(rng.choice([16, 32, 64]))
        uK = int(rng.choice([16, 32]))
        lines.append(f"kernel k{i} {uM} {uN} {uK} {int(rng.integers(1, 4))}")
        names.append(f"k{i}")
    for n in names:
        base = rng.uniform(0.2, 2.0)
        slope = rng.uniform(0.05, 1.0)
        pts = " ".join(f"{t}:{base + slope * t * rng.uniform(0.9, 1.1):.4f}" for t in (1, 3, 8, 20))
        lines.append(f"g {n} {pts}")
        if tails:
            for key in ("tail", "tailx"):
                fs = sorted(rng.uniform(0.05, 0.95, size=int(rng.integers(1, 4))))
                lines.append(f"{key} {n} " + " ".join(f"{f:.3f}:{rng.uniform(0.05, 1.0):.3f}" for f in fs))
    if skinny:
        # curves per tile-row class for most kernels and classes, cheaper or
        # dearer than the square ones
        classes = sorted(int(x) for x in rng.choice([1, 2, 3, 4, 6], size=int(rng.integers(1, 4)), replace=False))
        lines.append("rows " + " ".join(str(r) for r in classes))
        for n in names:
            for r in classes:
                if rng.uniform() < 0.3:
                    continue
                base = rng.uniform(0.2, 2.0)
                slope = rng.uniform(0.05, 1.0)
                pts = " ".join(f"{t}:{base + slope * t * rng.uniform(0.9, 1.1):.4f}" for t in (1, 4, 16))
                lines.append(f"g@{r} {n} {pts}")
                if tails:
                    for key in ("tail", "tailx"):
                        fs = sorted(rng.uniform(0.05, 0.95, size=int(rng.integers(1, 4))))
                        lines.append(f"{key}@{r} {n} " +
                                     " ".join(f"{f:.3f}:{rng.uniform(0.05, 1.0):.3f}" for f in fs))
    return "\n".join(lines) + "\n"


def test_pruned_search_is_exact(mkp):
    """Also: one-launch candidates stay out of the search unless enabled."""
    text = _with_pairs(np.random.default_rng(1), random_table(np.random.default_rng(1), 3))
    assert not mkp.mkp_plan_with_table(text, 1, 300, 300, 300)["fused"]
    rng = np.random.default_rng(2024)
    checked = 0
    for trial in range(40):
        text = random_table(rng, int(rng.integers(2, 4)))
        tab = cm.parse_table(text)
        M, N, K = (int(x) for x in rng.integers(1, 200, size=3))
        batch = int(rng.choice([1, 1, 3]))
        plan = mkp.mkp_plan_with_table(text, batch, M, N, K)
        ex = mkp.mkp_plan_with_table(text, batch, M, N, K, exhaustive=True)
        best = cm.exhaustive_best(tab, M, N, K, batch)
        assert plan["cost_us"] == pytest.approx(best[0], rel=1e-9), (trial, text, M, N, K)
        assert ex["cost_us"] == pytest.approx(best[0], rel=1e-9)
        regs = to_regions(plan)
        assert cm.plan_cost(tab, regs, K, batch) == pytest.approx(plan["cost_us"], rel=1e-9)
        tiles = {n: (k.uM, k.uN) for n, k in tab.kernels.items()}
        assert cm.covers_exactly(M, N, regs, tiles)
        assert plan["evaluated"] <= ex["evaluated"]
        checked += 1
    assert checked == 40


def test_library_table_plans_cover_output(mkp):
    """Plans from the active (shipped or analytic) table partition C."""
    names = mkp.mkp_kernel_names()
    rng = np.random.default_rng(5)
    for _ in range(30):
        M, N, K = int(rng.integers(1, 3000)), int(rng.integers(1, 3000)), int(rng.integers(1, 5000))
        p = mkp.mkp_plan_describe(1, M, N, K)
        regs = to_regions(p)
        tiles = {r["kernel"]: (r["uM"], r["uN"]) for r in p["regions"]}
        assert all(r.kernel in names for r in regs)
        # tiles cover the output exactly once (cheap check on a coarse grid)
        cnt = np.zeros((M, N), np.int8)
        for r in regs:
            cnt[r.m0:r.m0 + r.m, r.n0:r.n0 + r.n] += 1
        assert (cnt == 1).all()
        for r in p["regions"]:
            assert 1 <= r["s"] and r["steps"] * r["s"] * r["uK"] >= K
            assert (r["s"] - 1) * r["steps"] * r["uK"] < K   # no empty split


def test_pruned_search_is_exact_on_shipped_table(mkp):
    """The bounds that cut the search (per-kernel tile-count bounds for the
    second region, the linear wave floor for the first) never drop the
    optimum: on the calibrated table, over shapes with many tile-aligned
    cuts, the pruned search costs the same as the exhaustive one."""
    path = os.path.join(os.path.dirname(mkp.__file__), "calib", "gfx950.tbl")
    text = open(path).read()
    rng = np.random.default_rng(17)
    for trial in range(40):
        M, N, K = int(rng.integers(1, 3000)), int(rng.integers(1, 3000)), int(rng.integers(1, 8000))
        batch = int(rng.choice([1, 1, 1, 2, 5]))
        bt = bool(trial & 1)
        plan = mkp.mkp_plan_with_table(text, batch, M, N, K, bt=bt)
        ex = mkp.mkp_plan_with_table(text, batch, M, N, K, exhaustive=True, bt=bt)
        assert plan["cost_us"] == pytest.approx(ex["cost_us"], rel=1e-12), (M, N, K, batch, bt)
        assert plan["evaluated"] <= ex["evaluated"]


def test_plan_time_is_microseconds(mkp):
    import statistics
    ts = []
    rng = np.random.default_rng(6)
    for _ in range(50):
        shape = (int(rng.integers(1, 8192)), int(rng.integers(1, 8192)), int(rng.integers(1, 8192)))
        # the fastest of three searches of the shape: other load on the host
        # only ever adds to a search's time
        ts.append(min(mkp.mkp_plan_describe(1, *shape)["plan_us"] for _ in range(3)))
    # the page reports 2 us per shape; this host is slower and unpinned: report, bound loosely
    print(f"median plan time {statistics.median(ts):.1f} us")
    assert statistics.median(ts) < 1000


@pytest.mark.parametrize("mode", ["wave", "pipe"])
def test_ablation_search_matches_oracle(mkp, mode):
    """MikPoly-WAVE / MikPoly-PIPE (one factor of the cost dropped): the
    library's search returns the oracle's exhaustive minimum of that cost."""
    rng = np.random.default_rng(31 if mode == "wave" else 32)
    try:
        mkp.mkp_set_option("cost_model", mode)
        for trial in range(25):
            text = random_table(rng, int(rng.integers(2, 4)))
            tab = cm.parse_table(text)
            M, N, K = (int(x) for x in rng.integers(1, 200, size=3))
            batch = int(rng.choice([1, 2]))
            plan = mkp.mkp_plan_with_table(text, batch, M, N, K)
            best = cm.exhaustive_best(tab, M, N, K, batch, mode)
            assert plan["cost_us"] == pytest.approx(best[0], rel=1e-9), (mode, trial, M, N, K)
            regs = to_regions(plan)
            assert cm.plan_cost(tab, regs, K, batch, mode) == pytest.approx(plan["cost_us"], rel=1e-9)
            assert cm.covers_exactly(M, N, regs, {n: (k.uM, k.uN) for n, k in tab.kernels.items()})
    finally:
        mkp.mkp_set_option("cost_model", "full")


def test_ranked_candidates_match_oracle(mkp):
    """plan_rank r returns the r-th cheapest distinct candidate of the space,
    the list having as many entries as the oracle enumerates."""
    rng = np.random.default_rng(33)
    try:
        for trial in range(15):
            text = random_table(rng, int(rng.integers(2, 4)))
            tab = cm.parse_table(text)
            M, N, K = (int(x) for x in rng.integers(1, 160, size=3))
            cands = cm.distinct_candidates(tab, M, N, K, 1)
            n = len(cands)
            for r in sorted({1, 2, max(1, n // 2), n}):
                mkp.mkp_set_option("plan_rank", str(r))
                p = mkp.mkp_plan_with_table(text, 1, M, N, K)
                assert p["rank"] == r and p["candidates"] == n, (trial, r, n, p)
                assert p["cost_us"] == pytest.approx(cands[r - 1][0], rel=1e-9), (trial, r)
                regs = to_regions(p)
                assert cm.plan_cost(tab, regs, K, 1) == pytest.approx(p["cost_us"], rel=1e-9)
                assert cm.covers_exactly(M, N, regs, {k: (v.uM, v.uN) for k, v in tab.kernels.items()})
            mkp.mkp_set_option("plan_rank", str(n + 1))
            p = mkp.mkp_plan_with_table(text, 1, M, N, K)
            assert p["regions"] == [] and p["candidates"] == n
    finally:
        mkp.mkp_set_option("plan_rank", "0")


def test_partial_wave_search_is_exact(mkp):
    """With partial-wave (tail) points in the table, the pruned search still
    reaches the oracle's exhaustive minimum, and every chosen plan's cost
    recomputes to the oracle's."""
    rng = np.random.default_rng(77)
    for trial in range(40):
        text = random_table(rng, int(rng.integers(2, 4)), tails=True)
        tab = cm.parse_table(text)
        M, N, K = (int(x) for x in rng.integers(1, 220, size=3))
        batch = int(rng.choice([1, 1, 2]))
        plan = mkp.mkp_plan_with_table(text, batch, M, N, K)
        best = cm.exhaustive_best(tab, M, N, K, batch)
        assert plan["cost_us"] == pytest.approx(best[0], rel=1e-9), (trial, text, M, N, K, batch)
        regs = to_regions(plan)
        assert cm.plan_cost(tab, regs, K, batch) == pytest.approx(plan["cost_us"], rel=1e-9)
        assert cm.covers_exactly(M, N, regs, {n: (k.uM, k.uN) for n, k in tab.kernels.items()})


def test_row_class_curves_search_is_exact(mkp):
    """Tables whose kernels carry curves per tile-row class: the pruned
    search (whose bounds for a growing region take the smallest of the sets
    it may still reach) still reaches the oracle's exhaustive minimum, and
    the chosen plan recomputes to the oracle's cost.  Shapes of a few tile
    rows make several sets appear in one plan."""
    rng = np.random.default_rng(4242)
    for trial in range(60):
        text = random_table(rng, int(rng.integers(2, 4)), tails=bool(trial % 2), skinny=True)
        tab = cm.parse_table(text)
        M = int(rng.integers(1, 260)) if trial % 3 else int(rng.integers(1, 100))
        N, K = (int(x) for x in rng.integers(1, 220, size=2))
        batch = int(rng.choice([1, 1, 2]))
        plan = mkp.mkp_plan_with_table(text, batch, M, N, K)
        ex = mkp.mkp_plan_with_table(text, batch, M, N, K, exhaustive=True)
        best = cm.exhaustive_best(tab, M, N, K, batch)
        assert plan["cost_us"] == pytest.approx(best[0], rel=1e-9), (trial, text, M, N, K, batch)
        assert ex["cost_us"] == pytest.approx(best[0], rel=1e-9)
        regs = to_regions(plan)
        assert cm.plan_cost(tab, regs, K, batch) == pytest.approx(plan["cost_us"], rel=1e-9)
        assert cm.covers_exactly(M, N, regs, {n: (k.uM, k.uN) for n, k in tab.kernels.items()})
        assert plan["evaluated"] <= ex["evaluated"]


def test_layout_restricts_the_search(mkp):
    """A table holding kernels for both B layouts: the search for B given as
    N x K uses only the nk kernels and reaches the oracle's exhaustive
    minimum over them (and likewise for K x N)."""
    rng = np.random.default_rng(91)
    for trial in range(25):
        text = random_table(rng, int(rng.integers(2, 4)), tails=bool(trial % 2))
        # a second family of kernels, marked nk, with their own timings
        extra = random_table(rng, int(rng.integers(1, 4)), tails=bool(trial % 2))
        lines = []
        for line in extra.splitlines():
            tok = line.split()
            if tok[0] == "kernel":
                lines.append(" ".join(["kernel", tok[1] + "_nk"] + tok[2:] + ["nk"]))
            elif tok[0] in ("g", "tail", "tailx"):
                lines.append(" ".join([tok[0], tok[1] + "_nk"] + tok[2:]))
        text = text + "\n".join(lines) + "\n"
        tab = cm.parse_table(text)
        M, N, K = (int(x) for x in rng.integers(1, 200, size=3))
        for bt in (False, True):
            plan = mkp.mkp_plan_with_table(text, 1, M, N, K, bt=bt)
            best = cm.exhaustive_best(tab, M, N, K, 1, bt=bt)
            assert plan["cost_us"] == pytest.approx(best[0], rel=1e-9), (trial, bt)
            assert all(r["kernel"].endswith("_nk") == bt for r in plan["regions"])


def test_transpose_then_nk_choice_matches_oracle(mkp):
    """With N x K kernels and transpose figures in the table, a K x N call
    takes the cheaper of its own plan and transpose + N x K plan, as the
    oracle computes it."""
    rng = np.random.default_rng(123)
    chosen = {False: 0, True: 0}
    for trial in range(30):
        text = random_table(rng, int(rng.integers(2, 4)))
        extra = random_table(rng, int(rng.integers(1, 3)))
        lines = [f"transpose {rng.uniform(0.5, 5):.3f} {rng.uniform(200, 20000):.1f}"]
        for line in extra.splitlines():
            tok = line.split()
            if tok[0] == "kernel":
                lines.append(" ".join(["kernel", tok[1] + "_nk"] + tok[2:] + ["nk"]))
            elif tok[0] == "g":
                # the N x K family runs 0.3x - 1.5x the time of its K x N draw
                scale = rng.uniform(0.3, 1.5)
                pts = " ".join(f"{p.split(':')[0]}:{float(p.split(':')[1]) * scale:.4f}" for p in tok[2:])
                lines.append(f"g {tok[1]}_nk {pts}")
        text = text + "\n".join(lines) + "\n"
        tab = cm.parse_table(text)
        M, N, K = (int(x) for x in rng.integers(1, 300, size=3))
        plan = mkp.mkp_plan_with_table(text, 1, M, N, K)
        cost, transposed = cm.best_call(tab, M, N, K, 1)
        assert plan["cost_us"] == pytest.approx(cost, rel=1e-9), (trial, M, N, K)
        assert plan["transpose_b"] == transposed
        assert all(r["kernel"].endswith("_nk") == transposed for r in plan["regions"])
        if transposed:
            assert plan["transpose_us"] == pytest.approx(cm.transpose_cost(tab, 1, N, K), rel=1e-9)
        chosen[transposed] += 1
    assert chosen[True] > 0 and chosen[False] > 0


SHIPPED = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       "dynamic_shape_gemm_amd", "calib", "gfx950.tbl")


def _check_grouped(mkp, tab, M, K, Ns, bt):
    plan = mkp.mkp_plan_describe_grouped(M, K, Ns, bt=bt)
    best = cm.grouped_best(tab, M, K, Ns, bt=bt)
    assert plan["cost_us"] == pytest.approx(best[0], rel=1e-9), (M, K, Ns, bt)
    (r,) = plan["regions"]
    assert r["n"] == sum(Ns) and r["m"] == M
    assert tab.kernels[r["kernel"]].bt == bt
    # the chosen (kernel, split) is priced by the oracle at the same cost
    assert cm.grouped_cost(tab, r["kernel"], r["s"], M, K, Ns) == pytest.approx(plan["cost_us"], rel=1e-9)


def test_grouped_plan_matches_oracle_on_shipped_table(mkp):
    """Grouped calls (BladeDISC page, GEMM merge of the first kind) are
    planned as one launch over every group's tiles; the library's choice
    is the oracle's minimum over kernels x splits."""
    mkp.mkp_load_calibration(None)
    tab = cm.parse_table(open(SHIPPED).read())
    rng = np.random.default_rng(8)
    for _ in range(40):
        M = int(rng.choice([1, 16, 100, 512, 2048, 8192]))
        K = int(rng.choice([64, 200, 768, 1024, 4096]))
        Ns = [int(x) for x in rng.integers(1, 5000, size=int(rng.integers(1, 5)))]
        for bt in (False, True):
            _check_grouped(mkp, tab, M, K, Ns, bt)
    # the attention projections of a 768-wide model
    for M in (128, 4096):
        _check_grouped(mkp, tab, M, 768, [768, 768, 768], True)


def test_grouped_plan_matches_oracle_on_random_tables(mkp, tmp_path):
    shipped = cm.parse_table(open(SHIPPED).read())
    rng = np.random.default_rng(44)
    try:
        for trial in range(12):
            lines = [f"device {int(rng.integers(4, 300))}", f"launch_us {rng.uniform(0, 3):.3f}",
                     "splitk 1 2 3 4 8", f"reduce {rng.uniform(0, 2):.3f} {rng.uniform(100, 20000):.1f}"]
            for name, k in shipped.kernels.items():
                lines.append(f"kernel {name} {k.uM} {k.uN} {k.uK} {int(rng.integers(1, 3))} "
                             f"{'nk' if k.bt else 'kn'}")
                base, slope = rng.uniform(1, 20), rng.uniform(0.1, 3)
                lines.append(f"g {name} " + " ".join(f"{t}:{base + slope * t * rng.uniform(0.9, 1.1):.4f}"
                                                      for t in (1, 4, 16, 64)))
                if trial % 2:
                    fs = sorted(rng.uniform(0.05, 0.95, size=2))
                    lines.append(f"tail {name} " + " ".join(f"{f:.3f}:{rng.uniform(0.1, 1):.3f}" for f in fs))
                    lines.append(f"tailx {name} " + " ".join(f"{f:.3f}:{rng.uniform(0.1, 1):.3f}" for f in fs))
                if trial >= 8:
                    # curves for regions of one and of two tile rows
                    for r in (1, 2):
                        lines.append(f"g@{r} {name} " + " ".join(
                            f"{t}:{base * 2 + slope * t * rng.uniform(0.5, 2):.4f}" for t in (1, 4, 16, 64)))
                        lines.append(f"tail@{r} {name} 0.5:{rng.uniform(0.1, 1):.3f}")
            if trial >= 8:
                lines.append("rows 1 2")
            text = "\n".join(lines) + "\n"
            path = tmp_path / f"t{trial}.tbl"
            path.write_text(text)
            mkp.mkp_load_calibration(str(path))
            tab = cm.parse_table(text)
            for i in range(6):
                M, K = (int(x) for x in rng.integers(1, 3000, size=2))
                if trial >= 8 and i % 2:
                    M = int(rng.integers(1, 300))
                Ns = [int(x) for x in rng.integers(1, 3000, size=int(rng.integers(1, 5)))]
                _check_grouped(mkp, tab, M, K, Ns, bool(rng.integers(0, 2)))
    finally:
        mkp.mkp_load_calibration(None)


def _with_pairs(rng, text):
    """Append pair lines for kernels of equal workgroups per CU (and layout)."""
    tab = cm.parse_table(text)
    names = sorted(tab.kernels)
    lines = []
    for a in names:
        for b in names:
            ka, kb = tab.kernels[a], tab.kernels[b]
            if a != b and ka.wg_per_cu == kb.wg_per_cu and ka.bt == kb.bt and rng.uniform() < 0.7:
                lines.append(f"pair {a} {b}")
    return text + "\n".join(lines) + "\n"


@pytest.fixture
def fuse_on(mkp):
    mkp.mkp_set_option("fuse_regions", 1)
    yield
    mkp.mkp_set_option("fuse_regions", 0)


def test_one_launch_plans_match_oracle(mkp, fuse_on):
    """Tables with kernel pairs: the planner's choice (one-launch Pattern II
    plans scored by the merged-wave makespan, with its bounds) reaches the
    oracle's exhaustive minimum, whose makespan is simulated task by task."""
    rng = np.random.default_rng(77)
    fused_seen = 0
    for trial in range(80):
        text = random_table(rng, int(rng.integers(2, 5)), tails=bool(trial % 2), skinny=trial >= 60)
        # equal workgroups per CU for most kernels, so that pairs exist
        text = "\n".join(l if not l.startswith("kernel") else " ".join(l.split()[:5] + ["2"])
                         for l in text.splitlines()) + "\n"
        text = _with_pairs(rng, text)
        tab = cm.parse_table(text)
        M, N, K = (int(x) for x in rng.integers(1, 400, size=3))
        batch = int(rng.choice([1, 1, 2]))
        plan = mkp.mkp_plan_with_table(text, batch, M, N, K)
        ex = mkp.mkp_plan_with_table(text, batch, M, N, K, exhaustive=True)
        best = cm.exhaustive_best(tab, M, N, K, batch)
        assert plan["cost_us"] == pytest.approx(best[0], rel=1e-9), (trial, M, N, K, batch, best[1])
        assert ex["cost_us"] == pytest.approx(best[0], rel=1e-9)
        regs = to_regions(plan)
        pat = plan["pattern"] + ("+1" if plan["fused"] else "")
        assert cm.candidate_cost(tab, pat, regs, K, batch) == pytest.approx(plan["cost_us"], rel=1e-9)
        if plan["fused"]:
            fused_seen += 1
            assert (regs[0].kernel, regs[1].kernel) in tab.pairs
        assert cm.covers_exactly(M, N, regs, {n: (k.uM, k.uN) for n, k in tab.kernels.items()})
    assert fused_seen >= 5


def test_ranked_list_includes_one_launch_candidates(mkp, fuse_on):
    """With kernel pairs the ranked space holds the one-launch form of each
    paired Pattern II candidate; plan_rank walks it in the oracle's order."""
    rng = np.random.default_rng(78)
    try:
        for trial in range(8):
            text = random_table(rng, 3)
            text = "\n".join(l if not l.startswith("kernel") else " ".join(l.split()[:5] + ["1"])
                             for l in text.splitlines()) + "\n"
            text = _with_pairs(rng, text)
            tab = cm.parse_table(text)
            M, N, K = (int(x) for x in rng.integers(20, 150, size=3))
            cands = cm.distinct_candidates(tab, M, N, K, 1)
            n = len(cands)
            assert any(c[1].endswith("+1") for c in cands)
            for r in sorted({1, 2, max(1, n // 3), n}):
                mkp.mkp_set_option("plan_rank", str(r))
                p = mkp.mkp_plan_with_table(text, 1, M, N, K)
                assert p["candidates"] == n and p["cost_us"] == pytest.approx(cands[r - 1][0], rel=1e-9), (trial, r)
                pat = p["pattern"] + ("+1" if p["fused"] else "")
                assert cm.candidate_cost(tab, pat, to_regions(p), K, 1) == pytest.approx(p["cost_us"], rel=1e-9)
    finally:
        mkp.mkp_set_option("plan_rank", "0")
