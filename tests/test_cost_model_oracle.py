"""Pins of the cost-model oracle against the MikPoly page's own arithmetic
(section 6 case study, stored with its citation in
tests/golden/mikpoly_case_study.json) and against brute-force invariants."""
import json
import math
import os

import numpy as np
import pytest

from oracle import cost_model as cm

GOLD = os.path.join(os.path.dirname(__file__), "golden", "mikpoly_case_study.json")


def case_table(Ta, Tb, launch=0.0, patterns="I II-M II-N"):
    gold = json.load(open(GOLD))
    sms = gold["sms"]
    per_sm = gold["resident_warps_per_sm"]
    A, B = gold["kernel_A"], gold["kernel_B"]
    # workgroups resident per SM = resident warps / warps per workgroup
    wa = per_sm // A["warps"]
    wb = per_sm // B["warps"]
    fa = gold["shape"][2] // A["tile"][2]  # K steps of A = 128
    fb = gold["shape"][2] // B["tile"][2]  # K steps of B = 64
    text = f"""
device {sms}
launch_us {launch}
splitk 1
patterns {patterns}
kernel A {A['tile'][0]} {A['tile'][1]} {A['tile'][2]} {wa}
kernel B {B['tile'][0]} {B['tile'][1]} {B['tile'][2]} {wb}
g A 1:{Ta / fa} {fa}:{Ta}
g B 1:{Tb / fb} {fb}:{Tb}
"""
    return cm.parse_table(text), gold


def test_case_study_wave_arithmetic():
    tab, gold = case_table(10.0, 3.0)
    M, N, K = gold["shape"]
    kA, kB = tab.kernels["A"], tab.kernels["B"]
    # slots per kernel reproduce the page's resident-warp counts
    assert tab.slots(kA) * gold["kernel_A"]["warps"] == gold["warps_per_wave"]
    assert tab.slots(kB) * gold["kernel_B"]["warps"] == gold["warps_per_wave"]
    tasks_a = math.ceil(M / kA.uM) * math.ceil(N / kA.uN)
    assert tasks_a == gold["single_A"]["tasks"]
    assert tasks_a * gold["kernel_A"]["warps"] == gold["single_A"]["warps"]
    assert math.ceil(tasks_a / tab.slots(kA)) == gold["single_A"]["waves"]
    cut = gold["pattern_II"]["cut_m"]
    t1 = math.ceil(cut / kA.uM) * math.ceil(N / kA.uN)
    t2 = math.ceil((M - cut) / kB.uM) * math.ceil(N / kB.uN)
    assert t1 == gold["pattern_II"]["region_1"]["tasks"]
    assert t2 == gold["pattern_II"]["region_2"]["tasks"]
    warps = t1 * gold["kernel_A"]["warps"] + t2 * gold["kernel_B"]["warps"]
    assert warps == gold["pattern_II"]["total_warps"]
    assert math.ceil(warps / gold["warps_per_wave"]) == gold["pattern_II"]["waves"]


@pytest.mark.parametrize("Ta,Tb", [(10.0, 3.0), (10.0, 4.9), (10.0, 5.1), (10.0, 8.0)])
def test_case_study_costs(Ta, Tb):
    tab, gold = case_table(Ta, Tb)
    M, N, K = gold["shape"]
    cut = gold["pattern_II"]["cut_m"]
    single = cm.plan_cost(tab, [cm.Region(0, 0, M, N, "A", 1)], K, 1)
    poly = cm.plan_cost(tab, [cm.Region(0, 0, cut, N, "A", 1), cm.Region(cut, 0, M - cut, N, "B", 1)], K, 1)
    assert single == pytest.approx(2 * Ta, rel=1e-12)
    assert poly == pytest.approx(Ta + 2 * Tb, rel=1e-12)
    assert single / poly == pytest.approx(2 * Ta / (Ta + 2 * Tb), rel=1e-12)
    # the page's choice between the two: polymerize iff Ta > 2 Tb
    assert (poly < single) == (Ta > 2 * Tb)
    # the exhaustive search over the whole space is never worse than either
    best = cm.exhaustive_best(tab, M, N, K)
    assert best[0] <= min(single, poly) + 1e-9


def test_g_interpolation():
    tab = cm.parse_table("device 4\nkernel X 16 16 16 1\ng X 1:2 4:5 8:13\n")
    k = tab.kernels["X"]
    assert cm.g_predict(k.pts, 1) == 2 and cm.g_predict(k.pts, 4) == 5 and cm.g_predict(k.pts, 8) == 13
    assert cm.g_predict(k.pts, 2) == pytest.approx(3.0)
    assert cm.g_predict(k.pts, 6) == pytest.approx(9.0)
    assert cm.g_predict(k.pts, 10) == pytest.approx(17.0)


def test_split_accounting():
    assert cm.split_steps(10, 4) == (3, 4)
    assert cm.split_steps(10, 8) == (2, 5)
    assert cm.split_steps(64, 16) == (4, 16)
    tab = cm.parse_table("device 8\nsplitk 1 2 4\nreduce 1.0 1000\nkernel X 16 16 16 1\ng X 1:1 100:100\n")
    c1 = cm.region_cost(tab, cm.Region(0, 0, 16, 16, "X", 1), 160, 1)
    c2 = cm.region_cost(tab, cm.Region(0, 0, 16, 16, "X", 2), 160, 1)
    assert c1 == pytest.approx(10.0)
    assert c2 == pytest.approx(5.0 + 1.0 + 5 * 4 * 256 / 1e6)


def test_plans_cover_output_exactly():
    tab = cm.parse_table("""device 4
splitk 1 2
kernel P 32 16 16 1
kernel Q 16 32 16 2
g P 1:1 10:8
g Q 1:0.7 10:5
""")
    tiles = {n: (k.uM, k.uN) for n, k in tab.kernels.items()}
    rng = np.random.default_rng(3)
    for _ in range(6):
        M, N, K = (int(x) for x in rng.integers(1, 90, size=3))
        count = 0
        for pat, regs in cm.enumerate_plans(tab, M, N, K):
            assert cm.covers_exactly(M, N, regs, tiles), (pat, regs)
            count += 1
        assert count > 0


def test_ablation_costs_of_case_study():
    """The section 5 ablations on the section 6 case study: with only f_wave
    the single-kernel plan scores its 2 waves and the split plan 1 + 2
    waves; with only f_pipe they score Ta and Ta + Tb (one g per region)."""
    Ta, Tb = 10.0, 3.0
    tab, gold = case_table(Ta, Tb)
    M, N, K = gold["shape"]
    cut = gold["pattern_II"]["cut_m"]
    single = [cm.Region(0, 0, M, N, "A", 1)]
    split = [cm.Region(0, 0, cut, N, "A", 1), cm.Region(cut, 0, M - cut, N, "B", 1)]
    assert cm.plan_cost(tab, single, K, 1, "wave") == pytest.approx(gold["single_A"]["waves"])
    # the page's timeline Ta + 2 Tb: one wave of A then two of B = its 3 waves
    assert cm.plan_cost(tab, split, K, 1, "wave") == pytest.approx(gold["pattern_II"]["waves"])
    assert cm.plan_cost(tab, single, K, 1, "pipe") == pytest.approx(Ta)
    assert cm.plan_cost(tab, split, K, 1, "pipe") == pytest.approx(Ta + Tb)
    # the full model is the product per region (the page's 2 Ta and Ta + 2 Tb)
    assert cm.plan_cost(tab, single, K, 1) == pytest.approx(2 * Ta)
    assert cm.plan_cost(tab, split, K, 1) == pytest.approx(Ta + 2 * Tb)


def test_distinct_candidates_brute_force():
    """The ranked list holds each distinct plan once, sorted, and its head is
    the exhaustive minimum; on the case study it holds exactly the plans a
    hand count gives: 2 Pattern I plans; II-M cuts at every multiple of 256
    (A first: 15) or of 64 (B first: 63) inside 4096 rows; II-N cuts at
    every multiple of 128 (A first: 7) or of 64 (B first: 15) inside 1024
    columns -- 102 in all."""
    tab, gold = case_table(10.0, 3.0)
    M, N, K = gold["shape"]
    c = cm.distinct_candidates(tab, M, N, K)
    costs = [x[0] for x in c]
    assert costs == sorted(costs)
    assert costs[0] == pytest.approx(cm.exhaustive_best(tab, M, N, K)[0])
    assert sum(1 for x in c if x[1] == "I") == 2
    assert sum(1 for x in c if x[1] == "II-M") == 15 + 63
    assert sum(1 for x in c if x[1] == "II-N") == 7 + 15
    assert len(c) == 102
    # with one split factor every enumerated plan is already distinct
    assert len(c) == sum(1 for _ in cm.enumerate_plans(tab, M, N, K))


@pytest.mark.parametrize("Ta,Tb", [(10.0, 3.0), (10.0, 6.0)])
def test_case_study_plan_is_a_candidate(Ta, Tb):
    """The page's own strategy -- kernel A on rows [0, 3072), kernel B on
    rows [3072, 4096) -- is in the enumerated space at cost Ta + 2 Tb (its
    first region is 96 tasks of a 108-slot wave, not a whole wave).  Under
    the page's ceil(f_parallel / |P|) the search may still find a cheaper
    cut (3328 rows of A: 104 tasks, one wave; the rest on B in one wave)."""
    tab, gold = case_table(Ta, Tb)
    M, N, K = gold["shape"]
    cut = gold["pattern_II"]["cut_m"]
    found = [regs for pat, regs in cm.enumerate_plans(tab, M, N, K)
             if pat == "II-M" and regs[0].kernel == "A" and regs[0].m == cut and regs[1].kernel == "B"]
    assert len(found) == 1
    assert cm.plan_cost(tab, found[0], K, 1) == pytest.approx(Ta + 2 * Tb, rel=1e-12)
    cheaper = [regs for pat, regs in cm.enumerate_plans(tab, M, N, K)
               if pat == "II-M" and regs[0].kernel == "A" and regs[0].m == 3328]
    assert cm.plan_cost(tab, cheaper[0], K, 1) == pytest.approx(Ta + Tb, rel=1e-12)
    assert cm.exhaustive_best(tab, M, N, K)[0] <= Ta + Tb + 1e-12


def test_best_call_hand_worked():
    """best_call against costs worked by hand: one slot, no launch cost,
    g proportional to t.  A 16 x 16 x 16 call is one task of one K step: on
    the K x N kernel 10 us; on the N x K kernel 2 us after a transpose of
    1 us + 4 * 16 * 16 bytes at 1000 GB/s = 1.001024 us.  The copy wins at
    3.001024 us, and loses once its fixed part reaches 20 us.  With batch 3
    every term triples except the copy's fixed part."""
    base = """device 1
launch_us 0
splitk 1
kernel kn 16 16 16 1
kernel nk 16 16 16 1 nk
g kn 1:10
g nk 1:2
"""
    tab = cm.parse_table(base + "transpose 1.0 1000\n")
    cost, tr = cm.best_call(tab, 16, 16, 16)
    assert tr is True and cost == pytest.approx(3.001024, rel=1e-12)
    # B already N x K: no copy, the N x K kernel alone
    assert cm.best_call(tab, 16, 16, 16, bt=True) == (pytest.approx(2.0), False)
    # batch 3: three tasks on one slot -> 30 us direct, 6 + 1 + 3 * 0.001024 via the copy
    cost3, tr3 = cm.best_call(tab, 16, 16, 16, batch=3)
    assert tr3 is True and cost3 == pytest.approx(7.003072, rel=1e-12)
    slow = cm.parse_table(base + "transpose 20.0 1000\n")
    assert cm.best_call(slow, 16, 16, 16) == (pytest.approx(10.0), False)
    # two K steps: 20 us direct against 4 + 1.002048 (the copy of a 32 x 16 B)
    assert cm.best_call(tab, 16, 16, 32)[0] == pytest.approx(5.002048, rel=1e-12)


def test_fused_cost_hand_worked():
    """One launch for both regions, against a schedule worked by hand: 2
    slots, launch 0.5 us, K = 32 (two K steps of 16), g_a(t) = 3t, g_b(t) =
    t.  Region 1: 48 x 16 on kernel a, 3 tasks of 6 us; region 2: 32 x 16 on
    kernel b with 2 splits, 4 tasks of 1 us.  Slots: a1, a2 at 0-6; a3 at
    6-12 on one slot, b1..b4 at 6-7, 7-8, 8-9, 9-10 on the other: makespan
    12.  Region 2's reduction: 0.25 + (2*2 + 1) * 4 * 32 * 16 bytes at 1000
    GB/s = 0.26024.  Total 12.76024 us; regions launched one after the
    other would cost 0.5 + 2 * 6 and 0.5 + 2 * 1 + 0.26024 = 15.26024."""
    tab = cm.parse_table("""device 2
launch_us 0.5
splitk 1 2
reduce 0.25 1000
kernel a 16 16 16 1
kernel b 16 16 16 1
g a 1:3
g b 1:1
pair a b
""")
    r1 = cm.Region(0, 0, 48, 16, "a", 1)
    r2 = cm.Region(48, 0, 32, 16, "b", 2)
    assert cm.fused_cost(tab, (r1, r2), 32, 1) == pytest.approx(12.76024, rel=1e-12)
    assert cm.plan_cost(tab, (r1, r2), 32, 1) == pytest.approx(15.26024, rel=1e-12)
    # without splits: a1, a2 at 0-6, a3 at 6-12, b1 at 6-8, b2 at 8-10 -> 12.5
    r2s = cm.Region(48, 0, 32, 16, "b", 1)
    assert cm.fused_cost(tab, (r1, r2s), 32, 1) == pytest.approx(12.5, rel=1e-12)
    # batch 2 doubles the tasks: a: 6 tasks (3 waves of 6 us, 0-18); b: 4 tasks
    # of 2 us after them, 18-22 -> 22.5 us
    assert cm.fused_cost(tab, (r1, r2s), 32, 2) == pytest.approx(22.5, rel=1e-12)


def test_partial_wave_term_closed_form():
    """The partial-last-wave refinement: tail points interpolate linearly up
    to (1, 1), hold their first value below the first point, and a region of
    w*slots + r tasks costs (w + tail(r/slots)) * g, with the `tail` points
    when w = 0 and the `tailx` points when w > 0; with no points the term is
    the page's ceil(tasks/slots)."""
    text = """device 4
launch_us 0.5
splitk 1
kernel k 16 16 16 2
g k 1:2 10:11
tail k 0.25:0.4 0.5:0.7
tailx k 0.5:0.2
"""
    tab = cm.parse_table(text)
    k = tab.kernels["k"]
    assert tab.slots(k) == 8
    assert cm.tail_ratio(k.tail, 0.1) == pytest.approx(0.4)          # below the first point
    assert cm.tail_ratio(k.tail, 0.25) == pytest.approx(0.4)
    assert cm.tail_ratio(k.tail, 0.375) == pytest.approx(0.55)       # halfway 0.4 -> 0.7
    assert cm.tail_ratio(k.tail, 0.75) == pytest.approx(0.85)        # halfway 0.7 -> 1
    assert cm.tail_ratio(k.tail, 1.0) == 1.0
    assert cm.tail_ratio(k.tailx, 0.3) == pytest.approx(0.2)         # the tailx points
    assert cm.tail_ratio(k.tailx, 0.75) == pytest.approx(0.6)        # halfway 0.2 -> 1
    # 16 x 16 output, K = 16: 1 task of g(1) = 2 us; 1 of 8 slots filled, alone
    assert cm.region_cost(tab, cm.Region(0, 0, 16, 16, "k", 1), 16, 1) == pytest.approx(0.5 + 0.4 * 2)
    # 11 tasks of t = 10 steps: one full wave (8) + 3/8 filled after it -> (1 + 0.2) * 11
    r = cm.Region(0, 0, 16, 176, "k", 1)
    assert cm.region_cost(tab, r, 160, 1) == pytest.approx(0.5 + 1.2 * 11)
    # exactly two full waves: no partial term
    assert cm.region_cost(tab, cm.Region(0, 0, 16, 256, "k", 1), 160, 1) == pytest.approx(0.5 + 2 * 11)
    # the WAVE ablation keeps ceil(tasks / slots)
    assert cm.region_cost(tab, r, 160, 1, "wave") == pytest.approx(0.5 + 2)
    # without tail lines the full model is the page's ceil
    tab0 = cm.parse_table(text.replace("tail k 0.25:0.4 0.5:0.7\n", "").replace("tailx k 0.5:0.2\n", ""))
    assert cm.region_cost(tab0, r, 160, 1) == pytest.approx(0.5 + 2 * 11)


def test_row_class_curves_closed_form():
    """Curves per tile-row class: a region of r tile rows takes g and both
    tail curves of the smallest listed class >= r when its kernel has a g
    line for that class; a kernel without one, a region above every class
    and a table without a rows line take the square curves.  Grouped and
    one-launch costs follow the same rule."""
    text = """device 4
launch_us 0.5
splitk 1
rows 2 4
kernel k 16 16 16 1
kernel j 16 16 16 1
g k 1:2 10:11
g@2 k 1:4 10:31
tail@2 k 0.5:0.8
tailx@2 k 0.5:0.3
g@4 k 1:3 10:21
tail k 0.5:0.5
g j 1:2 10:11
g@4 j 1:1 10:5
pair k j
"""
    tab = cm.parse_table(text)
    k, j = tab.kernels["k"], tab.kernels["j"]
    assert tab.row_classes == [2, 4]
    assert k.by_rows[2] == ([(1.0, 4.0), (10.0, 31.0)], [(0.5, 0.8)], [(0.5, 0.3)])
    assert k.by_rows[4][0] == [(1.0, 3.0), (10.0, 21.0)] and 2 not in j.by_rows
    # 32 rows = 2 tile rows (class 2), 2 columns, K = 160 (10 steps): 4
    # tasks, one full wave of g@2(10) = 31
    assert cm.region_cost(tab, cm.Region(0, 0, 32, 32, "k", 1), 160, 1) == pytest.approx(0.5 + 31)
    # 1 row, 1 column: class 2; 1 task of 4 slots alone: tail@2(0.25) = 0.8
    # (held below the first point) on g@2(1) = 4
    assert cm.region_cost(tab, cm.Region(0, 0, 1, 16, "k", 1), 16, 1) == pytest.approx(0.5 + 0.8 * 4)
    # 16 rows, 6 columns: 1 full wave + 2 of 4 slots after it: tailx@2(0.5) = 0.3
    assert cm.region_cost(tab, cm.Region(0, 0, 16, 96, "k", 1), 16, 1) == pytest.approx(0.5 + 1.3 * 4)
    # 33 rows = 3 tile rows: class 4, whose set has no tail points: 6 tasks =
    # 1 full wave + a partial one counted whole, on g@4(10) = 21
    assert cm.region_cost(tab, cm.Region(0, 0, 33, 32, "k", 1), 160, 1) == pytest.approx(0.5 + 2 * 21)
    # 65 rows = 5 tile rows: above every class, the square set: 10 tasks =
    # 2 full waves + 2 of 4 after them (no square tailx points: whole)
    assert cm.region_cost(tab, cm.Region(0, 0, 65, 32, "k", 1), 160, 1) == pytest.approx(0.5 + 3 * 11)
    # j has no class-2 curves: a 2-row region takes the square set (not
    # class 4's), 4 tasks of g(10) = 11; a 3-row one takes g@4
    assert cm.region_cost(tab, cm.Region(0, 0, 32, 32, "j", 1), 160, 1) == pytest.approx(0.5 + 11)
    assert cm.region_cost(tab, cm.Region(0, 0, 48, 16, "j", 1), 160, 1) == pytest.approx(0.5 + 5)
    # curves of a class that no rows line lists are refused
    with pytest.raises(ValueError):
        cm.parse_table(text.replace("rows 2 4", "rows 2"))
    # without class curves every region takes the square set
    tab0 = cm.parse_table("\n".join(l for l in text.splitlines() if not l.startswith("rows") and "@" not in l) + "\n")
    assert cm.region_cost(tab0, cm.Region(0, 0, 32, 32, "k", 1), 160, 1) == pytest.approx(0.5 + 11)
    # grouped: M = 20 (2 tile rows) over two widths of 16: 4 tasks, one wave of g@2(10)
    assert cm.grouped_cost(tab, "k", 1, 20, 160, [16, 16]) == pytest.approx(0.5 + 31)
    # one launch of a 2-tile-row region on k (4 tasks of 31) then one tile
    # row on j (class 2, which j lacks: 2 square tasks of 11): the 4 slots
    # are busy until 31, then j's tasks run to 42
    regs = (cm.Region(0, 0, 32, 32, "k", 1), cm.Region(32, 0, 16, 32, "j", 1))
    assert cm.fused_cost(tab, regs, 160, 1) == pytest.approx(0.5 + 42)


def test_partial_wave_fill_follows_busiest_cu():
    """A partial wave of r tasks on C CUs with two slots each: up to r = C
    its fill is r/slots; beyond, some CU runs two tasks, so the wave takes as
    long as a full one.  Measured fills go through the same map (the point
    at 3/4, six tasks on four CUs, lands on a whole wave and drops out)."""
    assert cm.busiest_fill(3, 8, 4) == pytest.approx(0.375)
    assert cm.busiest_fill(4, 8, 4) == pytest.approx(0.5)
    assert cm.busiest_fill(5, 8, 4) == 1.0
    assert cm.busiest_fill(5, 12, 4) == pytest.approx(8 / 12)    # three slots per CU: two on the busiest
    assert cm.busiest_fill(9, 12, 4) == 1.0
    text = """device 4
launch_us 0
splitk 1
kernel k 16 16 16 2
g k 1:2
tail k 0.25:0.4 0.5:0.6 0.75:0.9
"""
    tab = cm.parse_table(text)
    region = lambda tiles_n: cm.region_cost(tab, cm.Region(0, 0, 16, 16 * tiles_n, "k", 1), 16, 1)
    assert region(3) == pytest.approx(0.5 * 2)    # 3/8: halfway between 0.4 and 0.6
    assert region(4) == pytest.approx(0.6 * 2)
    assert region(5) == pytest.approx(1.0 * 2)    # a CU runs two tasks: a whole wave
    assert region(6) == pytest.approx(1.0 * 2)    # not the measured 0.9 at 6/8
    assert region(1) == pytest.approx(0.4 * 2)


def test_transpose_cost_closed_form():
    """The copy of a K x N B to N x K costs launch + 4*K*N*batch bytes at the
    table's bandwidth; without a transpose line it is never taken."""
    tab = cm.parse_table("device 4\ntranspose 1.5 2000\nkernel k 16 16 16 1\ng k 1:1\n")
    assert cm.transpose_cost(tab, 3, 1000, 500) == pytest.approx(1.5 + 4.0 * 500 * 1000 * 3 / 2e6)
    tab0 = cm.parse_table("device 4\nkernel k 16 16 16 1\ng k 1:1\n")
    assert cm.transpose_cost(tab0, 1, 64, 64) == float("inf")
    assert cm.best_call(tab0, 64, 64, 64)[1] is False


# ---- grouped calls (BladeDISC page, GEMM merge of the first kind) ----------

def _grouped_table(cus=3, wg=2, launch=1.5, red=(0.7, 900.0)):
    return cm.parse_table(f"""device {cus}
launch_us {launch}
splitk 1 2 4
reduce {red[0]} {red[1]}
kernel a 64 64 32 {wg}
kernel b 32 128 32 1
kernel c 128 256 32 1
g a 1:0.9 4:2.0 16:6.5
g b 1:0.5 4:1.7 16:5.0
g c 1:2.0 4:4.5 16:13.0
tail a 0.25:0.4 0.5:0.7
tailx a 0.5:0.6
""")


def test_grouped_equals_concatenated_gemm_for_tile_multiples():
    """Merging products that share A is the product with the B_g side by
    side: when every width is a multiple of every kernel's uN, the grouped
    launch has exactly the tasks of one GEMM of width sum(N_g), so its cost
    is that Pattern I region's, plus one more reduction launch per extra
    group when split."""
    tab = _grouped_table()
    for Ns in ([256], [256, 512], [768, 256, 256], [256, 256, 256, 1024]):
        for M, K in ((64, 96), (300, 512), (1000, 40)):
            for name in tab.kernels:
                for s in (1, 2, 4):
                    g = cm.grouped_cost(tab, name, s, M, K, Ns)
                    one = cm.region_cost(tab, cm.Region(0, 0, M, sum(Ns), name, s), K, 1)
                    s_eff = cm.split_steps(cm.ceil_div(K, tab.kernels[name].uK), s)[1]
                    extra = (len(Ns) - 1) * tab.red_launch_us if s_eff > 1 else 0.0
                    assert g == pytest.approx(one + extra, rel=1e-12), (Ns, M, K, name, s)


def test_grouped_single_group_is_pattern_one():
    tab = _grouped_table()
    for M, N, K in ((1, 1, 1), (77, 130, 200), (513, 37, 4096)):
        for name in tab.kernels:
            for s in (1, 2, 4):
                assert cm.grouped_cost(tab, name, s, M, K, [N]) == pytest.approx(
                    cm.region_cost(tab, cm.Region(0, 0, M, N, name, s), K, 1), rel=1e-12)


def test_grouped_task_count_by_brute_force():
    """With one slot, no launch cost and g = 1 per wave at one K step, the
    cost is the task count; count the tiles by walking every output element
    of every group and collecting the distinct (group, tile row, tile col)."""
    tab = cm.parse_table("""device 1
launch_us 0
splitk 1
reduce 0 1
kernel k 48 40 64 1
g k 1:1 2:2
""")
    rng = np.random.default_rng(5)
    for _ in range(20):
        M = int(rng.integers(1, 120))
        Ns = [int(x) for x in rng.integers(1, 150, size=int(rng.integers(1, 5)))]
        tiles = set()
        for g, n in enumerate(Ns):
            for i in range(M):
                for j in range(n):
                    tiles.add((g, i // 48, j // 40))
        assert cm.grouped_cost(tab, "k", 1, M, 64, Ns) == pytest.approx(len(tiles)), (M, Ns)


def test_grouped_best_is_minimum_over_enumeration():
    tab = _grouped_table()
    rng = np.random.default_rng(17)
    for _ in range(30):
        M, K = (int(x) for x in rng.integers(1, 700, size=2))
        Ns = [int(x) for x in rng.integers(1, 700, size=int(rng.integers(1, 5)))]
        best = cm.grouped_best(tab, M, K, Ns)
        costs = [cm.grouped_cost(tab, n, s, M, K, Ns) for n in tab.kernels for s in (1, 2, 4)
                 if s <= max(cm.ceil_div(K, tab.kernels[n].uK), 1)]
        assert best[0] == pytest.approx(min(costs), rel=1e-12)


# ---- one launch for two regions: the merged-wave schedule ------------------

def test_makespan_hand_worked():
    # S = 4 slots, 6 tasks of 3 us then 5 of 1 us: the first wave of 4 ends
    # at 3; two slots finish region 1 (3..6), the other two run region 2 at
    # 3, 3, 4, 4, 5 -> the last ends at 6
    assert cm.makespan_sim(4, 6, 3.0, 5, 1.0) == 6.0
    # S = 3, 4 tasks of 2 then 7 of 1: starts 2, 2, 3, 3, 4, 4 (two slots)
    # and 4 (the third slot, free at 4): last start 4, end 5
    assert cm.makespan_sim(3, 4, 2.0, 7, 1.0) == 5.0
    # the second region shorter than the first's last wave: the first region decides
    assert cm.makespan_sim(4, 5, 10.0, 3, 1.0) == 20.0


def test_makespan_equal_durations_is_merged_waves():
    """With equal task times the launch runs ceil((n1 + n2) / S) waves --
    the page's merged-warp count (its case study: 1792 warps in waves of
    864 -> 3 waves)."""
    assert cm.makespan_sim(864, 768, 1.0, 1024, 1.0) == 3.0
    rng = np.random.default_rng(12)
    for _ in range(50):
        S = int(rng.integers(1, 40))
        n1, n2 = (int(x) for x in rng.integers(0, 200, size=2))
        assert cm.makespan_sim(S, n1, 2.5, n2, 2.5) == pytest.approx(math.ceil((n1 + n2) / S) * 2.5)


def test_makespan_whole_waves_are_additive():
    """When the first region fills whole waves the second starts on all
    slots at once: the serial sum of the two regions' waves."""
    rng = np.random.default_rng(13)
    for _ in range(50):
        S = int(rng.integers(1, 30))
        w = int(rng.integers(0, 5))
        n2 = int(rng.integers(1, 100))
        d1, d2 = rng.uniform(0.5, 4, size=2)
        assert cm.makespan_sim(S, w * S, d1, n2, d2) == pytest.approx(w * d1 + math.ceil(n2 / S) * d2)


def test_fused_candidates_only_for_pairs():
    text = """device 2
launch_us 1
splitk 1
kernel a 32 32 32 1
kernel b 16 16 32 1
kernel c 16 32 32 2
g a 1:4
g b 1:1
g c 1:1
pair a b
"""
    tab = cm.parse_table(text)
    pats = [p for p, _ in cm.enumerate_plans(tab, 100, 64, 32, fused=True)]
    fused = [p for p in pats if p.endswith("+1")]
    assert fused and len(fused) == sum(1 for p, r in cm.enumerate_plans(tab, 100, 64, 32, fused=True)
                                      if p.endswith("+1") and r[0].kernel == "a" and r[1].kernel == "b")
    with pytest.raises(ValueError):
        cm.parse_table(text + "pair a c\n")   # different workgroups per CU
