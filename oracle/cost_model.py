"""Oracle for the polymerization cost model and its exhaustive search.

TEST INFRASTRUCTURE ONLY: imported by tests (and nothing on the product path).
It shares no code with the C++ planner; the two only agree on the text format
of the performance table, which both parse on their own.

Source: MikPoly page, section 3 "polymerization cost model" equations:
    Cost(S, H) = sum over regions (R_i, K_i) of f_wave * f_pipe
    f_wave     = ceil(f_parallel(R_i, K_i) / |P_multi|)
    f_pipe     = g_predict(f_num(R_i, K_i), K_i, H)
with f_parallel the number of pipeline tasks (output tiles) in region R_i and
f_num the micro-kernel instances (K steps) one task runs; g_predict is the
per-micro-kernel table measured offline for t in [1, T]  (section 3
"micro-kernel performance model", T = 5120 by experience).

Readings where the page is silent (each is listed in the design doc):
  * |P_multi| for kernel k is slots(k) = CUs x resident workgroups per CU,
    i.e. the case study's resident-warp count (8 warps/SM on 108 SMs) divided
    by the warps one workgroup uses.
  * regions run one after another (additive cost), each as its own launch;
    a per-launch overhead `launch_us` is added per region (0 reproduces the
    page's formula exactly).
  * split-K (not on the page): s splits multiply the tasks by s, divide the K
    steps per task to ceil(t3/s), and add a reduction term
    red_launch_us + (2s+1)*4*m*n*batch bytes / red_GBps.
  * g between measured points is linear; beyond the last point it continues
    the last segment's slope.
  * a partial last wave (not on the page): with tasks = w*slots + r, r > 0,
    the wave term is w + tail(r/slots), where tail(f) is the measured time
    of a wave filling a fraction f of the slots relative to a full wave
    (linear between measured points and up to tail(1) = 1, the first
    point's value below it) -- the `tail` points when w = 0 (the wave runs
    alone), the `tailx` points when w > 0 (it follows full waves).  Without
    points it is ceil(tasks/slots), the page's f_wave.  The WAVE ablation
    keeps the page's ceil.
  * the fill of a partial wave (not on the page): the dispatcher gives
    every CU one workgroup before any CU a second, so a wave of r tasks
    keeps its busiest CU as busy as a wave of ceil(r/CUs) * CUs tasks once
    r exceeds the CU count.  The fill f above is r/slots up to r = CUs and
    min(1, ceil(r/CUs) * CUs / slots) beyond; the measured fills of the
    tail points are taken through the same map, and points that land on a
    whole wave drop out.
  * wave layouts by tile rows (not on the page, whose g_predict depends on
    the micro-kernel and t only): the table may list row classes
    (`rows r1 r2 ...`, ascending) and, per kernel, the three curves again
    for each class (`g@r`, `tail@r`, `tailx@r`), measured on a wave of r
    tile rows.  A region of ceil(m/uM) tile rows takes the curves of the
    smallest class >= that count if its kernel has a `g@` line for that
    class, else (and above every class) the plain `g`, `tail`, `tailx`.
  * the ablations of section 5 "cost-model effectiveness" (MikPoly-WAVE,
    MikPoly-PIPE) keep one factor of the product and take the other as 1
    (f_pipe = 1 us, resp. f_wave = 1); the launch and reduction terms stay.
  * B layouts (not on the page): a kernel takes B as K x N or as N x K; a
    call searches the kernels of its layout.  A K x N call may instead pay
    for a transpose of B (launch + 4*K*N*batch bytes / bandwidth) and run
    the N x K search; the cheaper of the two is the plan.
  * one launch for both regions (not on the page as an interface; its case
    study merges the two regions' warps into common waves): for a kernel
    pair listed in the table, a Pattern II candidate may run as one launch
    whose tasks are taken in order by the earliest free slot; its cost is
    launch + the makespan of that schedule (each task lasting its kernel's
    full-wave time) + the reductions.  Not additive over the regions.
  * Pattern I: one region = whole output, one kernel.  Pattern II-M (II-N):
    a cut of the M (N) extent, the two parts on two different kernels (the
    case study's 3072 | 1024 split).  The cut may be any multiple of kernel
    a's tile height (width) strictly inside the extent, so the first region
    is tile-aligned and only the second carries the ragged edge; in the case
    study the first region holds 96 tasks of a 108-slot wave, which is not a
    whole wave.  Each region has its own split factor.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple


@dataclasses.dataclass
class Kernel:
    name: str
    uM: int
    uN: int
    uK: int
    wg_per_cu: int
    pts: List[Tuple[float, float]]  # (t, microseconds) sorted by t
    bt: bool = False  # serves B given as N x K
    tail: List[Tuple[float, float]] = dataclasses.field(default_factory=list)   # (fill, ratio), alone
    tailx: List[Tuple[float, float]] = dataclasses.field(default_factory=list)  # after full waves
    # row class r -> (g points, tail points, tailx points) on a wave of r tile rows
    by_rows: Dict[int, Tuple[list, list, list]] = dataclasses.field(default_factory=dict)


@dataclasses.dataclass
class Table:
    cus: int
    launch_us: float
    red_launch_us: float
    red_gbps: float
    splits: List[int]
    patterns: List[str]
    kernels: Dict[str, Kernel]
    tr_launch_us: float = 0.0
    tr_gbps: float = 0.0
    pairs: List[Tuple[str, str]] = dataclasses.field(default_factory=list)  # one-launch kernel pairs
    row_classes: List[int] = dataclasses.field(default_factory=list)  # tile-row classes, ascending

    def slots(self, k: Kernel) -> int:
        return self.cus * k.wg_per_cu

    def curves(self, k: Kernel, m: int):
        """(g points, tail points, tailx points) that price an m-row region
        on kernel k."""
        rows = ceil_div(m, k.uM)
        for r in self.row_classes:
            if rows <= r:
                if r in k.by_rows and k.by_rows[r][0]:
                    return k.by_rows[r]
                break
        return k.pts, k.tail, k.tailx


def parse_table(text: str) -> Table:
    """Parse the line-oriented performance-table text (own parser)."""
    cus = 0
    launch = 0.0
    red_l, red_bw = 0.0, 1.0
    tr_l, tr_bw = 0.0, 0.0
    splits = [1]
    patterns = ["I", "II-M", "II-N"]
    kernels: Dict[str, Kernel] = {}
    pairs: List[Tuple[str, str]] = []
    row_classes: List[int] = []
    # (curve kind, row class or 0) -> kernel name -> points
    curves: Dict[Tuple[str, int], Dict[str, List[Tuple[float, float]]]] = {}
    for raw in text.splitlines():
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        tok = line.split()
        key = tok[0]
        if key == "device":
            cus = int(tok[1])
        elif key == "launch_us":
            launch = float(tok[1])
        elif key == "reduce":
            red_l, red_bw = float(tok[1]), float(tok[2])
        elif key == "transpose":
            tr_l, tr_bw = float(tok[1]), float(tok[2])
        elif key == "splitk":
            splits = [int(x) for x in tok[1:]]
        elif key == "patterns":
            patterns = tok[1:]
        elif key == "measured":
            pass  # sustained-rate figures: reported, not part of the cost model
        elif key == "kernel":
            layout = tok[6] if len(tok) > 6 else "kn"
            if layout not in ("kn", "nk"):
                raise ValueError(f"bad kernel layout: {raw!r}")
            kernels[tok[1]] = Kernel(tok[1], int(tok[2]), int(tok[3]), int(tok[4]), int(tok[5]), [], layout == "nk")
        elif key.split("@")[0] in ("g", "tail", "tailx"):
            kind, _, rows = key.partition("@")
            pts = curves.setdefault((kind, int(rows) if rows else 0), {}).setdefault(tok[1], [])
            for p in tok[2:]:
                x, y = p.split(":")
                pts.append((float(x), float(y)))
        elif key == "rows":
            row_classes = [int(x) for x in tok[1:]]
            if any(b <= a for a, b in zip(row_classes, row_classes[1:])) or min(row_classes) < 1:
                raise ValueError(f"bad rows line: {raw!r}")
        elif key == "pair":
            pairs.append((tok[1], tok[2]))
        else:
            raise ValueError(f"unknown table line: {raw!r}")
    for (kind, rows), per_kernel in curves.items():
        if rows and rows not in row_classes:
            raise ValueError(f"curves for row class {rows} not listed in rows")
        for name, pts in per_kernel.items():
            k = kernels[name]
            if not rows:
                setattr(k, {"g": "pts", "tail": "tail", "tailx": "tailx"}[kind], sorted(pts))
            else:
                sets = k.by_rows.setdefault(rows, ([], [], []))
                sets[("g", "tail", "tailx").index(kind)].extend(pts)
    for k in kernels.values():
        for sets in k.by_rows.values():
            for pts in sets:
                pts.sort()
    for k in kernels.values():
        if not k.pts:
            raise ValueError(f"kernel {k.name} has no g points")
    for a, b in pairs:
        ka, kb = kernels[a], kernels[b]
        if a == b or ka.bt != kb.bt or ka.wg_per_cu != kb.wg_per_cu:
            raise ValueError(f"bad pair {a} {b}")
    return Table(cus, launch, red_l, red_bw, splits, patterns, kernels, tr_l, tr_bw, pairs, row_classes)


def g_predict(pts: List[Tuple[float, float]], t: float) -> float:
    """Time of one wave of tasks that each run t micro-kernel instances,
    from one kernel's measured (t, us) points."""
    if len(pts) == 1 or t <= pts[0][0]:
        if len(pts) == 1:
            return pts[0][1] * t / pts[0][0]
        return pts[0][1]
    for (t0, v0), (t1, v1) in zip(pts, pts[1:]):
        if t <= t1:
            return v0 + (v1 - v0) * (t - t0) / (t1 - t0)
    (t0, v0), (t1, v1) = pts[-2], pts[-1]
    return v1 + (v1 - v0) * (t - t1) / (t1 - t0)


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def tail_ratio(points: List[Tuple[float, float]], f: float) -> float:
    """Relative time of a wave filling a fraction f of the slots."""
    if not points or f >= 1.0:
        return 1.0
    pts = list(points) + [(1.0, 1.0)]
    if f <= pts[0][0]:
        return pts[0][1]
    for (f0, r0), (f1, r1) in zip(pts, pts[1:]):
        if f <= f1:
            return r0 + (r1 - r0) * (f - f0) / (f1 - f0)
    return 1.0


def busiest_fill(r: int, slots: int, cus: int) -> float:
    """Fill of a wave of r tasks as its busiest CU sees it."""
    if r <= cus:
        return r / slots
    busiest = -(-r // cus)          # tasks on the busiest CU
    return min(1.0, busiest * cus / slots)


def wave_term(tail: List[Tuple[float, float]], tailx: List[Tuple[float, float]], tasks: int, slots: int,
              cus: int) -> float:
    full, rem = divmod(tasks, slots)
    if not rem:
        return full
    pts = []
    for f, ratio in (tailx if full else tail):
        x = busiest_fill(math.floor(f * slots + 0.5), slots, cus)   # the point's task count, halves up
        if x >= 1.0:
            break
        pts.append((x, ratio))
    return full + tail_ratio(pts, busiest_fill(rem, slots, cus))


def split_steps(t3: int, s: int) -> Tuple[int, int]:
    """(K steps per split, splits actually used) for a requested factor s."""
    per = ceil_div(t3, s)
    return per, ceil_div(t3, per)


@dataclasses.dataclass(frozen=True)
class Region:
    m0: int
    n0: int
    m: int
    n: int
    kernel: str
    s: int


MODES = ("full", "wave", "pipe")


def region_cost(tab: Table, r: Region, K: int, batch: int, mode: str = "full") -> float:
    k = tab.kernels[r.kernel]
    t3 = ceil_div(K, k.uK)
    per, s_eff = split_steps(t3, r.s)
    f_parallel = ceil_div(r.m, k.uM) * ceil_div(r.n, k.uN) * s_eff * batch
    g, tail, tailx = tab.curves(k, r.m)
    f_wave = wave_term(tail, tailx, f_parallel, tab.slots(k), tab.cus)
    f_pipe = g_predict(g, per)
    if mode == "wave":
        f_wave = ceil_div(f_parallel, tab.slots(k))
        f_pipe = 1.0
    elif mode == "pipe":
        f_wave = 1
    c = tab.launch_us + f_wave * f_pipe
    if s_eff > 1:
        c += tab.red_launch_us + (2 * s_eff + 1) * 4.0 * r.m * r.n * batch / (tab.red_gbps * 1e3)
    return c


def plan_cost(tab: Table, regions: Sequence[Region], K: int, batch: int, mode: str = "full") -> float:
    return sum(region_cost(tab, r, K, batch, mode) for r in regions)


def _valid_splits(tab: Table, k: Kernel, K: int) -> List[int]:
    t3 = ceil_div(K, k.uK)
    return [s for s in tab.splits if 1 <= s <= max(t3, 1)]


def makespan_sim(S: int, n1: int, d1: float, n2: int, d2: float) -> float:
    """Finish time of n1 tasks of duration d1 followed by n2 tasks of
    duration d2 on S slots, each task taken in order by the earliest free
    slot -- simulated task by task (the merged-wave view of one launch that
    holds two regions, MikPoly page case study: the second region's warps
    fill the waves the first leaves free)."""
    import heapq

    free = [0.0] * S
    end = 0.0
    for d, n in ((d1, n1), (d2, n2)):
        for _ in range(n):
            t = heapq.heappop(free)
            heapq.heappush(free, t + d)
            end = max(end, t + d)
    return end


def fused_cost(tab: Table, regions: Sequence[Region], K: int, batch: int) -> float:
    """Both regions of a Pattern II plan in one launch over a kernel pair:
    launch + the simulated makespan of the two task lists, each task taking
    its kernel's full-wave time g(f_num), + each region's split-K reduction."""
    r1, r2 = regions
    k1, k2 = tab.kernels[r1.kernel], tab.kernels[r2.kernel]
    S = tab.slots(k1)
    parts = []
    c = tab.launch_us
    for r, k in ((r1, k1), (r2, k2)):
        per, s_eff = split_steps(ceil_div(K, k.uK), r.s)
        parts.append((ceil_div(r.m, k.uM) * ceil_div(r.n, k.uN) * s_eff * batch, g_predict(tab.curves(k, r.m)[0], per)))
        if s_eff > 1:
            c += tab.red_launch_us + (2 * s_eff + 1) * 4.0 * r.m * r.n * batch / (tab.red_gbps * 1e3)
    return c + makespan_sim(S, parts[0][0], parts[0][1], parts[1][0], parts[1][1])


def candidate_cost(tab: Table, pat: str, regions: Sequence[Region], K: int, batch: int, mode: str = "full") -> float:
    """Modelled cost of one candidate: one-launch candidates (pattern names
    ending in '+1') are scored whole, the others region by region."""
    if pat.endswith("+1"):
        return fused_cost(tab, regions, K, batch)
    return plan_cost(tab, regions, K, batch, mode)


def enumerate_plans(tab: Table, M: int, N: int, K: int, batch: int = 1, bt: bool = False, fused: bool = False):
    """Every candidate strategy of the search space, no pruning; only the
    kernels that take B in the call's layout (K x N, or N x K when bt).
    With `fused`, also the one-launch form ('II-M+1', 'II-N+1') of every
    Pattern II candidate over a kernel pair of the table."""
    names = sorted(n for n, k in tab.kernels.items() if k.bt == bt)
    if "I" in tab.patterns:
        for a in names:
            for s in _valid_splits(tab, tab.kernels[a], K):
                yield "I", (Region(0, 0, M, N, a, s),)
    for pat in ("II-M", "II-N"):
        if pat not in tab.patterns:
            continue
        ext = M if pat == "II-M" else N
        for a in names:
            ka = tab.kernels[a]
            step = ka.uM if pat == "II-M" else ka.uN
            for s1 in _valid_splits(tab, ka, K):
                # every tile-aligned cut strictly inside the extent
                for cut in range(step, ext, step):
                    for b in names:
                        if b == a:
                            continue
                        for s2 in _valid_splits(tab, tab.kernels[b], K):
                            if pat == "II-M":
                                r1 = Region(0, 0, cut, N, a, s1)
                                r2 = Region(cut, 0, M - cut, N, b, s2)
                            else:
                                r1 = Region(0, 0, M, cut, a, s1)
                                r2 = Region(0, cut, M, N - cut, b, s2)
                            yield pat, (r1, r2)
                            if fused and (a, b) in tab.pairs:
                                yield pat + "+1", (r1, r2)


def exhaustive_best(tab: Table, M: int, N: int, K: int, batch: int = 1, mode: str = "full", bt: bool = False):
    """Minimum modelled cost over the whole space (the page's ORACLE variant
    searches exhaustively; here only the modelled cost is minimised)."""
    best: Optional[Tuple[float, str, tuple]] = None
    for pat, regs in enumerate_plans(tab, M, N, K, batch, bt, fused=mode == "full"):
        c = candidate_cost(tab, pat, regs, K, batch, mode)
        if best is None or c < best[0]:
            best = (c, pat, regs)
    return best


def distinct_candidates(tab: Table, M: int, N: int, K: int, batch: int = 1, mode: str = "full"):
    """Every distinct candidate (two requested split factors that give the
    same number of splits are one candidate) with its modelled cost, sorted
    by cost."""
    seen = {}
    for pat, regs in enumerate_plans(tab, M, N, K, batch, fused=mode == "full"):
        key = [pat]
        for r in regs:
            t3 = ceil_div(K, tab.kernels[r.kernel].uK)
            key.append((r.m0, r.n0, r.m, r.n, r.kernel, split_steps(t3, r.s)[1]))
        key = tuple(key)
        if key not in seen:
            seen[key] = (candidate_cost(tab, pat, regs, K, batch, mode), pat, regs)
    return sorted(seen.values(), key=lambda x: x[0])


def covers_exactly(M: int, N: int, regions: Sequence[Region], tiles: Dict[str, Tuple[int, int]]) -> bool:
    """Count, per output element, how many tiles of the plan write it (brute force)."""
    import numpy as np

    cnt = np.zeros((M, N), dtype=np.int32)
    for r in regions:
        uM, uN = tiles[r.kernel]
        for i0 in range(r.m0, r.m0 + r.m, uM):
            for j0 in range(r.n0, r.n0 + r.n, uN):
                cnt[i0:min(i0 + uM, r.m0 + r.m), j0:min(j0 + uN, r.n0 + r.n)] += 1
    return bool((cnt == 1).all())


def grouped_cost(tab: Table, kernel: str, s: int, M: int, K: int, Ns: Sequence[int]) -> float:
    """Modelled time of one launch computing A.B_g for every width N_g in Ns
    (BladeDISC page, GEMM merge of the first kind: products that share A
    run as A times the B_g placed side by side).  The launch holds every
    group's tiles: sum over g of ceil(M/uM) * ceil(N_g/uN) * s_eff tasks, one
    wave term and one g_predict over them (MikPoly page, section 3 cost, one
    Pattern I region); with split-K each group has its own reduction."""
    k = tab.kernels[kernel]
    t3 = ceil_div(K, k.uK)
    per, s_eff = split_steps(t3, s)
    columns = sum(ceil_div(n, k.uN) for n in Ns)
    tasks = ceil_div(M, k.uM) * columns * s_eff
    g, tail, tailx = tab.curves(k, M)
    c = tab.launch_us + wave_term(tail, tailx, tasks, tab.slots(k), tab.cus) * g_predict(g, per)
    if s_eff > 1:
        for n in Ns:
            c += tab.red_launch_us + (2 * s_eff + 1) * 4.0 * M * n / (tab.red_gbps * 1e3)
    return c


def grouped_best(tab: Table, M: int, K: int, Ns: Sequence[int], bt: bool = False):
    """(cost, kernel, split) minimising grouped_cost over the kernels of the
    call's B layout and every split factor, by enumeration."""
    best = None
    for name in sorted(n for n, k in tab.kernels.items() if k.bt == bt):
        for s in _valid_splits(tab, tab.kernels[name], K):
            c = grouped_cost(tab, name, s, M, K, Ns)
            if best is None or c < best[0]:
                best = (c, name, s)
    return best


def transpose_cost(tab: Table, batch: int, N: int, K: int) -> float:
    """Modelled time of copying a K x N B to N x K (infinite without figures)."""
    if tab.tr_gbps <= 0:
        return float("inf")
    return tab.tr_launch_us + 4.0 * K * N * batch / (tab.tr_gbps * 1e3)


def best_call(tab: Table, M: int, N: int, K: int, batch: int = 1, bt: bool = False):
    """(cost, transposed?) of the best plan of a call: for B given as K x N,
    the K x N plan or a transpose followed by the N x K plan."""
    direct = exhaustive_best(tab, M, N, K, batch, bt=bt)
    if bt:
        return (direct[0] if direct else float("inf")), False
    via = exhaustive_best(tab, M, N, K, batch, bt=True)
    tc = transpose_cost(tab, batch, N, K)
    if via is not None and (direct is None or via[0] + tc < direct[0]):
        return via[0] + tc, True
    return (direct[0] if direct else float("inf")), False
