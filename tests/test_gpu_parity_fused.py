"""GPU parity of one-launch Pattern II plans: both regions of a cut run in a
single launch of a two-tile kernel, the second region's workgroups filling
the slots the first region's last wave leaves free (the merged-wave view of
the MikPoly page's case study).  Results are compared element by element with
the CPU oracle, NaN guard bands around C.
"""
import os

import numpy as np
import pytest

import oracle
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

from _gpu_util import GuardedC, assert_close, dev_bf16  # noqa: E402


@pytest.fixture(scope="module")
def mkp(gpu):
    import dynamic_shape_gemm_amd as m

    m.mkp_load_calibration(None)
    opts = (("force_kernel", ""), ("force_splitk", 0), ("fused_reduce", 1), ("plan_rank", 0), ("transpose_b", 1))
    for k, v in opts:
        m.mkp_set_option(k, v)
    m.mkp_set_option("fuse_regions", 1)   # off by default
    yield m
    for k, v in opts:
        m.mkp_set_option(k, v)
    m.mkp_set_option("fuse_regions", 0)


def rand_bits(rng, shape):
    return f32_to_bf16_bits(rng.uniform(-1, 1, size=shape).astype(np.float32))


def run(mkp, a, b, bt, what):
    import torch

    M, K = a.shape
    N = b.shape[0] if bt else b.shape[1]
    plan = mkp.mkp_plan_describe(1, M, N, K, bt=bt)
    desc = [(r["kernel"], r["s"], r["m0"], r["n0"], r["m"], r["n"]) for r in plan["regions"]]
    print(f"[case] {what} M={M} N={N} K={K} bt={bt} fused={plan['fused']} {desc}", flush=True)
    ta, pa = dev_bf16(a)
    tb, pb = dev_bf16(b)
    gc = GuardedC(1, M, N)
    fn = mkp.mkp_gemm_bt if bt else mkp.mkp_gemm
    fn(M, N, K, pa, K, pb, K if bt else N, gc.addr, gc.ld)
    torch.cuda.synchronize()
    got, untouched = gc.result()
    assert untouched, f"{what}: write outside C"
    ref, refabs = oracle.gemm(a, np.ascontiguousarray(b.T) if bt else b, with_abs=True)
    assert_close(got[0], ref, refabs, K, what)
    return plan


@pytest.mark.parametrize("bt", [False, True], ids=["kn", "nk"])
def test_planner_chosen_one_launch_plans(mkp, bt):
    """Shapes of the encoder linears whose plan the cost model makes a
    one-launch pair."""
    rng = np.random.default_rng(3 + bt)
    seen = 0
    # which shapes get a one-launch plan depends on the calibrated table:
    # walk the encoder linears' FFN-up rows and decoder-sized projections,
    # and run the first three
    shapes = ([(16 * L, N, 768) for L in range(128, 513) for N in (3072, 2304)] + [(336, 6000, 4096)] +
              [(16 * L, N, K) for L in range(8, 64) for (N, K) in ((4096, 11008), (11008, 4096))])
    for (M, N, K) in shapes:
        if seen == 3:
            break
        p = mkp.mkp_plan_describe(1, M, N, K, bt=bt)
        if not p["fused"]:
            continue
        a = rand_bits(rng, (M, K))
        b = rand_bits(rng, (N, K) if bt else (K, N))
        run(mkp, a, b, bt, "chosen")
        seen += 1
    assert seen >= 1


def _walk_fused(mkp, shapes, bt, limit, want):
    """(shape, rank) of the first one-launch candidate of each key that
    want(plan) returns, walking the ranked list of each shape up to limit."""
    found = {}
    for (M, N, K) in shapes:
        for r in range(1, limit + 1):
            mkp.mkp_set_option("plan_rank", r)
            p = mkp.mkp_plan_describe(1, M, N, K, bt=bt)
            if r > p["candidates"]:
                break
            key = want(p) if p["fused"] else None
            if key is not None and key not in found:
                found[key] = ((M, N, K), r)
    return found


SHIPPED = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "dynamic_shape_gemm_amd", "calib",
                       "gfx950.tbl")


def _pair_table(a, b, path):
    """The shipped table with kernels a and b made 100x cheaper and the pair
    (a, b) its only one-launch pair: the ranked candidate lists then start
    with plans on a and b, so one-launch plans over the pair come early."""
    out = []
    for line in open(SHIPPED).read().splitlines():
        tok = line.split("#", 1)[0].split()
        if tok and tok[0] == "pair":
            continue
        if tok and tok[0].split("@")[0] == "g" and tok[1] in (a, b):   # every wave layout's g
            pts = " ".join(f"{x.split(':')[0]}:{float(x.split(':')[1]) * 0.01:.6f}" for x in tok[2:])
            line = f"{tok[0]} {tok[1]} {pts}"
        out.append(line)
    out.append(f"pair {a} {b}")
    open(path, "w").write("\n".join(out) + "\n")


@pytest.mark.parametrize("bt", [False, True], ids=["kn", "nk"])
def test_ranked_one_launch_plans(mkp, bt, tmp_path):
    """Run one-launch plans of every kernel pair of the layout, with split-K
    off and on in either region, under both split-K reductions (the
    last-arriving split, with each region's own counters, and the second
    pass): for each pair, a table that makes the pair's kernels the cheap
    ones, and the first one-launch candidates of its ranked lists."""
    from oracle import cost_model as cm

    rng = np.random.default_rng(10 + bt)
    pairs = [(x, y) for x, y in cm.parse_table(open(SHIPPED).read()).pairs if x.endswith("_nk") == bt]
    assert len(pairs) == 8, pairs   # every pair of the layout
    key = lambda p: (p["regions"][0]["s"] > 1, p["regions"][1]["s"] > 1)
    both = 0
    try:
        mkp.mkp_set_option("transpose_b", 0)
        for a, b in pairs:
            path = str(tmp_path / f"{a}_{b}.tbl")
            _pair_table(a, b, path)
            mkp.mkp_load_calibration(path)
            want = lambda p: key(p) if (p["regions"][0]["kernel"], p["regions"][1]["kernel"]) == (a, b) else None
            found = _walk_fused(mkp, [(1500, 1600, 256), (700, 900, 6144)], bt, 150, want)
            print(f"[case] pair {a} + {b}: one-launch candidates {sorted(found.items())}", flush=True)
            assert found, (a, b)
            both += sum(1 for k in found if k[0] and k[1])
            for k, ((M, N, K), r) in sorted(found.items(), key=lambda x: x[1]):
                a_bits = rand_bits(rng, (M, K))
                b_bits = rand_bits(rng, (N, K) if bt else (K, N))
                mkp.mkp_set_option("plan_rank", r)
                for fused_reduce in (1, 0):
                    mkp.mkp_set_option("fused_reduce", fused_reduce)
                    run(mkp, a_bits, b_bits, bt, f"pair {a}+{b} rank {r} splits {k} fused_reduce={fused_reduce}")
                mkp.mkp_set_option("plan_rank", 0)
        assert both > 0
    finally:
        mkp.mkp_set_option("plan_rank", 0)
        mkp.mkp_set_option("fused_reduce", 1)
        mkp.mkp_set_option("transpose_b", 1)
        mkp.mkp_load_calibration(None)


def test_one_launch_off_matches_oracle(mkp):
    """fuse_regions 0 (the default) keeps the two-launch form of the same shapes."""
    rng = np.random.default_rng(21)
    M, N, K = 2720, 3072, 768
    a = rand_bits(rng, (M, K))
    b = rand_bits(rng, (K, N))
    try:
        mkp.mkp_set_option("fuse_regions", 0)
        p = run(mkp, a, b, False, "fuse off")
        assert not p["fused"]
    finally:
        mkp.mkp_set_option("fuse_regions", 1)
