"""GPU parity of the HIP path against the CPU oracle, through the C-ABI.

Every case prints its name before it touches the GPU.  Full-element checks
at sizes the oracle finishes in seconds (several tiles plus ragged tails);
sampled entries at the workloads' full sizes.  The gate is
|dC| <= 1e-3*sqrt(K) per element, plus the binary32 summation bound.
"""
import json
import math
import os
import tempfile

import numpy as np
import pytest

import oracle
import workloads
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

from _gpu_util import GuardedC, assert_close, dev_bf16, padded  # noqa: E402


@pytest.fixture(scope="module")
def mkp(gpu):
    import dynamic_shape_gemm_amd as m

    m.mkp_load_calibration(None)
    m.mkp_set_option("force_kernel", "")
    m.mkp_set_option("force_splitk", 0)
    m.mkp_set_option("patterns", "I,II")
    yield m
    m.mkp_set_option("force_kernel", "")
    m.mkp_set_option("force_splitk", 0)


def rand_bits(rng, shape, law="u"):
    if law == "u":
        v = rng.uniform(-1, 1, size=shape)
    else:
        v = rng.normal(0, 1, size=shape)
    return f32_to_bf16_bits(v.astype(np.float32))


def run_case(mkp, a, b, *, lda=None, ldb=None, ldc=None, offA=0, offB=0, offC=0, what=""):
    """a (M,K), b (K,N) bf16 bits; full-element compare with guard bands."""
    import torch

    M, K = a.shape
    N = b.shape[1]
    lda = lda or max(K, 1)
    ldb = ldb or max(N, 1)
    print(f"[case] {what} M={M} N={N} K={K} lda={lda} ldb={ldb} ldc={ldc} off=({offA},{offB},{offC})", flush=True)
    ta, pa = dev_bf16(padded(a, lda) if K else a, offA)
    tb, pb = dev_bf16(padded(b, ldb) if N else b, offB)
    gc = GuardedC(1, M, N, ld=ldc, offset=offC)
    mkp.mkp_gemm(M, N, K, pa, lda, pb, ldb, gc.addr, gc.ld)
    torch.cuda.synchronize()
    got, untouched = gc.result()
    ref, refabs = oracle.gemm(a, b, with_abs=True)
    assert untouched, f"{what}: write outside C"
    return assert_close(got[0], ref, refabs, K, what)


def test_config1_full(mkp):
    case = workloads.config_cases(1)[0]
    a, b = workloads.make_operands(case)
    run_case(mkp, a[0], b[0], what="config1")


RAGGED = [(1, 1, 1), (1, 4096, 64), (17, 33, 65), (64, 64, 64), (65, 129, 257), (300, 257, 129),
          (255, 511, 1023), (513, 1000, 777), (16, 5000, 300), (1000, 17, 2049), (7, 300, 12544)]


@pytest.mark.parametrize("shape", RAGGED, ids=[f"{m}x{n}x{k}" for m, n, k in RAGGED])
def test_ragged_auto(mkp, shape):
    M, N, K = shape
    rng = np.random.default_rng(M * 1_000_003 + N * 1009 + K)
    run_case(mkp, rand_bits(rng, (M, K)), rand_bits(rng, (K, N)), what=f"auto {shape}")


EDGE = [(1, 1, 1), (15, 17, 63), (129, 250, 200), (257, 385, 130)]


@pytest.mark.parametrize("split", [1, 3])
def test_each_kernel_forced(mkp, split):
    rng = np.random.default_rng(split)
    try:
        mkp.mkp_set_option("force_splitk", split)
        for name in [n for n in mkp.mkp_kernel_names() if not n.endswith("_nk")]:
            mkp.mkp_set_option("force_kernel", name)
            for (M, N, K) in EDGE:
                run_case(mkp, rand_bits(rng, (M, K)), rand_bits(rng, (K, N)), what=f"{name} s={split}")
    finally:
        mkp.mkp_set_option("force_kernel", "")
        mkp.mkp_set_option("force_splitk", 0)


@pytest.mark.parametrize("split", [1, 3])
def test_each_kernel_forced_padded_b(mkp, split):
    """Every K x N micro-kernel where N is not a multiple of 8 but B's rows
    are 16-byte aligned (ldb = N rounded up to 8, the padding NaN): the last
    tile column takes the direct loads, whose last chunk of each B row
    reaches past N, and none of that may reach C."""
    rng = np.random.default_rng(40 + split)
    try:
        mkp.mkp_set_option("force_splitk", split)
        for name in [n for n in mkp.mkp_kernel_names() if not n.endswith("_nk")]:
            mkp.mkp_set_option("force_kernel", name)
            for (M, N, K) in ((129, 250, 200), (257, 385, 130), (65, 1001, 256), (16, 7, 64)):
                ldb = (N + 7) // 8 * 8
                run_case(mkp, rand_bits(rng, (M, K)), rand_bits(rng, (K, N)), ldb=ldb,
                         what=f"{name} s={split} padded B")
    finally:
        mkp.mkp_set_option("force_kernel", "")
        mkp.mkp_set_option("force_splitk", 0)


@pytest.mark.parametrize("nt", [0, 2, 38])
def test_each_kernel_store_policies(mkp, nt):
    """Every micro-kernel under the C-store policies other than the default:
    plain stores (0), streaming stores of every vector-aligned C (2), and
    streaming plus shared-level write-through of split-K partials with the
    second pass streaming (38); one split, and three with either reduction.
    C rows are dense (ldc = N: 256 is a multiple of 32 floats, 388 of 4 only)."""
    rng = np.random.default_rng(700 + nt)
    try:
        mkp.mkp_set_option("nt_stores", nt)
        for split, fused in ((1, 0), (3, 1), (3, 0)):
            mkp.mkp_set_option("force_splitk", split)
            mkp.mkp_set_option("fused_reduce", fused)
            for name in [n for n in mkp.mkp_kernel_names() if not n.endswith("_nk")]:
                mkp.mkp_set_option("force_kernel", name)
                for (M, N, K) in ((129, 256, 200), (257, 388, 130)):
                    run_case(mkp, rand_bits(rng, (M, K)), rand_bits(rng, (K, N)), ldc=N,
                             what=f"{name} s={split} fused={fused} nt={nt}")
    finally:
        mkp.mkp_set_option("force_kernel", "")
        mkp.mkp_set_option("force_splitk", 0)
        mkp.mkp_set_option("fused_reduce", 0)
        mkp.mkp_set_option("nt_stores", 33)


@pytest.mark.parametrize("fused", [1, 0])
@pytest.mark.parametrize("s", [2, 4, 8, 32])
def test_splitk(mkp, s, fused):
    rng = np.random.default_rng(100 + s)
    try:
        mkp.mkp_set_option("force_splitk", s)
        mkp.mkp_set_option("fused_reduce", fused)
        for (M, N, K) in [(33, 700, 4097), (200, 300, 2000), (1, 4096, 4096)]:
            run_case(mkp, rand_bits(rng, (M, K)), rand_bits(rng, (K, N)), what=f"splitk {s} fused={fused}")
    finally:
        mkp.mkp_set_option("force_splitk", 0)
        mkp.mkp_set_option("fused_reduce", 0)


@pytest.mark.parametrize("fused", [1])
def test_splitk_repeated_calls_reuse_counters(mkp, fused):
    """Back-to-back fused split-K calls on one stream (counters must return
    to zero after every launch) and batched split-K."""
    import torch
    rng = np.random.default_rng(321)
    try:
        mkp.mkp_set_option("force_splitk", 8)
        mkp.mkp_set_option("fused_reduce", fused)
        for it in range(3):
            run_case(mkp, rand_bits(rng, (70, 3000)), rand_bits(rng, (3000, 500)),
                     what=f"repeat {it}")
        batch, M, N, K = 5, 40, 300, 2048
        a = rand_bits(rng, (batch, M, K))
        b = rand_bits(rng, (batch, K, N))
        print("[case] batched split-K", flush=True)
        ta, pa = dev_bf16(a)
        tb, pb = dev_bf16(b)
        tc = torch.full((batch * M * N + 64,), float("nan"), dtype=torch.float32, device="cuda")
        mkp.mkp_gemm_batched(batch, M, N, K, pa, K, M * K, pb, N, K * N, tc.data_ptr(), N, M * N)
        torch.cuda.synchronize()
        h = tc.cpu().numpy()
        assert np.isnan(h[batch * M * N:]).all()
        got = h[:batch * M * N].reshape(batch, M, N).astype(np.float64)
        ref, refabs = oracle.gemm(a, b, with_abs=True)
        for z in range(batch):
            assert_close(got[z], ref[z], refabs[z], K, f"batched split-K [{z}]")
    finally:
        mkp.mkp_set_option("force_splitk", 0)
        mkp.mkp_set_option("fused_reduce", 0)


@pytest.mark.parametrize("pack", [1, 0])
def test_unaligned(mkp, pack):
    rng = np.random.default_rng(5)
    try:
        mkp.mkp_set_option("pack_unaligned", pack)
        M, N, K = 77, 131, 301
        a, b = rand_bits(rng, (M, K)), rand_bits(rng, (K, N))
        run_case(mkp, a, b, lda=K + 1, what=f"lda odd pack={pack}")
        run_case(mkp, a, b, ldb=N + 3, what=f"ldb odd pack={pack}")
        run_case(mkp, a, b, ldc=N + 1, what=f"ldc odd pack={pack}")
        run_case(mkp, a, b, offA=1, offB=3, offC=1, what=f"misaligned pointers pack={pack}")
        M, N, K = 256, 256, 256
        a, b = rand_bits(rng, (M, K)), rand_bits(rng, (K, N))
        run_case(mkp, a, b, offB=1, what=f"aligned shape, B pointer off by one pack={pack}")
        M, N, K = 300, 509, 64
        a, b = rand_bits(rng, (M, K)), rand_bits(rng, (K, N))
        run_case(mkp, a, b, lda=K + 3, ldb=N, ldc=N, what=f"odd N, ldb=N pack={pack}")
        # deep enough K for the staging copy of re-read unaligned operands
        # (the launch trace shows whether the copy ran)
        M, N, K = 260, 301, 520
        a, b = rand_bits(rng, (M, K)), rand_bits(rng, (K, N))
        mkp.mkp_set_option("trace", 1)
        mkp.mkp_trace_dump()
        run_case(mkp, a, b, lda=K + 1, ldb=N, ldc=N + 1, what=f"deep K, lda odd, odd N pack={pack}")
        packed = [r for r in mkp.mkp_trace_dump() if r["kernel"] == "pack_rows"]
        assert bool(packed) == bool(pack), packed
        run_case(mkp, a, b, offA=1, offB=1, what=f"deep K, misaligned pointers pack={pack}")
        M, N, K = 260, 301, 64   # shallow K: read in place either way
        a, b = rand_bits(rng, (M, K)), rand_bits(rng, (K, N))
        mkp.mkp_trace_dump()
        run_case(mkp, a, b, lda=K + 1, what=f"shallow K, lda odd pack={pack}")
        assert not [r for r in mkp.mkp_trace_dump() if r["kernel"] == "pack_rows"]
    finally:
        mkp.mkp_set_option("pack_unaligned", 1)
        mkp.mkp_set_option("trace", 0)
        mkp.mkp_trace_dump()


UNALIGNED_C_KERNELS = ["m256n256k64", "m128n128k64", "m128n64k64", "m64n64k64", "m16n128k64", "m32n64k64"]


@pytest.mark.parametrize("name", UNALIGNED_C_KERNELS)
def test_unaligned_rows_every_phase(mkp, name):
    """C rows that start at every 4-byte phase of a 16-byte boundary (the
    stores go out as whole 16-byte chunks plus up to three floats at each
    end), strips narrower than the head, and B rows at odd and even element
    offsets (word loads shifted by 16 bits, or not)."""
    rng = np.random.default_rng(500 + UNALIGNED_C_KERNELS.index(name))
    try:
        mkp.mkp_set_option("force_kernel", name)
        mkp.mkp_set_option("pack_unaligned", 0)
        for (M, N, K) in [(70, 67, 72), (33, 130, 64), (9, 3, 40), (150, 258, 136)]:
            a, b = rand_bits(rng, (M, K)), rand_bits(rng, (K, N))
            for ldc, offC, ldb, offB in [(N + 1, 0, N + 1, 0), (N + 2, 1, N, 1), (N + 3, 2, N + 2, 0),
                                         (N, 3, N + 3, 1)]:
                run_case(mkp, a, b, ldb=ldb, ldc=ldc, offB=offB, offC=offC,
                         what=f"{name} ldc={ldc} offC={offC} ldb={ldb} offB={offB}")
    finally:
        mkp.mkp_set_option("force_kernel", "")
        mkp.mkp_set_option("pack_unaligned", 1)


def test_k0_and_empty(mkp):
    import torch

    print("[case] K=0 / M=0 / N=0", flush=True)
    gc = GuardedC(1, 37, 41)
    mkp.mkp_gemm(37, 41, 0, 0, 1, 0, 41, gc.addr, gc.ld)
    torch.cuda.synchronize()
    got, untouched = gc.result()
    assert untouched and np.all(got == 0.0)
    gc = GuardedC(1, 5, 5)
    mkp.mkp_gemm(0, 5, 7, 0, 7, 0, 5, gc.addr, gc.ld)
    mkp.mkp_gemm(5, 0, 7, 0, 7, 0, 5, gc.addr, gc.ld)
    mkp.mkp_gemm_batched(0, 5, 5, 7, 0, 7, 0, 0, 5, 0, gc.addr, gc.ld, 0)
    torch.cuda.synchronize()
    h = gc.t.cpu().numpy()
    assert np.isnan(h).all()


def test_batched_config5_members(mkp):
    import torch

    cases = workloads.config_cases(5)
    for case in [cases[i] for i in (0, 1, 7, 31)] + [workloads.GemmCase(17, 17, 64, 48, ("normal", 0, 1),
                                                                        ("normal", 0, 1), (1,), (2,))]:
        a, b = workloads.make_operands(case)
        S, B = case.M, case.batch
        print(f"[case] batched {case.tag} S={S} batch={B}", flush=True)
        ta, pa = dev_bf16(a)
        tb, pb = dev_bf16(b)
        gc = GuardedC(B, S, S, ld=S)
        gc.stride = S * S  # packed like the workload
        gc.t = torch.full((B * S * S + 64 * S,), float("nan"), dtype=torch.float32, device="cuda")
        gc.addr = gc.t.data_ptr()
        mkp.mkp_gemm_batched(B, S, S, 64, pa, 64, S * 64, pb, S, 64 * S, gc.addr, S, S * S)
        torch.cuda.synchronize()
        h = gc.t.cpu().numpy()
        got = h[:B * S * S].reshape(B, S, S).astype(np.float64)
        assert np.isnan(h[B * S * S:]).all()
        ref, refabs = oracle.gemm(a, b, with_abs=True)
        for z in range(B):
            assert_close(got[z], ref[z], refabs[z], 64, f"{case.tag}[{z}]")


def sampled_check(mkp, case, nsamp=2048, a=None, b=None):
    import torch

    if a is None:
        a, b = workloads.make_operands(case)
    M, N, K = case.M, case.N, case.K
    print(f"[case] sampled {case.tag} M={M} N={N} K={K}", flush=True)
    ta, pa = dev_bf16(a)
    tb, pb = dev_bf16(b)
    tc = torch.full((M * N + 256,), float("nan"), dtype=torch.float32, device="cuda")
    mkp.mkp_gemm(M, N, K, pa, K, pb, N, tc.data_ptr(), N)
    torch.cuda.synchronize()
    h = tc.cpu().numpy()
    assert np.isnan(h[M * N:]).all(), "write beyond C"
    c = h[:M * N].reshape(M, N)
    assert np.isfinite(c).all(), "hole in C"
    rng = np.random.default_rng(M * 7 + N * 13 + K)
    rows = np.concatenate([rng.integers(0, M, nsamp), [0, M - 1, M - 1, 0]])
    cols = np.concatenate([rng.integers(0, N, nsamp), [0, N - 1, 0, N - 1]])
    ref, refabs = oracle.gemm_entries(a[0], b[0], rows, cols)
    assert_close(c[rows, cols].astype(np.float64), ref, refabs, K, case.tag)


def test_config2_sampled(mkp):
    for case in workloads.config_cases(2):
        sampled_check(mkp, case, nsamp=1024)


def test_config3_full_size_sampled(mkp):
    for case in workloads.config_cases(3):
        sampled_check(mkp, case, nsamp=4096)


def test_config4_sampled(mkp):
    weights = {}
    for case in workloads.config_cases(4)[::5]:
        if case.seed_b not in weights:
            weights[case.seed_b] = workloads.make_b(case)
        sampled_check(mkp, case, nsamp=1024, a=workloads.make_a(case), b=weights[case.seed_b])


def test_determinism(mkp):
    import torch

    rng = np.random.default_rng(77)
    M, N, K = 300, 1000, 5000
    a, b = rand_bits(rng, (M, K)), rand_bits(rng, (K, N))
    print("[case] determinism", flush=True)
    ta, pa = dev_bf16(a)
    tb, pb = dev_bf16(b)
    outs = []
    for s in (0, 0, 4, 4):
        mkp.mkp_set_option("force_splitk", s)
        tc = torch.empty((M, N), dtype=torch.float32, device="cuda")
        mkp.mkp_gemm(M, N, K, pa, K, pb, N, tc, N)
        torch.cuda.synchronize()
        outs.append(tc.cpu().numpy())
    mkp.mkp_set_option("force_splitk", 0)
    assert np.array_equal(outs[0], outs[1])
    assert np.array_equal(outs[2], outs[3])


def test_pattern_II_regions(mkp):
    """A table whose costs make two-region plans win; the II plans must still
    produce the exact product (regions partition C)."""
    names = mkp.mkp_kernel_names()
    big, small = "m128n128k64", "m64n64k64"
    assert big in names and small in names
    text = """device 2
launch_us 0
splitk 1
patterns II-M II-N
kernel m128n128k64 128 128 64 1
kernel m64n64k64 64 64 64 1
g m128n128k64 1:1 1000:1000
g m64n64k64 1:0.3 1000:300
"""
    path = os.path.join(tempfile.mkdtemp(), "ii.tbl")
    open(path, "w").write(text)
    rng = np.random.default_rng(9)
    try:
        mkp.mkp_load_calibration(path)
        for (M, N, K) in [(300, 200, 130), (129, 513, 64), (1000, 70, 99)]:
            plan = mkp.mkp_plan_describe(1, M, N, K)
            assert plan["pattern"] in ("II-M", "II-N"), plan
            run_case(mkp, rand_bits(rng, (M, K)), rand_bits(rng, (K, N)), what=f"II {plan['pattern']}")
    finally:
        mkp.mkp_load_calibration(None)


def test_ranked_and_ablated_plans(mkp):
    """Every plan the measured search launches (the ranked candidates of the
    shipped table, the WAVE and PIPE ablations, each kernel at 16 splits)
    computes the product."""
    rng = np.random.default_rng(12)
    try:
        for (M, N, K) in [(300, 257, 129), (1000, 700, 300)]:
            a, b = rand_bits(rng, (M, K)), rand_bits(rng, (K, N))
            for r in range(1, 17):
                mkp.mkp_set_option("plan_rank", r)
                plan = mkp.mkp_plan_describe(1, M, N, K)
                if not plan["regions"]:
                    break
                run_case(mkp, a, b, what=f"rank {r} {plan['pattern']}")
            mkp.mkp_set_option("plan_rank", 0)
            for mode in ("wave", "pipe"):
                mkp.mkp_set_option("cost_model", mode)
                run_case(mkp, a, b, what=f"cost_model {mode}")
            mkp.mkp_set_option("cost_model", "full")
        a, b = rand_bits(rng, (300, 1100)), rand_bits(rng, (1100, 257))
        mkp.mkp_set_option("force_splitk", 16)
        for name in [n for n in mkp.mkp_kernel_names() if not n.endswith("_nk")]:
            mkp.mkp_set_option("force_kernel", name)
            run_case(mkp, a, b, what=f"{name} s=16")
    finally:
        mkp.mkp_set_option("plan_rank", 0)
        mkp.mkp_set_option("cost_model", "full")
        mkp.mkp_set_option("force_kernel", "")
        mkp.mkp_set_option("force_splitk", 0)


def test_package_imported_before_torch(tmp_path):
    """A process that imports the package before torch still runs the GEMM
    (one HIP runtime per process); checked in a child process."""
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = tmp_path / "c.npy"
    code = f"""
import sys
sys.path.insert(0, {root!r})
import dynamic_shape_gemm_amd as m
import numpy as np
import torch
import workloads
case = workloads.config_cases(1)[0]
a, b = workloads.make_operands(case)
ta = torch.from_numpy(a[0].view(np.int16)).cuda().view(torch.bfloat16)
tb = torch.from_numpy(b[0].view(np.int16)).cuda().view(torch.bfloat16)
c = m.gemm(ta, tb)
torch.cuda.synchronize()
np.save({str(out)!r}, c.cpu().numpy())
"""
    print("[case] child process: package imported before torch, config1", flush=True)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=180)
    assert r.returncode == 0, r.stderr[-2000:]
    case = workloads.config_cases(1)[0]
    a, b = workloads.make_operands(case)
    ref, refabs = oracle.gemm(a[0], b[0], with_abs=True)
    assert_close(np.load(out), ref, refabs, case.K, "package-first child")


def test_transposed_b_path(mkp):
    """K x N calls run as a transpose of B into the workspace followed by the
    N x K kernels (forced here with transpose_b = 2): ragged, unaligned,
    split-K and batched cases."""
    rng = np.random.default_rng(4242)
    try:
        mkp.mkp_set_option("transpose_b", 2)
        # K and N multiples of 8 (register-block transpose) and not
        for (M, N, K) in [(1, 1, 1), (17, 33, 65), (300, 257, 129), (513, 1000, 777), (7, 300, 3000), (3, 8, 8),
                          (100, 200, 136), (260, 768, 3072)]:
            plan = mkp.mkp_plan_describe(1, M, N, K)
            assert plan["transpose_b"] and all(r["kernel"].endswith("_nk") for r in plan["regions"]), plan
            run_case(mkp, rand_bits(rng, (M, K)), rand_bits(rng, (K, N)), what=f"transposed B {M}x{N}x{K}")
        M, N, K = 77, 131, 301
        a, b = rand_bits(rng, (M, K)), rand_bits(rng, (K, N))
        run_case(mkp, a, b, ldb=N + 3, offB=1, what="transposed B, unaligned")
        mkp.mkp_set_option("force_splitk", 4)
        run_case(mkp, rand_bits(rng, (200, 2000)), rand_bits(rng, (2000, 300)), what="transposed B, split 4")
        mkp.mkp_set_option("force_splitk", 0)
        for batch, M, N, K in [(6, 90, 150, 64), (5, 40, 200, 72)]:
            _batched_transposed(mkp, rng, batch, M, N, K)
    finally:
        mkp.mkp_set_option("transpose_b", 1)
        mkp.mkp_set_option("force_splitk", 0)


def _batched_transposed(mkp, rng, batch, M, N, K):
    """One batched K x N call on the transposed-B path, NaN guard after C."""
    import torch

    a = rand_bits(rng, (batch, M, K))
    b = rand_bits(rng, (batch, K, N))
    print(f"[case] transposed B, batched {batch}x{M}x{N}x{K}", flush=True)
    ta, pa = dev_bf16(a)
    tb, pb = dev_bf16(b)
    tc = torch.full((batch * M * N + 64,), float("nan"), dtype=torch.float32, device="cuda")
    mkp.mkp_gemm_batched(batch, M, N, K, pa, K, M * K, pb, N, K * N, tc.data_ptr(), N, M * N)
    torch.cuda.synchronize()
    h = tc.cpu().numpy()
    assert np.isnan(h[batch * M * N:]).all()
    ref, refabs = oracle.gemm(a, b, with_abs=True)
    got = h[:batch * M * N].reshape(batch, M, N).astype(np.float64)
    for z in range(batch):
        assert_close(got[z], ref[z], refabs[z], K, f"transposed B batched [{z}]")


def test_concurrent_callers_on_separate_streams(mkp):
    """Two host threads call the library at once, each on its own stream with
    its own shapes (split-K workspaces are per stream, the plan cache is
    shared): every result matches the oracle."""
    import threading

    import torch

    rng = np.random.default_rng(99)
    jobs = []
    for t in range(2):
        cases = []
        for i in range(6):
            M, N, K = int(rng.integers(50, 700)), int(rng.integers(50, 700)), int(rng.integers(64, 3000))
            cases.append((rand_bits(rng, (M, K)), rand_bits(rng, (K, N))))
        jobs.append(cases)
    results = [[None] * 6 for _ in range(2)]
    errors = []
    print("[case] two threads, two streams", flush=True)

    def worker(t):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                outs = []
                for i, (a, b) in enumerate(jobs[t]):
                    M, K = a.shape
                    N = b.shape[1]
                    ta, pa = dev_bf16(a)
                    tb, pb = dev_bf16(b)
                    tc = torch.empty((M, N), dtype=torch.float32, device="cuda")
                    for _ in range(3):   # repeated calls: cache hits and workspace reuse
                        mkp.mkp_gemm(M, N, K, pa, K, pb, N, tc, N, stream.cuda_stream)
                    outs.append((ta, tb, tc))
                stream.synchronize()
                for i, (_, _, tc) in enumerate(outs):
                    results[t][i] = tc.cpu().numpy().astype(np.float64)
        except Exception as e:  # reported below
            errors.append(repr(e))

    try:
        mkp.mkp_set_option("force_splitk", 4)
        threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
        for th in threads:
            th.start()
        for th in threads:
            th.join()
    finally:
        mkp.mkp_set_option("force_splitk", 0)
    assert not errors, errors
    for t in range(2):
        for i, (a, b) in enumerate(jobs[t]):
            ref, refabs = oracle.gemm(a, b, with_abs=True)
            assert_close(results[t][i], ref, refabs, a.shape[1], f"thread {t} case {i}")


def test_concurrent_callers_on_one_stream(mkp):
    """Two host threads call the library at once on the SAME stream, every
    call using the stream's workspace (split-K partials forced, B copied to
    N x K first), with shapes that grow so the workspace is regrown between
    calls: each call holds the workspace until its launches are enqueued,
    so no call's partials or transposed B are overwritten or freed by the
    other's; every result matches the oracle."""
    import threading

    import torch

    rng = np.random.default_rng(101)
    jobs = []
    for t in range(2):
        cases = []
        for i in range(8):
            # sizes rise call by call (workspace regrowth), ragged and deep enough for 4 splits
            M = int(rng.integers(40, 120)) * (i + 1)
            N = int(rng.integers(40, 150)) * (i + 1)
            K = int(rng.integers(256, 1500))
            cases.append((rand_bits(rng, (M, K)), rand_bits(rng, (K, N))))
        jobs.append(cases)
    results = [[None] * 8 for _ in range(2)]
    errors = []
    stream = torch.cuda.Stream()
    barrier = threading.Barrier(2)
    print("[case] two threads, one shared stream, split 4, transposed B", flush=True)

    def worker(t):
        try:
            with torch.cuda.stream(stream):
                ins = []
                for a, b in jobs[t]:
                    M, K = a.shape
                    N = b.shape[1]
                    ta, pa = dev_bf16(a)
                    tb, pb = dev_bf16(b)
                    tc = torch.empty((M, N), dtype=torch.float32, device="cuda")
                    ins.append((ta, tb, tc, pa, pb, M, N, K))
                torch.cuda.current_stream().synchronize()
                barrier.wait()
                for _ in range(3):
                    for ta, tb, tc, pa, pb, M, N, K in ins:
                        rc = mkp.mkp_gemm(M, N, K, pa, K, pb, N, tc, N, stream.cuda_stream)
                        assert rc == 0
                stream.synchronize()
                for i, (_, _, tc, *_rest) in enumerate(ins):
                    results[t][i] = tc.cpu().numpy().astype(np.float64)
        except Exception as e:  # reported below
            errors.append(repr(e))

    try:
        mkp.mkp_set_option("force_splitk", 4)
        mkp.mkp_set_option("transpose_b", 2)
        mkp.mkp_cache_clear()   # start from an empty workspace, so it grows under both threads
        threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
        for th in threads:
            th.start()
        for th in threads:
            th.join()
    finally:
        mkp.mkp_set_option("force_splitk", 0)
        mkp.mkp_set_option("transpose_b", 1)
    assert not errors, errors
    for t in range(2):
        for i, (a, b) in enumerate(jobs[t]):
            ref, refabs = oracle.gemm(a, b, with_abs=True)
            assert_close(results[t][i], ref, refabs, a.shape[1], f"shared stream: thread {t} case {i}")
