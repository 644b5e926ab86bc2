"""GPU parity of C = A . B^T with B given as N x K (mkp_gemm_bt, the layout
of a linear layer's weights and of attention's K), through the C-ABI,
against the CPU oracle of C = A . B on the transposed operand.

Every case prints its name before it touches the GPU; the gate is the one of
the K x N path (|dC| <= 1e-3*sqrt(K) and the binary32 summation bound).
"""
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
    yield m
    m.mkp_set_option("force_kernel", "")
    m.mkp_set_option("force_splitk", 0)


def rand_bits(rng, shape):
    return f32_to_bf16_bits(rng.uniform(-1, 1, size=shape).astype(np.float32))


def reference(a, w, with_abs=True):
    """C = A . W^T: the oracle's product with W^T laid out as K x N."""
    return oracle.gemm(a, np.ascontiguousarray(np.swapaxes(w, -1, -2)), with_abs=with_abs)


def run_case_bt(mkp, a, w, *, lda=None, ldb=None, ldc=None, offA=0, offB=0, offC=0, what=""):
    """a (M,K), w (N,K) bf16 bits; full-element compare with guard bands."""
    import torch

    M, K = a.shape
    N = w.shape[0]
    lda = lda or max(K, 1)
    ldb = ldb or max(K, 1)
    print(f"[case] bt {what} M={M} N={N} K={K} lda={lda} ldb={ldb} ldc={ldc} off=({offA},{offB},{offC})",
          flush=True)
    ta, pa = dev_bf16(padded(a, lda) if K else a, offA)
    tb, pb = dev_bf16(padded(w, ldb) if K else w, offB)
    gc = GuardedC(1, M, N, ld=ldc, offset=offC)
    mkp.mkp_gemm_bt(M, N, K, pa, lda, pb, ldb, gc.addr, gc.ld)
    torch.cuda.synchronize()
    got, untouched = gc.result()
    ref, refabs = reference(a, w)
    assert untouched, f"{what}: write outside C"
    return assert_close(got[0], ref, refabs, K, what)


RAGGED = [(1, 1, 1), (1, 4096, 64), (17, 33, 65), (64, 64, 64), (300, 257, 129), (255, 511, 1023),
          (513, 1000, 777), (16, 5000, 300), (1000, 17, 2049), (7, 300, 12544)]


@pytest.mark.parametrize("shape", RAGGED, ids=[f"{m}x{n}x{k}" for m, n, k in RAGGED])
def test_bt_ragged_auto(mkp, shape):
    M, N, K = shape
    rng = np.random.default_rng(M * 7919 + N * 31 + K)
    run_case_bt(mkp, rand_bits(rng, (M, K)), rand_bits(rng, (N, K)), what=f"auto {shape}")


EDGE = [(1, 1, 1), (15, 17, 63), (129, 250, 200), (257, 385, 130)]


@pytest.mark.parametrize("split", [1, 3])
def test_bt_each_kernel_forced(mkp, split):
    rng = np.random.default_rng(40 + split)
    names = [n for n in mkp.mkp_kernel_names() if n.endswith("_nk")]
    assert len(names) >= 8
    try:
        mkp.mkp_set_option("force_splitk", split)
        for name in names:
            mkp.mkp_set_option("force_kernel", name)
            for (M, N, K) in EDGE:
                run_case_bt(mkp, rand_bits(rng, (M, K)), rand_bits(rng, (N, K)), what=f"{name} s={split}")
    finally:
        mkp.mkp_set_option("force_kernel", "")
        mkp.mkp_set_option("force_splitk", 0)


@pytest.mark.parametrize("s", [2, 8, 32])
def test_bt_splitk(mkp, s):
    rng = np.random.default_rng(200 + s)
    try:
        mkp.mkp_set_option("force_splitk", s)
        for (M, N, K) in [(33, 700, 4097), (200, 300, 2000), (1, 4096, 4096)]:
            run_case_bt(mkp, rand_bits(rng, (M, K)), rand_bits(rng, (N, K)), what=f"splitk {s}")
    finally:
        mkp.mkp_set_option("force_splitk", 0)


@pytest.mark.parametrize("pack", [1, 0])
def test_bt_unaligned(mkp, pack):
    rng = np.random.default_rng(15)
    try:
        mkp.mkp_set_option("pack_unaligned", pack)
        M, N, K = 300, 131, 301
        a, w = rand_bits(rng, (M, K)), rand_bits(rng, (N, K))
        run_case_bt(mkp, a, w, what=f"K odd pack={pack}")
        run_case_bt(mkp, a, w, ldb=K + 4, what=f"ldb = K+4 pack={pack}")
        run_case_bt(mkp, a, w, offA=1, offB=3, offC=1, what=f"misaligned pointers pack={pack}")
        M, N, K = 256, 256, 256
        a, w = rand_bits(rng, (M, K)), rand_bits(rng, (N, K))
        run_case_bt(mkp, a, w, offB=1, what=f"aligned shape, B pointer off by one pack={pack}")
        # deep enough K for the staging copy of re-read unaligned operands
        M, N, K = 300, 260, 777
        a, w = rand_bits(rng, (M, K)), rand_bits(rng, (N, K))
        run_case_bt(mkp, a, w, what=f"deep K odd pack={pack}")
        run_case_bt(mkp, a, w, offA=1, offB=1, what=f"deep K, misaligned pointers pack={pack}")
    finally:
        mkp.mkp_set_option("pack_unaligned", 1)


BT_PHASE_KERNELS = ["m256n256k64_nk", "m128n128k64_nk", "m64n64k64_nk", "m32n128k64_nk"]


@pytest.mark.parametrize("name", BT_PHASE_KERNELS)
def test_bt_unaligned_rows_every_phase(mkp, name):
    """N x K kernels on rows of every alignment: A and B rows at odd and even
    element offsets (whole chunks read as shifted 4-byte words) and C rows at
    every 4-byte phase of a 16-byte boundary (16-byte chunk stores plus up to
    three floats at each end)."""
    rng = np.random.default_rng(700 + BT_PHASE_KERNELS.index(name))
    try:
        mkp.mkp_set_option("force_kernel", name)
        mkp.mkp_set_option("pack_unaligned", 0)
        for (M, N, K) in [(70, 67, 72), (33, 130, 136), (9, 3, 40)]:
            a, w = rand_bits(rng, (M, K)), rand_bits(rng, (N, K))
            for lda, ldb, ldc, offA, offB, offC in [(K + 1, K + 1, N + 1, 0, 0, 0), (K, K + 2, N + 2, 1, 1, 1),
                                                    (K + 3, K, N + 3, 0, 1, 2), (K + 1, K + 3, N, 1, 0, 3)]:
                run_case_bt(mkp, a, w, lda=lda, ldb=ldb, ldc=ldc, offA=offA, offB=offB, offC=offC,
                            what=f"{name} lda={lda} ldb={ldb} ldc={ldc} off=({offA},{offB},{offC})")
    finally:
        mkp.mkp_set_option("force_kernel", "")
        mkp.mkp_set_option("pack_unaligned", 1)


def test_bt_k0_and_empty(mkp):
    import torch

    print("[case] bt K=0 / M=0 / N=0", flush=True)
    gc = GuardedC(1, 37, 41)
    mkp.mkp_gemm_bt(37, 41, 0, 0, 1, 0, 1, gc.addr, gc.ld)
    torch.cuda.synchronize()
    got, untouched = gc.result()
    assert untouched and np.all(got == 0.0)
    gc = GuardedC(1, 5, 5)
    mkp.mkp_gemm_bt(0, 5, 7, 0, 7, 0, 7, gc.addr, gc.ld)
    mkp.mkp_gemm_bt(5, 0, 7, 0, 7, 0, 7, gc.addr, gc.ld)
    mkp.mkp_gemm_batched_bt(0, 5, 5, 7, 0, 7, 0, 0, 7, 0, gc.addr, gc.ld, 0)
    torch.cuda.synchronize()
    assert np.isnan(gc.t.cpu().numpy()).all()


def test_bt_batched_attention_scores(mkp):
    """Per-head scores Q . K^T with K kept as S x 64 rows (config 5's
    shapes): B given as N x K is the natural layout."""
    import torch

    cases = workloads.config_cases(5)
    for case in [cases[i] for i in (0, 3, 31)]:
        q, k_t = workloads.make_operands(case)            # q: (B,S,64); k_t: (B,64,S) as K x N
        k = np.ascontiguousarray(np.swapaxes(k_t, 1, 2))  # the same keys as S x 64 rows
        S, B = case.M, case.batch
        print(f"[case] bt batched {case.tag} S={S} batch={B}", flush=True)
        tq, pq = dev_bf16(q)
        tk, pk = dev_bf16(k)
        tc = torch.full((B * S * S + 64 * S,), float("nan"), dtype=torch.float32, device="cuda")
        mkp.mkp_gemm_batched_bt(B, S, S, 64, pq, 64, S * 64, pk, 64, S * 64, tc.data_ptr(), S, S * S)
        torch.cuda.synchronize()
        h = tc.cpu().numpy()
        assert np.isnan(h[B * S * S:]).all()
        got = h[:B * S * S].reshape(B, S, S).astype(np.float64)
        ref, refabs = oracle.gemm(q, k_t, with_abs=True)
        for z in range(B):
            assert_close(got[z], ref[z], refabs[z], 64, f"{case.tag}[{z}]")


def test_bt_config2_weights_sampled(mkp):
    """The encoder linears with their weights stored N x K, sampled entries
    at full size."""
    import torch

    for case in workloads.config_cases(2)[:8]:
        a, b = workloads.make_operands(case)
        w = np.ascontiguousarray(b[0].T)
        M, N, K = case.M, case.N, case.K
        print(f"[case] bt sampled {case.tag} M={M} N={N} K={K}", flush=True)
        ta, pa = dev_bf16(a)
        tw, pw = dev_bf16(w)
        tc = torch.full((M * N + 256,), float("nan"), dtype=torch.float32, device="cuda")
        mkp.mkp_gemm_bt(M, N, K, pa, K, pw, K, tc.data_ptr(), N)
        torch.cuda.synchronize()
        h = tc.cpu().numpy()
        assert np.isnan(h[M * N:]).all(), "write beyond C"
        c = h[:M * N].reshape(M, N)
        rng = np.random.default_rng(M + N + K)
        rows = np.concatenate([rng.integers(0, M, 1024), [0, M - 1]])
        cols = np.concatenate([rng.integers(0, N, 1024), [N - 1, 0]])
        ref, refabs = oracle.gemm_entries(a[0], b[0], rows, cols)
        assert_close(c[rows, cols].astype(np.float64), ref, refabs, K, case.tag)
