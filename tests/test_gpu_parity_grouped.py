"""GPU parity of grouped calls (mkp_gemm_grouped / mkp_gemm_grouped_bt): one
launch computes C_g = A . B_g for up to four B_g that share A -- the merge
of products with a common operand (BladeDISC page, GEMM merge, first kind;
the query/key/value projections are the typical case).  Each group's C is
checked element by element against the CPU oracle, with NaN guard bands
around every C; the gate is the one of the single-product path.
"""
import numpy as np
import pytest

import oracle
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


def run_grouped(mkp, a, ws, *, bt=False, lda=None, ldbs=None, ldcs=None, offA=0, offBs=None, offCs=None,
                what="", check=True):
    """a (M,K); ws[g] (K,N_g), or (N_g,K) when bt; all bf16 bits.  Returns
    the per-group results (float64) after checking each against the oracle."""
    import torch

    M, K = a.shape
    G = len(ws)
    Ns = [w.shape[0] if bt else w.shape[1] for w in ws]
    lda = lda or max(K, 1)
    ldbs = ldbs or [max(K if bt else n, 1) for n in Ns]
    offBs = offBs or [0] * G
    offCs = offCs or [0] * G
    print(f"[case] grouped {'nk' if bt else 'kn'} {what} M={M} K={K} N={Ns} lda={lda} ldb={ldbs} "
          f"ldc={ldcs} offA={offA} offB={offBs} offC={offCs}", flush=True)
    ta, pa = dev_bf16(padded(a, lda) if K else a, offA)
    keep, pbs, gcs = [ta], [], []
    for g in range(G):
        tb, pb = dev_bf16(padded(ws[g], ldbs[g]) if ws[g].size else ws[g], offBs[g])
        keep.append(tb)
        pbs.append(pb)
        gcs.append(GuardedC(1, M, Ns[g], ld=None if ldcs is None else ldcs[g], offset=offCs[g]))
    fn = mkp.mkp_gemm_grouped_bt if bt else mkp.mkp_gemm_grouped
    fn(M, K, pa, lda, Ns, pbs, ldbs, [gc.addr for gc in gcs], [gc.ld for gc in gcs])
    torch.cuda.synchronize()
    outs = []
    for g in range(G):
        got, untouched = gcs[g].result()
        assert untouched, f"{what}: write outside C of group {g}"
        if check and Ns[g] > 0:
            b = np.ascontiguousarray(ws[g].T) if bt else ws[g]
            ref, refabs = oracle.gemm(a, b, with_abs=True)
            assert_close(got[0], ref, refabs, K, f"{what} group {g}")
        outs.append(got[0])
    return outs


def make_ws(rng, K, Ns, bt):
    return [rand_bits(rng, (n, K) if bt else (K, n)) for n in Ns]


CASES = [
    (300, 768, [768, 768, 768]),        # query/key/value of a 768-wide layer
    (1, 256, [64, 64, 64]),
    (77, 129, [17, 300, 5, 129]),       # ragged widths, ragged K
    (513, 200, [1000]),                 # one group
    (16, 4096, [256, 512]),
    (255, 65, [255, 1, 33]),
]


@pytest.mark.parametrize("bt", [False, True], ids=["kn", "nk"])
@pytest.mark.parametrize("case", CASES, ids=[f"{m}x{k}x{'+'.join(map(str, n))}" for m, k, n in CASES])
def test_grouped_auto(mkp, case, bt):
    M, K, Ns = case
    rng = np.random.default_rng(M * 31 + K + len(Ns))
    run_grouped(mkp, rand_bits(rng, (M, K)), make_ws(rng, K, Ns, bt), bt=bt, what="auto")


@pytest.mark.parametrize("bt", [False, True], ids=["kn", "nk"])
def test_grouped_each_kernel_forced(mkp, bt):
    """Every micro-kernel of the layout, with and without split-K, over
    groups whose widths end mid-tile (tile columns of neighbouring groups
    meet inside one launch)."""
    rng = np.random.default_rng(61 + bt)
    names = [n for n in mkp.mkp_kernel_names() if n.endswith("_nk") == bt]
    M, K = 133, 200
    Ns = [70, 257, 3]
    a = rand_bits(rng, (M, K))
    ws = make_ws(rng, K, Ns, bt)
    try:
        for split in (1, 3):
            mkp.mkp_set_option("force_splitk", split)
            for name in names:
                mkp.mkp_set_option("force_kernel", name)
                run_grouped(mkp, a, ws, bt=bt, what=f"{name} s={split}")
    finally:
        mkp.mkp_set_option("force_kernel", "")
        mkp.mkp_set_option("force_splitk", 0)


@pytest.mark.parametrize("nt", [33, 0, 38])
@pytest.mark.parametrize("bt", [False, True], ids=["kn", "nk"])
def test_grouped_store_policies(mkp, bt, nt):
    """Every micro-kernel over vector-aligned groups under the default
    C-store policy (33: streaming stores where C is 128-byte aligned with a
    leading dimension of 32 floats), plain stores (0), and streaming stores
    with shared-level write-through of split-K partials (38); one split and
    three."""
    rng = np.random.default_rng(800 + nt + bt)
    names = [n for n in mkp.mkp_kernel_names() if n.endswith("_nk") == bt]
    M, K = 200, 160
    Ns = [64, 256, 96]
    a = rand_bits(rng, (M, K))
    ws = make_ws(rng, K, Ns, bt)
    try:
        mkp.mkp_set_option("nt_stores", nt)
        for split in (1, 3):
            mkp.mkp_set_option("force_splitk", split)
            for name in names:
                mkp.mkp_set_option("force_kernel", name)
                run_grouped(mkp, a, ws, bt=bt, ldcs=list(Ns), what=f"{name} s={split} nt={nt}")
    finally:
        mkp.mkp_set_option("force_kernel", "")
        mkp.mkp_set_option("force_splitk", 0)
        mkp.mkp_set_option("nt_stores", 33)


@pytest.mark.parametrize("s", [2, 8])
def test_grouped_splitk(mkp, s):
    rng = np.random.default_rng(300 + s)
    try:
        mkp.mkp_set_option("force_splitk", s)
        for bt in (False, True):
            run_grouped(mkp, rand_bits(rng, (40, 3000)), make_ws(rng, 3000, [130, 64, 700], bt), bt=bt,
                        what=f"splitk {s}")
    finally:
        mkp.mkp_set_option("force_splitk", 0)


def test_grouped_matches_separate_calls_bitwise(mkp):
    """With the kernel and split fixed, a grouped launch does each group's
    arithmetic in the same order as a call of its own: the outputs agree
    bit for bit."""
    import torch

    rng = np.random.default_rng(7)
    M, K, Ns = 200, 512, [256, 96, 640]
    a = rand_bits(rng, (M, K))
    ws = make_ws(rng, K, Ns, True)
    try:
        for name, split in (("m128n128k64_nk", 1), ("m64n64k64_nk", 4)):
            mkp.mkp_set_option("force_kernel", name)
            mkp.mkp_set_option("force_splitk", split)
            grouped = run_grouped(mkp, a, ws, bt=True, what=f"{name} s={split} vs separate")
            ta, pa = dev_bf16(a)
            for g, w in enumerate(ws):
                tw, pw = dev_bf16(w)
                gc = GuardedC(1, M, Ns[g])
                mkp.mkp_gemm_bt(M, Ns[g], K, pa, K, pw, K, gc.addr, gc.ld)
                torch.cuda.synchronize()
                got, untouched = gc.result()
                assert untouched
                assert np.array_equal(got[0], grouped[g]), (name, split, g)
    finally:
        mkp.mkp_set_option("force_kernel", "")
        mkp.mkp_set_option("force_splitk", 0)


def test_grouped_unaligned(mkp):
    """Leading dimensions and pointers that rule out 128-bit accesses, for
    some groups only: each group keeps its own access width."""
    rng = np.random.default_rng(19)
    M, K = 150, 301
    for bt in (False, True):
        Ns = [131, 64, 257]
        a = rand_bits(rng, (M, K))
        ws = make_ws(rng, K, Ns, bt)
        run_grouped(mkp, a, ws, bt=bt, what="K odd")
        ldbs = [K + 3, K, K + 8] if bt else [Ns[0] + 1, Ns[1], Ns[2] + 8]
        run_grouped(mkp, a, ws, bt=bt, ldbs=ldbs, ldcs=[Ns[0] + 1, Ns[1] + 4, Ns[2] + 3],
                    what="mixed leading dimensions")
        run_grouped(mkp, a, ws, bt=bt, offA=1, offBs=[0, 3, 0], offCs=[1, 0, 2], what="misaligned pointers")


def test_grouped_zero_width_groups_and_k0(mkp):
    rng = np.random.default_rng(23)
    M, K = 90, 100
    for bt in (False, True):
        ws = make_ws(rng, K, [40, 0, 65, 0], bt)
        run_grouped(mkp, rand_bits(rng, (M, K)), ws, bt=bt, what="zero-width groups")
    # K = 0: every C is zero filled, nothing else written
    outs = run_grouped(mkp, rand_bits(rng, (M, 0)), [np.zeros((0, 33), np.uint16), np.zeros((0, 7), np.uint16)],
                       what="K=0", check=False)
    assert all(np.all(o == 0.0) for o in outs)


def test_grouped_qkv_full_size_sampled(mkp):
    """Query/key/value projections at full size (M = 8192 tokens, 768 wide,
    weights kept N x K) in one launch; sampled entries against the oracle."""
    import torch

    rng = np.random.default_rng(99)
    M, K, Ns = 8192, 768, [768, 768, 768]
    a = rand_bits(rng, (M, K))
    ws = make_ws(rng, K, Ns, True)
    print(f"[case] grouped qkv sampled M={M} K={K} N={Ns}", flush=True)
    ta, pa = dev_bf16(a)
    tws = [dev_bf16(w) for w in ws]
    tcs = [torch.full((M * n + 256,), float("nan"), dtype=torch.float32, device="cuda") for n in Ns]
    mkp.mkp_gemm_grouped_bt(M, K, pa, K, Ns, [p for _, p in tws], [K] * 3, [t.data_ptr() for t in tcs], Ns)
    torch.cuda.synchronize()
    for g, n in enumerate(Ns):
        h = tcs[g].cpu().numpy()
        assert np.isnan(h[M * n:]).all(), "write beyond C"
        c = h[:M * n].reshape(M, n)
        rows = np.concatenate([rng.integers(0, M, 1024), [0, M - 1]])
        cols = np.concatenate([rng.integers(0, n, 1024), [n - 1, 0]])
        ref, refabs = oracle.gemm_entries(a, np.ascontiguousarray(ws[g].T), rows, cols)
        assert_close(c[rows, cols].astype(np.float64), ref, refabs, K, f"qkv group {g}")
