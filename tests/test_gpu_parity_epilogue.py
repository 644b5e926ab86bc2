"""GPU parity of the fused epilogue (mkp_gemm_ex): C := act(alpha * A.op(B) +
beta * C + bias), Bolt page, epilogue fusion.  Each result is checked element
by element against the oracle product followed by the oracle epilogue
(oracle/epilogue.py), with NaN guard bands around C.

Tolerance: the product's gate carried through the epilogue,
  |dC| <= L * (|alpha| * e_K + 4u * (|alpha.acc| + |beta.C| + |bias|)) + 8u * (|v| + |C_ref|),
with e_K = 1e-3 * sqrt(K) (the product's gate), then again with e_K the
binary32 summation bound; L = sup |act'|, u = 2^-24, v the pre-activation.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import epilogue as ep
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

from _gpu_util import GuardedC, dev_bf16, padded  # noqa: E402

U = 2.0 ** -24


@pytest.fixture(scope="module")
def mkp(gpu):
    import dynamic_shape_gemm_amd as m

    m.mkp_load_calibration(None)
    for k, v in (("force_kernel", ""), ("force_splitk", 0), ("fused_reduce", 1), ("patterns", "I,II")):
        m.mkp_set_option(k, v)
    yield m
    for k, v in (("force_kernel", ""), ("force_splitk", 0), ("fused_reduce", 1), ("patterns", "I,II")):
        m.mkp_set_option(k, v)


def rand_bits(rng, shape):
    return f32_to_bf16_bits(rng.uniform(-1, 1, size=shape).astype(np.float32))


def check_epilogue(got, acc, acc_abs, K, alpha, beta, c_old, bias, act, what):
    v = ep.pre_activation(acc, alpha, beta, c_old, bias)
    ref = ep.activation(act, v)
    L = ep.LIPSCHITZ[act]
    terms = np.abs(alpha * acc)
    if beta != 0.0:
        terms = terms + np.abs(beta * c_old)
    if bias is not None:
        terms = terms + np.abs(bias)
    tail = 8 * U * (np.abs(v) + np.abs(ref)) + 1e-30
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    gate = L * (abs(alpha) * 1e-3 * math.sqrt(max(K, 1)) + 4 * U * terms) + tail
    assert (err <= gate).all(), f"{what}: max|dC| {err.max():.3e}, worst excess {(err - gate).max():.3e}"
    bound = L * (abs(alpha) * oracle.error_bound(K, acc_abs) + 4 * U * terms) + tail
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond the summation bound carried through"


def run_ex(mkp, a, b, *, nk=False, batch=1, alpha=1.0, beta=0.0, act="none", bias=True, ldc=None, offC=0,
           rng=None, what="", check=True):
    """a (batch,M,K), b (batch,K,N) or (batch,N,K) when nk; returns got (batch,M,N)."""
    import torch

    batch, M, K = a.shape
    N = b.shape[1] if nk else b.shape[2]
    rng = rng or np.random.default_rng(0)
    print(f"[case] epilogue {what} batch={batch} M={M} N={N} K={K} nk={nk} alpha={alpha} beta={beta} "
          f"act={act} bias={bias} ldc={ldc} offC={offC}", flush=True)
    ta, pa = dev_bf16(a)
    tb, pb = dev_bf16(b)
    gc = GuardedC(batch, M, N, ld=ldc, offset=offC)
    c_old = None
    if beta != 0.0:
        c_old = rng.uniform(-2, 2, size=(batch, M, N)).astype(np.float32)
        h = gc.t.cpu().numpy()
        for z in range(batch):
            for i in range(M):
                base = gc.offset + z * gc.stride + i * gc.ld
                h[base:base + N] = c_old[z, i]
        gc.t.copy_(torch.from_numpy(h))
    bias_h = rng.uniform(-1, 1, size=N).astype(np.float32) if bias else None
    tbias = torch.from_numpy(bias_h).cuda() if bias else None
    ldb = K if nk else N
    mkp.mkp_gemm_ex(batch, M, N, K, pa, K, M * K, pb, ldb, N * K, mkp.MKP_B_NK if nk else mkp.MKP_B_KN,
                    gc.addr, gc.ld, gc.stride, alpha, beta, tbias, act)
    torch.cuda.synchronize()
    got, untouched = gc.result()
    assert untouched, f"{what}: write outside C"
    if check:
        bk = np.ascontiguousarray(np.swapaxes(b, 1, 2)) if nk else b
        acc, acc_abs = oracle.gemm(a, bk, with_abs=True)
        for z in range(batch):
            check_epilogue(got[z], acc[z], acc_abs[z], K, alpha, beta, None if c_old is None else c_old[z],
                           bias_h, act, f"{what}[{z}]")
    return got


ACTS = ["none", "relu", "gelu", "gelu_tanh", "silu"]
SHAPES = [(1, 64, 64), (77, 130, 200), (300, 257, 129)]


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("nk", [False, True], ids=["kn", "nk"])
def test_activations_bias_alpha_beta(mkp, act, nk):
    rng = np.random.default_rng(11 + ACTS.index(act) + 7 * nk)
    for (M, N, K) in SHAPES:
        a = rand_bits(rng, (1, M, K))
        b = rand_bits(rng, (1, N, K) if nk else (1, K, N))
        run_ex(mkp, a, b, nk=nk, alpha=1.5, act=act, rng=rng, what=f"{act} alpha")
        run_ex(mkp, a, b, nk=nk, beta=0.5, act=act, rng=rng, what=f"{act} beta")
        run_ex(mkp, a, b, nk=nk, alpha=-0.75, beta=-1.0, act=act, bias=False, rng=rng, what=f"{act} no bias")


@pytest.mark.parametrize("fused", [1, 0], ids=["fused", "two-pass"])
def test_epilogue_with_split_k(mkp, fused):
    """Split partials never see the epilogue; the fused last-arrival sum or
    the second pass applies it once."""
    rng = np.random.default_rng(40 + fused)
    try:
        mkp.mkp_set_option("fused_reduce", fused)
        for s in (2, 5):
            mkp.mkp_set_option("force_splitk", s)
            for nk in (False, True):
                a = rand_bits(rng, (1, 96, 1500))
                b = rand_bits(rng, (1, 200, 1500) if nk else (1, 1500, 200))
                run_ex(mkp, a, b, nk=nk, alpha=0.5, beta=1.0, act="gelu", rng=rng, what=f"s={s}")
    finally:
        mkp.mkp_set_option("force_splitk", 0)
        mkp.mkp_set_option("fused_reduce", 1)


def test_epilogue_each_kernel_forced(mkp):
    rng = np.random.default_rng(5)
    a = rand_bits(rng, (1, 133, 150))
    bkn = rand_bits(rng, (1, 150, 261))
    bnk = rand_bits(rng, (1, 261, 150))
    try:
        for name in mkp.mkp_kernel_names():
            nk = name.endswith("_nk")
            mkp.mkp_set_option("force_kernel", name)
            run_ex(mkp, a, bnk if nk else bkn, nk=nk, beta=0.25, act="silu", rng=rng, what=name)
    finally:
        mkp.mkp_set_option("force_kernel", "")


def test_epilogue_batched_and_unaligned(mkp):
    rng = np.random.default_rng(8)
    a = rand_bits(rng, (3, 70, 96))
    b = rand_bits(rng, (3, 96, 45))
    run_ex(mkp, a, b, batch=3, beta=2.0, act="relu", rng=rng, what="batched")
    # C rows not 16-byte aligned: the element-wise store path carries the epilogue
    run_ex(mkp, a, b, batch=3, beta=0.5, act="gelu_tanh", ldc=47, offC=1, rng=rng, what="unaligned C")


def test_epilogue_k0(mkp):
    """K = 0: the product is an empty sum, C := act(beta * C + bias)."""
    rng = np.random.default_rng(9)
    a = np.zeros((1, 33, 0), np.uint16)
    b = np.zeros((1, 0, 70), np.uint16)
    got = run_ex(mkp, a, b, beta=0.5, act="silu", rng=np.random.default_rng(1), what="K=0", check=False)
    # rebuild the same c_old and bias draws as run_ex (same generator seed and order)
    r = np.random.default_rng(1)
    c_old = r.uniform(-2, 2, size=(1, 33, 70)).astype(np.float32)
    bias = r.uniform(-1, 1, size=70).astype(np.float32)
    ref = ep.epilogue(np.zeros((33, 70)), 1.0, 0.5, c_old[0], bias, "silu")
    assert np.allclose(got[0], ref, rtol=0, atol=8 * U * (np.abs(ref) + 2))


def test_identity_and_power_of_two_alpha_bitwise(mkp):
    """The identity epilogue is the plain product bit for bit, and alpha = 2
    doubles it bit for bit -- also through split-K and a two-region plan --
    so alpha is applied once, to the final sum."""
    import torch

    rng = np.random.default_rng(21)
    cases = [(200, 300, 700, 0, 1), (200, 300, 700, 3, 1), (200, 300, 700, 3, 0), (2720, 3072, 768, 0, 1)]
    try:
        for (M, N, K, s, fused) in cases:
            mkp.mkp_set_option("force_splitk", s)
            mkp.mkp_set_option("fused_reduce", fused)
            a = rand_bits(rng, (M, K))
            b = rand_bits(rng, (K, N))
            ta, pa = dev_bf16(a)
            tb, pb = dev_bf16(b)
            print(f"[case] epilogue bitwise M={M} N={N} K={K} s={s} fused={fused}", flush=True)
            plain = torch.empty((M, N), dtype=torch.float32, device="cuda")
            ident = torch.empty_like(plain)
            twice = torch.empty_like(plain)
            mkp.mkp_gemm(M, N, K, pa, K, pb, N, plain, N)
            mkp.mkp_gemm_ex(1, M, N, K, pa, K, 0, pb, N, 0, mkp.MKP_B_KN, ident, N, 0, 1.0, 0.0, None, "none")
            mkp.mkp_gemm_ex(1, M, N, K, pa, K, 0, pb, N, 0, mkp.MKP_B_KN, twice, N, 0, 2.0, 0.0, None, "none")
            torch.cuda.synchronize()
            assert torch.equal(plain, ident)
            assert torch.equal(2.0 * plain, twice)
    finally:
        mkp.mkp_set_option("force_splitk", 0)
        mkp.mkp_set_option("fused_reduce", 1)


def test_epilogue_on_two_region_plan_sampled(mkp):
    """A plan that cuts N (two regions, split-K in both): the bias of the
    second region starts at the cut.  Sampled entries on both sides of it."""
    import torch

    M, N, K = 336, 6000, 4096
    plan = mkp.mkp_plan_describe(1, M, N, K)
    print(f"[case] epilogue two-region plan {plan['pattern']} "
          f"{[(r['kernel'], r['s'], r['n0'], r['n']) for r in plan['regions']]}", flush=True)
    rng = np.random.default_rng(31)
    a = rand_bits(rng, (M, K))
    b = rand_bits(rng, (K, N))
    bias = rng.uniform(-1, 1, size=N).astype(np.float32)
    c_old = rng.uniform(-1, 1, size=(M, N)).astype(np.float32)
    ta, pa = dev_bf16(a)
    tb, pb = dev_bf16(b)
    tc = torch.from_numpy(c_old.copy()).cuda()
    tbias = torch.from_numpy(bias).cuda()
    mkp.mkp_gemm_ex(1, M, N, K, pa, K, 0, pb, N, 0, mkp.MKP_B_KN, tc, N, 0, 1.0, 1.0, tbias, "gelu")
    torch.cuda.synchronize()
    got = tc.cpu().numpy().astype(np.float64)
    cut = plan["regions"][1]["n0"] if len(plan["regions"]) > 1 else N // 2
    cols = np.concatenate([np.arange(max(cut - 40, 0), min(cut + 40, N)), rng.integers(0, N, 300), [0, N - 1]])
    rows = rng.integers(0, M, cols.size)
    rows[:2] = [0, M - 1]
    acc, acc_abs = oracle.gemm_entries(a, b, rows, cols)
    check_epilogue(got[rows, cols], acc, acc_abs, K, 1.0, 1.0, c_old[rows, cols].astype(np.float64), bias[cols],
                   "gelu", "two-region")


def test_linear_helper(mkp):
    """mkp.linear: a . w^T + bias through gelu, the weight kept N x K."""
    import torch

    rng = np.random.default_rng(77)
    M, N, K = 100, 3 * 96, 200
    a = rand_bits(rng, (M, K))
    w = rand_bits(rng, (N, K))
    bias = rng.uniform(-1, 1, size=N).astype(np.float32)
    print("[case] linear helper", flush=True)
    ta = torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    tw = torch.from_numpy(w.view(np.int16)).cuda().view(torch.bfloat16)
    out = mkp.linear(ta, tw, torch.from_numpy(bias).cuda(), "gelu")
    torch.cuda.synchronize()
    acc, acc_abs = oracle.gemm(a, np.ascontiguousarray(w.T), with_abs=True)
    check_epilogue(out.cpu().numpy().astype(np.float64), acc, acc_abs, K, 1.0, 0.0, None, bias, "gelu", "linear")
