"""The allocation-free entry point (for callers that cannot allocate device
memory) against the allocating one, through the C-ABI: the same products
within the parity tolerance, on two calls in a row, the second smaller,
with split-K partials and a transposed B living in the library's fixed
scratch array, and on a shape whose usual plan would not fit in it."""
import numpy as np
import pytest

import oracle
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

from _gpu_util import assert_close, dev_bf16  # noqa: E402


@pytest.fixture(scope="module")
def mkp(gpu):
    import dynamic_shape_gemm_amd as m

    m.mkp_load_calibration(None)
    for k, v in (("force_kernel", ""), ("force_splitk", 0), ("transpose_b", 1), ("fused_reduce", 0)):
        m.mkp_set_option(k, v)
    return m


def bits(rng, shape):
    return f32_to_bf16_bits(rng.uniform(-1, 1, size=shape).astype(np.float32))


def both(mkp, a, b):
    """(allocation-free result, allocating result, oracle, |a b| sums) of one batched call."""
    import torch

    batch, M, K = a.shape
    N = b.shape[2]
    ta, pa = dev_bf16(a)
    tb, pb = dev_bf16(b)
    c0 = torch.full((batch * M * N + 64,), float("nan"), dtype=torch.float32, device="cuda")
    c1 = torch.full((batch * M * N + 64,), float("nan"), dtype=torch.float32, device="cuda")
    mkp.mkp_gemm_batched_noalloc(batch, M, N, K, pa, K, M * K, pb, N, K * N, c0.data_ptr(), N, M * N)
    mkp.mkp_gemm_batched(batch, M, N, K, pa, K, M * K, pb, N, K * N, c1.data_ptr(), N, M * N)
    torch.cuda.synchronize()
    h0, h1 = c0.cpu().numpy(), c1.cpu().numpy()
    assert np.isnan(h0[batch * M * N:]).all() and np.isnan(h1[batch * M * N:]).all(), "write beyond C"
    ref, refabs = oracle.gemm(a, b, with_abs=True)
    shape = (batch, M, N)
    return h0[:batch * M * N].reshape(shape), h1[:batch * M * N].reshape(shape), ref, refabs


def check(mkp, rng, batch, M, N, K, what):
    print(f"[case] no-alloc {what} batch={batch} M={M} N={N} K={K}", flush=True)
    a, b = bits(rng, (batch, M, K)), bits(rng, (batch, K, N))
    got, usual, ref, refabs = both(mkp, a, b)
    for z in range(batch):
        # the allocation-free call against the allocating one, to the parity bar
        assert_close(got[z].astype(np.float64), usual[z].astype(np.float64), refabs[z], K, f"{what} vs usual [{z}]")
        assert_close(got[z].astype(np.float64), ref[z], refabs[z], K, f"{what} vs oracle [{z}]")


def test_noalloc_matches_allocating_call(mkp):
    rng = np.random.default_rng(2718)
    assert mkp.mkp_noalloc_scratch_bytes() == 64 << 20
    try:
        # split-K partials and a transposed B in the scratch array, two
        # calls in a row, the second smaller
        mkp.mkp_set_option("force_splitk", 4)
        mkp.mkp_set_option("transpose_b", 2)
        check(mkp, rng, 3, 300, 700, 2000, "split 4, transposed B")
        check(mkp, rng, 2, 77, 130, 600, "split 4, transposed B, smaller")
        mkp.mkp_set_option("transpose_b", 1)
        mkp.mkp_set_option("force_splitk", 8)
        check(mkp, rng, 1, 500, 900, 4096, "split 8")
        check(mkp, rng, 1, 40, 64, 1024, "split 8, smaller")
        mkp.mkp_set_option("force_splitk", 0)
        # a plan whose partials would exceed the scratch (16 splits of a
        # 1024 x 4096 fp32 tile = 256 MiB) is replaced by one that fits
        mkp.mkp_set_option("force_splitk", 16)
        check(mkp, rng, 1, 1024, 4096, 4096, "usual plan too large for the scratch")
        check(mkp, rng, 1, 96, 200, 1100, "after it, smaller")
    finally:
        mkp.mkp_set_option("force_splitk", 0)
        mkp.mkp_set_option("transpose_b", 1)


def test_noalloc_argument_errors(mkp):
    # errors come back before anything is launched, as for the allocating call
    assert mkp._lib.mkp_gemm_batched_noalloc(2, 4, 4, 8, 1, 7, 32, 1, 4, 32, 1, 4, 16, None) == mkp.MKP_ERR_INVALID_ARG
    assert "lda < K" in mkp.last_error()
    assert mkp._lib.mkp_gemm_batched_noalloc(0, 4, 4, 8, 0, 8, 0, 0, 4, 0, 0, 4, 0, None) == mkp.MKP_OK
