"""GPU parity at the workloads' full sizes on every element.

The HIP path (through the C-ABI, in the launch configuration the benchmark
times: default options, the shipped table) against the binary64 oracle
over the same bf16 inputs, every element of C compared:

* both GEMMs of the irregular/square pair, (105, 1024, 12544) and 4096^3;
* one skinny-M decoder GEMM per (N, K) projection (the largest M drawn for
  it), each on its shared weight matrix;
* all 32 batched per-head score calls, every batch entry;
* one encoder-linear GEMM per (N, K) (the largest M drawn for it).

Gate per element: |dC| <= 1e-3 sqrt(K) and the binary32 summation bound.
C is pre-filled with NaN and followed by a NaN guard band.
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

from _gpu_util import assert_close, dev_bf16  # noqa: E402


@pytest.fixture(scope="module")
def mkp(gpu):
    import dynamic_shape_gemm_amd as m

    m.mkp_load_calibration(None)
    m.mkp_set_option("force_kernel", "")
    m.mkp_set_option("force_splitk", 0)
    m.mkp_set_option("patterns", "I,II")
    return m


def full_check(mkp, case, a, b):
    """One (batched) call of `case` on operands a (batch, M, K), b (batch, K, N);
    every element against the oracle."""
    import torch

    B, M, N, K = case.batch, case.M, case.N, case.K
    plan = mkp.mkp_plan_describe(B, M, N, K)
    desc = "+".join(f"{r['kernel']}/s{r['s']}" for r in plan["regions"])
    print(f"[case] full {case.tag} batch={B} M={M} N={N} K={K} plan {plan['pattern']} {desc}", flush=True)
    ta, pa = dev_bf16(a)
    tb, pb = dev_bf16(b)
    tc = torch.full((B * M * N + 1024,), float("nan"), dtype=torch.float32, device="cuda")
    if B == 1:
        mkp.mkp_gemm(M, N, K, pa, K, pb, N, tc.data_ptr(), N)
    else:
        mkp.mkp_gemm_batched(B, M, N, K, pa, K, M * K, pb, N, K * N, tc.data_ptr(), N, M * N)
    torch.cuda.synchronize()
    h = tc.cpu().numpy()
    assert np.isnan(h[B * M * N:]).all(), f"{case.tag}: write beyond C"
    got = h[:B * M * N].reshape(B, M, N).astype(np.float64)
    ref, refabs = oracle.gemm(a, b, with_abs=True)
    for z in range(B):
        assert_close(got[z], ref[z], refabs[z], K, f"{case.tag}[{z}]")
    del ta, tb, tc


def test_config3_every_element(mkp):
    for case in workloads.config_cases(3):
        a, b = workloads.make_operands(case)
        full_check(mkp, case, a, b)


def test_config4_every_element_per_projection(mkp):
    cases = workloads.config_cases(4)
    for nk in sorted({(c.N, c.K) for c in cases}):
        case = max((c for c in cases if (c.N, c.K) == nk), key=lambda c: c.M)
        full_check(mkp, case, workloads.make_a(case), workloads.make_b(case))
    # and the smallest M of each projection (the most split-K)
    for nk in sorted({(c.N, c.K) for c in cases}):
        case = min((c for c in cases if (c.N, c.K) == nk), key=lambda c: c.M)
        full_check(mkp, case, workloads.make_a(case), workloads.make_b(case))


def test_config5_every_call_every_element(mkp):
    for case in workloads.config_cases(5):
        a, b = workloads.make_operands(case)
        full_check(mkp, case, a, b)


def test_config2_every_element_per_shape_class(mkp):
    cases = workloads.config_cases(2)
    for nk in sorted({(c.N, c.K) for c in cases}):
        case = max((c for c in cases if (c.N, c.K) == nk), key=lambda c: c.M)
        a, b = workloads.make_operands(case)
        full_check(mkp, case, a, b)
