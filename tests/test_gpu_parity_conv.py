"""GPU parity of convolution as an implicit GEMM (mkp_conv2d): NHWC input,
KRSC filters, NPQK fp32 output, against the CPU oracle of the convolution's
definition (oracle/conv.py).  The gate is the GEMM's, with K = R S C:
|dy| <= 1e-3 sqrt(K) and the binary32 summation bound.  Every case prints
its geometry before it touches the GPU.
"""
import numpy as np
import pytest

from oracle import conv as ocv
from oracle import epilogue as ep
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

from _gpu_util import assert_close, dev_bf16  # noqa: E402


@pytest.fixture(scope="module")
def mkp(gpu):
    import dynamic_shape_gemm_amd as m

    m.mkp_load_calibration(None)
    m.mkp_set_option("force_kernel", "")
    m.mkp_set_option("force_splitk", 0)
    yield m
    m.mkp_set_option("force_kernel", "")
    m.mkp_set_option("force_splitk", 0)


def bits(rng, shape):
    return f32_to_bf16_bits(rng.uniform(-1, 1, size=shape).astype(np.float32))


def run_conv(mkp, x, w, stride=(1, 1), pad=(0, 0), dil=(1, 1), bias=None, act="none", offx=0, what=""):
    import torch

    N, H, W, C = x.shape
    K, R, S, _ = w.shape
    P, Q = ocv.out_size(H, R, stride[0], pad[0], dil[0]), ocv.out_size(W, S, stride[1], pad[1], dil[1])
    print(f"[case] conv {what} N={N} H={H} W={W} C={C} K={K} R={R} S={S} stride={stride} pad={pad} dil={dil} "
          f"P={P} Q={Q} act={act} bias={bias is not None} offx={offx}", flush=True)
    tx, px = dev_bf16(x, offx)
    tw, pw = dev_bf16(w)
    guard = 256
    ty = torch.full((N * P * Q * K + guard,), float("nan"), dtype=torch.float32, device="cuda")
    tb = torch.from_numpy(bias).cuda() if bias is not None else None
    mkp.mkp_conv2d(N, H, W, C, K, R, S, stride[0], stride[1], pad[0], pad[1], dil[0], dil[1], px, pw, ty, tb, act)
    torch.cuda.synchronize()
    h = ty.cpu().numpy()
    assert np.isnan(h[N * P * Q * K:]).all(), f"{what}: write beyond y"
    got = h[:N * P * Q * K].reshape(N, P, Q, K).astype(np.float64)
    ref, refabs = ocv.conv2d(x, w, stride, pad, dil, with_abs=True)
    Kg = R * S * C
    if bias is None and act == "none":
        assert_close(got.reshape(-1, K), ref.reshape(-1, K), refabs.reshape(-1, K), Kg, what)
    else:
        v = ep.pre_activation(ref, bias=bias)
        want = ep.activation(act, v)
        tol = ep.LIPSCHITZ[act] * (1e-3 * np.sqrt(Kg) + 4 * 2.0 ** -24 * (np.abs(ref) + np.abs(bias))) + \
            8 * 2.0 ** -24 * (np.abs(v) + np.abs(want))
        assert np.isfinite(got).all() and (np.abs(got - want) <= tol).all(), f"{what}: epilogue mismatch"
    return got


CASES = [
    # (N, H, W, C, K, R, S, stride, pad, dil)
    (2, 9, 9, 64, 80, 3, 3, (1, 1), (1, 1), (1, 1)),      # channels a multiple of 64: direct loads
    (3, 7, 6, 128, 64, 1, 1, (1, 1), (0, 0), (1, 1)),     # 1 x 1
    (2, 11, 10, 64, 96, 3, 3, (2, 2), (1, 1), (1, 1)),    # stride 2
    (1, 12, 9, 64, 40, 3, 2, (1, 2), (2, 0), (2, 1)),     # dilation, asymmetric
    (2, 8, 8, 40, 48, 3, 3, (1, 1), (1, 1), (1, 1)),      # C % 8 == 0: 8-channel gathers
    (2, 15, 15, 3, 64, 7, 7, (2, 2), (3, 3), (1, 1)),     # C = 3 (a stem): element gathers
    (1, 5, 5, 64, 17, 5, 5, (1, 1), (0, 0), (1, 1)),      # ragged K (output channels), one output row
    (4, 6, 6, 256, 300, 3, 3, (1, 1), (1, 1), (1, 1)),    # deep K
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_conv_geometries(mkp, case):
    N, H, W, C, K, R, S, stride, pad, dil = case
    rng = np.random.default_rng(sum(case[:7]))
    run_conv(mkp, bits(rng, (N, H, W, C)), bits(rng, (K, R, S, C)), stride, pad, dil, what="auto")


@pytest.mark.parametrize("C", [64, 40, 3])
def test_conv_each_kernel_forced(mkp, C):
    """The convolution form of every N x K tile that has one, on the direct-load (C = 64),
    8-channel (C = 40) and element (C = 3) paths."""
    rng = np.random.default_rng(C)
    x = bits(rng, (2, 9, 8, C))
    w = bits(rng, (70, 3, 3, C))
    try:
        # (the skinny tiles whose waves split K, uK = 256, have no convolution form)
        for name in [n for n in mkp.mkp_kernel_names() if n.endswith("_nk") and "k256" not in n]:
            mkp.mkp_set_option("force_kernel", name)
            run_conv(mkp, x, w, (1, 1), (1, 1), (1, 1), what=name)
    finally:
        mkp.mkp_set_option("force_kernel", "")


@pytest.mark.parametrize("s", [2, 5])
def test_conv_splitk(mkp, s):
    rng = np.random.default_rng(50 + s)
    try:
        mkp.mkp_set_option("force_splitk", s)
        run_conv(mkp, bits(rng, (2, 10, 10, 64)), bits(rng, (96, 3, 3, 64)), (1, 1), (1, 1), (1, 1), what=f"s={s}")
        run_conv(mkp, bits(rng, (1, 9, 7, 40)), bits(rng, (33, 3, 3, 40)), (2, 1), (1, 1), (1, 1), what=f"s={s}")
    finally:
        mkp.mkp_set_option("force_splitk", 0)


def test_conv_bias_relu_and_unaligned(mkp):
    rng = np.random.default_rng(77)
    x = bits(rng, (2, 9, 9, 64))
    w = bits(rng, (64, 3, 3, 64))
    bias = rng.uniform(-1, 1, size=64).astype(np.float32)
    run_conv(mkp, x, w, (1, 1), (1, 1), (1, 1), bias=bias, act="relu", what="bias relu")
    run_conv(mkp, x, w, (1, 1), (1, 1), (1, 1), bias=bias, act="silu", what="bias silu")
    # input not 16-byte aligned: element gathers
    run_conv(mkp, x, w, (1, 1), (1, 1), (1, 1), offx=1, what="unaligned x")


def test_conv_resnet_layer_full(mkp):
    """A 3 x 3, 64 -> 64 layer on 56 x 56 at batch 8 (M = 25088), every
    output checked."""
    rng = np.random.default_rng(9)
    run_conv(mkp, bits(rng, (8, 56, 56, 64)), bits(rng, (64, 3, 3, 64)), (1, 1), (1, 1), (1, 1), what="resnet 3x3")


def test_conv_torch_helper(mkp):
    import torch

    rng = np.random.default_rng(4)
    x = bits(rng, (2, 10, 10, 64))
    w = bits(rng, (32, 3, 3, 64))
    print("[case] conv2d helper", flush=True)
    tx = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    tw = torch.from_numpy(w.view(np.int16)).cuda().view(torch.bfloat16)
    y = mkp.conv2d(tx, tw, stride=2, padding=1)
    torch.cuda.synchronize()
    ref, refabs = ocv.conv2d(x, w, (2, 2), (1, 1), (1, 1), with_abs=True)
    assert tuple(y.shape) == ref.shape
    assert_close(y.cpu().numpy().astype(np.float64).reshape(-1, 32), ref.reshape(-1, 32), refabs.reshape(-1, 32),
                 9 * 64, "helper")
