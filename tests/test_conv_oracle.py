"""Pins of the convolution oracle (oracle/conv.py): the definition by loops,
the 1 x 1 case as the GEMM oracle, a one-hot filter that copies a shifted
input channel, and all-ones operands whose output counts the in-image taps."""
import numpy as np
import pytest

import oracle
from oracle import conv as cv
from workloads import f32_to_bf16_bits


def bits(rng, shape, lo=-1, hi=1):
    return f32_to_bf16_bits(rng.uniform(lo, hi, size=shape).astype(np.float32))


GEOMS = [((1, 1), (0, 0), (1, 1)), ((1, 1), (1, 1), (1, 1)), ((2, 2), (1, 0), (1, 1)), ((1, 2), (2, 1), (2, 1)),
         ((3, 1), (0, 2), (1, 3))]


@pytest.mark.parametrize("geom", GEOMS)
def test_matches_loops(geom):
    stride, pad, dil = geom
    rng = np.random.default_rng(hash(geom) & 0xFFFF)
    x = bits(rng, (2, 7, 6, 3))
    w = bits(rng, (4, 3, 2, 3))
    a = cv.conv2d(x, w, stride, pad, dil)
    b = cv.conv2d_loops(x, w, stride, pad, dil)
    assert a.shape == b.shape
    assert np.allclose(a, b, rtol=1e-13, atol=1e-13)


def test_one_by_one_is_gemm():
    rng = np.random.default_rng(1)
    x = bits(rng, (3, 5, 4, 24))
    w = bits(rng, (10, 1, 1, 24))
    y = cv.conv2d(x, w)
    g = oracle.gemm(x.reshape(-1, 24), np.ascontiguousarray(w.reshape(10, 24).T))
    assert np.allclose(y.reshape(-1, 10), g, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("geom", GEOMS)
def test_one_hot_filter_copies_input(geom):
    """w[k][r0][s0][c0] = 1 (others 0): y[..., k] is input channel c0 at the
    position tap (r0, s0) reads, zero where that falls outside the image."""
    stride, pad, dil = geom
    rng = np.random.default_rng(2)
    N, H, W, C, K, R, S = 2, 8, 7, 5, 3, 3, 2
    x = bits(rng, (N, H, W, C))
    w = np.zeros((K, R, S, C), np.uint16)
    picks = [(0, 0, 0, 1), (1, 2, 1, 4), (2, 1, 0, 0)]
    for k, r, s, c in picks:
        w[k, r, s, c] = 0x3F80   # 1.0 in bf16
    y = cv.conv2d(x, w, stride, pad, dil)
    xf = cv.bf16_to_f64(x)
    P, Q = y.shape[1:3]
    for k, r, s, c in picks:
        for p in range(P):
            for q in range(Q):
                h, ww = p * stride[0] - pad[0] + r * dil[0], q * stride[1] - pad[1] + s * dil[1]
                want = xf[:, h, ww, c] if (0 <= h < H and 0 <= ww < W) else 0.0
                assert np.array_equal(y[:, p, q, k], np.broadcast_to(want, (N,)))


def test_all_ones_counts_taps():
    """All-ones operands: every output is C times the number of filter taps
    that land inside the image -- (R S C) in the interior, fewer at the
    padded border."""
    N, H, W, C, K, R, S = 1, 6, 5, 4, 2, 3, 3
    x = np.full((N, H, W, C), 0x3F80, np.uint16)
    w = np.full((K, R, S, C), 0x3F80, np.uint16)
    y = cv.conv2d(x, w, (1, 1), (1, 1), (1, 1))
    assert y.shape == (N, H, W, K)
    for p in range(H):
        for q in range(W):
            rows = sum(1 for r in range(R) if 0 <= p - 1 + r < H)
            cols = sum(1 for s in range(S) if 0 <= q - 1 + s < W)
            assert np.all(y[0, p, q] == rows * cols * C)
    assert y[0, 2, 2, 0] == R * S * C and y[0, 0, 0, 0] == 4 * C


def test_output_size():
    assert cv.out_size(224, 7, 2, 3, 1) == 112      # the classic 7x7 stride-2 stem
    assert cv.out_size(56, 3, 1, 1, 1) == 56
    assert cv.out_size(56, 1, 2, 0, 1) == 28
    assert cv.out_size(9, 3, 1, 2, 2) == 9
