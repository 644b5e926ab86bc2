"""Oracle of 2-D convolution (test infrastructure only).

The MikPoly page runs convolutions as GEMMs on its micro-kernels; what is
computed is the convolution itself, written here from its definition in
binary64 over the exact bf16 inputs (NHWC input, KRSC filters, NPQK output):

  y[n][p][q][k] = sum_{r < R, s < S, c < C}
                    x[n][p*sh - ph + r*dh][q*sw - pw + s*dw][c] * w[k][r][s][c]

with input positions outside the H x W image contributing zero.  `conv2d`
adds, per filter tap (r, s), the product of the shifted input window with
that tap's K x C filter slice (a matrix product as a library step);
`conv2d_loops` is the same sum by explicit loops, for tiny cases.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def out_size(H: int, R: int, stride: int, pad: int, dil: int) -> int:
    return (H + 2 * pad - dil * (R - 1) - 1) // stride + 1


def conv2d(x_bits, w_bits, stride=(1, 1), pad=(0, 0), dil=(1, 1), with_abs=False):
    """y (N,P,Q,K) in binary64 (and sum |x*w| over the same terms if with_abs)."""
    x = bf16_to_f64(x_bits)
    wt = bf16_to_f64(w_bits)
    N, H, W, C = x.shape
    K, R, S, C2 = wt.shape
    assert C2 == C
    sh, sw = stride
    ph, pw = pad
    dh, dw = dil
    P, Q = out_size(H, R, sh, ph, dh), out_size(W, S, sw, pw, dw)
    xp = np.zeros((N, H + 2 * ph, W + 2 * pw, C))
    xp[:, ph:ph + H, pw:pw + W, :] = x
    y = np.zeros((N, P, Q, K))
    ya = np.zeros((N, P, Q, K)) if with_abs else None
    for r in range(R):
        for s in range(S):
            h0, w0 = r * dh, s * dw
            win = xp[:, h0:h0 + sh * (P - 1) + 1:sh, w0:w0 + sw * (Q - 1) + 1:sw, :]   # (N,P,Q,C)
            y += win @ wt[:, r, s, :].T
            if with_abs:
                ya += np.abs(win) @ np.abs(wt[:, r, s, :]).T
    return (y, ya) if with_abs else y


def conv2d_loops(x_bits, w_bits, stride=(1, 1), pad=(0, 0), dil=(1, 1)):
    """The same sum element by element (tiny cases only)."""
    x = bf16_to_f64(x_bits)
    wt = bf16_to_f64(w_bits)
    N, H, W, C = x.shape
    K, R, S, _ = wt.shape
    P, Q = out_size(H, R, stride[0], pad[0], dil[0]), out_size(W, S, stride[1], pad[1], dil[1])
    y = np.zeros((N, P, Q, K))
    for n in range(N):
        for p in range(P):
            for q in range(Q):
                for k in range(K):
                    acc = 0.0
                    for r in range(R):
                        for s in range(S):
                            h = p * stride[0] - pad[0] + r * dil[0]
                            ww = q * stride[1] - pad[1] + s * dil[1]
                            if 0 <= h < H and 0 <= ww < W:
                                for c in range(C):
                                    acc += x[n, h, ww, c] * wt[k, r, s, c]
                    y[n, p, q, k] = acc
    return y
