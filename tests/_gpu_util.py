"""Helpers for the GPU parity tests: device buffers with NaN guard bands,
runs through the C-ABI, and the comparison against the oracle."""
from __future__ import annotations

import math

import numpy as np

import oracle


def dev_bf16(bits: np.ndarray, offset_elems: int = 0):
    """Copy bf16 bits to the GPU; optionally shift the start by whole elements
    (to get pointers that are not 16-byte aligned).  Returns (tensor, address)."""
    import torch

    flat = np.ascontiguousarray(bits, dtype=np.uint16).reshape(-1)
    buf = np.zeros(flat.size + offset_elems + 8, dtype=np.uint16)
    buf[offset_elems:offset_elems + flat.size] = flat
    t = torch.from_numpy(buf.view(np.int16)).cuda()
    return t, t.data_ptr() + 2 * offset_elems


def padded(bits2d: np.ndarray, ld: int) -> np.ndarray:
    """Row-major copy with leading dimension ld >= columns (pad = 0x7FC0, a NaN)."""
    r, c = bits2d.shape
    out = np.full((r, ld), 0x7FC0, dtype=np.uint16)
    out[:, :c] = bits2d
    return out


class GuardedC:
    """fp32 output buffer of `rows` x `ld` per batch entry plus a guard band,
    pre-filled with NaN so holes and stray writes both show."""

    def __init__(self, batch: int, M: int, N: int, ld: int | None = None, guard: int = 64, offset: int = 0):
        import torch

        self.batch, self.M, self.N = batch, M, N
        self.ld = ld if ld is not None else N + 3
        self.stride = (M + 1) * self.ld
        self.offset = offset
        total = offset + batch * self.stride + guard * self.ld + guard
        self.t = torch.full((total,), float("nan"), dtype=torch.float32, device="cuda")
        self.addr = self.t.data_ptr() + 4 * offset

    def result(self):
        """(batch, M, N) float64 result, and whether every other element is untouched."""
        h = self.t.cpu().numpy()
        body = h[self.offset:self.offset + self.batch * self.stride].reshape(self.batch, M1 := self.M + 1, self.ld)
        c = body[:, :self.M, :self.N].astype(np.float64)
        mask = np.ones(h.shape, dtype=bool)
        for b in range(self.batch):
            base = self.offset + b * self.stride
            for i in range(self.M):
                mask[base + i * self.ld: base + i * self.ld + self.N] = False
        untouched = bool(np.isnan(h[mask]).all())
        return c, untouched


def tolerance(K: int) -> float:
    """Parity gate: |dC| <= 1e-3 * sqrt(K) per element."""
    return 1e-3 * math.sqrt(max(K, 1))


def assert_close(got: np.ndarray, ref: np.ndarray, refabs: np.ndarray, K: int, what: str = ""):
    assert np.isfinite(got).all(), f"{what}: non-finite output (hole or NaN)"
    err = np.abs(got - ref)
    tol = tolerance(K)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"{what}: max|dC| = {worst:.3e} > {tol:.3e}"
    # forward error bound of binary32 summation (2x slack for the MFMA's
    # internal adds); zero products must give exact zeros
    bound = oracle.error_bound(K, refabs) + 1e-30
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond the summation error bound"
    return worst
