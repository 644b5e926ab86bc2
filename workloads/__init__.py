"""Seeded synthetic inputs for the dynamic-shape GEMM workloads.

This module holds no GEMM arithmetic: it draws shapes and values from numpy's
PCG64 generator and rounds fp32 draws to bf16 bit patterns (round to nearest,
ties to even).  Both the CPU oracle and the HIP path consume the same uint16
arrays it returns, so parity never depends on how either side would round.

Workload recipes (shapes and value laws) follow the dynamic-shape scenarios of
the MikPoly page (section 2, dynamic sequence length / batch size) and the
shape pair of its Introduction table; see the design doc for the full recipe.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import List, Tuple

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "GemmCase",
    "config_cases",
    "make_operands",
    "make_a",
    "make_b",
    "CONFIG_NAMES",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class GemmCase:
    """One (batched) GEMM call C = A.B with row-major operands.

    ``law_a``/``law_b`` name the value distribution: ``("uniform", lo, hi)`` or
    ``("normal", mean, std)``.  ``seed`` is a tuple fed to numpy's SeedSequence
    so each case regenerates independently of the others.
    """

    M: int
    N: int
    K: int
    batch: int
    law_a: tuple
    law_b: tuple
    seed_a: tuple
    seed_b: tuple
    tag: str = ""

    @property
    def flops(self) -> int:
        return 2 * self.batch * self.M * self.N * self.K

    @property
    def bytes(self) -> int:
        return self.batch * (2 * self.M * self.K + 2 * self.K * self.N + 4 * self.M * self.N)


CONFIG_NAMES = {
    1: "single GEMM (105,256,512)",
    2: "encoder linears, 64 GEMMs, M=16L, L~U{1..512}",
    3: "irregular vs square pair (105,1024,12544) and (4096,4096,4096)",
    4: "skinny-M decoder projections, 128 GEMMs, M~U{1..256}",
    5: "batched per-head scores, 32 calls of 48x(S,S,64), S~U{17..509}",
}

_U11 = ("uniform", -1.0, 1.0)


def config_cases(cfg: int) -> List[GemmCase]:
    """Shapes of the five synthetic workloads, drawn first from the config seed."""
    if cfg == 1:
        return [GemmCase(105, 256, 512, 1, _U11, _U11, (101, 0, 0), (101, 0, 1), "c1")]
    if cfg == 2:
        rng = np.random.default_rng(102)
        L = rng.integers(1, 512, size=64, endpoint=True)
        nk = [(2304, 768), (768, 768), (3072, 768), (768, 3072)]
        out = []
        for i in range(64):
            n, k = nk[i % 4]
            out.append(GemmCase(int(16 * L[i]), n, k, 1, _U11, _U11, (102, i, 0), (102, i, 1), f"c2[{i}]"))
        return out
    if cfg == 3:
        return [
            GemmCase(105, 1024, 12544, 1, _U11, _U11, (103, 0, 0), (103, 0, 1), "c3[irregular]"),
            GemmCase(4096, 4096, 4096, 1, _U11, _U11, (103, 1, 0), (103, 1, 1), "c3[square]"),
        ]
    if cfg == 4:
        rng = np.random.default_rng(104)
        Ms = rng.integers(1, 256, size=128, endpoint=True)
        nk = [(4096, 4096), (11008, 4096), (4096, 11008)]
        out = []
        for i in range(128):
            n, k = nk[i % 3]
            # one weight matrix per (N,K) projection, shared by every decode step
            out.append(GemmCase(int(Ms[i]), n, k, 1, ("normal", 0.0, 1.0), ("normal", 0.0, 0.02),
                                (104, i, 0), (104, 1000 + i % 3, 1), f"c4[{i}]"))
        return out
    if cfg == 5:
        rng = np.random.default_rng(105)
        S = rng.integers(17, 509, size=32, endpoint=True)
        law = ("normal", 0.0, 1.0)
        return [GemmCase(int(s), int(s), 64, 48, law, law, (105, i, 0), (105, i, 1), f"c5[{i}]")
                for i, s in enumerate(S)]
    raise ValueError(f"unknown config {cfg}")


def _draw(law: tuple, seed: tuple, count: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed))))
    kind = law[0]
    if kind == "uniform":
        v = rng.uniform(law[1], law[2], size=count).astype(np.float32)
    elif kind == "normal":
        v = rng.normal(law[1], law[2], size=count).astype(np.float32)
    else:
        raise ValueError(kind)
    return f32_to_bf16_bits(v)


def make_a(case: GemmCase) -> np.ndarray:
    """Packed bf16 bits of A, shape (batch, M, K), row-major."""
    return _draw(case.law_a, case.seed_a, case.batch * case.M * case.K).reshape(case.batch, case.M, case.K)


def make_b(case: GemmCase) -> np.ndarray:
    """Packed bf16 bits of B, shape (batch, K, N), row-major."""
    return _draw(case.law_b, case.seed_b, case.batch * case.K * case.N).reshape(case.batch, case.K, case.N)


def make_operands(case: GemmCase) -> Tuple[np.ndarray, np.ndarray]:
    """Packed bf16 bit arrays A (batch, M, K) and B (batch, K, N), row-major.

    Batch entries are contiguous: strides M*K for A and K*N for B.
    """
    return make_a(case), make_b(case)


def digest(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()[:16]


# ---- convolution sweep -------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class ConvCase:
    """One convolution call: NHWC input, KRSC filters, NPQK output."""
    N: int
    H: int
    W: int
    C: int
    K: int
    R: int
    S: int
    stride: int
    pad: int
    seed_x: tuple
    seed_w: tuple
    tag: str

    @property
    def P(self) -> int:
        return (self.H + 2 * self.pad - self.R) // self.stride + 1

    @property
    def Q(self) -> int:
        return (self.W + 2 * self.pad - self.S) // self.stride + 1

    # the GEMM view: M = N P Q, N = K, K = R S C
    @property
    def M(self) -> int:
        return self.N * self.P * self.Q

    @property
    def Kg(self) -> int:
        return self.R * self.S * self.C

    batch = 1

    @property
    def flops(self) -> int:
        return 2 * self.M * self.K * self.Kg

    @property
    def bytes(self) -> int:
        # input, filters and output once each
        return 2 * self.N * self.H * self.W * self.C + 2 * self.K * self.Kg + 4 * self.M * self.K


# Distinct convolution layers of a ResNet-50 (bottleneck blocks, stride on the
# 3 x 3 convolution, 224 x 224 input): (H, C, K, R, stride, pad).
RESNET50_LAYERS = [
    (224, 3, 64, 7, 2, 3),                                                   # stem
    (56, 64, 64, 1, 1, 0), (56, 64, 64, 3, 1, 1), (56, 64, 256, 1, 1, 0), (56, 256, 64, 1, 1, 0),
    (56, 256, 128, 1, 1, 0), (56, 128, 128, 3, 2, 1), (28, 128, 512, 1, 1, 0), (56, 256, 512, 1, 2, 0),
    (28, 512, 128, 1, 1, 0), (28, 128, 128, 3, 1, 1),
    (28, 512, 256, 1, 1, 0), (28, 256, 256, 3, 2, 1), (14, 256, 1024, 1, 1, 0), (28, 512, 1024, 1, 2, 0),
    (14, 1024, 256, 1, 1, 0), (14, 256, 256, 3, 1, 1),
    (14, 1024, 512, 1, 1, 0), (14, 512, 512, 3, 2, 1), (7, 512, 2048, 1, 1, 0), (14, 1024, 2048, 1, 2, 0),
    (7, 2048, 512, 1, 1, 0), (7, 512, 512, 3, 1, 1),
]

CONV_NAME = "ResNet-50 conv layers (23 distinct), batch N~U{1..32} per call, NHWC bf16"


def conv_cases() -> List[ConvCase]:
    """Every distinct ResNet-50 convolution once, each with its own batch
    size drawn from seed 106 (the dynamic dimension of CNN inference)."""
    rng = np.random.default_rng(106)
    Ns = rng.integers(1, 32, size=len(RESNET50_LAYERS), endpoint=True)
    out = []
    for i, ((H, C, K, R, stride, pad), N) in enumerate(zip(RESNET50_LAYERS, Ns)):
        out.append(ConvCase(int(N), H, H, C, K, R, R, stride, pad, (106, i, 0), (106, i, 1), f"conv[{i}]"))
    return out


def make_conv_operands(case: ConvCase) -> Tuple[np.ndarray, np.ndarray]:
    """bf16 bits of x (N,H,W,C) ~ U[-1,1] and w (K,R,S,C) ~ U[-1,1]."""
    x = _draw(_U11, case.seed_x, case.N * case.H * case.W * case.C).reshape(case.N, case.H, case.W, case.C)
    w = _draw(_U11, case.seed_w, case.K * case.R * case.S * case.C).reshape(case.K, case.R, case.S, case.C)
    return x, w
