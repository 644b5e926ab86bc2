"""Oracle of the fused GEMM epilogue (test infrastructure only).

Bolt page, "Enabling deeper operator fusion" (epilogue fusion) and its
persistent-kernel section, which writes each GEMM as D = alpha.A.W + beta.C;
the activation follows.  Here, in binary64 on top of the oracle product:

    out = act(alpha * (A.B) + beta * C_old + bias[n])

Activations, from their definitions:
  relu(x)      = max(x, 0)
  gelu(x)      = x * Phi(x), Phi(x) = (1 + erf(x / sqrt 2)) / 2, the standard
                 normal distribution function
  gelu_tanh(x) = x/2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3))), the tanh
                 approximation of x * Phi(x)
  silu(x)      = x * sigmoid(x) = x / (1 + exp(-x))
"""
from __future__ import annotations

import math

import numpy as np

ACT_CODES = {"none": 0, "relu": 1, "gelu": 2, "gelu_tanh": 3, "silu": 4}

# sup |act'(x)|, for propagating an input error through the activation:
# gelu' = Phi + x phi peaks at x = sqrt 2 (1.1289); the tanh form at 1.1289
# to 4 digits; silu' = s (1 + x (1 - s)) peaks near x = 2.40 (1.0998)
LIPSCHITZ = {"none": 1.0, "relu": 1.0, "gelu": 1.13, "gelu_tanh": 1.13, "silu": 1.10}

_erf = np.vectorize(math.erf, otypes=[np.float64])


def activation(name: str, x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    if name == "none":
        return x.copy()
    if name == "relu":
        return np.where(x > 0.0, x, 0.0)
    if name == "gelu":
        return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))
    if name == "gelu_tanh":
        return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))
    if name == "silu":
        with np.errstate(over="ignore"):
            return x / (1.0 + np.exp(-x))
    raise ValueError(name)


def epilogue(acc: np.ndarray, alpha: float = 1.0, beta: float = 0.0, c_old=None, bias=None,
             act: str = "none") -> np.ndarray:
    """act(alpha * acc + beta * c_old + bias) in binary64; acc (..., M, N),
    bias (N,) broadcast over rows, c_old read only when beta != 0."""
    v = float(alpha) * np.asarray(acc, dtype=np.float64)
    if beta != 0.0:
        v = v + float(beta) * np.asarray(c_old, dtype=np.float64)
    if bias is not None:
        v = v + np.asarray(bias, dtype=np.float64)
    return activation(act, v)


def pre_activation(acc, alpha=1.0, beta=0.0, c_old=None, bias=None) -> np.ndarray:
    return epilogue(acc, alpha, beta, c_old, bias, "none")
