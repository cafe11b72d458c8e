"""Elementwise activations in float64 (test infrastructure; see ``oracle``).

GeLU is named but never written out on the pages ([HJ] MLP, single-card
forward; [TP1] row/column split).  Reading taken: the exact form
``GeLU(x) = x * Phi(x)`` with ``Phi`` the standard normal CDF, i.e.
``0.5 * x * (1 + erf(x / sqrt(2)))``; the tanh approximation is not used.

SwiGLU's formula was lost from [L11] section 3; its prose names the gate,
up and down projections.  Reading taken: the Llama form
``H = SiLU(X W_gate) * (X W_up)`` with ``SiLU(x) = x * sigmoid(x)``.
"""
import numpy as np
from scipy.special import erf, expit

_SQRT2 = np.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / np.sqrt(2.0 * np.pi)


def normal_cdf(x):
    return 0.5 * (1.0 + erf(np.asarray(x, dtype=np.float64) / _SQRT2))


def normal_pdf(x):
    x = np.asarray(x, dtype=np.float64)
    return _INV_SQRT_2PI * np.exp(-0.5 * x * x)


def gelu(x):
    x = np.asarray(x, dtype=np.float64)
    return x * normal_cdf(x)


def gelu_grad(x):
    """d/dx [x Phi(x)] = Phi(x) + x phi(x)."""
    x = np.asarray(x, dtype=np.float64)
    return normal_cdf(x) + x * normal_pdf(x)


def sigmoid(x):
    return expit(np.asarray(x, dtype=np.float64))


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def silu_grad(x):
    """d/dx [x sigma(x)] = sigma(x) (1 + x (1 - sigma(x)))."""
    x = np.asarray(x, dtype=np.float64)
    s = sigmoid(x)
    return s * (1.0 + x * (1.0 - s))
