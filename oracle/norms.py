"""Residual add followed by LayerNorm or RMSNorm over the last axis, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests and the bench's
cpu_baseline leg, never by the GPU library.

Definitions followed ([SNS] section 5, "the numerical problems of LayerNorm and RMSNorm"):

    LayerNorm:  y = (h - mu) / sqrt(var + eps) * gamma + beta,
                mu = mean(h), var = mean((h - mu)^2)       (over the hidden dimension)
    RMSNorm:    y = h / sqrt(mean(h^2) + eps) * gamma

The same section recommends 16-bit inputs and outputs with 32-bit statistics, a stable
variance algorithm, and fusing the residual add, the normalisation and the type
conversion into one pass.  Readings taken where it is silent: the
fused operation first forms h = x + residual, returns h (the updated residual stream)
next to y, and normalises h; the variance is the biased one (divided by the row length,
as in the formula); gamma and beta are per-column vectors.  Here h is the exact sum of
the float64 upcasts and every statistic is computed from it in float64.
"""

import numpy as np

from .attention import _as_f64


def residual_sum(x, residual=None):
    """h = x + residual (exactly, in float64); residual None means h = x."""
    h = _as_f64(x)
    if residual is not None:
        r = _as_f64(residual)
        if r.shape != h.shape:
            raise ValueError("x and residual must have the same shape")
        h = h + r
    return h


def layer_norm(x, gamma, beta, eps, residual=None):
    """(y, h) for LayerNorm of h = x + residual over the last axis."""
    h = residual_sum(x, residual)
    g, b = _as_f64(gamma), _as_f64(beta)
    if g.shape != h.shape[-1:] or b.shape != h.shape[-1:]:
        raise ValueError("gamma and beta must have the row length")
    mu = np.mean(h, axis=-1, keepdims=True)
    var = np.mean((h - mu) ** 2, axis=-1, keepdims=True)
    return (h - mu) / np.sqrt(var + float(eps)) * g + b, h


def rms_norm(x, gamma, eps, residual=None):
    """(y, h) for RMSNorm of h = x + residual over the last axis."""
    h = residual_sum(x, residual)
    g = _as_f64(gamma)
    if g.shape != h.shape[-1:]:
        raise ValueError("gamma must have the row length")
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + float(eps)) * g, h
