"""Pins for the residual + LayerNorm / RMSNorm oracle (float64).

Each check takes the implementation under test and also runs on copies with a planted
mistake (unbiased variance, eps dropped, LayerNorm without centring, RMSNorm without the
square root, residual ignored) that must fail at least one check.
"""

from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads


def _rand(shape, seed, sd=1.0):
    return workloads.generator(seed).normal(0.0, sd, size=shape)


def check_torch_layer_norm(ln):
    """torch.nn.functional.layer_norm in float64 (library routine)."""
    for rows, cols, eps in ((5, 17, 1e-5), (3, 1024, 1e-6), (2, 1, 1e-5)):
        x, r = _rand((rows, cols), cols), _rand((rows, cols), cols + 1)
        g, b = _rand((cols,), 2), _rand((cols,), 3)
        y, h = ln(x, g, b, eps, residual=r)
        ref = F.layer_norm(torch.from_numpy(x + r), (cols,), torch.from_numpy(g), torch.from_numpy(b), eps)
        if not (np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12) and np.array_equal(h, x + r)):
            return False
    return True


def check_torch_rms_norm(rms):
    """torch.nn.functional.rms_norm in float64 (library routine)."""
    for rows, cols, eps in ((5, 17, 1e-5), (3, 1024, 1e-6)):
        x, r = _rand((rows, cols), cols + 7), _rand((rows, cols), cols + 8)
        g = _rand((cols,), 4)
        y, h = rms(x, g, eps, residual=r)
        ref = F.rms_norm(torch.from_numpy(x + r), (cols,), torch.from_numpy(g), eps)
        if not (np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12) and np.array_equal(h, x + r)):
            return False
    return True


def check_decimal(ln, rms):
    """A 6-element row against a 50-digit decimal evaluation of both formulas."""
    getcontext().prec = 50
    x = _rand((1, 6), 11)
    g, b = _rand((6,), 12), _rand((6,), 13)
    eps = 1e-3
    xs = [Decimal(float(v)) for v in x[0]]
    n = Decimal(6)
    mu = sum(xs) / n
    var = sum((v - mu) ** 2 for v in xs) / n
    ln_ref = [float((v - mu) / (var + Decimal(eps)).sqrt() * Decimal(float(gi)) + Decimal(float(bi)))
              for v, gi, bi in zip(xs, g, b)]
    ms = sum(v * v for v in xs) / n
    rms_ref = [float(v / (ms + Decimal(eps)).sqrt() * Decimal(float(gi))) for v, gi in zip(xs, g)]
    y1, _ = ln(x, g, b, eps)
    y2, _ = rms(x, g, eps)
    return np.allclose(y1[0], ln_ref, rtol=1e-14, atol=1e-15) and np.allclose(y2[0], rms_ref, rtol=1e-14, atol=1e-15)


def check_closed_forms(ln, rms):
    cols = 64
    g, b = _rand((cols,), 21), _rand((cols,), 22)
    # a constant row has no deviation: LayerNorm returns beta exactly
    c = np.full((1, cols), 3.5)
    y, _ = ln(c, g, b, 1e-5)
    if not np.allclose(y[0], b, rtol=0, atol=1e-15):
        return False
    # RMSNorm of a constant row c: c / sqrt(c^2 + eps) * gamma
    y, _ = rms(c, g, 1e-5)
    if not np.allclose(y[0], 3.5 / np.sqrt(3.5 ** 2 + 1e-5) * g, rtol=1e-14):
        return False
    # with eps = 0: LayerNorm ignores a shift and a positive scale, RMSNorm a positive scale
    x = _rand((3, cols), 23)
    y0, _ = ln(x, g, b, 0.0)
    y1, _ = ln(2.5 * x + 7.0, g, b, 0.0)
    y2, _ = rms(x, g, 0.0)
    y3, _ = rms(4.0 * x, g, 0.0)
    if not (np.allclose(y0, y1, rtol=1e-12, atol=1e-12) and np.allclose(y2, y3, rtol=1e-13)):
        return False
    # unit gamma, zero beta: LayerNorm rows have mean 0 and mean square var/(var+eps);
    # RMSNorm rows have mean square ms/(ms+eps)
    ones, zeros = np.ones(cols), np.zeros(cols)
    y, _ = ln(x, ones, zeros, 0.25)
    var = x.var(axis=1)
    if not (np.allclose(y.mean(axis=1), 0, atol=1e-14) and np.allclose((y ** 2).mean(axis=1), var / (var + 0.25))):
        return False
    y, _ = rms(x, ones, 0.25)
    ms = (x ** 2).mean(axis=1)
    return np.allclose((y ** 2).mean(axis=1), ms / (ms + 0.25), rtol=1e-13)


def test_layer_norm_matches_torch():
    assert check_torch_layer_norm(oracle.layer_norm)


def test_rms_norm_matches_torch():
    assert check_torch_rms_norm(oracle.rms_norm)


def test_norms_decimal():
    assert check_decimal(oracle.layer_norm, oracle.rms_norm)


def test_norms_closed_forms():
    assert check_closed_forms(oracle.layer_norm, oracle.rms_norm)


def test_residual_optional_and_exact():
    x = workloads.attention_inputs(1, 1, 8, 64, seed=3)[0][0, 0]   # bf16 [8, 64]
    r = workloads.attention_inputs(1, 1, 8, 64, seed=4)[0][0, 0]
    h = oracle.residual_sum(x, r)
    assert np.array_equal(h, x.double().numpy() + r.double().numpy())
    y1, h1 = oracle.rms_norm(x, np.ones(64), 1e-5)
    assert np.array_equal(h1, x.double().numpy())
    with pytest.raises(ValueError):
        oracle.rms_norm(x, np.ones(63), 1e-5)


# --------------------------------------------------------------------------
# Planted mistakes
# --------------------------------------------------------------------------

def _ln_unbiased(x, g, b, eps, residual=None):
    h = oracle.residual_sum(x, residual)
    mu = h.mean(-1, keepdims=True)
    var = h.var(-1, ddof=1, keepdims=True)      # mistake: divides by n - 1
    return (h - mu) / np.sqrt(var + eps) * g + b, h


def _ln_no_eps(x, g, b, eps, residual=None):
    return oracle.layer_norm(x, g, b, 0.0, residual)


def _ln_uncentred(x, g, b, eps, residual=None):
    h = oracle.residual_sum(x, residual)
    var = h.var(-1, keepdims=True)
    return h / np.sqrt(var + eps) * g + b, h    # mistake: no mean subtraction


def _ln_no_residual(x, g, b, eps, residual=None):
    y, _ = oracle.layer_norm(x, g, b, eps)       # mistake: residual ignored
    return y, oracle.residual_sum(x, residual)


def _rms_no_sqrt(x, g, eps, residual=None):
    h = oracle.residual_sum(x, residual)
    return h / (np.mean(h * h, -1, keepdims=True) + eps) * g, h


def _rms_no_eps(x, g, eps, residual=None):
    return oracle.rms_norm(x, g, 0.0, residual)


def _rms_mean_centred(x, g, eps, residual=None):
    h = oracle.residual_sum(x, residual)
    c = h - h.mean(-1, keepdims=True)            # mistake: centres like LayerNorm
    return c / np.sqrt(np.mean(c * c, -1, keepdims=True) + eps) * g, h


def _fails(checks):
    with np.errstate(all="ignore"):
        res = []
        for c in checks:
            try:
                res.append(c())
            except Exception:
                res.append(False)
    return not all(res)


@pytest.mark.parametrize("mut", [_ln_unbiased, _ln_no_eps, _ln_uncentred, _ln_no_residual])
def test_pins_catch_layer_norm_mutants(mut):
    assert _fails([lambda: check_torch_layer_norm(mut), lambda: check_decimal(mut, oracle.rms_norm),
                   lambda: check_closed_forms(mut, oracle.rms_norm)])


@pytest.mark.parametrize("mut", [_rms_no_sqrt, _rms_no_eps, _rms_mean_centred])
def test_pins_catch_rms_norm_mutants(mut):
    assert _fails([lambda: check_torch_rms_norm(mut), lambda: check_decimal(oracle.layer_norm, mut),
                   lambda: check_closed_forms(oracle.layer_norm, mut)])
