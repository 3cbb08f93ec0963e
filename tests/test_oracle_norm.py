"""Pins of the RMSNorm oracle (oracle/norm.py) against closed forms and
invariants that do not go through its own code path."""
import math

import numpy as np
import pytest

from oracle import mx as omx
from oracle import norm


def _bf16(a):
    """Round float64 values to bf16 (RNE) and back."""
    f = np.asarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def test_constant_row_gives_the_gain_exactly():
    # x_d = 3: mean square 9, rstd = fl32(1/3), fl32(3 fl32(1/3)) = 1, so y = gamma exactly
    rng = np.random.default_rng(0)
    gamma = rng.standard_normal(128).astype(np.float32).astype(np.float64)
    x = np.full((2, 128), 3.0)
    y = norm.rmsnorm(x, gamma, 0.0)
    assert np.array_equal(y, np.broadcast_to(gamma, y.shape))


def test_power_of_two_scaling_is_exact():
    rng = np.random.default_rng(1)
    x = _bf16(rng.standard_normal((16, 64)))
    gamma = (1 + 0.1 * rng.standard_normal(64)).astype(np.float32).astype(np.float64)
    y = norm.rmsnorm(x, gamma, 0.0)
    for k in (-20, -3, 5, 40):
        assert np.array_equal(norm.rmsnorm(x * 2.0 ** k, gamma, 0.0), y)


def test_unit_mean_square_and_textbook_formula():
    rng = np.random.default_rng(2)
    x = _bf16(rng.standard_normal((64, 128)) * 7.5)
    y = norm.rmsnorm(x, np.ones(128), 0.0)
    assert np.max(np.abs(np.mean(y * y, axis=1) - 1)) < 1e-6
    gamma = (1 + 0.1 * rng.standard_normal(128)).astype(np.float32).astype(np.float64)
    eps = 1e-5
    ref = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + float(np.float32(eps))) * gamma
    y = norm.rmsnorm(x, gamma, eps)
    assert np.max(np.abs(y - ref) / np.abs(ref).max()) < 4 * 2.0 ** -24


def test_epsilon_and_zero_rows():
    x = np.zeros((1, 64))
    assert np.array_equal(norm.rmsnorm(x, np.ones(64), 1e-6), x)
    x = np.full((1, 64), 0.5)
    # eps dominates: rstd ~ 1/sqrt(1e6) = 1e-3
    y = norm.rmsnorm(x, np.ones(64), 1e6)
    assert np.allclose(y, 0.5 / math.sqrt(0.25 + 1e6), rtol=1e-6)


def test_normalized_then_quantized_codes():
    # y = gamma (constant-row closed form), so the codes are the quantizer's codes of gamma
    gamma = np.array([1.5, -0.25, 448.0, 2.0 ** -9] * 16)
    x = np.full((1, 2, 1, 64), -2.0)   # sign flips y
    out = norm.rmsnorm_quantize(x, gamma, 0.0, layouts=("row32",))
    codes, k = out["row32"]
    ref_codes, ref_k = omx.quantize_row32(np.broadcast_to(-gamma, (1, 2, 1, 64)))
    assert np.array_equal(codes, ref_codes) and np.array_equal(k, ref_k)
