"""Pins of the RMSNorm oracle (oracle/rmsnorm.py) to closed forms and
invariants, and planted mistakes that those pins must reject."""
import numpy as np
import pytest

from oracle.rmsnorm import rms_norm


def pins(f):
    """Run every pin on the function f(x, weight, eps); raises on a miss."""
    rng = np.random.default_rng(5)
    D = 96
    # constant row c: y = c * w / sqrt(c^2 + eps)
    for c, eps in ((0.75, 1e-6), (-3.0, 0.5), (1e-3, 1e-2)):
        w = rng.standard_normal(D)
        y = f(np.full((1, D), c), w, eps)
        np.testing.assert_allclose(y[0], c * w / np.sqrt(c * c + eps), rtol=1e-12, atol=0)
    # one non-zero element a at j: y_j = a / sqrt(a^2 / D + eps), the rest 0
    x = np.zeros((1, D))
    x[0, 17] = 2.5
    y = f(x, None, 1e-3)
    assert y[0, 17] == pytest.approx(2.5 / np.sqrt(2.5 ** 2 / D + 1e-3), rel=1e-12)
    assert np.count_nonzero(y) == 1
    # zero row stays zero (eps > 0)
    assert np.all(f(np.zeros((2, D)), None, 1e-6) == 0.0)
    # eps = 0, no weight: every output row has root-mean-square exactly 1
    x = rng.standard_normal((7, D)) * rng.uniform(0.1, 10.0, (7, 1))
    y = f(x, None, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-12)
    # a row of +-1 already has unit RMS: unchanged
    s = np.where(rng.random((1, D)) < 0.5, -1.0, 1.0)
    np.testing.assert_allclose(f(s, None, 0.0), s, rtol=1e-12)
    # eps = 0: scale invariance and odd symmetry
    np.testing.assert_allclose(f(4.0 * x, None, 0.0), y, rtol=1e-12)
    np.testing.assert_allclose(f(-x, None, 0.0), -y, rtol=1e-12)
    # weight: elementwise and linear; rows are independent
    w = rng.standard_normal(D)
    np.testing.assert_allclose(f(x, w, 0.0), y * w[None, :], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(f(x, 3.0 * w, 1e-4), 3.0 * f(x, w, 1e-4), rtol=1e-12)
    np.testing.assert_allclose(f(x[2:3], w, 1e-4), f(x, w, 1e-4)[2:3], rtol=1e-12)
    # eps enters under the square root: for a row of RMS 1, y = x / sqrt(1 + eps)
    np.testing.assert_allclose(f(s, None, 0.25), s / np.sqrt(1.25), rtol=1e-12)


def test_oracle_meets_every_pin():
    pins(rms_norm)


def _sum_not_mean(x, w=None, eps=1e-6):
    x = np.asarray(x, float)
    y = x / np.sqrt(np.sum(x * x, axis=1, keepdims=True) + eps)
    return y if w is None else y * w


def _no_sqrt(x, w=None, eps=1e-6):
    x = np.asarray(x, float)
    y = x / (np.mean(x * x, axis=1, keepdims=True) + eps)
    return y if w is None else y * w


def _eps_outside(x, w=None, eps=1e-6):
    x = np.asarray(x, float)
    y = x / (np.sqrt(np.mean(x * x, axis=1, keepdims=True)) + eps)
    return y if w is None else y * w


def _column_mean(x, w=None, eps=1e-6):
    x = np.asarray(x, float)
    y = x / np.sqrt(np.mean(x * x, axis=0, keepdims=True) + eps)
    return y if w is None else y * w


def _mean_abs(x, w=None, eps=1e-6):
    x = np.asarray(x, float)
    y = x / np.sqrt(np.mean(np.abs(x), axis=1, keepdims=True) ** 2 + eps)
    return y if w is None else y * w


def _weight_divides(x, w=None, eps=1e-6):
    y = rms_norm(x, None, eps)
    return y if w is None else y / w


def _mean_subtracted(x, w=None, eps=1e-6):
    x = np.asarray(x, float)
    xc = x - x.mean(axis=1, keepdims=True)
    y = x / np.sqrt(np.mean(xc * xc, axis=1, keepdims=True) + eps)
    return y if w is None else y * w


@pytest.mark.parametrize("mutant", [_sum_not_mean, _no_sqrt, _eps_outside, _column_mean,
                                    _mean_abs, _weight_divides, _mean_subtracted])
def test_pins_reject_planted_mistakes(mutant):
    with pytest.raises(AssertionError):
        pins(mutant)
