"""Pins for the oracle's gated RMSNorm, each against something other than itself:
closed forms for constant rows and a zero gate, invariance under scaling the row,
the unit-RMS property of the normalised row, and planted mistakes that must fail."""

import math

import numpy as np
import pytest

from oracle import kda_oracle as O

RNG = np.random.default_rng(21)


def test_constant_row_closed_form():
    D, c, eps = 128, 0.75, 1e-6
    x = np.full((3, D), c)
    g = np.array([[0.0] * D, [math.log(3.0)] * D, [-2.0] * D])
    w = np.linspace(0.5, 1.5, D)
    y, rstd = O.gated_rmsnorm(x, g, w, eps)
    assert np.allclose(rstd, 1.0 / math.sqrt(c * c + eps), rtol=1e-15, atol=0)
    sig = np.array([0.5, 0.75, 1.0 / (1.0 + math.exp(2.0))])
    want = (c / math.sqrt(c * c + eps)) * w[None, :] * sig[:, None]
    assert np.allclose(y, want, rtol=1e-14, atol=0)


def test_scale_invariance_and_unit_rms_without_eps():
    x = RNG.standard_normal((5, 128))
    g = RNG.standard_normal((5, 128))
    w = RNG.uniform(0.5, 2.0, 128)
    y1, r1 = O.gated_rmsnorm(x, g, w, 0.0)
    y2, r2 = O.gated_rmsnorm(7.5 * x, g, w, 0.0)
    assert np.allclose(y1, y2, rtol=1e-13, atol=0)
    assert np.allclose(r1, 7.5 * r2, rtol=1e-13, atol=0)
    # With weight 1 and the gate at +inf (sigmoid 1), each output row has RMS 1.
    y3, _ = O.gated_rmsnorm(x, np.full_like(g, 800.0), np.ones(128), 0.0)
    assert np.allclose(np.sqrt(np.mean(y3 ** 2, axis=-1)), 1.0, rtol=1e-13)


def _sum_not_mean(x, gate, weight, eps):
    x = np.asarray(x, np.float64)
    rstd = 1.0 / np.sqrt(np.sum(x * x, axis=-1) + eps)
    return x * rstd[..., None] * weight * O.sigmoid(gate), rstd


def _no_gate(x, gate, weight, eps):
    x = np.asarray(x, np.float64)
    rstd = 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)
    return x * rstd[..., None] * weight, rstd


@pytest.mark.parametrize("bad", [_sum_not_mean, _no_gate])
def test_planted_norm_mistakes_are_caught(bad):
    D, c, eps = 128, 0.75, 1e-6
    x = np.full((1, D), c)
    g = np.zeros((1, D))
    w = np.ones(D)
    y, _ = bad(x, g, w, eps)
    want = (c / math.sqrt(c * c + eps)) * 0.5
    assert not np.allclose(y, want, rtol=1e-6, atol=0)
