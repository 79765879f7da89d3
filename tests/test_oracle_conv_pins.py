"""Pins for the oracle's short causal convolution, each against something other than
itself: tap impulses with closed-form outputs, the window shift of a short sequence,
splitting a sequence with the window carried, the multi-step update against prefill,
and planted mistakes that must fail."""

import math

import numpy as np
import pytest

from oracle import kda_oracle as O

RNG = np.random.default_rng(31)
C, W = 24, 4


def _taps(i):
    w = np.zeros((C, W))
    w[:, i] = 1.0
    return w


def test_identity_tap_and_silu_closed_form():
    x = RNG.standard_normal((10, C))
    y, _ = O.conv1d_prefill(x, _taps(W - 1), None, [0, 10], None, None, silu=False)
    assert np.array_equal(y, x)
    y2, _ = O.conv1d_prefill(x, _taps(W - 1), None, [0, 10], None, None, silu=True)
    want = x / (1.0 + np.exp(-x))
    assert np.allclose(y2, want, rtol=1e-14, atol=0)
    assert abs(O.conv1d_prefill(np.full((1, C), math.log(3.0)), _taps(W - 1), None, [0, 1],
                                None, None)[0][0, 0] - 0.75 * math.log(3.0)) < 1e-15


def test_oldest_tap_reads_the_window_then_the_sequence():
    x = RNG.standard_normal((9, C))
    state = RNG.standard_normal((2, W - 1, C))
    y, new = O.conv1d_prefill(x, _taps(0), None, [0, 9], state, [1], silu=False)
    assert np.array_equal(y[: W - 1], state[1])            # y_t = x_{t-3}: the window first
    assert np.array_equal(y[W - 1:], x[: 9 - (W - 1)])
    assert np.array_equal(new[1], x[-(W - 1):])            # window after the sequence
    assert np.array_equal(new[0], state[0])                # other rows unchanged


def test_short_sequence_shifts_the_window():
    x = RNG.standard_normal((1, C))
    state = RNG.standard_normal((1, W - 1, C))
    _, new = O.conv1d_prefill(x, RNG.standard_normal((C, W)), None, [0, 1], state, [0])
    assert np.array_equal(new[0], np.concatenate([state[0, 1:], x]))


def test_split_with_window_carried_equals_one_call():
    x = RNG.standard_normal((23, C))
    w, b = RNG.standard_normal((C, W)), RNG.standard_normal(C)
    s0 = RNG.standard_normal((1, W - 1, C))
    y, s_all = O.conv1d_prefill(x, w, b, [0, 23], s0, [0])
    ya, sa = O.conv1d_prefill(x[:8], w, b, [0, 8], s0, [0])
    yb, sb = O.conv1d_prefill(x[8:], w, b, [0, 15], sa, [0])
    assert np.allclose(np.concatenate([ya, yb]), y, rtol=0, atol=1e-13)
    assert np.array_equal(sb, s_all)


def test_update_rows_equal_prefill_and_windows_after_each_token():
    B, T = 3, 5
    x = RNG.standard_normal((B * T, C))
    w, b = RNG.standard_normal((C, W)), RNG.standard_normal(C)
    pool = RNG.standard_normal((6, W - 1, C))
    idx = np.array([4, -1, 2])
    y, inter = O.conv1d_update(x, w, b, pool, idx, T)
    for r in (0, 2):
        for t in range(T):
            yp, sp = O.conv1d_prefill(x[r * T:r * T + t + 1], w, b, [0, t + 1], pool, [idx[r]])
            assert np.allclose(y[r * T + t], yp[-1], rtol=0, atol=1e-13)
            assert np.array_equal(inter[r, t], sp[idx[r]])
    assert np.all(y[T:2 * T] == 0) and np.all(inter[1] == 0)   # padding row


def _off_by_one(x, weight, bias, cu, state, idx, silu=True):
    # planted: taps aligned one token late (the current input never used)
    w2 = np.zeros_like(np.asarray(weight, np.float64))
    w2[:, 1:] = np.asarray(weight, np.float64)[:, :-1]
    return O.conv1d_prefill(x, w2, bias, cu, state, idx, silu)


def _no_bias(x, weight, bias, cu, state, idx, silu=True):
    return O.conv1d_prefill(x, weight, None, cu, state, idx, silu)


@pytest.mark.parametrize("bad", [_off_by_one, _no_bias])
def test_planted_conv_mistakes_are_caught(bad):
    x = RNG.standard_normal((6, C))
    b = RNG.standard_normal(C)
    y_bad, _ = bad(x, _taps(W - 1), b, [0, 6], None, None, silu=False)
    assert not np.allclose(y_bad, x + b, rtol=0, atol=1e-9)
