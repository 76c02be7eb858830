"""Pins of the oracle's causal depthwise conv1d (+ silu) against routes that do
not retype its loop: numpy.convolve (a library convolution), the impulse
response, scipy.special.expit for the gate, and the split property of a
causal filter (lmnt page, sections 3.1 and 3.2: depthwise conv of width about
4 with width-1 left padding, output cut to L steps, then silu)."""
import numpy as np
import pytest
from scipy.special import expit

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _inputs(seed, batch=2, L=37, Dn=5, width=4):
    r = _rng(seed)
    return (r.standard_normal((batch, L, Dn)), r.standard_normal((Dn, width)),
            r.standard_normal(Dn))


@pytest.mark.parametrize("width", [1, 2, 3, 4])
def test_conv_equals_numpy_convolve(width):
    """Causal conv = the first L outputs of a full convolution with the
    flipped kernel (conv1d layers compute a cross-correlation)."""
    x, w, bias = _inputs(1, width=width)
    pre = oracle.conv1d(x, w, bias, silu=False)
    for b in range(x.shape[0]):
        for d in range(x.shape[2]):
            ref = np.convolve(x[b, :, d], w[d, ::-1])[: x.shape[1]] + bias[d]
            np.testing.assert_allclose(pre[b, :, d], ref, rtol=1e-13, atol=1e-13)


def test_silu_gate_is_x_times_sigmoid():
    x, w, bias = _inputs(2)
    pre = oracle.conv1d(x, w, bias, silu=False)
    u = oracle.conv1d(x, w, bias, silu=True)
    np.testing.assert_allclose(u, pre * expit(pre), rtol=1e-13, atol=1e-15)


def test_impulse_response_is_reversed_kernel():
    """A unit impulse at t0 gives bias + w[width-1-j] at t0 + j, bias elsewhere."""
    width, L, t0 = 4, 12, 5
    w = np.array([[0.5, -1.0, 2.0, 3.0]])
    x = np.zeros((1, L, 1))
    x[0, t0, 0] = 1.0
    pre = oracle.conv1d(x, w, np.array([0.25]), silu=False)[0, :, 0]
    expect = np.full(L, 0.25)
    for j in range(width):
        expect[t0 + j] += w[0, width - 1 - j]
    np.testing.assert_array_equal(pre, expect)


def test_history_continues_the_sequence():
    """Convolving [x_prev ; x] from zeros and keeping the last L outputs equals
    convolving x with x_prev as its history (a causal filter splits)."""
    x, w, bias = _inputs(3, L=20)
    width = w.shape[1]
    r = _rng(4)
    prev = r.standard_normal((x.shape[0], width - 1, x.shape[2]))
    whole = oracle.conv1d(np.concatenate([prev, x], axis=1), w, bias)
    part = oracle.conv1d(x, w, bias, x_prev=prev)
    np.testing.assert_allclose(part, whole[:, width - 1:], rtol=1e-13, atol=1e-15)
    # and the zero history is the same as no history
    zero = oracle.conv1d(x, w, bias, x_prev=np.zeros_like(prev))
    np.testing.assert_array_equal(zero, oracle.conv1d(x, w, bias))


def test_width_one_is_pointwise():
    x, w, bias = _inputs(5, width=1)
    pre = w[:, 0] * x + bias
    np.testing.assert_allclose(oracle.conv1d(x, w, bias), pre * expit(pre), rtol=1e-13)


def test_pins_would_catch_a_flipped_kernel():
    """A plausible mistake -- the kernel applied unflipped -- must fail the
    convolution pin (planted on the CPU, in the inputs of the oracle)."""
    x, w, bias = _inputs(6)
    wrong = oracle.conv1d(x, w[:, ::-1].copy(), bias, silu=False)
    ref = np.convolve(x[0, :, 0], w[0, ::-1])[: x.shape[1]] + bias[0]
    assert not np.allclose(wrong[0, :, 0], ref, rtol=1e-6)
