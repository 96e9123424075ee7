"""Pins for the oracle's short causal convolution (CPU only): a hand-worked
example, closed forms (identity and shift taps, SiLU), sequence isolation,
linearity, the bf16 rounding step, and two planted mistakes."""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(T, H, d, seed, cu):
    r = np.random.default_rng(seed)
    return r.standard_normal((T, H, d)), np.asarray(cu, dtype=np.int32), r.standard_normal((H * d, 4))


def pin_golden(conv):
    g = json.load(open(os.path.join(GOLDEN, "conv_d1_example.json")))
    w = np.asarray(g["weight"]).reshape(1, 4)
    x = np.asarray(g["x"]).reshape(-1, 1, 1)
    y = conv(x, [0, len(g["x"])], w, silu=False)
    ok = np.allclose(y.ravel(), g["y_linear"], rtol=0, atol=1e-15)
    ys = conv(x, [0, len(g["x"])], w, silu=True)
    lin = np.asarray(g["y_linear"])
    ok &= np.allclose(ys.ravel(), lin / (1 + np.exp(-lin)), rtol=1e-15, atol=0)
    xp = np.asarray(g["x"] + g["packed_second_sequence"]["x"]).reshape(-1, 1, 1)
    yp = conv(xp, [0, 4, 6], w, silu=False).ravel()
    ok &= np.allclose(yp[4:], g["packed_second_sequence"]["y_linear"], rtol=0, atol=1e-15)
    return bool(ok)


def pin_identity_and_shift(conv):
    x, cu, _ = _rand(30, 2, 4, 1, [0, 11, 11, 30])
    ident = np.tile([0.0, 0.0, 0.0, 1.0], (8, 1))
    shift = np.tile([0.0, 0.0, 1.0, 0.0], (8, 1))
    ok = np.array_equal(conv(x, cu, ident, silu=False), x)
    y = conv(x, cu, shift, silu=False)
    exp = np.zeros_like(x)
    for a, b in ((0, 11), (11, 30)):
        exp[a + 1:b] = x[a:b - 1]
    ok &= np.array_equal(y, exp)
    bias = np.arange(8.0)
    ok &= np.allclose(conv(x, cu, ident, bias=bias, silu=False), x + bias.reshape(1, 2, 4),
                      rtol=0, atol=1e-15)
    return bool(ok)


def pin_sequence_isolation_and_linearity(conv):
    x, cu, w = _rand(40, 2, 4, 2, [0, 17, 40])
    y = conv(x, cu, w, silu=False)
    x2 = x.copy()
    x2[:17] *= -3.0
    ok = np.array_equal(conv(x2, cu, w, silu=False)[17:], y[17:])
    ok &= np.allclose(conv(2.5 * x, cu, w, silu=False), 2.5 * y, rtol=1e-13, atol=1e-13)
    sub = conv(x[17:], [0, 23], w, silu=False)
    ok &= np.array_equal(sub, y[17:])
    return bool(ok)


def pin_bf16_rounding():
    x = np.array([1.0 + 2 ** -9, 1.0 + 3 * 2 ** -9, -(1.0 + 2 ** -8 + 2 ** -10), 3.0e-3]).reshape(-1, 1, 1)
    ident = np.array([[0.0, 0.0, 0.0, 1.0]])
    y = oracle.short_conv(x, [0, 4], ident, silu=False, round_bf16=True).ravel()
    # ties to even: 1 + 2^-9 -> 1; 1 + 3*2^-9 -> 1 + 2^-7; -(1 + 2^-8 + 2^-10) -> -(1 + 2^-7)
    exp = [1.0, 1.0 + 2 ** -7, -(1.0 + 2 ** -7)]
    # elsewhere: within half a bf16 step, which is at most 2^-8 of the value
    return bool(np.array_equal(y[:3], exp) and abs(y[3] - 3.0e-3) <= 3.0e-3 * 2 ** -8)


CONV_PINS = [pin_golden, pin_identity_and_shift, pin_sequence_isolation_and_linearity]


@pytest.mark.parametrize("pin", CONV_PINS, ids=lambda p: p.__name__)
def test_conv_pin(pin):
    assert pin(oracle.short_conv)


def test_conv_bf16_rounding_ties_to_even():
    assert pin_bf16_rounding()


@pytest.mark.parametrize("plant", sorted(oracle.CONV_PLANT), ids=str)
def test_conv_planted_mistake_is_caught(plant):
    def bad(*a, **kw):
        return oracle.short_conv(*a, plant=oracle.CONV_PLANT[plant], **kw)
    assert [p.__name__ for p in CONV_PINS if not p(bad)], plant
