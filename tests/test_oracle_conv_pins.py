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


# ----------------------------------------------------------------- backward
def _conv_loss(x, cu, w, b, dy, silu):
    return float(np.sum(dy * oracle.short_conv(x, cu, w, bias=b, silu=silu)))


def pin_vjp_finite_differences(vjp):
    """Central differences of L = <dy, short_conv(x)> for every element of x,
    the taps and the bias (packed sequences with an empty one, with and
    without SiLU)."""
    r = np.random.default_rng(11)
    cu = np.asarray([0, 5, 5, 12], dtype=np.int32)
    x = r.standard_normal((12, 1, 2))
    w = r.standard_normal((2, 4))
    b = r.standard_normal(2)
    dy = r.standard_normal((12, 1, 2))
    ok = True
    for silu in (False, True):
        dx, dw, db = vjp(x, dy, cu, w, b, silu)
        h = 1e-6
        for arr, grad in ((x, dx), (w, dw), (b, db)):
            flat = arr.reshape(-1)
            for j in range(flat.size):
                keep = flat[j]
                flat[j] = keep + h
                lp = _conv_loss(x, cu, w, b, dy, silu)
                flat[j] = keep - h
                lm = _conv_loss(x, cu, w, b, dy, silu)
                flat[j] = keep
                ok &= abs((lp - lm) / (2 * h) - grad.reshape(-1)[j]) <= 1e-7 * (1 + abs(grad.reshape(-1)[j]))
    return bool(ok)


def pin_vjp_identity_taps(vjp):
    """Taps (0, 0, 0, 1), no bias, no SiLU: dx = dy exactly; the gradient of
    tap i is the sum of dy_t x_{t-3+i} over tokens with that history inside
    the sequence; the bias gradient is the sum of dy."""
    r = np.random.default_rng(12)
    cu = np.asarray([0, 7, 20], dtype=np.int32)
    x = r.standard_normal((20, 2, 3))
    dy = r.standard_normal((20, 2, 3))
    ident = np.tile([0.0, 0.0, 0.0, 1.0], (6, 1))
    dx, dw, db = vjp(x, dy, cu, ident, None, False)
    ok = np.array_equal(dx, dy)
    xf, dyf = x.reshape(20, 6), dy.reshape(20, 6)
    for i in range(4):
        exp = np.zeros(6)
        for a, bnd in ((0, 7), (7, 20)):
            for t in range(a, bnd):
                u = t - 3 + i
                if u >= a:
                    exp += dyf[t] * xf[u]
        ok &= np.allclose(dw[:, i], exp, rtol=1e-13, atol=1e-13)
    ok &= np.allclose(db, dyf.sum(0), rtol=1e-13, atol=1e-13)
    return bool(ok)


def pin_vjp_sequence_isolation(vjp):
    """A gradient that reaches only the second sequence leaves the first
    sequence's input gradient exactly zero."""
    r = np.random.default_rng(13)
    cu = np.asarray([0, 9, 25], dtype=np.int32)
    x = r.standard_normal((25, 1, 4))
    w = r.standard_normal((4, 4))
    dy = r.standard_normal((25, 1, 4))
    dy[:9] = 0.0
    dx, _, _ = vjp(x, dy, cu, w, r.standard_normal(4), True)
    return bool(np.count_nonzero(dx[:9]) == 0 and np.count_nonzero(dx[9:]) > 0)


CONV_VJP_PINS = [pin_vjp_finite_differences, pin_vjp_identity_taps, pin_vjp_sequence_isolation]


def _vjp(plant=0):
    return lambda x, dy, cu, w, b, silu: oracle.short_conv_vjp(x, dy, cu, w, bias=b, silu=silu,
                                                               plant=plant)


@pytest.mark.parametrize("pin", CONV_VJP_PINS, ids=lambda p: p.__name__)
def test_conv_vjp_pin(pin):
    assert pin(_vjp())


@pytest.mark.parametrize("plant", sorted(oracle.CONVB_PLANT), ids=str)
def test_conv_vjp_planted_mistake_is_caught(plant):
    bad = _vjp(oracle.CONVB_PLANT[plant])
    assert [p.__name__ for p in CONV_VJP_PINS if not p(bad)], plant
