"""Pins of the oracle's backward (vector-Jacobian product of the token
recurrence) to facts outside it.

The pages check the chunked operator's gradients for q, k, v, the gate and beta
against an independent FP64 recurrence VJP, with a planted 25 % gradient
scaling error that must fail (xtuner PR #2301, section Validation).  The VJP
here is pinned by:
  * central finite differences of the (separately pinned) FP64 forward, element
    by element on tiny inputs and along random directions at the production
    head size (d = 128), including packed sequences, a chunk boundary, an
    initial state and a final-state gradient;
  * the closed form of a single token;
  * exact zeros where beta saturates or the gate is switched off;
  * every planted backward mistake failing the finite-difference pin.
"""
import numpy as np
import pytest

import oracle


def _inputs(seed, lens, H, dk, dv):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N = len(lens)
    x = dict(
        q=rng.standard_normal((T, H, dk)), k=rng.standard_normal((T, H, dk)),
        v=rng.standard_normal((T, H, dv)), f_raw=rng.standard_normal((T, H, dk)),
        b_raw=rng.standard_normal((T, H)), A_log=rng.uniform(0, np.log(16), H),
        dt_bias=rng.normal(0, 0.5, (H, dk)),
        initial_state=0.3 * rng.standard_normal((N, H, dk, dv)))
    dout = rng.standard_normal((T, H, dv))
    dfin = rng.standard_normal((N, H, dk, dv))
    return x, cu, dout, dfin


ORDER = ("q", "k", "v", "f_raw", "b_raw", "A_log", "dt_bias", "initial_state")
GRAD = {"q": "dq", "k": "dk", "v": "dv", "f_raw": "df", "b_raw": "db", "A_log": "dA_log",
        "dt_bias": "ddt_bias", "initial_state": "dinit"}


def _loss(x, cu, dout, dfin):
    out, fin = oracle.kda_forward_rect(x["q"], x["k"], x["v"], x["f_raw"], x["b_raw"], x["A_log"],
                                       x["dt_bias"], cu, initial_state=x["initial_state"],
                                       return_final_state=True)
    return float(np.sum(out * dout) + np.sum(fin * dfin))


def _vjp(x, cu, dout, dfin, plant=0):
    return oracle.kda_backward(x["q"], x["k"], x["v"], x["f_raw"], x["b_raw"], x["A_log"],
                               x["dt_bias"], cu, dout, initial_state=x["initial_state"],
                               dfinal_state=dfin, plant=plant)


def _fd_all(x, cu, dout, dfin, h=1e-6):
    fd = {}
    for name in ORDER:
        a = x[name]
        g = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            old = a[idx]
            a[idx] = old + h
            lp = _loss(x, cu, dout, dfin)
            a[idx] = old - h
            lm = _loss(x, cu, dout, dfin)
            a[idx] = old
            g[idx] = (lp - lm) / (2 * h)
        fd[GRAD[name]] = g
    return fd


@pytest.fixture(scope="module")
def tiny():
    x, cu, dout, dfin = _inputs(11, [3, 4], 2, 4, 3)
    return x, cu, dout, dfin, _fd_all(x, cu, dout, dfin)


def _worst(got, fd):
    return max(float(np.max(np.abs(got[k] - fd[k]) / (1.0 + np.abs(fd[k])))) for k in fd)


def test_vjp_matches_finite_differences_elementwise(tiny):
    x, cu, dout, dfin, fd = tiny
    g = _vjp(x, cu, dout, dfin)
    for key in fd:
        err = np.max(np.abs(g[key] - fd[key]) / (1.0 + np.abs(fd[key])))
        assert err < 1e-7, (key, err)
        assert np.any(g[key] != 0), key


@pytest.mark.parametrize("plant", sorted(oracle.BWD_PLANT))
def test_planted_backward_mistakes_fail_finite_differences(tiny, plant):
    x, cu, dout, dfin, fd = tiny
    g = _vjp(x, cu, dout, dfin, plant=oracle.BWD_PLANT[plant])
    assert _worst(g, fd) > 1e-4, plant


def test_planted_beta_scale_fails_by_the_pages_margin(tiny):
    """A 25 % scaling of one gradient is seen as a 25 % relative error of db."""
    x, cu, dout, dfin, fd = tiny
    g = _vjp(x, cu, dout, dfin, plant=oracle.BWD_PLANT["bwd_beta_scale"])
    rel = np.linalg.norm(g["db"] - fd["db"]) / np.linalg.norm(fd["db"])
    assert abs(rel - 0.25) < 1e-6


@pytest.mark.parametrize("lens,H", [([37, 28], 2), ([129], 1)])
def test_vjp_directional_derivative_production_head(lens, H):
    """d = 128 (the production head), packed 37/28 and a 129-token sequence
    (two chunk boundaries at 64 tokens): <grad, delta> against a central
    difference of the forward along a random direction of every input."""
    x, cu, dout, dfin = _inputs(23 + len(lens), lens, H, 128, 128)
    rng = np.random.default_rng(5)
    delta = {n: rng.standard_normal(x[n].shape) for n in ORDER}
    g = _vjp(x, cu, dout, dfin)
    for name in ORDER:
        h = 1e-5
        xp = dict(x); xp[name] = x[name] + h * delta[name]
        xm = dict(x); xm[name] = x[name] - h * delta[name]
        fd = (_loss(xp, cu, dout, dfin) - _loss(xm, cu, dout, dfin)) / (2 * h)
        an = float(np.sum(g[GRAD[name]] * delta[name]))
        assert abs(an - fd) <= 1e-6 * (1.0 + abs(fd)), (name, an, fd)


def test_single_token_closed_form():
    """T = 1 from a zero state: o = scale beta (k^.q^) v, so with
    L = <dout, o>:  dv = scale beta (k^.q^) dout,  dbeta = scale (k^.q^)(v.dout),
    dq^ = scale beta (v.dout) k^  and dq = (dq^ - q^ (q^.dq^)) / sqrt(|q|^2+eps)."""
    rng = np.random.default_rng(3)
    d, eps = 8, 1e-6
    q, k, v, f = (rng.standard_normal((1, 1, d)) for _ in range(4))
    b = rng.standard_normal((1, 1))
    A_log, dtb = np.array([0.7]), rng.standard_normal((1, d))
    dout = rng.standard_normal((1, 1, d))
    g = oracle.kda_backward(q, k, v, f, b, A_log, dtb, [0, 1], dout, eps=eps)
    scale = 1 / np.sqrt(d)
    rq = 1 / np.sqrt(np.sum(q ** 2) + eps)
    rk = 1 / np.sqrt(np.sum(k ** 2) + eps)
    qn, kn = q[0, 0] * rq, k[0, 0] * rk
    beta = 1 / (1 + np.exp(-b[0, 0]))
    kq, vd = kn @ qn, v[0, 0] @ dout[0, 0]
    np.testing.assert_allclose(g["dv"][0, 0], scale * beta * kq * dout[0, 0], rtol=1e-13)
    np.testing.assert_allclose(g["db"][0, 0], scale * kq * vd * beta * (1 - beta), rtol=1e-12)
    dqn = scale * beta * vd * kn
    np.testing.assert_allclose(g["dq"][0, 0], rq * (dqn - qn * (qn @ dqn)), rtol=1e-11, atol=1e-15)
    dkn = scale * beta * vd * qn
    np.testing.assert_allclose(g["dk"][0, 0], rk * (dkn - kn * (kn @ dkn)), rtol=1e-11, atol=1e-15)
    # the decay of a zero state has no effect: the gate gets no gradient
    assert np.all(g["df"] == 0) and np.all(g["dA_log"] == 0) and np.all(g["ddt_bias"] == 0)


def test_saturated_beta_and_switched_off_gate_give_exact_zeros():
    x, cu, dout, dfin = _inputs(7, [5, 3], 2, 6, 6)
    x["b_raw"][1, 0] = np.inf
    x["b_raw"][4, 1] = -np.inf
    x["A_log"][1] = -np.inf
    g = _vjp(x, cu, dout, dfin)
    assert g["db"][1, 0] == 0.0 and g["db"][4, 1] == 0.0
    assert np.all(g["df"][:, 1] == 0) and g["dA_log"][1] == 0.0 and np.all(g["ddt_bias"][1] == 0)
    assert np.all(np.isfinite(g["dq"])) and np.any(g["df"][:, 0] != 0)


def test_packed_equals_separate_and_parameter_gradients_add():
    x, cu, dout, dfin = _inputs(9, [4, 6], 2, 5, 4)
    g = _vjp(x, cu, dout, dfin)
    sums = {"dA_log": 0.0, "ddt_bias": 0.0}
    for n in range(2):
        s, e = cu[n], cu[n + 1]
        xs = {name: x[name][s:e] for name in ("q", "k", "v", "f_raw", "b_raw")}
        gs = oracle.kda_backward(xs["q"], xs["k"], xs["v"], xs["f_raw"], xs["b_raw"], x["A_log"],
                                 x["dt_bias"], [0, e - s], dout[s:e],
                                 initial_state=x["initial_state"][n:n + 1],
                                 dfinal_state=dfin[n:n + 1])
        for key in ("dq", "dk", "dv", "df", "db"):
            assert np.array_equal(gs[key], g[key][s:e]), key
        assert np.array_equal(gs["dinit"][0], g["dinit"][n])
        for key in sums:
            sums[key] = sums[key] + gs[key]
    for key in sums:
        np.testing.assert_allclose(g[key], sums[key], rtol=1e-14, atol=1e-15)
