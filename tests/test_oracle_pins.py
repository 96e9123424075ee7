"""Pins for the FP64 oracle (CPU only).

The oracle is checked against things other than itself: hand-derived worked
examples (tests/golden), closed forms, special cases, structural invariants,
and agreement with an independently written chunk-form implementation.  The
final test plants each plausible mistake in the oracle and shows that at least
one pin catches it.
"""
import functools
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_inputs(T, H, d, seed, gate_scale=1.0, cu=None):
    r = _rng(seed)
    q = r.standard_normal((T, H, d))
    k = r.standard_normal((T, H, d))
    v = r.standard_normal((T, H, d))
    f = r.standard_normal((T, H, d)) * gate_scale
    b = r.standard_normal((T, H))
    A_log = r.uniform(0, math.log(16), H)
    dtb = 0.5 * r.standard_normal((H, d))
    if cu is None:
        cu = [0, T]
    return dict(q=q, k=k, v=v, f_raw=f, b_raw=b, A_log=A_log, dt_bias=dtb,
                cu_seqlens=np.asarray(cu, dtype=np.int32))


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def _load_golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def _num(x):
    return float(x)


# --------------------------------------------------------------------------
# Pins written over a forward callable fwd(**inputs, eps=..., scale=...) -> out.
# Each returns True when the pin holds.
# --------------------------------------------------------------------------

def pin_golden_d1(fwd):
    g = _load_golden("kda_d1_ema.json")
    T = len(g["q"])
    arr = lambda x: np.asarray(x, dtype=np.float64).reshape(T, 1, 1)
    ok = True
    for case in g["cases"]:
        out = fwd(q=arr(g["q"]), k=arr(g["k"]), v=arr(g["v"]), f_raw=arr(g["f_raw"]),
                  b_raw=np.asarray(g["b_raw"], dtype=np.float64).reshape(T, 1),
                  A_log=np.asarray(g["A_log"], dtype=np.float64),
                  dt_bias=np.asarray(g["dt_bias"], dtype=np.float64),
                  cu_seqlens=np.asarray(case["cu_seqlens"], dtype=np.int32),
                  eps=g["eps"], scale=g["scale"])
        ok &= np.allclose(out.reshape(-1), case["out"], rtol=0, atol=1e-14)
    return bool(ok)


def pin_golden_d2(fwd):
    g = _load_golden("kda_d2_retrieval.json")
    T, d = len(g["q"]), g["d"]
    arr = lambda x: np.asarray(x, dtype=np.float64).reshape(T, 1, d)
    out = fwd(q=arr(g["q"]), k=arr(g["k"]), v=arr(g["v"]), f_raw=arr(g["f_raw"]),
              b_raw=np.asarray([_num(x) for x in g["b_raw"]]).reshape(T, 1),
              A_log=np.asarray([_num(x) for x in g["A_log"]]),
              dt_bias=np.asarray(g["dt_bias"], dtype=np.float64),
              cu_seqlens=np.asarray(g["cu_seqlens"], dtype=np.int32), eps=g["eps"])
    return bool(np.allclose(out.reshape(T, d), np.asarray(g["out"]), rtol=0, atol=1e-14))


def pin_single_token(fwd):
    """T=1: o = scale * beta * (k^ . q^) * v with k^, q^ the L2-normalised vectors."""
    x = _rand_inputs(1, 3, 8, seed=11)
    out = fwd(**x, eps=0.0)
    ok = True
    for h in range(3):
        q = x["q"][0, h] / np.linalg.norm(x["q"][0, h])
        k = x["k"][0, h] / np.linalg.norm(x["k"][0, h])
        beta = 1.0 / (1.0 + math.exp(-x["b_raw"][0, h]))
        exp = (1 / math.sqrt(8)) * beta * float(k @ q) * x["v"][0, h]
        ok &= np.allclose(out[0, h], exp, rtol=1e-13, atol=1e-15)
    return bool(ok)


def pin_pure_decay(fwd):
    """beta_1 = 1 then beta = 0 (b = +inf, -inf): the state only decays, so
    o_t = scale * v_1 * sum_c k^_1c q^_tc exp(sum_{j=2..t} g_jc).  The gate
    inputs are chosen so g is known in closed form: A_log = ln(lam), x = f + dt
    with softplus(0) = ln 2, softplus(ln 3) = ln 4, so g = -lam ln 2 or -lam ln 4."""
    T, d = 5, 6
    r = _rng(5)
    q = r.standard_normal((T, 1, d))
    k = r.standard_normal((T, 1, d))
    v = r.standard_normal((T, 1, d))
    lam = 0.75
    # x = 0 on even channels, ln 3 on odd channels, split between f_raw and dt_bias
    dtb = np.where(np.arange(d) % 2 == 0, 0.25, 0.25 + math.log(3)).reshape(1, d)
    f = np.full((T, 1, d), -0.25)
    b = np.full((T, 1), -np.inf)
    b[0, 0] = np.inf
    out = fwd(q=q, k=k, v=v, f_raw=f, b_raw=b, A_log=np.array([math.log(lam)]), dt_bias=dtb,
              cu_seqlens=np.array([0, T], dtype=np.int32), eps=0.0)
    g = -lam * np.where(np.arange(d) % 2 == 0, math.log(2), math.log(4))
    k1 = k[0, 0] / np.linalg.norm(k[0, 0])
    ok = True
    for t in range(T):
        qt = q[t, 0] / np.linalg.norm(q[t, 0])
        dec = np.exp(g * t)  # tokens 2..t+1 (1-based) each decay by exp(g)
        exp = (1 / math.sqrt(d)) * float(np.sum(k1 * qt * dec)) * v[0, 0]
        ok &= np.allclose(out[t, 0], exp, rtol=1e-13, atol=1e-15)
    return bool(ok)


def pin_long_memory(fwd):
    """No decay (A_log = -inf) and beta_1 = 1, beta = 0 afterwards: the state
    written by token 1 is read unchanged by every later token, across chunk
    sizes: o_t = scale * (k^_1 . q^_t) * v_1 for all t (here up to 130)."""
    T, d = 130, 8
    r = _rng(9)
    q = r.standard_normal((T, 1, d)); k = r.standard_normal((T, 1, d)); v = r.standard_normal((T, 1, d))
    b = np.full((T, 1), -np.inf); b[0, 0] = np.inf
    out = fwd(q=q, k=k, v=v, f_raw=r.standard_normal((T, 1, d)), b_raw=b, A_log=np.array([-np.inf]),
              dt_bias=np.zeros((1, d)), cu_seqlens=np.array([0, T], dtype=np.int32), eps=0.0)
    k1 = k[0, 0] / np.linalg.norm(k[0, 0])
    qn = q[:, 0] / np.linalg.norm(q[:, 0], axis=-1, keepdims=True)
    exp = (qn @ k1)[:, None] * v[0, 0][None, :] / math.sqrt(d)
    return bool(np.allclose(out[:, 0], exp, rtol=1e-13, atol=1e-14))


def pin_retrieval_orthonormal(fwd):
    """g = 0, beta = 1, orthonormal keys: reading with q = k_j returns v_j
    exactly (scaled); re-writing a key returns the newest value."""
    d, m = 16, 10
    r = _rng(7)
    Q, _ = np.linalg.qr(r.standard_normal((d, d)))
    keys = Q[:, :m].T  # m orthonormal rows
    T = 2 * m + 3
    k = np.zeros((T, 1, d)); q = np.zeros((T, 1, d)); v = r.standard_normal((T, 1, d))
    wkey = [t for t in range(m)] + [t - m for t in range(m, 2 * m)] + [t % m for t in range(2 * m, T)]
    rkey = [t for t in range(m)] + [(t - m + 3) % m for t in range(m, 2 * m)] + [(t + 1) % m for t in range(2 * m, T)]
    latest = {}
    exp = np.zeros((T, d))
    for t in range(T):
        k[t, 0] = keys[wkey[t]]; q[t, 0] = keys[rkey[t]]
        latest[wkey[t]] = t
        exp[t] = v[latest[rkey[t]], 0] if rkey[t] in latest else 0.0
    out = fwd(q=q, k=k, v=v, f_raw=np.zeros((T, 1, d)), b_raw=np.full((T, 1), np.inf),
              A_log=np.array([-np.inf]), dt_bias=np.zeros((1, d)),
              cu_seqlens=np.array([0, T], dtype=np.int32), eps=0.0)
    return bool(np.allclose(out[:, 0], exp / math.sqrt(d), rtol=0, atol=1e-12))


def pin_delta_on_decayed_state(fwd):
    """Write v1 at key k (beta=1), then, after one decay step by exactly 1/2,
    write v2 at the same key: the delta rule on the decayed state makes
    S^T k = v2 exactly, so reading with q = k gives scale*v2."""
    d = 4
    r = _rng(3)
    kk = r.standard_normal(d); kk /= np.linalg.norm(kk)
    v = r.standard_normal((2, 1, d))
    k = np.stack([kk, kk]).reshape(2, 1, d)
    out = fwd(q=k.copy(), k=k, v=v, f_raw=np.zeros((2, 1, d)), b_raw=np.full((2, 1), np.inf),
              A_log=np.array([0.0]), dt_bias=np.zeros((1, d)),
              cu_seqlens=np.array([0, 2], dtype=np.int32), eps=0.0)
    return bool(np.allclose(out[1, 0], v[1, 0] / math.sqrt(d), rtol=0, atol=1e-13))


def pin_sequence_reset(fwd):
    """Packed run == each sequence run on its own; perturbing sequence 1 leaves
    sequence 2 bit-for-bit unchanged."""
    cu = [0, 37, 65, 70]
    x = _rand_inputs(70, 2, 8, seed=21, cu=cu)
    out = fwd(**x)
    ok = True
    for n in range(3):
        a, b = cu[n], cu[n + 1]
        sub = {kk: (vv[a:b] if kk not in ("A_log", "dt_bias", "cu_seqlens") else vv)
               for kk, vv in x.items()}
        sub["cu_seqlens"] = np.array([0, b - a], dtype=np.int32)
        ok &= np.array_equal(fwd(**sub), out[a:b])
    y = {kk: vv.copy() for kk, vv in x.items()}
    y["v"][:37] += 1.0
    y["q"][:37] *= -1.0
    ok &= np.array_equal(fwd(**y)[37:], out[37:])
    return bool(ok)


def pin_causality(fwd):
    x = _rand_inputs(40, 2, 8, seed=31)
    out = fwd(**x)
    ok = True
    for tp in (0, 17, 39):
        y = {kk: vv.copy() for kk, vv in x.items()}
        y["k"][tp] += 0.5; y["v"][tp] -= 1.0; y["f_raw"][tp] += 2.0; y["b_raw"][tp] *= -1
        o2 = fwd(**y)
        ok &= np.array_equal(o2[:tp], out[:tp]) and not np.allclose(o2[tp:], out[tp:])
    return bool(ok)


def pin_linearity_in_v(fwd):
    x = _rand_inputs(30, 2, 8, seed=41)
    o1 = fwd(**x)
    y = dict(x); y["v"] = x["v"] * 2.5 + 1.0
    z = dict(x); z["v"] = np.ones_like(x["v"])
    o2 = fwd(**y); o3 = fwd(**z)
    return bool(np.allclose(o2, 2.5 * o1 + o3, rtol=1e-12, atol=1e-12))


def pin_head_permutation(fwd):
    x = _rand_inputs(20, 4, 8, seed=51)
    out = fwd(**x)
    perm = np.array([2, 0, 3, 1])
    y = {kk: (vv[:, perm] if kk in ("q", "k", "v", "f_raw", "b_raw") else vv)
         for kk, vv in x.items()}
    y["A_log"] = x["A_log"][perm]; y["dt_bias"] = x["dt_bias"][perm]
    return bool(np.array_equal(fwd(**y), out[:, perm]))


def pin_chunked_agreement(fwd, chunks=(1, 4, 16, 64), gate_scales=(1.0, 1e-3, 4.0), tol=1e-12):
    """An independently written FP64 chunk form agrees with the recurrence."""
    ok = True
    for gs in gate_scales:
        x = _rand_inputs(150, 2, 16, seed=61, gate_scale=gs, cu=[0, 130, 131, 150])
        if gs == 1e-3:
            x["A_log"] = np.array([-3.0, -5.0])  # weak decay: long memory across chunks
        ref = fwd(**x)
        for C in chunks:
            ok &= _rel(oracle.kda_chunked(**x, chunk=C), ref) < tol
    return bool(ok)


def pin_state_split(fwd):
    """Running each sequence in two pieces, the second starting from the first
    piece's final state, gives the whole run's outputs and final state; the
    whole run itself starts from a given (random) initial state.  Packed: three
    sequences with their own initial states, one of them empty (final state =
    initial state)."""
    cu = [0, 150, 150, 197]
    T, H, d = 197, 2, 8
    x = _rand_inputs(T, H, d, seed=71, cu=cu)
    r = _rng(72)
    S0 = 0.3 * r.standard_normal((3, H, d, d))
    out, fin = fwd(**x, initial_state=S0, return_final_state=True)
    ok = np.array_equal(fin[1], S0[1])
    cut = {0: 70, 2: 150 + 31}  # split points inside sequences 0 and 2
    for n, tc in cut.items():
        a, b = cu[n], cu[n + 1]

        def piece(lo, hi):
            return {kk: (vv[lo:hi] if kk not in ("A_log", "dt_bias", "cu_seqlens") else vv)
                    for kk, vv in x.items() if kk != "cu_seqlens"}
        one = np.array([0, tc - a], dtype=np.int32)
        two = np.array([0, b - tc], dtype=np.int32)
        o1, f1 = fwd(**piece(a, tc), cu_seqlens=one, initial_state=S0[n:n + 1],
                     return_final_state=True)
        o2, f2 = fwd(**piece(tc, b), cu_seqlens=two, initial_state=f1, return_final_state=True)
        ok &= _rel(np.concatenate([o1, o2]), out[a:b]) < 1e-12
        ok &= _rel(f2[0], fin[n]) < 1e-12
    return bool(ok)


def pin_state_closed_form(fwd):
    """No writes (beta = 0): the initial state only decays, with the closed-form
    gate of pin_pure_decay (g = -lam ln 2 or -lam ln 4 per key channel), so
    o_t = scale * (Diag(exp(t' g)) S_init)^T q^_t with t' = t + 1 tokens decayed,
    and the final state is Diag(exp(T g)) S_init."""
    T, d = 6, 6
    r = _rng(75)
    q = r.standard_normal((T, 1, d))
    S0 = r.standard_normal((1, 1, d, d))
    lam = 0.75
    dtb = np.where(np.arange(d) % 2 == 0, 0.25, 0.25 + math.log(3)).reshape(1, d)
    out, fin = fwd(q=q, k=r.standard_normal((T, 1, d)), v=r.standard_normal((T, 1, d)),
                   f_raw=np.full((T, 1, d), -0.25), b_raw=np.full((T, 1), -np.inf),
                   A_log=np.array([math.log(lam)]), dt_bias=dtb,
                   cu_seqlens=np.array([0, T], dtype=np.int32), eps=0.0, initial_state=S0,
                   return_final_state=True)
    g = -lam * np.where(np.arange(d) % 2 == 0, math.log(2), math.log(4))
    ok = True
    for t in range(T):
        St = np.exp(g * (t + 1))[:, None] * S0[0, 0]  # row i (key) scaled
        qt = q[t, 0] / np.linalg.norm(q[t, 0])
        ok &= np.allclose(out[t, 0], (St.T @ qt) / math.sqrt(d), rtol=1e-13, atol=1e-15)
    ok &= np.allclose(fin[0, 0], np.exp(g * T)[:, None] * S0[0, 0], rtol=1e-13, atol=1e-15)
    return bool(ok)


FORWARD_PINS = [pin_golden_d1, pin_golden_d2, pin_single_token, pin_pure_decay, pin_long_memory,
                pin_retrieval_orthonormal, pin_delta_on_decayed_state, pin_sequence_reset,
                pin_causality, pin_linearity_in_v, pin_head_permutation, pin_chunked_agreement,
                pin_state_split, pin_state_closed_form]


@pytest.mark.parametrize("pin", FORWARD_PINS, ids=lambda p: p.__name__)
def test_forward_pin(pin):
    assert pin(oracle.kda_forward)


@pytest.mark.parametrize("plant", sorted(oracle.PLANT), ids=str)
def test_planted_mistake_is_caught(plant):
    """Each plausible mistake planted in the oracle fails at least one pin."""
    bad = functools.partial(oracle.kda_forward, plant=oracle.PLANT[plant])
    failed = [p.__name__ for p in FORWARD_PINS if not p(bad)]
    assert failed, f"planted mistake {plant!r} passed every pin"


# --------------------------------------------------------------------------
# Stage-one (prep) closed forms
# --------------------------------------------------------------------------

def test_chunked_form_carries_initial_and_final_state():
    """The chunk-form oracle takes and returns the state like the recurrence
    (chunk sizes that split the sequences at different places)."""
    cu = [0, 100, 100, 163]
    x = _rand_inputs(163, 2, 16, seed=81, cu=cu)
    S0 = 0.5 * _rng(82).standard_normal((3, 2, 16, 16))
    ref, fref = oracle.kda_forward(**x, initial_state=S0, return_final_state=True)
    for C in (1, 16, 64):
        out, fin = oracle.kda_chunked(**x, chunk=C, initial_state=S0, return_final_state=True)
        assert _rel(out, ref) < 1e-12 and _rel(fin, fref) < 1e-12, C


def test_prep_l2norm_closed_form():
    r = _rng(1)
    q = r.standard_normal((5, 3, 128)) * 3.0
    k = r.standard_normal((5, 3, 128))
    eps = 1e-6
    qn, kn, _, _ = oracle.kda_prep(q, k, np.zeros_like(q), np.zeros((5, 3)), np.zeros(3),
                                   np.zeros((3, 128)), eps=eps)
    nq = np.linalg.norm(q, axis=-1)
    assert np.allclose(np.linalg.norm(qn, axis=-1), 1 / np.sqrt(1 + eps / nq ** 2), rtol=1e-14)
    # direction preserved
    cos = np.sum(qn * q, axis=-1) / (np.linalg.norm(qn, axis=-1) * nq)
    assert np.allclose(cos, 1.0, rtol=0, atol=1e-14)
    # zero vector stays zero (no division by zero)
    z, _, _, _ = oracle.kda_prep(np.zeros((1, 1, 4)), np.zeros((1, 1, 4)), np.zeros((1, 1, 4)),
                                 np.zeros((1, 1)), np.zeros(1), np.zeros((1, 4)), eps=eps)
    assert np.all(z == 0)


def test_prep_gate_closed_forms():
    # x = f + dt_bias; g = -exp(A_log) * softplus(x)
    A_log = np.array([0.0, math.log(3.0), -np.inf, math.log(16.0)])
    x = np.array([0.0, math.log(3.0), 40.0, -40.0, 5.0, -0.7])
    f = np.tile(x, (1, 4, 1))  # [1, 4, 6]
    dtb = np.zeros((4, 6))
    _, _, g, _ = oracle.kda_prep(np.ones_like(f), np.ones_like(f), f, np.zeros((1, 4)), A_log, dtb)
    sp = np.array([math.log(2), math.log(4), 40.0 + math.exp(-40.0), math.exp(-40.0),
                   5.0 + math.log1p(math.exp(-5.0)), math.log1p(math.exp(-0.7))])
    for h, lam in enumerate([1.0, 3.0, 0.0, 16.0]):
        assert np.allclose(g[0, h], -lam * sp, rtol=1e-14, atol=0)
    assert np.all(g[0, 2] == 0.0)  # A_log = -inf gives no decay, exactly
    # softplus(x) - softplus(-x) = x
    _, _, g2, _ = oracle.kda_prep(np.ones((1, 1, 6)), np.ones((1, 1, 6)), -f[:, :1], np.zeros((1, 1)),
                                  np.zeros(1), np.zeros((1, 6)))
    assert np.allclose(-g[0, 0] + g2[0, 0], x, rtol=0, atol=1e-12)
    # dt_bias adds to f_raw
    _, _, g3, _ = oracle.kda_prep(np.ones((1, 1, 6)), np.ones((1, 1, 6)), np.zeros((1, 1, 6)),
                                  np.zeros((1, 1)), np.zeros(1), x.reshape(1, 6))
    assert np.allclose(g3[0, 0], g[0, 0], rtol=1e-15)


def test_prep_beta_special_values():
    b = np.array([[0.0, np.inf, -np.inf, math.log(3.0), -800.0]])
    _, _, _, beta = oracle.kda_prep(np.ones((1, 5, 2)), np.ones((1, 5, 2)), np.zeros((1, 5, 2)), b,
                                    np.zeros(5), np.zeros((5, 2)))
    assert beta[0, 0] == 0.5 and beta[0, 1] == 1.0 and beta[0, 2] == 0.0
    assert abs(beta[0, 3] - 0.75) < 1e-15
    assert 0.0 <= beta[0, 4] < 1e-300


def test_chunk_records_consistent():
    """The chunk-form records satisfy their defining identities: (I + A) W =
    Diag(beta) (k^ * exp(G)), A strictly lower, P lower, Gamma = exp(G_last)."""
    x = _rand_inputs(70, 2, 8, seed=71, cu=[0, 70])
    out, rec = oracle.kda_chunked(**x, chunk=64, records=True)
    qn, kn, g, beta = oracle.kda_prep(x["q"], x["k"], x["f_raw"], x["b_raw"], x["A_log"],
                                      x["dt_bias"])
    for c, (t0, n) in enumerate([(0, 64), (64, 6)]):
        for h in range(2):
            A = rec["A"][c, h][:n, :n]
            P = rec["P"][c, h][:n, :n]
            assert np.all(np.triu(A) == 0) and np.all(np.triu(P, 1) == 0)
            G = np.cumsum(g[t0:t0 + n, h], axis=0)
            assert np.allclose(rec["G"][c, h][:n], G, rtol=1e-14, atol=1e-12)
            rhs = beta[t0:t0 + n, h, None] * kn[t0:t0 + n, h] * np.exp(G)
            assert np.allclose((np.eye(n) + A) @ rec["W"][c, h][:n], rhs, atol=1e-13)
            assert np.allclose(rec["Gamma"][c, h], np.exp(G[-1]), rtol=1e-14)
    assert np.allclose(rec["S0"][0], 0.0)


# --------------------------------------------------------------------------
# Rectangular state (d_k != d_v): reduced to the square recurrence by
# zero-padding, which adds only exact zeros to every sum.
# --------------------------------------------------------------------------

def _rect_inputs(T, H, dk, dv, seed, cu):
    r = _rng(seed)
    return dict(q=r.standard_normal((T, H, dk)), k=r.standard_normal((T, H, dk)),
                v=r.standard_normal((T, H, dv)), f_raw=r.standard_normal((T, H, dk)),
                b_raw=r.standard_normal((T, H)), A_log=r.uniform(0, math.log(16), H),
                dt_bias=0.5 * r.standard_normal((H, dk)), cu_seqlens=np.asarray(cu, dtype=np.int32))


def _pad(a, n, axis=-1):
    w = [(0, 0)] * a.ndim
    w[axis] = (0, n - a.shape[axis])
    return np.pad(a, w)


def test_rect_pad_keys_to_square():
    """dk = 16 < dv = 24 (the pages' failing rectangular case): padding q, k,
    f_raw, dt_bias (and the start state's key rows) with zeros to 24 gives the
    square recurrence the same outputs and final state."""
    cu = [0, 5, 5, 40]
    x = _rect_inputs(40, 2, 16, 24, 91, cu)
    S0 = _rng(92).standard_normal((3, 2, 16, 24))
    out, fin = oracle.kda_forward_rect(**x, scale=0.25, initial_state=S0, return_final_state=True)
    sq = dict(x)
    for key in ("q", "k", "f_raw"):
        sq[key] = _pad(x[key], 24)
    sq["dt_bias"] = _pad(x["dt_bias"], 24)
    out2, fin2 = oracle.kda_forward(**sq, scale=0.25, initial_state=_pad(S0, 24, axis=2),
                                    return_final_state=True)
    assert np.allclose(out, out2, rtol=1e-14, atol=1e-15)
    assert np.allclose(fin, fin2[:, :, :16, :], rtol=1e-14, atol=1e-15)
    assert np.all(fin2[:, :, 16:, :] == 0.0)


def test_rect_pad_values_to_square():
    """dk = 32 > dv = 16: padding v (and the start state's value columns) with
    zeros to 32 adds zero output columns and leaves the others unchanged."""
    cu = [0, 33, 70]
    x = _rect_inputs(70, 2, 32, 16, 93, cu)
    S0 = _rng(94).standard_normal((2, 2, 32, 16))
    out, fin = oracle.kda_forward_rect(**x, initial_state=S0, return_final_state=True)
    sq = dict(x)
    sq["v"] = _pad(x["v"], 32)
    out2, fin2 = oracle.kda_forward(**sq, scale=1 / math.sqrt(32), initial_state=_pad(S0, 32, axis=3),
                                    return_final_state=True)
    assert np.allclose(out, out2[..., :16], rtol=1e-14, atol=1e-15)
    assert np.all(out2[..., 16:] == 0.0)
    assert np.allclose(fin, fin2[..., :16], rtol=1e-14, atol=1e-15)


def test_rect_single_token_closed_form():
    x = _rect_inputs(1, 3, 16, 24, 95, [0, 1])
    out = oracle.kda_forward_rect(**x, eps=0.0)
    for h in range(3):
        qn = x["q"][0, h] / np.linalg.norm(x["q"][0, h])
        kn = x["k"][0, h] / np.linalg.norm(x["k"][0, h])
        beta = 1 / (1 + math.exp(-x["b_raw"][0, h]))
        assert np.allclose(out[0, h], 0.25 * beta * (kn @ qn) * x["v"][0, h], rtol=1e-13, atol=1e-15)
