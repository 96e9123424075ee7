"""FP64 CPU oracle for the KDA chunked forward -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``kda_oracle.c`` (plain C,
FP64, OpenMP over (sequence, head) pairs) through ctypes.  Nothing here is
shared with, imported by, or imported from the GPU library.

Functions follow the definitions written at the top of ``kda_oracle.c``: the
token-serial KDA recurrence (the serving-side FP32 recurrence the training
chunk path is compared against in xtuner PR #2301 "[Enhancement] Add opt-in
FP32 KDA chunk computation", sections Problem and Validation) and an FP64 chunk
form with exposed intermediates.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None

# Deliberate-mistake switches (see kda_oracle.c); used only by the pin tests.
PLANT = {
    "no_decay": 1 << 0,
    "delta_undecayed": 1 << 1,
    "read_before_write": 1 << 2,
    "transposed_read": 1 << 3,
    "delta_sign": 1 << 4,
    "no_beta": 1 << 5,
    "no_reset": 1 << 6,
    "no_l2norm": 1 << 7,
    "no_softplus": 1 << 8,
    "gate_sign": 1 << 9,
    "no_scale": 1 << 10,
    "outer_swap": 1 << 11,
    "drop_carry_64": 1 << 12,
    "init_transposed": 1 << 13,
    "final_early": 1 << 14,
}
# Deliberate mistakes of the backward (kda_oracle_bwd_rect).
BWD_PLANT = {
    "bwd_beta_scale": 1 << 17,
    "bwd_no_state_decay": 1 << 18,
    "bwd_no_norm_proj": 1 << 19,
    "bwd_gate_no_sigmoid": 1 << 20,
}
# Deliberate mistakes of the short convolution (kda_oracle_short_conv).
CONV_PLANT = {
    "conv_no_reset": 1 << 15,
    "conv_taps_reversed": 1 << 16,
}
# Deliberate mistakes of its backward (kda_oracle_short_conv_vjp).
CONVB_PLANT = {
    "convb_no_silu_deriv": 1 << 21,
    "convb_taps_forward": 1 << 22,
}


def build(force: bool = False) -> str:
    """Compile kda_oracle.c into libkda_oracle.so next to it (gcc -O2 -fopenmp)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    lib = ctypes.CDLL(build())
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.kda_oracle_fwd.restype = ctypes.c_int
    lib.kda_oracle_fwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, ip, ctypes.c_int, ctypes.c_int64,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_double, ctypes.c_double, ctypes.c_uint, dp, dp, dp]
    lib.kda_oracle_fwd_rect.restype = ctypes.c_int
    lib.kda_oracle_fwd_rect.argtypes = [dp, dp, dp, dp, dp, dp, dp, ip, ctypes.c_int,
                                        ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                        ctypes.c_double, ctypes.c_uint, dp, dp, dp]
    lib.kda_oracle_chunked.restype = ctypes.c_int
    lib.kda_oracle_chunked.argtypes = [dp, dp, dp, dp, dp, dp, dp, ip, ctypes.c_int, ctypes.c_int64,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_double, ctypes.c_double, ctypes.c_int, dp, dp, dp,
                                       dp]
    lib.kda_oracle_prep.restype = None
    lib.kda_oracle_prep.argtypes = [dp, dp, dp, dp, dp, dp, ctypes.c_int64, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_double, dp, dp, dp, dp]
    lib.kda_oracle_num_chunks.restype = ctypes.c_int64
    lib.kda_oracle_num_chunks.argtypes = [ip, ctypes.c_int, ctypes.c_int]
    lib.kda_oracle_chunk_record_len.restype = ctypes.c_int64
    lib.kda_oracle_chunk_record_len.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.kda_oracle_short_conv.restype = ctypes.c_int
    lib.kda_oracle_short_conv.argtypes = [dp, ip, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                          ctypes.c_int, dp, dp, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_uint]
    lib.kda_oracle_short_conv_vjp.restype = ctypes.c_int
    lib.kda_oracle_short_conv_vjp.argtypes = [dp, dp, ip, ctypes.c_int, ctypes.c_int64,
                                              ctypes.c_int, ctypes.c_int, dp, dp, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_uint, dp, dp, dp]
    lib.kda_oracle_bwd_rect.restype = ctypes.c_int
    lib.kda_oracle_bwd_rect.argtypes = [dp, dp, dp, dp, dp, dp, dp, ip, ctypes.c_int,
                                        ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_double, ctypes.c_double, ctypes.c_uint, dp, dp,
                                        dp, dp, dp, dp, dp, dp, dp, dp, dp]
    lib.kda_oracle_num_threads.restype = ctypes.c_int
    lib.kda_oracle_num_threads.argtypes = []
    lib.kda_oracle_set_num_threads.restype = None
    lib.kda_oracle_set_num_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, ct=ctypes.c_double):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def _check_shapes(q, k, v, f, b, A_log, dt_bias, cu):
    T, H, d = q.shape
    for x in (k, v, f):
        assert x.shape == (T, H, d), x.shape
    assert b.shape == (T, H) and A_log.shape == (H,) and dt_bias.shape == (H, d)
    assert cu.ndim == 1 and cu[0] == 0 and cu[-1] == T
    return T, H, d


def kda_forward_rect(q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, scale=None, eps=1e-6,
                     plant=0, initial_state=None, return_final_state=False):
    """Token-serial FP64 KDA forward with a rectangular state: q, k, f_raw
    [T, H, dk], dt_bias [H, dk], v [T, H, dv]; returns out [T, H, dv] (and the
    final state [N, H, dk, dv]).  scale defaults to 1/sqrt(dk)."""
    lib = _load()
    q, k, v, f_raw, b_raw, A_log, dt_bias = map(_f64, (q, k, v, f_raw, b_raw, A_log, dt_bias))
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    T, H, dk = q.shape
    dv = v.shape[2]
    assert k.shape == q.shape and f_raw.shape == q.shape and v.shape == (T, H, dv)
    assert b_raw.shape == (T, H) and A_log.shape == (H,) and dt_bias.shape == (H, dk)
    N = len(cu) - 1
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    out = np.zeros((T, H, dv), dtype=np.float64)
    init = None if initial_state is None else _f64(initial_state)
    if init is not None:
        assert init.shape == (N, H, dk, dv), init.shape
    fin = np.zeros((N, H, dk, dv), dtype=np.float64) if return_final_state else None
    rc = lib.kda_oracle_fwd_rect(_ptr(q), _ptr(k), _ptr(v), _ptr(f_raw), _ptr(b_raw), _ptr(A_log),
                                 _ptr(dt_bias), _ptr(cu, ctypes.c_int32), N, T, H, dk, dv, 0, H,
                                 float(scale), float(eps), int(plant),
                                 _ptr(init) if init is not None else None,
                                 _ptr(fin) if fin is not None else None, _ptr(out))
    if rc != 0:
        raise ValueError("kda_oracle_fwd_rect rejected its arguments")
    return (out, fin) if return_final_state else out


def _states(initial_state, return_final_state, N, H, d):
    init = None
    if initial_state is not None:
        init = _f64(initial_state)
        assert init.shape == (N, H, d, d), init.shape
    fin = np.zeros((N, H, d, d), dtype=np.float64) if return_final_state else None
    return init, fin


def kda_forward(q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, scale=None, eps=1e-6,
                heads=None, plant=0, out=None, initial_state=None, return_final_state=False):
    """Token-serial FP64 KDA forward.  Inputs are any real arrays (converted to
    float64 exactly); returns out [T, H, d] float64.  ``heads=(lo, hi)`` limits
    the computation to a head range (other heads' rows stay zero / as given).
    ``initial_state`` [N, H, d, d] (key, value) starts each sequence from the
    given state; with ``return_final_state`` the result is (out, final_state)."""
    lib = _load()
    q, k, v, f_raw, b_raw, A_log, dt_bias = map(_f64, (q, k, v, f_raw, b_raw, A_log, dt_bias))
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    T, H, d = _check_shapes(q, k, v, f_raw, b_raw, A_log, dt_bias, cu)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    lo, hi = (0, H) if heads is None else heads
    if out is None:
        out = np.zeros((T, H, d), dtype=np.float64)
    init, fin = _states(initial_state, return_final_state, len(cu) - 1, H, d)
    rc = lib.kda_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(f_raw), _ptr(b_raw), _ptr(A_log),
                            _ptr(dt_bias), _ptr(cu, ctypes.c_int32), len(cu) - 1, T, H, d, lo, hi,
                            float(scale), float(eps), int(plant),
                            _ptr(init) if init is not None else None,
                            _ptr(fin) if fin is not None else None, _ptr(out))
    if rc != 0:
        raise ValueError("kda_oracle_fwd rejected its arguments")
    return (out, fin) if return_final_state else out


def kda_chunked(q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, chunk=64, scale=None,
                eps=1e-6, heads=None, records=False, initial_state=None, return_final_state=False):
    """FP64 chunk-form forward.  Returns out, or (out, rec) with rec a dict of
    per-(chunk, head) intermediates shaped [num_chunks, H, ...]; with
    ``return_final_state`` the final state [N, H, d, d] is appended."""
    lib = _load()
    q, k, v, f_raw, b_raw, A_log, dt_bias = map(_f64, (q, k, v, f_raw, b_raw, A_log, dt_bias))
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    T, H, d = _check_shapes(q, k, v, f_raw, b_raw, A_log, dt_bias, cu)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    lo, hi = (0, H) if heads is None else heads
    C = int(chunk)
    out = np.zeros((T, H, d), dtype=np.float64)
    rec = None
    if records:
        nc = lib.kda_oracle_num_chunks(_ptr(cu, ctypes.c_int32), len(cu) - 1, C)
        RL = lib.kda_oracle_chunk_record_len(C, d)
        rec = np.zeros((nc, H, RL), dtype=np.float64)
    init, fin = _states(initial_state, return_final_state, len(cu) - 1, H, d)
    rc = lib.kda_oracle_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(f_raw), _ptr(b_raw), _ptr(A_log),
                                _ptr(dt_bias), _ptr(cu, ctypes.c_int32), len(cu) - 1, T, H, d, lo,
                                hi, float(scale), float(eps), C,
                                _ptr(init) if init is not None else None,
                                _ptr(fin) if fin is not None else None, _ptr(out),
                                _ptr(rec) if rec is not None else None)
    if rc != 0:
        raise ValueError("kda_oracle_chunked rejected its arguments")
    if not records:
        return (out, fin) if return_final_state else out
    parts = {}
    off = 0
    for name, shape in (("G", (C, d)), ("beta", (C,)), ("A", (C, C)), ("P", (C, C)),
                        ("W", (C, d)), ("U", (C, d)), ("Qt", (C, d)), ("Kb", (C, d)),
                        ("Gamma", (d,)), ("S0", (d, d))):
        n = int(np.prod(shape))
        parts[name] = rec[:, :, off:off + n].reshape(rec.shape[:2] + shape)
        off += n
    return (out, parts, fin) if return_final_state else (out, parts)


def kda_prep(q, k, f_raw, b_raw, A_log, dt_bias, eps=1e-6):
    """Stage-one quantities: (q^, k^, g, beta) for every token-head, FP64."""
    lib = _load()
    q, k, f_raw, b_raw, A_log, dt_bias = map(_f64, (q, k, f_raw, b_raw, A_log, dt_bias))
    T, H, d = q.shape
    qn = np.empty_like(q)
    kn = np.empty_like(k)
    g = np.empty_like(f_raw)
    beta = np.empty((T, H), dtype=np.float64)
    lib.kda_oracle_prep(_ptr(q), _ptr(k), _ptr(f_raw), _ptr(b_raw), _ptr(A_log), _ptr(dt_bias),
                        T, H, d, float(eps), _ptr(qn), _ptr(kn), _ptr(g), _ptr(beta))
    return qn, kn, g, beta


def short_conv(x, cu_seqlens, weight, bias=None, silu=True, round_bf16=False, plant=0):
    """Short causal convolution of one activation tensor x [T, H, d] (FP64
    result): y_t = act(bias + sum_i weight[:, i] x_{t-K+1+i}), zero history at
    every sequence start, act = SiLU or identity, optionally rounded to
    bfloat16.  weight is [H*d, K] (last tap = current token), bias [H*d]."""
    lib = _load()
    y = _f64(x).copy()
    T, H, d = y.shape
    w = _f64(weight).reshape(H * d, -1)
    K = w.shape[1]
    b = None if bias is None else _f64(bias).reshape(H * d)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    rc = lib.kda_oracle_short_conv(_ptr(y), _ptr(cu, ctypes.c_int32), len(cu) - 1, T, H, d, _ptr(w),
                                   _ptr(b) if b is not None else None, K, int(bool(silu)),
                                   int(bool(round_bf16)), int(plant))
    if rc != 0:
        raise ValueError("kda_oracle_short_conv rejected its arguments")
    return y


def short_conv_vjp(x, dy, cu_seqlens, weight, bias=None, silu=True, plant=0):
    """Vector-Jacobian product of short_conv (without rounding): for
    L = <dy, short_conv(x)>, returns (dx [T, H, d], dweight [H*d, K],
    dbias [H*d]), FP64.  See kda_oracle_short_conv_vjp."""
    lib = _load()
    x = _f64(x)
    dy = _f64(dy)
    T, H, d = x.shape
    assert dy.shape == x.shape
    w = _f64(weight).reshape(H * d, -1)
    K = w.shape[1]
    b = None if bias is None else _f64(bias).reshape(H * d)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    dx = np.zeros_like(x)
    dw = np.zeros_like(w)
    db = np.zeros(H * d)
    rc = lib.kda_oracle_short_conv_vjp(_ptr(x), _ptr(dy), _ptr(cu, ctypes.c_int32), len(cu) - 1, T,
                                       H, d, _ptr(w), _ptr(b) if b is not None else None, K,
                                       int(bool(silu)), int(plant), _ptr(dx), _ptr(dw), _ptr(db))
    if rc != 0:
        raise ValueError("kda_oracle_short_conv_vjp rejected its arguments")
    return dx, dw, db


def kda_backward(q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, dout, scale=None, eps=1e-6,
                 initial_state=None, dfinal_state=None, plant=0):
    """FP64 vector-Jacobian product of the token recurrence (rectangular state
    allowed: q, k, f_raw [T, H, dk], v and dout [T, H, dv]).  For the loss
    L = <dout, out> + <dfinal_state, final_state> it returns a dict with dq,
    dk, dv, df (= dL/df_raw), db (= dL/db_raw), dA_log [H], ddt_bias [H, dk]
    and dinit [N, H, dk, dv] (dL/d initial state; zero start if none given)."""
    lib = _load()
    q, k, v, f_raw, b_raw, A_log, dt_bias, dout = map(
        _f64, (q, k, v, f_raw, b_raw, A_log, dt_bias, dout))
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    T, H, dk = q.shape
    dv = v.shape[2]
    assert k.shape == q.shape and f_raw.shape == q.shape and v.shape == (T, H, dv)
    assert dout.shape == (T, H, dv)
    assert b_raw.shape == (T, H) and A_log.shape == (H,) and dt_bias.shape == (H, dk)
    N = len(cu) - 1
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    init = None if initial_state is None else _f64(initial_state)
    dfin = None if dfinal_state is None else _f64(dfinal_state)
    for x in (init, dfin):
        if x is not None:
            assert x.shape == (N, H, dk, dv), x.shape
    r = {"dq": np.zeros((T, H, dk)), "dk": np.zeros((T, H, dk)), "dv": np.zeros((T, H, dv)),
         "df": np.zeros((T, H, dk)), "db": np.zeros((T, H)), "dA_log": np.zeros(H),
         "ddt_bias": np.zeros((H, dk)), "dinit": np.zeros((N, H, dk, dv))}
    opt = lambda x: _ptr(x) if x is not None else None
    rc = lib.kda_oracle_bwd_rect(_ptr(q), _ptr(k), _ptr(v), _ptr(f_raw), _ptr(b_raw), _ptr(A_log),
                                 _ptr(dt_bias), _ptr(cu, ctypes.c_int32), N, T, H, dk, dv,
                                 float(scale), float(eps), int(plant), opt(init), _ptr(dout),
                                 opt(dfin), _ptr(r["dq"]), _ptr(r["dk"]), _ptr(r["dv"]),
                                 _ptr(r["df"]), _ptr(r["db"]), _ptr(r["dA_log"]),
                                 _ptr(r["ddt_bias"]), _ptr(r["dinit"]))
    if rc != 0:
        raise ValueError("kda_oracle_bwd_rect rejected its arguments")
    return r


def num_threads() -> int:
    return int(_load().kda_oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads used by the following oracle calls (timing only: each (sequence,
    head) pair is computed by one thread, so results do not depend on it)."""
    _load().kda_oracle_set_num_threads(int(n))
