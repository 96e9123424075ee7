"""Seeded synthetic inputs for the KDA chunked forward.

This module only draws random numbers and converts them to storage formats;
it holds none of the method's arithmetic.  The same arrays feed both the GPU
library and the CPU oracle, so both sides see identical bits.

Workloads follow the pages' fixtures and timing shapes: 64 heads x 128 dims
(xtuner PR #2301 "[Enhancement] Add opt-in FP32 KDA chunk computation",
sections Problem and Validation), packed lengths 37/28 and a 129-token chunk
boundary case (same page, Validation), and 2048 / 16384-token operator timings
(same page, timing table).

Recipe (all inputs drawn in float32 with numpy PCG64, seed given per config):
lengths first (ragged configs only), then q, k, v, f_raw ~ N(0,1) of shape
[T,H,d], b_raw ~ N(0,1) of shape [T,H], A_log ~ U(0, ln 16) of shape [H],
dt_bias ~ N(0, 0.5^2) of shape [H,d].  Activations are then rounded
to the activation dtype (bfloat16 by round-to-nearest-even, or kept float32);
A_log and dt_bias stay float32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

H_DEFAULT = 64
D_DEFAULT = 128


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite values are at most 0xFF7FFFFF, so adding 0x8000 cannot wrap
    bias = (u >> np.uint32(16)) & np.uint32(1)
    bias += np.uint32(0x7FFF)
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class KdaInputs:
    """Host copies of one workload.  Activation arrays are uint16 (bf16 bits)
    when act == 'bf16', else float32."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    f_raw: np.ndarray
    b_raw: np.ndarray
    A_log: np.ndarray
    dt_bias: np.ndarray
    cu_seqlens: np.ndarray
    act: str

    @property
    def T(self):
        return self.q.shape[0]

    @property
    def H(self):
        return self.q.shape[1]

    @property
    def d(self):
        return self.q.shape[2]

    def as_f64(self):
        """All inputs as float64 (exact conversion of the stored values)."""
        conv = (lambda a: bf16_bits_to_f32(a).astype(np.float64)) if self.act == "bf16" else (
            lambda a: a.astype(np.float64))
        return dict(q=conv(self.q), k=conv(self.k), v=conv(self.v), f_raw=conv(self.f_raw),
                    b_raw=conv(self.b_raw), A_log=self.A_log.astype(np.float64),
                    dt_bias=self.dt_bias.astype(np.float64), cu_seqlens=self.cu_seqlens.copy())


def ragged_lengths(rng: np.random.Generator, total: int, lo: int, hi: int) -> np.ndarray:
    """Lengths drawn uniformly from [lo, hi] until the sum reaches total; the
    last length is trimmed so the lengths sum to exactly total."""
    out = []
    s = 0
    while s < total:
        L = int(rng.integers(lo, hi + 1))
        L = min(L, total - s)
        out.append(L)
        s += L
    return np.asarray(out, dtype=np.int64)


def make_inputs(cu_seqlens, H=H_DEFAULT, d=D_DEFAULT, act="bf16", seed=0,
                rng: np.random.Generator | None = None) -> KdaInputs:
    cu = np.asarray(cu_seqlens, dtype=np.int32)
    T = int(cu[-1])
    if rng is None:
        rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, d), dtype=np.float32)
    k = rng.standard_normal((T, H, d), dtype=np.float32)
    v = rng.standard_normal((T, H, d), dtype=np.float32)
    f = rng.standard_normal((T, H, d), dtype=np.float32)
    b = rng.standard_normal((T, H), dtype=np.float32)
    A_log = rng.uniform(0.0, math.log(16.0), size=(H,)).astype(np.float32)
    dt_bias = (0.5 * rng.standard_normal((H, d), dtype=np.float32)).astype(np.float32)
    if act == "bf16":
        q, k, v, f, b = (f32_to_bf16_bits(a) for a in (q, k, v, f, b))
    elif act != "fp32":
        raise ValueError(act)
    return KdaInputs(q, k, v, f, b, A_log, dt_bias, cu, act)


def rect_inputs(cu_seqlens, H, dk, dv, seed, act="bf16") -> dict:
    """Inputs with a rectangular state: q, k, f_raw [T,H,dk], v [T,H,dv],
    b_raw [T,H], A_log [H], dt_bias [H,dk], all float32 (activations rounded
    to bf16 values when act == 'bf16'), drawn in that order with the
    distributions of make_inputs."""
    cu = np.asarray(cu_seqlens, dtype=np.int32)
    T = int(cu[-1])
    r = np.random.default_rng(seed)

    def act_round(a):
        a = a.astype(np.float32)
        return bf16_bits_to_f32(f32_to_bf16_bits(a)) if act == "bf16" else a

    return dict(q=act_round(r.standard_normal((T, H, dk))),
                k=act_round(r.standard_normal((T, H, dk))),
                v=act_round(r.standard_normal((T, H, dv))),
                f_raw=act_round(r.standard_normal((T, H, dk))),
                b_raw=act_round(r.standard_normal((T, H))),
                A_log=r.uniform(0, np.log(16), H).astype(np.float32),
                dt_bias=(0.5 * r.standard_normal((H, dk))).astype(np.float32),
                cu_seqlens=cu)


# The five workloads.  cfg 0/1 are small parity cases, 2 a scaling point, 3 the
# headline 16K-token case, 4 a ragged packed batch.
CONFIGS = {
    0: dict(name="kda_fwd_129tok_fp32", cu=[0, 129], act="fp32", modes=("fp32",)),
    1: dict(name="kda_fwd_varlen_37_28_bf16", cu=[0, 37, 65], act="bf16", modes=("bf16", "fp32")),
    2: dict(name="kda_fwd_2048tok_bf16", cu=[0, 2048], act="bf16", modes=("bf16", "fp32")),
    3: dict(name="kda_fwd_16384tok_bf16", cu=[0, 16384], act="bf16", modes=("bf16", "fp32")),
    4: dict(name="kda_fwd_ragged_65536tok_bf16", cu=None, act="bf16", modes=("fp32",),
            ragged=(65536, 1, 8192)),
}


def config_inputs(i: int, H=H_DEFAULT, d=D_DEFAULT) -> KdaInputs:
    c = CONFIGS[i]
    rng = np.random.default_rng(1000 + i)
    if c.get("cu") is None:
        total, lo, hi = c["ragged"]
        lens = ragged_lengths(rng, total, lo, hi)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    else:
        cu = np.asarray(c["cu"], dtype=np.int32)
    return make_inputs(cu, H=H, d=d, act=c["act"], rng=rng)
