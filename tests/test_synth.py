"""The seeded generators reproduce the pages' workload shapes and the stated
distributions; bfloat16 rounding is round-to-nearest-even."""
import json
import math
import os

import numpy as np

from chunked_gated_delta_07_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5, 0.0,
                  3.0e38, 1e-40], dtype=np.float32)
    b = synth.f32_to_bf16_bits(x)
    back = synth.bf16_bits_to_f32(b)
    # ties to even: 1+2^-8 is halfway between 1 and 1+2^-7 -> 1 ; 1+3*2^-8 -> 1+2^-6
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == np.float32(1.0 + 2 ** -6)
    assert back[3] == np.float32(1.0 + 2 ** -7)
    assert back[4] == -2.5 and back[5] == 0.0
    # every bf16 value is exactly representable: a second rounding is the identity
    assert np.array_equal(synth.f32_to_bf16_bits(back), b)


def test_configs_match_pages_fixtures():
    with open(os.path.join(GOLDEN, "pages_workloads.json")) as fh:
        g = json.load(fh)
    cus = [list(c["cu"]) for c in synth.CONFIGS.values() if c.get("cu") is not None]
    for fx in g["fixtures"]:
        assert fx["cu_seqlens"] in cus
    assert synth.H_DEFAULT == g["heads"] and synth.D_DEFAULT == g["head_dim"]


def test_distributions_and_determinism():
    x = synth.make_inputs([0, 4096], H=4, d=128, act="fp32", seed=3)
    y = synth.make_inputs([0, 4096], H=4, d=128, act="fp32", seed=3)
    assert np.array_equal(x.q, y.q) and np.array_equal(x.dt_bias, y.dt_bias)
    for a in (x.q, x.k, x.v, x.f_raw, x.b_raw):
        assert abs(a.mean()) < 0.02 and abs(a.std() - 1.0) < 0.02
    assert 0.0 <= x.A_log.min() and x.A_log.max() <= math.log(16.0)
    assert abs(x.dt_bias.std() - 0.5) < 0.05


def test_ragged_config_lengths():
    inp = synth.config_inputs(4, H=1, d=8)
    cu = inp.cu_seqlens
    lens = np.diff(cu)
    assert cu[0] == 0 and cu[-1] == 65536
    assert lens.min() >= 1 and lens.max() <= 8192
    assert inp.act == "bf16" and inp.q.dtype == np.uint16
