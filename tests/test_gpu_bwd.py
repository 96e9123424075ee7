"""GPU parity of kda_chunk_bwd (the FP32-recomputed backward) against the FP64
oracle's vector-Jacobian product of the token recurrence.

The pages check the chunked operator's input gradients against an FP64
recurrence VJP written apart from the kernels, on two packed sequences of 37
and 28 tokens, on a 129-token sequence that crosses chunk boundaries and on all
64 heads of width 128 at 65 tokens; each gradient that is not zero must stay
within 2 % relative error, and a gradient scaled by 25 % on purpose must be
caught (xtuner PR #2301, section Validation); FP32 budgets of 0.3 % (dq, dk, dv) and
0.5 % (gate, beta) are quoted in xtuner PR #2153.  Bars here, relative L2 over
each whole gradient tensor:
  * FP32 gradients (FP32 activations, or bf16 activations with KDA_OUT_FP32):
    1e-4 -- the forward's FP32 bar; the backward's arithmetic is FP32 with
    sums of at most a few hundred terms per output, far below it;
  * bf16 gradients: 2e-2, the pages' BF16 budget (rounding of a correct
    result to bf16 alone costs ~2e-3);
  * the parameter gradients dA_log and dt_bias (FP32 sums over every token
    and channel of a head): 1e-3.  Their terms cancel -- sum|term| / |sum| is
    ~330 at 2048 tokens and ~670 at 8192 (it grows like sqrt(T)) -- so FP32
    rounding of ~2e-7 per term becomes ~1e-4 of the sum at 64K tokens; the
    pages' FP32 budget for the gate gradient is 0.5 % and their worst FP32
    parameter-gradient error 0.374 % (xtuner PR #2153, KDA module section).
"""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(__file__))
import kda_testutil as U  # noqa: E402

import oracle  # noqa: E402
from chunked_gated_delta_07_amd import synth  # noqa: E402

pytestmark = pytest.mark.gpu

TOL_FP32 = 1e-4
TOL_BF16 = 2e-2
TOL_PARAM = 1e-3
PARAMS = ("dA_log", "ddt_bias")
KEYS = ("dq", "dk", "dv", "df", "db", "dA_log", "ddt_bias")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from chunked_gated_delta_07_amd import kda

    kda.load_library()
    yield


def _case(lens, H, act, seed, with_states=True, grad_fp32=True):
    """Seeded inputs, dout (rounded to its dtype) and optional states."""
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    inp = synth.make_inputs(cu, H=H, act=act, seed=seed)
    rng = np.random.default_rng(seed + 7)
    T, N = int(cu[-1]), len(lens)
    dout = rng.standard_normal((T, H, 128)).astype(np.float32)
    if not grad_fp32:
        dout = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(dout))
    init = dfin = None
    if with_states:
        init = (0.3 * rng.standard_normal((N, H, 128, 128))).astype(np.float32)
        dfin = rng.standard_normal((N, H, 128, 128)).astype(np.float32)
    return inp, dout, init, dfin


def _gpu_bwd(inp, dout, init, dfin, grad_fp32, heads=None):
    """GPU gradients as float64 numpy; with ``heads`` only those heads are
    copied back (per-head arrays keep their head axis)."""
    import torch

    from chunked_gated_delta_07_amd import kda

    dev = "cuda:0"
    args = U.to_device(inp, dev)
    dt = torch.float32 if (grad_fp32 or inp.act == "fp32") else torch.bfloat16
    g = kda.chunk_bwd(*args, torch.from_numpy(dout).to(dev).to(dt), out_fp32=grad_fp32,
                      initial_state=None if init is None else torch.from_numpy(init).to(dev),
                      dfinal_state=None if dfin is None else torch.from_numpy(dfin).to(dev),
                      return_dinitial_state=True)
    torch.cuda.synchronize()
    if heads is not None:
        hd = torch.as_tensor(heads, device=dev)
        g = {k: (v.index_select(0, hd) if k in ("dA_log", "ddt_bias") else v.index_select(1, hd))
             for k, v in g.items()}
    return {k: v.to(torch.float64).cpu().numpy() for k, v in g.items()}


def _oracle_bwd(inp, dout, init, dfin, plant=0):
    x = inp.as_f64()
    return oracle.kda_backward(x["q"], x["k"], x["v"], x["f_raw"], x["b_raw"], x["A_log"],
                               x["dt_bias"], x["cu_seqlens"], dout.astype(np.float64),
                               initial_state=init, dfinal_state=dfin, plant=plant)


def _errors(got, ref, keys=KEYS + ("dinit",)):
    return {k: U.rel_l2(got[k], ref[k]) for k in keys if k in got}


def _check(got, ref, tol, label):
    errs = _errors(got, ref)
    print(label, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, e in errs.items():
        assert np.all(np.isfinite(got[k])), (label, k)
        assert e < (max(tol, TOL_PARAM) if k in PARAMS else tol), (label, k, e)
    return errs


@pytest.mark.parametrize("act", ["fp32", "bf16"])
def test_bwd_parity_packed_37_28(act):
    """The pages' packed lengths 37/28, with start states and a final-state
    gradient; FP32 gradients."""
    inp, dout, init, dfin = _case([37, 28], 4, act, seed=1)
    _check(_gpu_bwd(inp, dout, init, dfin, True), _oracle_bwd(inp, dout, init, dfin), TOL_FP32,
           f"37/28 {act}")


def test_bwd_parity_chunk_boundary_129():
    """129 tokens: chunks of 64, 64 and 1 (FP32 activations, zero start)."""
    inp, dout, _, _ = _case([129], 4, "fp32", seed=2, with_states=False)
    _check(_gpu_bwd(inp, dout, None, None, True), _oracle_bwd(inp, dout, None, None), TOL_FP32,
           "129")


def test_bwd_parity_ragged_multi_chunk():
    """Several chunks per sequence, ragged tails, an empty and a one-token
    sequence, with states."""
    inp, dout, init, dfin = _case([300, 1, 0, 64, 130, 65], 3, "bf16", seed=3)
    _check(_gpu_bwd(inp, dout, init, dfin, True), _oracle_bwd(inp, dout, init, dfin), TOL_FP32,
           "ragged")


def test_bwd_production_geometry_65_tokens():
    """64 heads x 128 at 65 tokens (37/28), bf16 activations: FP32 gradients
    to the FP32 bar and bf16 gradients to the pages' 2 % budget."""
    inp, dout, init, dfin = _case([37, 28], 64, "bf16", seed=4, with_states=False, grad_fp32=False)
    ref = _oracle_bwd(inp, dout, None, None)
    _check(_gpu_bwd(inp, dout, None, None, True), ref, TOL_FP32, "H64 fp32-grad")
    _check(_gpu_bwd(inp, dout, None, None, False), ref, TOL_BF16, "H64 bf16-grad")


def test_bwd_bf16_dout_split_products_match_fp32_dout():
    """With bf16 dout the value products run on bf16 matrix cores from split
    operands (dout exact as one bf16 piece, D, dD, S0, dSn as three); with
    FP32 dout the same products run in FP32.  On one bf16-exact dout the two
    paths agree to FP32 accuracy: the FP32 outputs (dA_log, dt_bias, dS_init)
    to 1e-5 relative, and each bf16 gradient is within one bf16 rounding step
    (2^-8, relative L2) of the FP32 path's gradient rounded to bf16.  (df is
    a running sum over the chunk, so where it nearly cancels, differences of
    FP32 size in larger terms flip its bf16 rounding; dA_log and dt_bias,
    which sum df's FP32 values, agree to ~3e-6.)  Against the oracle the
    split path's FP32 outputs meet the FP32 bars and its bf16 gradients the
    pages' BF16 budget."""
    inp, dout, init, dfin = _case([300, 1, 0, 64, 130, 65], 3, "bf16", seed=13, grad_fp32=False)
    got16 = _gpu_bwd(inp, dout, init, dfin, False)
    got32 = _gpu_bwd(inp, dout, init, dfin, True)
    ref = _oracle_bwd(inp, dout, init, dfin)
    for k in ("dinit",) + PARAMS:
        e_ref = U.rel_l2(got16[k], ref[k])
        e_fp32 = U.rel_l2(got16[k], got32[k])
        print("split", k, f"oracle {e_ref:.2e} fp32-path {e_fp32:.2e}", flush=True)
        assert e_ref < (TOL_PARAM if k in PARAMS else TOL_FP32), (k, e_ref)
        assert e_fp32 < 1e-5, (k, e_fp32)
    for k in ("dq", "dk", "dv", "df", "db"):
        b = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(got32[k].astype(np.float32)))
        e_path = U.rel_l2(got16[k], b)
        e_ref = U.rel_l2(got16[k], ref[k])
        print("split", k, f"equal {np.mean(got16[k] == b):.6f} vs fp32 path {e_path:.2e} "
              f"oracle {e_ref:.2e}", flush=True)
        assert e_path < 2.0 ** -8, (k, e_path)
        assert e_ref < TOL_BF16, (k, e_ref)


def test_bwd_planted_scale_error_fails():
    """The pages' negative control: a 25 % scaling of one gradient (in the
    oracle) is far outside the bar the GPU result meets."""
    inp, dout, init, dfin = _case([37, 28], 2, "fp32", seed=5)
    got = _gpu_bwd(inp, dout, init, dfin, True)
    bad = _oracle_bwd(inp, dout, init, dfin, plant=oracle.BWD_PLANT["bwd_beta_scale"])
    assert U.rel_l2(got["db"], bad["db"]) > 100 * TOL_FP32


def test_bwd_strong_gates_and_special_values():
    """Strong decay (A_log up to ln 64), saturated beta (b = +-inf) and a head
    with the gate switched off (A_log = -inf)."""
    inp, dout, init, dfin = _case([200, 70], 4, "fp32", seed=6)
    inp.A_log[:] = np.array([np.log(64.0), -np.inf, 0.0, np.log(16.0)], dtype=np.float32)
    inp.b_raw[5, 0] = np.inf
    inp.b_raw[100, 2] = -np.inf
    got = _gpu_bwd(inp, dout, init, dfin, True)
    ref = _oracle_bwd(inp, dout, init, dfin)
    _check(got, ref, TOL_FP32, "strong/special")
    assert got["db"][5, 0] == 0.0 and got["db"][100, 2] == 0.0
    assert np.all(got["df"][:, 1] == 0) and got["dA_log"][1] == 0.0


def test_bwd_empty_batch_and_zero_dout():
    import torch

    from chunked_gated_delta_07_amd import kda

    dev = "cuda:0"
    # T = 0: dS_init = dS_final, parameter gradients zero
    inp = synth.make_inputs(np.array([0, 0, 0], dtype=np.int32), H=2, act="bf16", seed=8)
    args = U.to_device(inp, dev)
    dfin = torch.randn(2, 2, 128, 128, device=dev)
    g = kda.chunk_bwd(*args, torch.empty((0, 2, 128), dtype=torch.bfloat16, device=dev),
                      dfinal_state=dfin)
    torch.cuda.synchronize()
    assert torch.equal(g["dinit"], dfin)
    assert torch.all(g["dA_log"] == 0) and torch.all(g["ddt_bias"] == 0)
    # zero output gradient and no final-state gradient: every gradient is zero
    inp = synth.make_inputs(np.array([0, 90], dtype=np.int32), H=2, act="fp32", seed=9)
    got = _gpu_bwd(inp, np.zeros((90, 2, 128), np.float32), None, None, True)
    for k in KEYS:
        assert np.all(got[k] == 0), k


def test_bwd_headline_size_sampled_heads():
    """The benchmark's workload (16384 tokens x 64 heads, bf16 activations, one
    call in the benchmark's launch configuration): heads 0 and 41 against the
    oracle (heads are independent, so the oracle runs on those two alone)."""
    import torch

    inp = U.config_inputs(3)
    T, H = inp.T, inp.H
    rng = np.random.default_rng(77)
    dout = synth.bf16_bits_to_f32(
        synth.f32_to_bf16_bits(rng.standard_normal((T, H, 128)).astype(np.float32)))
    heads = np.array([0, 41])
    got32 = _gpu_bwd(inp, dout, None, None, True, heads=heads)
    got16 = _gpu_bwd(inp, dout, None, None, False, heads=heads)
    torch.cuda.empty_cache()
    x = inp.as_f64()
    ref = oracle.kda_backward(x["q"][:, heads], x["k"][:, heads], x["v"][:, heads],
                              x["f_raw"][:, heads], x["b_raw"][:, heads], x["A_log"][heads],
                              x["dt_bias"][heads], x["cu_seqlens"],
                              dout[:, heads].astype(np.float64))
    for got, tol, lab in ((got32, TOL_FP32, "fp32-grad"), (got16, TOL_BF16, "bf16-grad")):
        got = {k: got[k] for k in KEYS}
        _check(got, ref, tol, f"16384x64 {lab}")


def test_bwd_ragged_65536_sampled_head():
    """The ragged packed workload (lengths U{1..8192} totalling 65536 tokens,
    64 heads, bf16): every sequence of head 23 against the oracle, FP32
    gradients, with the final-state gradient of every sequence."""
    import torch

    inp = U.config_inputs(4)
    T, H = inp.T, inp.H
    N = len(inp.cu_seqlens) - 1
    rng = np.random.default_rng(78)
    dout = rng.standard_normal((T, H, 128)).astype(np.float32)
    dfin = rng.standard_normal((N, H, 128, 128)).astype(np.float32)
    hd = np.array([23])
    got = _gpu_bwd(inp, dout, None, dfin, True, heads=hd)
    torch.cuda.empty_cache()
    x = inp.as_f64()
    ref = oracle.kda_backward(x["q"][:, hd], x["k"][:, hd], x["v"][:, hd], x["f_raw"][:, hd],
                              x["b_raw"][:, hd], x["A_log"][hd], x["dt_bias"][hd], x["cu_seqlens"],
                              dout[:, hd].astype(np.float64),
                              dfinal_state=dfin[:, hd].astype(np.float64))
    _check(got, ref, TOL_FP32, f"ragged 65536 ({N} seqs) head 23")


def test_bwd_mode_bit_changes_nothing():
    """KDA_MODE_FP32_INTERMEDIATE is accepted by kda_chunk_bwd and changes
    nothing: the backward recomputes in FP32 whatever the forward used.
    Called through the C ABI with the bit clear and set; bitwise equal."""
    import ctypes

    import torch

    from chunked_gated_delta_07_amd import kda

    inp, dout, init, dfin = _case([70, 30], 2, "bf16", seed=12, grad_fp32=False)
    dev = "cuda:0"
    args = U.to_device(inp, dev)
    T, H, N = inp.T, inp.H, 2
    lib = kda.load_library()
    d = torch.from_numpy(dout).to(dev).to(torch.bfloat16)
    ws = torch.empty(kda.bwd_workspace_bytes(T, N, H, 128, 1), dtype=torch.uint8, device=dev)
    outs = []
    for mode in (0, kda.KDA_MODE_FP32_INTERMEDIATE):
        g = [torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev) for _ in range(4)]
        g.append(torch.empty((T, H), dtype=torch.bfloat16, device=dev))
        par = [torch.empty(H, device=dev), torch.empty((H, 128), device=dev)]
        st = lib.kda_chunk_bwd(*[kda._ptr(a) for a in args], N, T, H, 128, mode, None, kda._ptr(d),
                               None, *[kda._ptr(x) for x in g], *[kda._ptr(x) for x in par], None,
                               kda._ptr(ws), ws.numel(),
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == kda.KDA_OK
        torch.cuda.synchronize()
        outs.append(g + par)
    for a, b in zip(*outs):
        assert torch.equal(a, b)
