"""GPU parity: libkda (through its C ABI) against the FP64 oracle.

Tolerances (whole-tensor relative L2, per-element max abs): FP32-intermediate
mode <= 1e-4 / <= 1e-3 on a float32 output; BF16-intermediate mode <= 1e-2,
checked both on a float32 output and on the bf16 output the benchmark times
(that output has its own pack-and-store code in the state pass).
Large workloads are compared on a sample of heads that the oracle computes in
seconds (heads are independent, so every sampled head is a full-size check).
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from chunked_gated_delta_07_amd import kda

    kda.load_library()  # raises if the library is missing: no fallback
    yield


def _check(inp, fp32, heads=None, out_fp32=True, label="", bf16_out=None):
    """GPU output vs the FP64 oracle on the given heads.  ``bf16_out`` (default:
    in BF16-intermediate mode) also runs the same call with the output cast to
    bf16 (the benched form of the path) and holds it to the same bar against
    the unrounded oracle."""
    heads = list(range(inp.H)) if heads is None else list(heads)
    ref = U.oracle_heads(inp, heads)
    if bf16_out is None:
        bf16_out = not fp32 and inp.act == "bf16"
    args = U.to_device(inp, "cuda:0")
    variants = [out_fp32] + ([False] if bf16_out and out_fp32 else [])
    result = None
    for o32 in variants:
        out = U.out_to_f64(U.run_gpu(inp, fp32, o32, args=args))
        got = out[:, heads]
        rel, mab = U.rel_l2(got, ref), U.max_abs(got, ref)
        print(f"[{label}] mode={'fp32' if fp32 else 'bf16'} out={'fp32' if o32 else 'bf16'} "
              f"heads={len(heads)} rel_l2={rel:.3e} max_abs={mab:.3e}", flush=True)
        assert np.all(np.isfinite(out))
        if fp32 and o32:
            assert rel <= U.TOL_FP32_REL and mab <= U.TOL_FP32_MAXABS, (rel, mab)
        else:
            # BF16 intermediates, or a bf16 output (whose rounding alone costs
            # ~1.7e-3 relative L2): the BF16 bar
            assert rel <= U.TOL_BF16_REL, rel
        if result is None:
            result = (out, ref)
    return result


def test_cfg0_129_tokens_fp32():
    inp = synth.config_inputs(0)
    _check(inp, fp32=True, label="cfg0")


@pytest.mark.parametrize("fp32", [False, True], ids=["bf16", "fp32"])
def test_cfg1_packed_37_28(fp32):
    inp = synth.config_inputs(1)
    _check(inp, fp32=fp32, label="cfg1")


def test_cfg1_fp32_mode_bf16_output():
    """FP32 intermediates with the output cast to bf16 (the pages' visible
    output dtype): compared with the oracle rounded to bf16; a few flips of
    the last bf16 bit are expected, so the bound is the bf16 half-ulp."""
    inp = synth.config_inputs(1)
    out = U.out_to_f64(U.run_gpu(inp, True, out_fp32=False))
    ref = U.bf16_round_f64(U.oracle_heads(inp, range(inp.H)))
    rel = U.rel_l2(out, ref)
    print(f"[cfg1 fp32 bf16-out] rel_l2 vs rounded oracle={rel:.3e}", flush=True)
    assert rel <= 2 ** -8


@pytest.mark.parametrize("fp32", [False, True], ids=["bf16", "fp32"])
def test_cfg2_2048_tokens(fp32):
    inp = U.config_inputs(2)
    _check(inp, fp32=fp32, label="cfg2")


@pytest.mark.parametrize("fp32", [False, True], ids=["bf16", "fp32"])
def test_cfg3_16384_tokens_all_heads(fp32):
    """The headline workload, every head, in the launch configuration the
    benchmark times (BF16: eight 32-chunk segments, bf16 output too)."""
    inp = U.config_inputs(3)
    _check(inp, fp32=fp32, label="cfg3")


@pytest.mark.parametrize("fp32", [False, True], ids=["bf16", "fp32"])
def test_cfg4_ragged_65536_tokens_sampled_heads(fp32):
    """19 ragged sequences (33 segments in BF16 mode, most boundaries inside
    a sequence); 16 heads spread over the workgroup-to-XCD mapping."""
    inp = U.config_inputs(4)
    _check(inp, fp32=fp32, heads=list(range(1, 64, 4)), label="cfg4")


@pytest.mark.parametrize("cu", [
    [0, 1], [0, 64], [0, 65], [0, 63, 64, 127], [0, 0, 5, 5, 70, 70],
    [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 200], [0, 128, 129, 257, 300],
    [0, 15, 31, 48, 79, 111, 144, 191, 239, 288],
], ids=lambda c: "cu" + "_".join(map(str, c)))
@pytest.mark.parametrize("fp32", [False, True], ids=["bf16", "fp32"])
def test_edge_lengths(cu, fp32):
    """1-token sequences, exact chunk multiples, a ragged tail, empty sequences,
    many short sequences, lengths on either side of the 16-token contraction
    steps and the 32-token tiles of P (15, 16, 17, 31, 32, 33, 47, 48, 49);
    H = 3 exercises an odd head count."""
    inp = synth.make_inputs(cu, H=3, d=128, act="bf16", seed=sum(cu))
    _check(inp, fp32=fp32, label=f"edge {cu}")


def test_fp32_activations_bf16_intermediates():
    inp = synth.make_inputs([0, 100, 190], H=2, d=128, act="fp32", seed=5)
    _check(inp, fp32=False, label="act fp32 / bf16 inter")


@pytest.mark.parametrize("fp32", [False, True], ids=["bf16", "fp32"])
def test_fp32_activations_long_packed(fp32):
    """FP32 activations over 2,500 + 1,100 tokens (57 chunks: two segments of
    the BF16 schedule, one pass in FP32 mode), three heads."""
    inp = synth.make_inputs([0, 2500, 3600], H=3, d=128, act="fp32", seed=6)
    _check(inp, fp32=fp32, label="act fp32 long")


def test_special_values():
    """A_log = -inf (no decay) on one head; b_raw = +-inf (beta exactly 1 / 0)
    on some tokens; large |f_raw| (gate saturation both ways)."""
    inp = synth.make_inputs([0, 150], H=4, d=128, act="fp32", seed=9)
    inp.A_log[1] = -np.inf
    inp.b_raw[::7, :] = np.inf
    inp.b_raw[3::11, :] = -np.inf
    inp.f_raw[::5, 2, :] = 30.0
    inp.f_raw[1::5, 3, :] = -30.0
    _check(inp, fp32=True, label="special")


def test_zero_tokens_is_noop():
    import torch

    from chunked_gated_delta_07_amd import kda

    dev = "cuda:0"
    e = torch.empty((0, 4, 128), dtype=torch.bfloat16, device=dev)
    out = kda.chunk_fwd(e, e, e, e, torch.empty((0, 4), dtype=torch.bfloat16, device=dev),
                        torch.zeros(4, device=dev), torch.zeros((4, 128), device=dev),
                        torch.zeros(2, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert out.shape == (0, 4, 128)


def test_deterministic_bitwise():
    import torch

    inp = U.config_inputs(2)
    args = U.to_device(inp, "cuda:0")
    for fp32 in (False, True):
        a = U.run_gpu(inp, fp32, False, args=args)
        b = U.run_gpu(inp, fp32, False, args=args)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_single_sequence_without_chunk_table_matches_table_path():
    """A single sequence is run without the chunk table (chunk c starts at token
    64 c); the same tokens packed with an empty second sequence take the table
    path.  Both map chunks to tokens alike, so the outputs and end states must
    be bitwise equal, in both precision modes, for a ragged length."""
    import torch

    from chunked_gated_delta_07_amd import kda

    inp = synth.make_inputs([0, 1000], H=8, d=128, act="bf16", seed=31)
    args = U.to_device(inp, "cuda:0")
    cu2 = torch.tensor([0, 1000, 1000], dtype=torch.int32, device="cuda:0")
    for fp32 in (False, True):
        a, fa = kda.chunk_fwd(*args, fp32_intermediate=fp32, out_fp32=True, return_final_state=True)
        b, fb = kda.chunk_fwd(*args[:7], cu2, fp32_intermediate=fp32, out_fp32=True,
                              return_final_state=True)
        torch.cuda.synchronize()
        print(f"[no-table vs table] mode={'fp32' if fp32 else 'bf16'}", flush=True)
        assert torch.equal(a, b)
        assert torch.equal(fa[0], fb[0])
        assert torch.count_nonzero(fb[1]) == 0  # the empty sequence's end state = its zero start


def test_negative_control_dropped_carry_fails():
    """A planted mistake (state reset every 64 tokens, planted in the oracle on
    the CPU) must be rejected by the same tolerance the real check passes."""
    inp = U.config_inputs(2)
    heads = [0, 9]
    out = U.out_to_f64(U.run_gpu(inp, True, True))[:, heads]
    good = U.oracle_heads(inp, heads)
    bad = U.oracle_heads(inp, heads, plant=oracle.PLANT["drop_carry_64"])
    assert U.rel_l2(out, good) <= U.TOL_FP32_REL
    assert U.rel_l2(out, bad) > 10 * U.TOL_FP32_REL, U.rel_l2(out, bad)


@pytest.mark.parametrize("fp32", [True, False], ids=["fp32_records", "bf16_records"])
def test_intra_records_match_chunk_oracle(fp32):
    """Stage check: the per-chunk matrices the intra kernel leaves in the
    workspace equal the FP64 chunk-form oracle's records: FP32 records to
    1e-5, bf16 records (each entry rounded once more) to the BF16 bar; Gam is
    FP32 in both modes."""
    import torch

    from chunked_gated_delta_07_amd import kda

    inp = synth.config_inputs(1)
    H, T, N = inp.H, inp.T, len(inp.cu_seqlens) - 1
    mode = kda.make_mode(fp32, False, True)
    nbytes = kda.workspace_bytes(T, N, H, 128, mode)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda:0")
    U.run_gpu(inp, fp32, True, workspace=ws)
    wsb = ws.cpu().numpy()
    # layout: status word (256 B) | cfirst [(N+1) int32] | gam [C][H][128] f32 |
    # rec [C][H][REC] (256-aligned parts); a record holds P's three lower
    # 32x32 tiles only
    al = lambda x: (x + 255) // 256 * 256
    Cmax = (T + 63 * min(N, T)) // 64
    off_cfirst = 256
    off_gam = off_cfirst + al(4 * (N + 1))
    off_rec = off_gam + al(4 * Cmax * H * 128)
    cfirst = wsb[off_cfirst:off_cfirst + 4 * (N + 1)].view(np.int32)
    nc = int(cfirst[-1])
    REC = 4 * 64 * 128 + 3 * 32 * 32
    gam = wsb[off_gam:off_gam + 4 * nc * H * 128].view(np.float32).reshape(nc, H, 128)
    if fp32:
        rec = wsb[off_rec:off_rec + 4 * nc * H * REC].view(np.float32).reshape(nc, H, REC)
    else:
        bits = wsb[off_rec:off_rec + 2 * nc * H * REC].view(np.uint16).reshape(nc, H, REC)
        rec = synth.bf16_bits_to_f32(bits)
    f64 = inp.as_f64()
    _, R = oracle.kda_chunked(**f64, chunk=64, records=True)
    assert nc == R["W"].shape[0]
    # the library stores each matrix in its state pass's read order (the
    # index maps below restate that order; FE elements per 16 bytes)
    FE = 4 if fp32 else 8
    r, c = np.meshgrid(np.arange(64), np.arange(128), indexing="ij")
    ia = ((((r >> 5) * (64 // FE) + (c & 63) // FE) * 64 + 32 * (c >> 6) + (r & 31)) * FE
          + (c & 63) % FE)
    ch, t = np.meshgrid(np.arange(128), np.arange(64), indexing="ij")
    q16 = 4 * ((r & 31) >> 3) + (r & 3)  # r: token, c: value channel
    iu = (((((c >> 5) * 2 + (r >> 5)) * (16 // FE) + q16 // FE) * 64 + 32 * ((r >> 2) & 1)
           + (c & 31)) * FE + q16 % FE)
    rr, ii = np.meshgrid(np.arange(64), np.arange(64), indexing="ij")
    # token-contracted operands in steps of 16 tokens: tokens 16 s + 8 g .. + 7
    # in lane half g; P: rows 0..31 keep columns 0..31 (the first 16 / FE
    # fragments), rows 32..63 all columns (the next 32 / FE)
    ikb = ((((ch >> 5) * (32 // FE) + (t >> 4) * (8 // FE) + (t & 7) // FE) * 64
            + 32 * ((t >> 3) & 1) + (ch & 31)) * FE + t % FE)
    stored = ii < 32 * ((rr >> 5) + 1)
    ip = (((np.where(rr >> 5 == 0, 0, 16 // FE) + (ii >> 4) * (8 // FE) + (ii & 7) // FE) * 64
           + 32 * ((ii >> 3) & 1) + (rr & 31)) * FE + ii % FE)
    ip = np.where(stored, ip, 0)
    # Qt: row-major, 16-byte chunk index permuted by row: chunk ^ (r % 16)
    iq = r * 128 + FE * ((c // FE) ^ (r & 15)) + c % FE
    P = np.where(stored, rec[:, :, 32768:][:, :, ip], 0.0)
    assert not np.any(R["P"][:, :, ~stored]), "the unstored tile of P is zero"
    checks = {
        "W": (rec[:, :, 0:8192][:, :, ia], R["W"]),
        "Qt": (rec[:, :, 8192:16384][:, :, iq], R["Qt"]),
        "KbT": (rec[:, :, 16384:24576][:, :, ikb], np.swapaxes(R["Kb"], 2, 3)),
        "U": (rec[:, :, 24576:32768][:, :, iu], R["U"]),
        "P": (P, R["P"]),
        "Gam": (gam, R["Gamma"]),
    }
    for name, (got, ref) in checks.items():
        rel = U.rel_l2(got.astype(np.float64), ref)
        print(f"[records {'fp32' if fp32 else 'bf16'}] {name}: rel_l2={rel:.3e}", flush=True)
        assert rel < (1e-5 if fp32 or name == "Gam" else 1e-2), (name, rel)


@pytest.mark.parametrize("cu", [[0, 3000], [0, 1700, 1700, 1701, 4000, 4100]],
                         ids=["one_seq_3000", "packed_with_empty"])
def test_windowed_and_two_pass_schedules(cu):
    """BF16 intermediates run as two passes by default and as a pipeline of
    24-chunk windows with KDA_MODE_WINDOWED: both against the oracle, with
    start and end states, on sequences that cross window boundaries (the
    windowed state pass hands the state over between launches), an empty
    sequence and a one-token sequence."""
    import torch

    from chunked_gated_delta_07_amd import kda

    inp = synth.make_inputs(cu, H=6, d=128, act="bf16", seed=61)
    args = U.to_device(inp, "cuda:0")
    N = len(cu) - 1
    S0 = (0.3 * np.random.default_rng(62).standard_normal((N, 6, 128, 128))).astype(np.float32)
    ref, fin_ref = oracle.kda_forward(**inp.as_f64(), initial_state=S0.astype(np.float64),
                                      return_final_state=True)
    S0d = torch.from_numpy(S0).to("cuda:0")
    assert kda.num_stages(inp.T, N, 6, kda.KDA_MODE_WINDOWED) == 2
    outs = {}
    for windowed in (True, False):
        for o32 in (True, False):
            o, f = kda.chunk_fwd(*args, out_fp32=o32, initial_state=S0d, return_final_state=True,
                                 windowed=windowed)
            torch.cuda.synchronize()
            o = U.out_to_f64(o)
            f = f.double().cpu().numpy()
            ro, rf = U.rel_l2(o, ref), U.rel_l2(f, fin_ref)
            print(f"[schedules {cu}] windowed={windowed} out={'fp32' if o32 else 'bf16'} "
                  f"out rel_l2={ro:.3e} final rel_l2={rf:.3e}", flush=True)
            assert ro <= U.TOL_BF16_REL and rf <= U.TOL_BF16_REL
            outs[(windowed, o32)] = o
    # the schedules share the arithmetic up to summation order
    assert U.rel_l2(outs[(True, True)], outs[(False, True)]) <= 2e-3


@pytest.mark.parametrize("fp32", [False, True], ids=["bf16", "fp32"])
def test_windowed_headline_and_conv(fp32):
    """The windowed schedule at the headline size (16384 tokens x 64 heads,
    sampled heads against the oracle) and with the fused convolution; with
    FP32 intermediates the bit is ignored (two passes, bitwise the default)."""
    import torch

    from chunked_gated_delta_07_amd import kda

    inp = U.config_inputs(3)
    args = U.to_device(inp, "cuda:0")
    heads = [3, 60]
    a = kda.chunk_fwd(*args, fp32_intermediate=fp32, out_fp32=True, windowed=True)
    b = kda.chunk_fwd(*args, fp32_intermediate=fp32, out_fp32=True)
    torch.cuda.synchronize()
    if fp32:
        assert torch.equal(a, b)
        return
    ref = U.oracle_heads(inp, heads)
    got = U.out_to_f64(a)[:, heads]
    rel = U.rel_l2(got, ref)
    print(f"[windowed 16384x64] rel_l2={rel:.3e} vs two passes "
          f"{U.rel_l2(U.out_to_f64(a), U.out_to_f64(b)):.3e}", flush=True)
    assert rel <= U.TOL_BF16_REL
    # convolution fused into the windowed intra role: same as the two passes
    g = torch.Generator().manual_seed(63)
    w = (0.5 * torch.randn((3, 64, 128, 4), generator=g)).to("cuda:0")
    cb = (0.1 * torch.randn((3, 64, 128), generator=g)).to("cuda:0")
    sub = [x[:3000].contiguous() for x in args[:5]] + list(args[5:7]) + [
        torch.tensor([0, 3000], dtype=torch.int32, device="cuda:0")]
    cw = kda.chunk_fwd(*sub, out_fp32=True, conv_weight=w, conv_bias=cb, windowed=True)
    c2 = kda.chunk_fwd(*sub, out_fp32=True, conv_weight=w, conv_bias=cb)
    torch.cuda.synchronize()
    assert U.rel_l2(U.out_to_f64(cw), U.out_to_f64(c2)) <= 2e-3
