"""The segmented schedule (BF16 intermediates, more than 32 chunks): segments
of 32 chunks, each an intra-chunk launch and a state-pass launch, with the
state of a sequence that crosses a segment boundary carried in FP32.  A
chunk's arithmetic does not depend on which launch runs it, so the results
must be bit for bit those of the same tokens run as separate calls with the
state handed over, and those of each sequence of a packed batch run alone;
plus the oracle at the BF16 bar (1e-2)."""
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

    kda.load_library()
    yield


def _call(args, cu, S0, o32):
    import torch

    from chunked_gated_delta_07_amd import kda

    a = list(args[:7]) + [torch.tensor(cu, dtype=torch.int32, device="cuda:0")]
    return kda.chunk_fwd(*a, out_fp32=o32, initial_state=S0, return_final_state=True)


@pytest.mark.parametrize("o32", [False, True], ids=["out_bf16", "out_fp32"])
def test_one_call_equals_calls_with_state_handed_over(o32):
    """5000 tokens (79 chunks: three segments) in one call, and as calls of
    2048, 2048 and 904 tokens (one segment each) with the end state of each
    passed as the start state of the next."""
    import torch

    from chunked_gated_delta_07_amd import kda

    H = 8
    inp = synth.make_inputs([0, 5000], H=H, d=128, act="bf16", seed=91)
    args = U.to_device(inp, "cuda:0")
    assert kda.num_stages(5000, 1, H, 0) == 1 + 2 * 3
    S0 = (0.3 * torch.randn((1, H, 128, 128), generator=torch.Generator().manual_seed(92))).cuda()
    out, fin = _call(args, [0, 5000], S0, o32)
    S = S0.clone()
    parts = []
    for a, b in ((0, 2048), (2048, 4096), (4096, 5000)):
        sub = [x[a:b].contiguous() for x in args[:5]] + list(args[5:7])
        o, S = _call(sub, [0, b - a], S, o32)
        parts.append(o)
    torch.cuda.synchronize()
    assert torch.equal(out, torch.cat(parts)) and torch.equal(fin, S)
    ref, fref = oracle.kda_forward(**inp.as_f64(), initial_state=S0.double().cpu().numpy(),
                                   return_final_state=True)
    ro = U.rel_l2(U.out_to_f64(out), ref)
    rf = U.rel_l2(fin.double().cpu().numpy(), fref)
    print(f"[segments 5000] out={'fp32' if o32 else 'bf16'} rel={ro:.3e} final={rf:.3e}", flush=True)
    assert ro <= U.TOL_BF16_REL and rf <= U.TOL_BF16_REL


def test_packed_batch_equals_sequences_alone():
    """Sequences of 1000, 2100, 0, 1900 and 1 tokens packed (segment
    boundaries fall inside sequences; an empty and a one-token sequence), with
    start states, against each sequence run alone."""
    import torch

    cu = [0, 1000, 3100, 3100, 5000, 5001]
    H = 4
    inp = synth.make_inputs(cu, H=H, d=128, act="bf16", seed=93)
    args = U.to_device(inp, "cuda:0")
    N = len(cu) - 1
    S0 = (0.3 * torch.randn((N, H, 128, 128), generator=torch.Generator().manual_seed(94))).cuda()
    out, fin = _call(args, cu, S0, True)
    for n in range(N):
        a, b = cu[n], cu[n + 1]
        sub = [x[a:b].contiguous() for x in args[:5]] + list(args[5:7])
        o, f = _call(sub, [0, b - a], S0[n:n + 1].contiguous(), True)
        torch.cuda.synchronize()
        assert torch.equal(out[a:b], o), n
        assert torch.equal(fin[n:n + 1], f), n
    ref, fref = oracle.kda_forward(**inp.as_f64(), initial_state=S0.double().cpu().numpy(),
                                   return_final_state=True)
    ro = U.rel_l2(U.out_to_f64(out), ref)
    print(f"[segments packed] rel={ro:.3e}", flush=True)
    assert ro <= U.TOL_BF16_REL and U.rel_l2(fin.double().cpu().numpy(), fref) <= U.TOL_BF16_REL


def test_segmented_rectangular_and_convolution():
    """The rectangular-state and fused-convolution forwards also run in
    segments: 3000 tokens against the oracle (d_k = 16, d_v = 24) and against
    the same tokens run as two calls (convolution: each call restarts the
    convolution history, so the comparison is per call, one sequence each)."""
    import torch

    from chunked_gated_delta_07_amd import kda

    cu = [0, 3000]
    r = synth.rect_inputs(cu, 2, 16, 24, seed=95)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    bf = lambda a: dev(a).to(torch.bfloat16)
    args = [bf(r["q"]), bf(r["k"]), bf(r["v"]), bf(r["f_raw"]), bf(r["b_raw"]), dev(r["A_log"]),
            dev(r["dt_bias"]), torch.tensor(cu, dtype=torch.int32, device="cuda:0")]
    out = kda.chunk_fwd(*args, out_fp32=True)
    torch.cuda.synchronize()
    ref = oracle.kda_forward_rect(**{k: r[k].astype(np.float64) for k in
                                     ("q", "k", "v", "f_raw", "b_raw", "A_log", "dt_bias")},
                                  cu_seqlens=np.asarray(cu, dtype=np.int32))
    ro = U.rel_l2(out.double().cpu().numpy(), ref)
    print(f"[segments rect 16x24] rel={ro:.3e}", flush=True)
    assert ro <= U.TOL_BF16_REL
    # convolution: 4200 tokens in one call = two sequences of 2100 run alone
    inp = synth.make_inputs([0, 2100, 4200], H=2, d=128, act="bf16", seed=96)
    a2 = U.to_device(inp, "cuda:0")
    g = torch.Generator().manual_seed(97)
    w = (0.5 * torch.randn((3, 2, 128, 4), generator=g)).cuda()
    o = kda.chunk_fwd(*a2, out_fp32=True, conv_weight=w)
    for s0, s1 in ((0, 2100), (2100, 4200)):
        sub = [x[s0:s1].contiguous() for x in a2[:5]] + list(a2[5:7]) + [
            torch.tensor([0, s1 - s0], dtype=torch.int32, device="cuda:0")]
        oo = kda.chunk_fwd(*sub, out_fp32=True, conv_weight=w)
        torch.cuda.synchronize()
        assert torch.equal(o[s0:s1], oo)


@pytest.mark.parametrize("H", [3, 5])
def test_segments_many_sequences_odd_heads(H):
    """Seven packed sequences (4500, 0, 65, 2100, 1, 3000 and 64 tokens: 153
    chunks, five segments; the first sequence crosses two segment boundaries)
    with a head count that leaves the state pass's last grid row partly
    empty (7 H pairs, not a multiple of 8), start states on: every sequence
    equals its run alone bit for bit, and the batch meets the BF16 bar
    against the oracle (output and end states)."""
    import torch

    lens = [4500, 0, 65, 2100, 1, 3000, 64]
    cu = [0] + np.cumsum(lens).tolist()
    inp = synth.make_inputs(cu, H=H, d=128, act="bf16", seed=98 + H)
    args = U.to_device(inp, "cuda:0")
    N = len(lens)
    S0 = (0.3 * torch.randn((N, H, 128, 128), generator=torch.Generator().manual_seed(H))).cuda()
    out, fin = _call(args, cu, S0, True)
    for n in range(N):
        a, b = cu[n], cu[n + 1]
        sub = [x[a:b].contiguous() for x in args[:5]] + list(args[5:7])
        o, f = _call(sub, [0, b - a], S0[n:n + 1].contiguous(), True)
        torch.cuda.synchronize()
        assert torch.equal(out[a:b], o), n
        assert torch.equal(fin[n:n + 1], f), n
    ref, fref = oracle.kda_forward(**inp.as_f64(), initial_state=S0.double().cpu().numpy(),
                                   return_final_state=True)
    ro = U.rel_l2(U.out_to_f64(out), ref)
    rf = U.rel_l2(fin.double().cpu().numpy(), fref)
    print(f"[segments odd heads H={H}] rel={ro:.3e} final={rf:.3e}", flush=True)
    assert ro <= U.TOL_BF16_REL and rf <= U.TOL_BF16_REL
