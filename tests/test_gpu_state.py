"""GPU parity of kda_chunk_fwd_state (start and end state per sequence and
head) against the FP64 oracle, and the property the states exist for: a
sequence run in two calls, the second starting from the first call's final
state, equals one call over the whole sequence.

Tolerances as for the output (relative L2 over the whole tensor): FP32 mode
1e-4 (and max abs 1e-3 on out), BF16 mode 1e-2; the final state is FP32 in
both modes and is held to the same relative bound.
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

    kda.load_library()
    yield


def _tol(fp32):
    return U.TOL_FP32_REL if fp32 else U.TOL_BF16_REL


def _run(args, fp32, init=None, final=None, ret=True):
    import torch

    from chunked_gated_delta_07_amd import kda

    res = kda.chunk_fwd(*args, fp32_intermediate=fp32, out_fp32=True, initial_state=init,
                        final_state=final, return_final_state=ret)
    torch.cuda.synchronize()
    return res


def _state(seed, N, H, scale=0.5):
    return (scale * np.random.default_rng(seed).standard_normal((N, H, 128, 128))).astype(np.float32)


@pytest.mark.parametrize("fp32", [False, True], ids=["bf16", "fp32"])
def test_state_parity_packed(fp32):
    """Random start states, packed sequences (one empty, one of one token,
    ragged tails): out and final state against the oracle."""
    import torch

    cu = [0, 100, 100, 229, 230]
    inp = synth.make_inputs(cu, H=3, d=128, act="bf16", seed=77)
    S0 = _state(78, len(cu) - 1, 3)
    args = U.to_device(inp, "cuda:0")
    out, fin = _run(args, fp32, init=torch.from_numpy(S0).cuda())
    ref, fref = oracle.kda_forward(**inp.as_f64(), initial_state=S0.astype(np.float64),
                                   return_final_state=True)
    o = out.double().cpu().numpy()
    f = fin.double().cpu().numpy()
    ro, rf = U.rel_l2(o, ref), U.rel_l2(f, fref)
    print(f"[state packed] mode={'fp32' if fp32 else 'bf16'} out rel={ro:.3e} "
          f"max_abs={U.max_abs(o, ref):.3e} final rel={rf:.3e}", flush=True)
    assert ro <= _tol(fp32) and rf <= _tol(fp32)
    if fp32:
        assert U.max_abs(o, ref) <= U.TOL_FP32_MAXABS
    assert np.array_equal(f[1], S0[1].astype(np.float64))  # empty sequence: end = start


def test_final_state_from_zero_start():
    inp = synth.config_inputs(1)
    args = U.to_device(inp, "cuda:0")
    out, fin = _run(args, True)
    ref, fref = oracle.kda_forward(**inp.as_f64(), return_final_state=True)
    rf = U.rel_l2(fin.double().cpu().numpy(), fref)
    print(f"[state zero start] final rel={rf:.3e}", flush=True)
    assert U.rel_l2(out.double().cpu().numpy(), ref) <= U.TOL_FP32_REL
    assert rf <= U.TOL_FP32_REL


def test_empty_batch_copies_state():
    """total_tokens = 0: the final state is the initial state (zero without one)."""
    import torch

    from chunked_gated_delta_07_amd import kda

    dev = "cuda:0"
    e = torch.empty((0, 2, 128), dtype=torch.bfloat16, device=dev)
    cu = torch.zeros(4, dtype=torch.int32, device=dev)
    S0 = torch.from_numpy(_state(5, 3, 2)).to(dev)
    args = (e, e, e, e, torch.empty((0, 2), dtype=torch.bfloat16, device=dev),
            torch.zeros(2, device=dev), torch.zeros((2, 128), device=dev), cu)
    _, fin = kda.chunk_fwd(*args, initial_state=S0, return_final_state=True)
    fin0 = torch.full_like(S0, 7.0)
    kda.chunk_fwd(*args, final_state=fin0)
    torch.cuda.synchronize()
    assert torch.equal(fin, S0) and torch.count_nonzero(fin0).item() == 0


@pytest.mark.parametrize("fp32", [False, True], ids=["bf16", "fp32"])
def test_state_update_in_place(fp32):
    """final_state may be the initial_state tensor: same bits as out of place."""
    import torch

    inp = synth.make_inputs([0, 90, 200], H=2, d=128, act="bf16", seed=12)
    args = U.to_device(inp, "cuda:0")
    S0 = torch.from_numpy(_state(13, 2, 2)).cuda()
    out_a, fin_a = _run(args, fp32, init=S0)
    S1 = S0.clone()
    out_b, _ = _run(args, fp32, init=S1, final=S1)
    assert torch.equal(out_a, out_b) and torch.equal(fin_a, S1)


@pytest.mark.parametrize("fp32", [False, True], ids=["bf16", "fp32"])
def test_split_handoff_16384_tokens(fp32):
    """16384 tokens x 64 heads run in two calls (split at token 5000, inside a
    chunk) with the state handed over, against one call over all tokens: the
    outputs and final states agree; two sampled heads are also checked
    against the oracle over the whole sequence."""
    import torch

    inp = U.config_inputs(3)
    full = U.to_device(inp, "cuda:0")
    out, fin = _run(full, fp32)
    cut = 5000

    def piece(lo, hi):
        a = [t[lo:hi].contiguous() for t in full[:5]] + list(full[5:7])
        a.append(torch.tensor([0, hi - lo], dtype=torch.int32, device="cuda:0"))
        return a
    o1, f1 = _run(piece(0, cut), fp32)
    o2, f2 = _run(piece(cut, inp.T), fp32, init=f1)
    o_split = torch.cat([o1, o2]).double().cpu().numpy()
    o_full = out.double().cpu().numpy()
    r_out = U.rel_l2(o_split, o_full)
    r_fin = U.rel_l2(f2.double().cpu().numpy(), fin.double().cpu().numpy())
    heads = [5, 38]
    f64 = inp.as_f64()
    ref = np.zeros((inp.T, inp.H, 128))
    fref = None
    for h in heads:
        o_h, f_h = oracle.kda_forward(**f64, heads=(h, h + 1), return_final_state=True)
        ref[:, h] = o_h[:, h]
        fref = f_h if fref is None else fref + f_h  # blocks of other heads stay zero
    r_or = U.rel_l2(o_split[:, heads], ref[:, heads])
    r_orf = U.rel_l2(f2.double().cpu().numpy()[0, heads], fref[0, heads])
    print(f"[split 16384] mode={'fp32' if fp32 else 'bf16'} split-vs-whole out={r_out:.3e} "
          f"final={r_fin:.3e}; vs oracle out={r_or:.3e} final={r_orf:.3e}", flush=True)
    assert r_out <= _tol(fp32) and r_fin <= _tol(fp32)
    assert r_or <= _tol(fp32) and r_orf <= _tol(fp32)


@pytest.mark.parametrize("fp32", [False, True], ids=["bf16", "fp32"])
def test_segmented_scan_with_transition_matrices(fp32):
    """The sequence-parallel scheme on one GPU: a 16384-token sequence cut into
    four pieces (not at chunk multiples) that are processed side by side as one
    packed batch.  Per piece r, S_end = M_r S_start + L_r with
    M_r = prod over its chunks of (Diag(Gamma) - Kb^T W): L_r is the final state
    from a zero start, M_r the final state with v = 0 from the identity (the
    recurrence is affine in the state).  An exclusive prefix
    S_in[r+1] = M_r S_in[r] + L_r (host, FP64) gives each piece its true start
    state; a third packed call then reproduces one call over the whole
    sequence."""
    import torch

    inp = synth.make_inputs([0, 16384], H=8, d=128, act="bf16", seed=91)
    full = U.to_device(inp, "cuda:0")
    out_whole, fin_whole = _run(full, fp32)
    cuts = [0, 4000, 8192, 12001, 16384]
    R = len(cuts) - 1
    packed = list(full[:7]) + [torch.tensor(cuts, dtype=torch.int32, device="cuda:0")]
    _, L = _run(packed, fp32)                                   # local end states
    zero_v = list(packed)
    zero_v[2] = torch.zeros_like(packed[2])
    eye = torch.eye(128, device="cuda:0").expand(R, inp.H, 128, 128).contiguous()
    _, M = _run(zero_v, fp32, init=eye)                         # transition matrices
    Ld, Md = L.double().cpu(), M.double().cpu()
    S_in = torch.zeros((R, inp.H, 128, 128), dtype=torch.float64)
    for r in range(R - 1):
        S_in[r + 1] = Md[r] @ S_in[r] + Ld[r]
    out_seg, fin_seg = _run(packed, fp32, init=S_in.float().cuda())
    r_out = U.rel_l2(out_seg.double().cpu().numpy(), out_whole.double().cpu().numpy())
    r_fin = U.rel_l2(fin_seg[-1].double().cpu().numpy(), fin_whole[0].double().cpu().numpy())
    r_end = U.rel_l2((Md[-1] @ S_in[-1] + Ld[-1]).numpy(), fin_whole[0].double().cpu().numpy())
    print(f"[segmented] mode={'fp32' if fp32 else 'bf16'} out={r_out:.3e} final={r_fin:.3e} "
          f"affine end={r_end:.3e}", flush=True)
    assert r_out <= _tol(fp32) and r_fin <= _tol(fp32) and r_end <= _tol(fp32)
