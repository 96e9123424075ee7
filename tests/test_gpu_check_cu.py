"""KDA_MODE_CHECK_CU: the device-side check of cu_seqlens (a debugging aid).

Valid offsets: status 0 and results bit for bit those of the unchecked call
(a single sequence then goes through the chunk table, which the unchecked call
skips).  Invalid offsets -- a decrease, a first offset other than 0, a last
offset other than the token count -- give the documented status bits, and no
token data is read or written: out and the input gradients keep a sentinel
value, end states equal the start states, parameter gradients are zero and the
start-state gradient is the end-state gradient.  The invalid offsets used here
stay inside the tensors' rows, so even an unchecked call would stay in bounds.
"""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(__file__))
import kda_testutil as U  # noqa: E402

from chunked_gated_delta_07_amd import synth  # noqa: E402

pytestmark = pytest.mark.gpu

INVALID = [([0, 40, 30, 65], 2), ([5, 37, 65], 1), ([0, 37, 60], 4), ([3, 20, 10, 50], 1 | 2 | 4)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from chunked_gated_delta_07_amd import kda

    kda.load_library()
    yield


def _ws(T, N, H, mode, bwd=False):
    import torch

    from chunked_gated_delta_07_amd import kda

    q = kda.bwd_workspace_bytes if bwd else kda.workspace_bytes
    return torch.empty(q(T, N, H, 128, mode), dtype=torch.uint8, device="cuda:0")


@pytest.mark.parametrize("sched", ["two_pass", "windowed", "fp32"])
@pytest.mark.parametrize("cu", [[0, 300], [0, 37, 65, 130, 130, 200]], ids=["one_seq", "packed"])
def test_valid_offsets_change_nothing(cu, sched):
    import torch

    from chunked_gated_delta_07_amd import kda

    inp = synth.make_inputs(cu, H=4, d=128, act="bf16", seed=81)
    args = U.to_device(inp, "cuda:0")
    N, T = len(cu) - 1, inp.T
    fp32, win = sched == "fp32", sched == "windowed"
    ws = _ws(T, N, 4, kda.make_mode(fp32, False, True, win, True))
    S0 = torch.randn((N, 4, 128, 128), device="cuda:0") * 0.3
    a, fa = kda.chunk_fwd(*args, fp32_intermediate=fp32, out_fp32=True, windowed=win,
                          initial_state=S0, return_final_state=True, workspace=ws, check_cu=True)
    b, fb = kda.chunk_fwd(*args, fp32_intermediate=fp32, out_fp32=True, windowed=win,
                          initial_state=S0, return_final_state=True)
    torch.cuda.synchronize()
    assert kda.check_status(ws) == 0
    assert torch.equal(a, b) and torch.equal(fa, fb)


@pytest.mark.parametrize("sched", ["two_pass", "windowed", "fp32"])
@pytest.mark.parametrize("cu,code", INVALID, ids=["decrease", "first_not_0", "last_not_T", "all"])
def test_invalid_offsets_are_reported_and_touch_no_tokens(cu, code, sched):
    import torch

    from chunked_gated_delta_07_amd import kda

    T = 65 if cu[-1] <= 65 else cu[-1]
    inp = synth.make_inputs([0, T], H=4, d=128, act="bf16", seed=82)
    args = U.to_device(inp, "cuda:0")[:7] + [torch.tensor(cu, dtype=torch.int32, device="cuda:0")]
    N = len(cu) - 1
    fp32, win = sched == "fp32", sched == "windowed"
    ws = _ws(T, N, 4, kda.make_mode(fp32, False, True, win, True))
    out = torch.full((T, 4, 128), 7.0, dtype=torch.float32, device="cuda:0")
    S0 = torch.randn((N, 4, 128, 128), device="cuda:0")
    fin = torch.full_like(S0, 5.0)
    kda.chunk_fwd(*args, fp32_intermediate=fp32, out_fp32=True, windowed=win, out=out,
                  initial_state=S0, final_state=fin, workspace=ws, check_cu=True)
    torch.cuda.synchronize()
    got = kda.check_status(ws)
    print(f"[check_cu {sched}] cu={cu} status={got}", flush=True)
    assert got == code
    assert bool((out == 7.0).all())
    assert torch.equal(fin, S0)


@pytest.mark.parametrize("conv", [False, True], ids=["core", "conv"])
def test_backward_invalid_offsets(conv):
    import torch

    from chunked_gated_delta_07_amd import kda

    cu = [0, 40, 30, 65]
    inp = synth.make_inputs([0, 65], H=2, d=128, act="bf16", seed=83)
    args = U.to_device(inp, "cuda:0")[:7] + [torch.tensor(cu, dtype=torch.int32, device="cuda:0")]
    g = torch.Generator().manual_seed(84)
    dout = torch.randn((65, 2, 128), generator=g).to("cuda:0")
    dfin = torch.randn((3, 2, 128, 128), generator=g).to("cuda:0")
    mode = kda.make_mode(True, False, True, check_cu=True)
    extra = {}
    if conv:
        extra = {"conv_weight": (0.5 * torch.randn((3, 2, 128, 4), generator=g)).to("cuda:0")}
        ws = torch.empty(kda.bwd_conv_workspace_bytes(65, 3, 2, 128, mode), dtype=torch.uint8,
                         device="cuda:0")
    else:
        ws = _ws(65, 3, 2, mode, bwd=True)
    ws.fill_(0xAB)
    grads = kda.chunk_bwd(*args, dout, out_fp32=True, dfinal_state=dfin, workspace=ws,
                          check_cu=True, **extra)
    torch.cuda.synchronize()
    assert kda.check_status(ws) == 2
    assert torch.count_nonzero(grads["dA_log"]) == 0 and torch.count_nonzero(grads["ddt_bias"]) == 0
    assert torch.equal(grads["dinit"], dfin)
    if conv:
        assert torch.count_nonzero(grads["dconv_weight"]) == 0
