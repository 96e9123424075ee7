"""kda_chunk_fwd is allocation-free and stream-ordered, so it can be captured
into a HIP graph.  Capture it once, replay it several times with eager work and
synchronisations in between, and check every replay bit for bit against the
eager call (both precision modes, packed ragged input)."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(__file__))
import kda_testutil as U  # noqa: E402

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


@pytest.mark.parametrize("cu", [[0, 100, 100, 357, 1000], [0, 2500, 2500, 4300]],
                         ids=["short", "three_segments"])
@pytest.mark.parametrize("fp32", [False, True], ids=["bf16", "fp32"])
def test_graph_replay_matches_eager(fp32, cu):
    """A captured forward replays bit for bit, also when the BF16 forward runs
    as several 32-chunk segments (the second case: 70 chunks)."""
    import torch

    from chunked_gated_delta_07_amd import kda

    inp = synth.make_inputs(cu, H=8, d=128, act="bf16", seed=55)
    args = U.to_device(inp, "cuda:0")
    T, H, N = inp.T, inp.H, len(inp.cu_seqlens) - 1
    mode = kda.make_mode(fp32, False, False)
    ws = torch.empty(kda.workspace_bytes(T, N, H, 128, mode), dtype=torch.uint8, device="cuda:0")
    eager = kda.chunk_fwd(*args, fp32_intermediate=fp32, workspace=ws).clone()
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the capture stream once
        kda.chunk_fwd(*args, fp32_intermediate=fp32, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        kda.chunk_fwd(*args, fp32_intermediate=fp32, out=out, workspace=ws)
    for i in range(4):
        out.zero_()
        ws.fill_(0x5A)  # scribble on the workspace between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i}"


def test_backward_graph_replay_and_determinism():
    """kda_chunk_bwd is allocation-free too: captured once, every replay (with
    the outputs cleared and the workspace scribbled on in between) equals the
    eager call bit for bit; two eager calls are also bitwise identical (the
    backward uses no atomics, its reductions run in a fixed order)."""
    import torch

    from chunked_gated_delta_07_amd import kda

    inp = synth.make_inputs([0, 100, 100, 357, 1000], H=8, d=128, act="bf16", seed=56)
    args = U.to_device(inp, "cuda:0")
    T, H, N = inp.T, inp.H, len(inp.cu_seqlens) - 1
    gen = torch.Generator().manual_seed(3)
    dout = torch.randn((T, H, 128), generator=gen).to(torch.bfloat16).to("cuda:0")
    init = (0.3 * torch.randn((N, H, 128, 128), generator=gen)).to("cuda:0")
    dfin = torch.randn((N, H, 128, 128), generator=gen).to("cuda:0")
    ws = torch.empty(kda.bwd_workspace_bytes(T, N, H, 128, kda.make_mode(True)), dtype=torch.uint8,
                     device="cuda:0")
    call = lambda: kda.chunk_bwd(*args, dout, initial_state=init, dfinal_state=dfin, workspace=ws)
    eager = {k: v.clone() for k, v in call().items()}
    again = call()
    torch.cuda.synchronize()
    for k in eager:
        assert torch.equal(eager[k], again[k]), f"eager run not reproducible: {k}"
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = call()
    for i in range(3):
        for v in out.values():
            v.zero_()
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in eager:
            assert torch.equal(out[k], eager[k]), f"replay {i}: {k}"
