"""kda_chunk_fwd_noalloc (the forward without a workspace argument, for
callers that cannot allocate) against kda_chunk_fwd with a caller-owned
workspace: the same kernels on the same inputs, so the outputs must be
bitwise equal.  Two calls in a row, the second with a smaller input, check
that nothing left in the shared array by one call leaks into the next."""
import ctypes
import os
import sys

import numpy as np
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

    kda.load_library()  # raises if the library is missing: no fallback
    yield


@pytest.mark.parametrize("fp32,out_fp32", [(False, False), (False, True), (True, True),
                                           (True, False)],
                         ids=["bf16-out16", "bf16-out32", "fp32-out32", "fp32-out16"])
def test_noalloc_matches_workspace_entry_point(fp32, out_fp32):
    import torch

    from chunked_gated_delta_07_amd import kda

    # a larger call, then a smaller one with a different packing; with BF16
    # intermediates the records live in a ring (one 32-chunk segment, or two
    # windows with KDA_MODE_WINDOWED), so the 16384-token, 64-head shape fits
    cases = [([0, 700, 1500, 1792], 32, 41, False), ([0, 37, 65, 300], 8, 42, False)]
    if not fp32:
        cases = [([0, 16384], 64, 43, False), ([0, 16384], 64, 43, True),
                 ([0, 700, 1500, 1792], 32, 41, True)] + cases
    for cu, H, seed, win in cases:
        inp = synth.make_inputs(cu, H=H, d=128, act="bf16", seed=seed)
        args = U.to_device(inp, "cuda:0")
        T = inp.T
        mode = kda.make_mode(fp32, False, out_fp32, win)
        assert kda.workspace_bytes(T, len(cu) - 1, H, 128, mode) <= kda.NOALLOC_SCRATCH_BYTES
        odt = torch.float32 if out_fp32 else torch.bfloat16
        ref = kda.chunk_fwd(*args, fp32_intermediate=fp32, out_fp32=out_fp32, windowed=win)
        # poison the output buffer: every element must be written
        got = torch.full((T, H, 128), float("nan"), dtype=odt, device="cuda:0")
        kda.chunk_fwd(*args, fp32_intermediate=fp32, out_fp32=out_fp32, out=got, noalloc=True,
                      windowed=win)
        torch.cuda.synchronize()
        print(f"[noalloc] cu={cu} H={H} mode={'fp32' if fp32 else 'bf16'} "
              f"out={'fp32' if out_fp32 else 'bf16'} windowed={win}", flush=True)
        assert torch.equal(ref.view(torch.int16) if not out_fp32 else ref.view(torch.int32),
                           got.view(torch.int16) if not out_fp32 else got.view(torch.int32))
        # and against the oracle on a few heads, at the mode's bar
        heads = [0, H - 1]
        o = U.out_to_f64(got)[:, heads]
        r = U.oracle_heads(inp, heads)
        bar = U.TOL_FP32_REL if (fp32 and out_fp32) else U.TOL_BF16_REL
        assert U.rel_l2(o, r) <= bar


def test_noalloc_rejects_shapes_beyond_its_array():
    """A shape whose workspace exceeds the library's array is refused before
    anything is launched."""
    from chunked_gated_delta_07_amd import kda

    lib = kda.load_library()
    p = ctypes.c_void_p(16)  # never dereferenced: the size check fails first
    T = 16384
    m32 = kda.KDA_MODE_FP32_INTERMEDIATE  # two passes: records for every chunk
    assert kda.workspace_bytes(T, 1, 64, 128, m32) > kda.NOALLOC_SCRATCH_BYTES
    assert lib.kda_chunk_fwd_noalloc(*([p] * 8), 1, T, 64, 128, m32, p, None) == \
        kda.KDA_ERR_WORKSPACE
    # BF16: a ring of one 32-chunk segment, about 2.5 MB per head
    assert kda.workspace_bytes(T, 1, 64, 128, 0) <= kda.NOALLOC_SCRATCH_BYTES
    assert kda.workspace_bytes(T, 1, 128, 128, 0) > kda.NOALLOC_SCRATCH_BYTES
    assert lib.kda_chunk_fwd_noalloc(*([p] * 8), 1, T, 128, 128, 0, p, None) == \
        kda.KDA_ERR_WORKSPACE
    assert kda.workspace_bytes(T, 1, 64, 128, kda.KDA_MODE_WINDOWED) <= kda.NOALLOC_SCRATCH_BYTES
    assert lib.kda_chunk_fwd_noalloc(*([p] * 8), 1, 10, 64, 96, 0, p, None) == \
        kda.KDA_ERR_UNSUPPORTED
    assert lib.kda_chunk_fwd_noalloc(*([p] * 8), 0, 10, 64, 128, 0, p, None) == \
        kda.KDA_ERR_INVALID_ARG
    assert lib.kda_chunk_fwd_noalloc(*([None] * 8), 1, 0, 64, 128, 0, None, None) == kda.KDA_OK
