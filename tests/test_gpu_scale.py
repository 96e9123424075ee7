"""Sizes at the edges: very many short sequences (chunk table over 20,000
sequences, one partial chunk each) and a 2^20-token sequence (16,384 chunks
per head).  The long run is checked by properties that hold at any size and
on a prefix the oracle computes in seconds: by causality, the first 16,384
outputs of the long run are the outputs of those tokens alone."""
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


@pytest.mark.parametrize("fp32", [False, True], ids=["bf16", "fp32"])
def test_twenty_thousand_short_sequences(fp32):
    lens = np.random.default_rng(71).integers(1, 8, size=20000)
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    inp = synth.make_inputs(cu, H=2, d=128, act="bf16", seed=72)
    out = U.out_to_f64(U.run_gpu(inp, fp32, True))
    ref = U.oracle_heads(inp, [0, 1])
    rel = U.rel_l2(out, ref)
    print(f"[20000 seqs, T={inp.T}] mode={'fp32' if fp32 else 'bf16'} rel={rel:.3e}", flush=True)
    assert rel <= (U.TOL_FP32_REL if fp32 else U.TOL_BF16_REL)


def test_million_token_sequence_fp32():
    import torch

    from chunked_gated_delta_07_amd import kda

    T, H, d = 1 << 20, 4, 128
    g = torch.Generator(device="cuda:0").manual_seed(73)
    mk = lambda *s: torch.randn(s, generator=g, device="cuda:0").to(torch.bfloat16)
    q, k, v, f = mk(T, H, d), mk(T, H, d), mk(T, H, d), mk(T, H, d)
    b = mk(T, H)
    A_log = torch.rand(H, generator=g, device="cuda:0") * float(np.log(16))
    dtb = 0.5 * torch.randn((H, d), generator=g, device="cuda:0")
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda:0")
    out, fin = kda.chunk_fwd(q, k, v, f, b, A_log, dtb, cu, fp32_intermediate=True, out_fp32=True,
                             return_final_state=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(fin).all())
    # two calls with the state handed over at an odd cut
    cut = 700001
    one = torch.tensor([0, cut], dtype=torch.int32, device="cuda:0")
    two = torch.tensor([0, T - cut], dtype=torch.int32, device="cuda:0")
    sl = lambda x, a, z: x[a:z].contiguous()
    o1, f1 = kda.chunk_fwd(sl(q, 0, cut), sl(k, 0, cut), sl(v, 0, cut), sl(f, 0, cut), sl(b, 0, cut),
                           A_log, dtb, one, fp32_intermediate=True, out_fp32=True,
                           return_final_state=True)
    o2, f2 = kda.chunk_fwd(sl(q, cut, T), sl(k, cut, T), sl(v, cut, T), sl(f, cut, T),
                           sl(b, cut, T), A_log, dtb, two, fp32_intermediate=True, out_fp32=True,
                           initial_state=f1, return_final_state=True)
    torch.cuda.synchronize()
    r_split = float(torch.linalg.vector_norm(torch.cat([o1, o2]) - out) / torch.linalg.vector_norm(out))
    r_fin = float(torch.linalg.vector_norm(f2 - fin) / torch.linalg.vector_norm(fin))
    # oracle on the first 16,384 tokens (all heads)
    P = 16384
    host = lambda x: x[:P].float().cpu().numpy().astype(np.float64)
    ref = oracle.kda_forward(host(q), host(k), host(v), host(f), host(b),
                             A_log.cpu().numpy().astype(np.float64), dtb.cpu().numpy().astype(np.float64),
                             np.array([0, P], dtype=np.int32))
    r_or = U.rel_l2(out[:P].double().cpu().numpy(), ref)
    print(f"[2^20 tokens x {H} heads] split={r_split:.3e} final={r_fin:.3e} prefix vs oracle={r_or:.3e}",
          flush=True)
    assert r_split <= 1e-5 and r_fin <= 1e-5 and r_or <= U.TOL_FP32_REL
