"""The matrix-core microbenchmarks and the streaming copy run and report
plausible figures: measured peaks within (20 %, 105 %] of the datasheet ones, per-iteration cycle counts of
the dependent chain and of the VALU block near their issue costs."""
import pytest

pytestmark = pytest.mark.gpu


def test_measured_peaks_plausible():
    from chunked_gated_delta_07_amd import peaks

    print("peaks: measure(iters=4000)", flush=True)
    m = peaks.measure(iters=4000)
    print(m, flush=True)
    assert 0.2 * 2500.0 < m["mfma_bf16_tflops"] <= 1.05 * 2500.0
    assert 0.2 * 157.3 < m["mfma_fp32_tflops"] <= 1.05 * 157.3
    cyc = m["chain_overlap"]["cycles_per_iter_at_2.4GHz"]
    # a dependent 32x32x16 bf16 product takes at least its 32 issue cycles; eight
    # wave64 FP32 FMAs at least 8 x 4 (16-lane SIMD)
    assert cyc["mfma_chain"] >= 30.0 and cyc["valu_8fma"] >= 30.0
    assert cyc["both"] >= max(cyc["mfma_chain"], cyc["valu_8fma"]) * 0.95
    assert -0.2 <= m["chain_overlap"]["overlap_frac"] <= 1.2


def test_streaming_copy_plausible():
    from chunked_gated_delta_07_amd import peaks

    print("peaks: copy_gbs(256 MiB)", flush=True)
    gbs = peaks.copy_gbs(1 << 28, repeats=3)
    print(gbs, flush=True)
    assert 0.2 * 8000.0 < gbs <= 1.05 * 8000.0
