"""Binding of libkda_peaks.so (include/kda_peaks.h): matrix-core and VALU
microbenchmarks timed with HIP events on the launch stream."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda_peaks.so")
SYMBOLS = ("kda_peaks_probe", "kda_peaks_copy")
MFMA_BF16, MFMA_FP32, CHAIN_BF16, CHAIN_BF16_VALU, VALU = range(5)
# FLOP per wave and loop iteration of each kind
FLOP_PER_ITER = {MFMA_BF16: 4 * 32 * 32 * 16 * 2, MFMA_FP32: 4 * 16 * 16 * 4 * 2,
                 CHAIN_BF16: 32 * 32 * 16 * 2, CHAIN_BF16_VALU: 32 * 32 * 16 * 2, VALU: 0}
_lib = None


def load_library(path: str = LIB_PATH):
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libkda_peaks.so not found at {path}; build it with __graft_entry__.build()")
    import torch  # noqa: F401  (same HIP runtime instance as torch)

    lib = ctypes.CDLL(path)
    lib.kda_peaks_probe.restype = ctypes.c_int
    lib.kda_peaks_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_void_p]
    lib.kda_peaks_copy.restype = ctypes.c_int
    lib.kda_peaks_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                   ctypes.c_void_p]
    _lib = lib
    return lib


def time_probe(kind: int, iters: int, blocks: int, threads: int, repeats: int = 5) -> float:
    """Median seconds of one launch (after one warm-up launch)."""
    import statistics

    import torch

    lib = load_library()
    sink = torch.empty(blocks * threads, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    times = []
    for r in range(repeats + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st = lib.kda_peaks_probe(kind, iters, blocks, threads, ctypes.c_void_p(sink.data_ptr()), sp)
        e1.record(stream)
        if st != 0:
            raise RuntimeError(f"kda_peaks_probe failed with status {st}")
        torch.cuda.synchronize()
        if r:
            times.append(e0.elapsed_time(e1) * 1e-3)
    if not bool(torch.isfinite(sink).all()):
        raise RuntimeError("kda_peaks_probe produced non-finite values")
    return statistics.median(times)


def copy_gbs(nbytes: int = 1 << 30, blocks: int = 256 * 8, repeats: int = 5) -> float:
    """HBM GB/s of the streaming copy kernel (2 x nbytes moved per launch, median)."""
    import statistics

    import torch

    lib = load_library()
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    times = []
    for r in range(repeats + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st = lib.kda_peaks_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                nbytes, blocks, sp)
        e1.record(stream)
        if st != 0:
            raise RuntimeError(f"kda_peaks_copy failed with status {st}")
        torch.cuda.synchronize()
        if r:
            times.append(e0.elapsed_time(e1) * 1e-3)
    if not bool(torch.equal(src[:: 1 << 20], dst[:: 1 << 20])):
        raise RuntimeError("kda_peaks_copy: copy mismatch")
    return 2 * nbytes / statistics.median(times) / 1e9


def measure(cus: int = 256, iters: int = 20000) -> dict:
    """Measured matrix-core peaks (all SIMDs, two waves each) and the overlap of
    a wave's VALU with its own dependent matrix-core chain (one wave per SIMD)."""
    out = {}
    for name, kind in (("mfma_bf16_tflops", MFMA_BF16), ("mfma_fp32_tflops", MFMA_FP32)):
        blocks, threads = 2 * cus, 256
        t = time_probe(kind, iters, blocks, threads)
        out[name] = round(FLOP_PER_ITER[kind] * iters * blocks * (threads // 64) / t / 1e12, 1)
    blocks, threads = cus, 256
    t_chain = time_probe(CHAIN_BF16, iters, blocks, threads)
    t_mix = time_probe(CHAIN_BF16_VALU, iters, blocks, threads)
    t_valu = time_probe(VALU, iters, blocks, threads)
    cyc = lambda t: t * 2.4e9 / iters  # noqa: E731  (at the 2.4 GHz peak clock)
    out["chain_overlap"] = {
        "note": "one wave per SIMD: dependent v_mfma_f32_32x32x16_bf16 chain, 8 independent FP32 FMAs, both",
        "cycles_per_iter_at_2.4GHz": {"mfma_chain": round(cyc(t_chain), 1), "valu_8fma": round(cyc(t_valu), 1),
                                      "both": round(cyc(t_mix), 1)},
        # 1 = the VALU hides entirely under the chain, 0 = the two add up
        "overlap_frac": round((t_chain + t_valu - t_mix) / min(t_chain, t_valu), 3),
    }
    return out
