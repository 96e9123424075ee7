"""The C-ABI library loads on a machine without a GPU, exports every symbol
include/kda.h declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")
LIB = os.path.join(ROOT, "chunked_gated_delta_07_amd", "libkda.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libkda.so not built")


def _declared():
    src = open(HEADER).read()
    return re.findall(r"KDA_API\s+[\w\s\*]+?\b(kda_\w+)\s*\(", src)


def test_exports_match_header():
    from chunked_gated_delta_07_amd import kda

    decl = _declared()
    assert decl and set(decl) == set(kda.SYMBOLS)
    out = subprocess.check_output(["nm", "-D", "--defined-only", LIB], text=True)
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for name in decl:
        assert name in exported, name
    # nothing else with C linkage leaks out under the kda_ prefix
    assert {n for n in exported if n.startswith("kda_")} == set(decl)
    lib = ctypes.CDLL(LIB)
    for name in decl:
        assert getattr(lib, name) is not None


def test_status_strings():
    from chunked_gated_delta_07_amd import kda

    names = [kda.status_string(i) for i in range(5)]
    assert names == ["KDA_OK", "KDA_ERR_INVALID_ARG", "KDA_ERR_UNSUPPORTED", "KDA_ERR_WORKSPACE",
                     "KDA_ERR_HIP"]
    assert kda.status_string(99) == "unknown"


def _call(lib, *, N=1, T=10, H=64, d=128, mode=0, ptrs=True, ws_bytes=None):
    p = ctypes.c_void_p(16) if ptrs else None  # never dereferenced: the checks fail first
    if ws_bytes is None:
        ws_bytes = 0
    return lib.kda_chunk_fwd(p, p, p, p, p, p, p, p, N, T, H, d, mode, p, p, ws_bytes, None)


def test_argument_errors_before_launch():
    from chunked_gated_delta_07_amd import kda

    lib = kda.load_library()
    assert _call(lib, ptrs=False) == kda.KDA_ERR_INVALID_ARG          # null pointers
    assert _call(lib, H=0) == kda.KDA_ERR_INVALID_ARG                 # H < 1
    assert _call(lib, N=0) == kda.KDA_ERR_INVALID_ARG                 # num_seqs < 1
    assert _call(lib, T=-1) == kda.KDA_ERR_INVALID_ARG                # negative T
    assert _call(lib, mode=0x20) == kda.KDA_ERR_INVALID_ARG           # unknown mode bit
    assert _call(lib, d=64) == kda.KDA_ERR_UNSUPPORTED                # d != 128
    assert _call(lib, ws_bytes=1) == kda.KDA_ERR_WORKSPACE            # workspace too small
    assert _call(lib, T=0, ptrs=False) == kda.KDA_OK                  # empty batch: no-op
    # timed variant needs n+1 non-null events
    p = ctypes.c_void_p(16)
    ev = (ctypes.c_void_p * 2)(None, None)
    n = kda.num_stages(10, 1, 4, 0)
    W = kda.KDA_MODE_WINDOWED
    assert n == 3 and kda.num_stages(10, 1, 4, W) == 2
    assert kda.num_stages(10, 1, 4, W | kda.KDA_MODE_FP32_INTERMEDIATE) == 3
    assert kda.num_stages(10, 65, 4, W) == 3  # many sequences: two passes
    assert lib.kda_chunk_fwd_timed(p, p, p, p, p, p, p, p, 1, 10, 4, 128, 0, p, p, 1 << 40, None,
                                   ev, 2) == kda.KDA_ERR_INVALID_ARG
    assert n >= 1
    # the state variant applies the same checks (states may be NULL)
    st = lambda **kw: lib.kda_chunk_fwd_state(
        *([kw.get("p", p)] * 8), kw.get("N", 1), kw.get("T", 10), 4, kw.get("d", 128), 0,
        kw.get("p", p), kw.get("p", p), kw.get("ws", 1 << 40), None, None, None)
    assert st(p=None) == kda.KDA_ERR_INVALID_ARG
    assert st(N=0) == kda.KDA_ERR_INVALID_ARG
    assert st(d=96) == kda.KDA_ERR_UNSUPPORTED
    assert st(ws=1) == kda.KDA_ERR_WORKSPACE
    assert st(T=0, p=None) == kda.KDA_OK  # no final state requested: nothing launched
    # the token-serial entry point checks the same before launching
    rc = lambda **kw: lib.kda_recurrent_fwd(
        *([kw.get("p", p)] * 8), kw.get("N", 1), kw.get("T", 10), kw.get("H", 4), kw.get("d", 128),
        kw.get("mode", 0), kw.get("p", p), None, None, None)
    assert rc(p=None) == kda.KDA_ERR_INVALID_ARG
    assert rc(N=0) == kda.KDA_ERR_INVALID_ARG
    assert rc(H=0) == kda.KDA_ERR_INVALID_ARG
    assert rc(mode=0x20) == kda.KDA_ERR_INVALID_ARG
    assert rc(d=64) == kda.KDA_ERR_UNSUPPORTED
    assert rc(mode=kda.KDA_MODE_CHECK_CU) == kda.KDA_ERR_UNSUPPORTED  # no workspace to report into
    assert rc(T=0, p=None) == kda.KDA_OK  # nothing to compute or copy
    rr = lambda dk, dv: lib.kda_recurrent_fwd_rect(*([p] * 8), 1, 10, 4, dk, dv, 0, p, None, None,
                                                   None)
    assert rr(48, 24) == kda.KDA_ERR_UNSUPPORTED   # key length not built
    assert rr(128, 200) == kda.KDA_ERR_UNSUPPORTED  # too many value channels for dk = 128
    assert rr(16, 600) == kda.KDA_ERR_UNSUPPORTED
    assert rr(16, 0) == kda.KDA_ERR_INVALID_ARG


def test_backward_argument_errors_before_launch():
    """kda_chunk_bwd rejects bad arguments before any HIP call (this runs on a
    machine without a GPU)."""
    from chunked_gated_delta_07_amd import kda

    lib = kda.load_library()
    p = ctypes.c_void_p(16)  # never dereferenced: the checks fail first

    def bw(N=1, T=10, H=4, d=128, mode=1, x=p, par=p, ws=1 << 40):
        return lib.kda_chunk_bwd(*([x] * 8), N, T, H, d, mode, None, x, None, x, x, x, x, x, par,
                                 par, None, x, ws, None)

    assert bw(x=None) == kda.KDA_ERR_INVALID_ARG      # null input / output pointers
    assert bw(par=None) == kda.KDA_ERR_INVALID_ARG    # parameter gradients are required
    assert bw(N=0) == kda.KDA_ERR_INVALID_ARG
    assert bw(H=0) == kda.KDA_ERR_INVALID_ARG
    assert bw(T=-1) == kda.KDA_ERR_INVALID_ARG
    assert bw(mode=0x20) == kda.KDA_ERR_INVALID_ARG
    assert bw(d=64) == kda.KDA_ERR_UNSUPPORTED
    assert bw(H=262144) == kda.KDA_ERR_UNSUPPORTED   # 32-bit row offsets: 64 x H x 128 < 2^31
    assert bw(ws=1) == kda.KDA_ERR_WORKSPACE
    assert bw(T=0, par=None) == kda.KDA_ERR_INVALID_ARG  # still required for an empty batch
    assert kda.bwd_workspace_bytes(0, 1, 64, 128, 1) == 0
    with pytest.raises(kda.KdaError):
        kda.bwd_workspace_bytes(10, 1, 64, 96, 1)
    b = [kda.bwd_workspace_bytes(T, 1, 64, 128, 1) for T in (1, 64, 65, 16384)]
    assert b == sorted(b) and all(x % 256 == 0 for x in b)
    # about 460 KB per (chunk, head): 16384 tokens x 64 heads = 256 x 64 chunk-heads
    assert 440e3 < b[-1] / (256 * 64) < 480e3


def test_conv_backward_argument_errors_before_launch():
    """kda_chunk_bwd_conv rejects bad arguments before any HIP call (this runs
    on a machine without a GPU); its workspace adds the convolution's buffers
    to the core backward's."""
    from chunked_gated_delta_07_amd import kda

    lib = kda.load_library()
    p = ctypes.c_void_p(16)  # never dereferenced: the checks fail first

    def bw(N=1, T=10, H=4, d=128, mode=1, x=p, par=p, cw=p, dcw=p, ws=1 << 40):
        return lib.kda_chunk_bwd_conv(*([x] * 8), N, T, H, d, mode, cw, None, 1, None, x, None,
                                      x, x, x, x, x, par, par, None, dcw, None, x, ws, None)

    assert bw(x=None) == kda.KDA_ERR_INVALID_ARG
    assert bw(par=None) == kda.KDA_ERR_INVALID_ARG
    assert bw(cw=None) == kda.KDA_ERR_INVALID_ARG     # the convolution's weights are required
    assert bw(dcw=None) == kda.KDA_ERR_INVALID_ARG    # and so is their gradient
    assert bw(T=0, dcw=None) == kda.KDA_ERR_INVALID_ARG
    assert bw(N=0) == kda.KDA_ERR_INVALID_ARG
    assert bw(mode=0x20) == kda.KDA_ERR_INVALID_ARG
    assert bw(d=64) == kda.KDA_ERR_UNSUPPORTED
    assert bw(H=262144) == kda.KDA_ERR_UNSUPPORTED
    assert bw(ws=1) == kda.KDA_ERR_WORKSPACE
    n = (1 << 23) - 1
    assert bw(N=n, T=n, H=1, ws=1) == kda.KDA_ERR_WORKSPACE
    assert bw(N=1 << 24, T=1 << 24, H=1) == kda.KDA_ERR_UNSUPPORTED
    assert kda.bwd_conv_workspace_bytes(0, 1, 64, 128, 1) == 0
    for T in (1, 64, 65, 16384):
        for mode in (1, 1 | kda.KDA_ACT_FP32):
            c = kda.bwd_conv_workspace_bytes(T, 1, 64, 128, mode)
            assert c % 256 == 0 and c > kda.bwd_workspace_bytes(T, 1, 64, 128, mode)
    c = kda.bwd_conv_workspace_bytes(16384, 1, 64, 128, 1)
    assert 620e3 < c / (256 * 64) < 690e3


def test_check_cu_bit_before_launch():
    """KDA_MODE_CHECK_CU (device-side cu_seqlens check) changes no workspace
    size, and the entry points without a workspace refuse it before any HIP
    call (this runs on a machine without a GPU)."""
    from chunked_gated_delta_07_amd import kda

    lib = kda.load_library()
    C = kda.KDA_MODE_CHECK_CU
    for T, N in ((1, 1), (16384, 1), (5000, 7)):
        for m in (0, 1, kda.KDA_MODE_WINDOWED):
            assert kda.workspace_bytes(T, N, 64, 128, m | C) == kda.workspace_bytes(T, N, 64, 128, m)
        assert kda.bwd_workspace_bytes(T, N, 64, 128, 1 | C) == kda.bwd_workspace_bytes(T, N, 64, 128, 1)
        assert kda.num_stages(T, N, 64, C) == kda.num_stages(T, N, 64, 0)
    p = ctypes.c_void_p(16)  # never dereferenced: the checks fail first
    assert lib.kda_chunk_fwd_noalloc(*([p] * 8), 1, 10, 4, 128, C, p, None) == kda.KDA_ERR_UNSUPPORTED
    assert lib.kda_chunk_fwd_noalloc(*([p] * 8), 1, 10, 4, 128, C | 0x20, p, None) == \
        kda.KDA_ERR_INVALID_ARG
    assert lib.kda_recurrent_fwd_rect(*([p] * 8), 1, 10, 4, 16, 24, C, p, None, None, None) == \
        kda.KDA_ERR_UNSUPPORTED


def test_grid_limits_rejected_before_launch():
    """A dispatch counts each grid dimension in work-items with a 32-bit field.
    Sizes whose grids would not fit return KDA_ERR_UNSUPPORTED from the host
    checks, before any HIP call (this runs on a machine without a GPU)."""
    from chunked_gated_delta_07_amd import kda

    lib = kda.load_library()
    p = ctypes.c_void_p(16)  # never dereferenced: the checks fail first
    big = ctypes.c_size_t(-1).value  # any workspace is large enough
    # forward: the intra grid's head dimension is H x 256 work-items
    H = (1 << 24) + 1
    assert lib.kda_chunk_fwd(*([p] * 8), 1, 1, H, 128, 0, p, p, big, None) == \
        kda.KDA_ERR_UNSUPPORTED
    # backward: chunks x 512 work-items; 2^24 one-token sequences are 2^24 chunks
    n = 1 << 24
    assert lib.kda_chunk_bwd(*([p] * 8), n, n, 1, 128, 1, None, p, None, p, p, p, p, p, p, p, None,
                             p, big, None) == kda.KDA_ERR_UNSUPPORTED
    # just inside the limit the same call reaches the workspace check instead
    n = (1 << 23) - 1
    assert lib.kda_chunk_bwd(*([p] * 8), n, n, 1, 128, 1, None, p, None, p, p, p, p, p, p, p, None,
                             p, 1, None) == kda.KDA_ERR_WORKSPACE
    # token-serial: one workgroup of 64 ceil(max(dk, dv) / 64) threads per (sequence, head)
    rr = lambda N, dk, dv: lib.kda_recurrent_fwd_rect(*([p] * 8), N, 10, 1, dk, dv, 0, p, None,
                                                      None, None)
    assert rr((1 << 23) + 1, 16, 512) == kda.KDA_ERR_UNSUPPORTED
    assert rr((1 << 25) + 1, 128, 128) == kda.KDA_ERR_UNSUPPORTED


def test_workspace_query():
    from chunked_gated_delta_07_amd import kda

    assert kda.workspace_bytes(0, 1, 64, 128, 0) == 0
    with pytest.raises(kda.KdaError):
        kda.workspace_bytes(10, 1, 64, 64, 0)
    with pytest.raises(kda.KdaError):
        kda.workspace_bytes(10, 1, 64, 128, 0x20)
    prev = 0
    for T in (1, 63, 64, 65, 1000, 16384):
        for N in (1, 2, 7):
            if N > T:
                continue
            b = kda.workspace_bytes(T, N, 64, 128, 0)
            bw = kda.workspace_bytes(T, N, 64, 128, kda.KDA_MODE_WINDOWED)
            b32 = kda.workspace_bytes(T, N, 64, 128, 1)
            assert b > 0 and bw > 0 and b32 > b and b % 256 == 0 and bw % 256 == 0
    # with BF16 intermediates the records live in a ring: one 32-chunk segment
    # (two passes, segmented) or two 24-chunk windows (windowed schedule); the
    # workspace stops growing with the length.  FP32 records cover every chunk.
    w = [kda.workspace_bytes(T, 1, 64, 128, kda.KDA_MODE_WINDOWED) for T in (48 * 64, 16384, 1 << 20)]
    sg = [kda.workspace_bytes(T, 1, 64, 128, 0) for T in (33 * 64, 16384, 1 << 20)]
    assert w[0] == w[1] == w[2] and sg[0] == sg[1] == sg[2] < 200e6
    assert kda.workspace_bytes(32 * 64, 1, 64, 128, 0) < sg[0]  # one segment: no carry buffers
    assert kda.workspace_bytes(16384, 1, 64, 128, 1) > 2e9
    # stages: the table, then intra and state pass per segment (32 chunks)
    assert kda.num_stages(16384, 1, 64, 0) == 1 + 2 * 8
    assert kda.num_stages(2048, 1, 64, 0) == 3 and kda.num_stages(16384, 1, 64, 1) == 3
    for T in range(1, 400, 7):
        b = kda.workspace_bytes(T, 3, 8, 128, 0)
        assert b >= prev
        prev = b
    prev = 0
    for N in range(1, 50):
        b = kda.workspace_bytes(1000, N, 8, 128, 0)
        assert b >= prev
        prev = b


PEAKS_HEADER = os.path.join(ROOT, "include", "kda_peaks.h")
PEAKS_LIB = os.path.join(ROOT, "chunked_gated_delta_07_amd", "libkda_peaks.so")


@pytest.mark.skipif(not os.path.exists(PEAKS_LIB), reason="libkda_peaks.so not built")
def test_peaks_exports_and_argument_errors():
    """The microbenchmark library exports exactly what its header declares and
    rejects bad arguments before any launch (so this runs without a GPU)."""
    from chunked_gated_delta_07_amd import peaks

    decl = re.findall(r"KDA_PEAKS_API\s+[\w\s\*]+?\b(kda_\w+)\s*\(", open(PEAKS_HEADER).read())
    assert decl and set(decl) == set(peaks.SYMBOLS)
    out = subprocess.check_output(["nm", "-D", "--defined-only", PEAKS_LIB], text=True)
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    assert {n for n in exported if n.startswith("kda_")} == set(decl)
    lib = peaks.load_library()
    sink = ctypes.c_void_p(16)  # never dereferenced: the checks fail first
    assert lib.kda_peaks_probe(9, 10, 1, 64, sink, None) == 1      # unknown kind
    assert lib.kda_peaks_probe(-1, 10, 1, 64, sink, None) == 1
    assert lib.kda_peaks_probe(0, 0, 1, 64, sink, None) == 1       # iters < 1
    assert lib.kda_peaks_probe(0, 10, 0, 64, sink, None) == 1      # blocks < 1
    assert lib.kda_peaks_probe(0, 10, 1, 100, sink, None) == 1     # threads not 64..512 pow2
    assert lib.kda_peaks_probe(0, 10, 1, 64, None, None) == 1      # null sink
    p16 = ctypes.c_void_p(16)
    assert lib.kda_peaks_copy(None, p16, 16, 1, None) == 1        # null source
    assert lib.kda_peaks_copy(p16, ctypes.c_void_p(24), 16, 1, None) == 1  # misaligned
    assert lib.kda_peaks_copy(p16, p16, 24, 1, None) == 1         # bytes not a multiple of 16
    assert lib.kda_peaks_copy(p16, p16, 16, 0, None) == 1         # blocks < 1
    assert lib.kda_peaks_copy(p16, p16, 0, 1, None) == 0          # nothing to copy: no launch
