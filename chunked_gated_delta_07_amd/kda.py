"""Thin ctypes binding over libkda (include/kda.h).

Argument marshalling only: every step of the forward runs in the library's
HIP kernels.  PyTorch provides device memory and the stream.  If the library
is missing, every call raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_OK = 0
KDA_ERR_INVALID_ARG = 1
KDA_ERR_UNSUPPORTED = 2
KDA_ERR_WORKSPACE = 3
KDA_ERR_HIP = 4

KDA_MODE_FP32_INTERMEDIATE = 0x1
KDA_ACT_FP32 = 0x2
KDA_OUT_FP32 = 0x4
KDA_MODE_WINDOWED = 0x8
KDA_MODE_CHECK_CU = 0x10

# Exported symbols, in declaration order of include/kda.h.
SYMBOLS = ("kda_chunk_fwd_workspace_bytes", "kda_chunk_fwd", "kda_chunk_fwd_state",
           "kda_chunk_fwd_conv", "kda_chunk_fwd_rect", "kda_recurrent_fwd", "kda_recurrent_fwd_rect",
           "kda_chunk_bwd_workspace_bytes", "kda_chunk_bwd", "kda_chunk_bwd_conv_workspace_bytes",
           "kda_chunk_bwd_conv", "kda_chunk_fwd_noalloc",
           "kda_chunk_fwd_num_stages", "kda_chunk_fwd_timed", "kda_status_string")

# Size of the library-owned workspace of kda_chunk_fwd_noalloc (kda.h).
NOALLOC_SCRATCH_BYTES = 256 << 20

_lib = None


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where} failed: {status_string(status)} ({status})")
        self.status = status


def load_library(path: str = LIB_PATH):
    """Load libkda.so (built in-tree by __graft_entry__.build()).  Raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libkda.so not found at {path}; build it with __graft_entry__.build()")
    # torch ships its own HIP runtime; loading it first makes libkda bind to the
    # same runtime instance (same soname) instead of a second one that would
    # not share devices, streams or allocations with torch.
    import torch  # noqa: F401

    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    lib.kda_chunk_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_chunk_fwd_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                  ctypes.c_int32, ctypes.c_uint32]
    fwd_args = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                ctypes.c_int32, ctypes.c_uint32, vp, vp, ctypes.c_size_t, vp]
    lib.kda_chunk_fwd.restype = ctypes.c_int
    lib.kda_chunk_fwd.argtypes = fwd_args
    lib.kda_chunk_fwd_state.restype = ctypes.c_int
    lib.kda_chunk_fwd_state.argtypes = fwd_args[:-1] + [vp, vp, vp]
    lib.kda_chunk_fwd_conv.restype = ctypes.c_int
    lib.kda_chunk_fwd_conv.argtypes = (fwd_args[:13] + [vp, vp, ctypes.c_int32] + fwd_args[13:16]
                                       + [vp, vp, vp])
    lib.kda_chunk_fwd_rect.restype = ctypes.c_int
    lib.kda_chunk_fwd_rect.argtypes = (fwd_args[:11] + [ctypes.c_int32, ctypes.c_int32,
                                                        ctypes.c_uint32, vp, vp, ctypes.c_size_t,
                                                        vp, vp, vp])
    lib.kda_recurrent_fwd.restype = ctypes.c_int
    lib.kda_recurrent_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32,
                                      ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_uint32, vp, vp, vp, vp]
    lib.kda_recurrent_fwd_rect.restype = ctypes.c_int
    lib.kda_recurrent_fwd_rect.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32,
                                           ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_uint32, vp, vp, vp, vp]
    lib.kda_chunk_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_chunk_bwd_workspace_bytes.argtypes = lib.kda_chunk_fwd_workspace_bytes.argtypes
    lib.kda_chunk_bwd.restype = ctypes.c_int
    lib.kda_chunk_bwd.argtypes = ([vp] * 8 + [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_uint32]
                                  + [vp] * 11 + [vp, ctypes.c_size_t, vp])
    lib.kda_chunk_bwd_conv_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_chunk_bwd_conv_workspace_bytes.argtypes = lib.kda_chunk_fwd_workspace_bytes.argtypes
    lib.kda_chunk_bwd_conv.restype = ctypes.c_int
    lib.kda_chunk_bwd_conv.argtypes = ([vp] * 8 + [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                                   ctypes.c_int32, ctypes.c_uint32]
                                       + [vp, vp, ctypes.c_int32] + [vp] * 13
                                       + [vp, ctypes.c_size_t, vp])
    lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.kda_chunk_fwd_noalloc.argtypes = fwd_args[:14] + [vp]
    lib.kda_chunk_fwd_timed.restype = ctypes.c_int
    lib.kda_chunk_fwd_timed.argtypes = fwd_args + [ctypes.POINTER(vp), ctypes.c_int32]
    lib.kda_chunk_fwd_num_stages.restype = ctypes.c_int
    lib.kda_chunk_fwd_num_stages.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_uint32]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().kda_status_string(int(status)).decode()


def workspace_bytes(total_tokens: int, num_seqs: int, H: int, d: int, mode: int) -> int:
    n = load_library().kda_chunk_fwd_workspace_bytes(int(total_tokens), int(num_seqs), int(H),
                                                     int(d), int(mode))
    if n == ctypes.c_size_t(-1).value:
        raise KdaError(KDA_ERR_INVALID_ARG, "kda_chunk_fwd_workspace_bytes")
    return int(n)


def num_stages(total_tokens: int, num_seqs: int, H: int, mode: int) -> int:
    n = int(load_library().kda_chunk_fwd_num_stages(int(total_tokens), int(num_seqs), int(H),
                                                    int(mode)))
    if n < 0:
        raise KdaError(KDA_ERR_INVALID_ARG, "kda_chunk_fwd_num_stages")
    return n


def make_mode(fp32_intermediate: bool, act_fp32: bool = False, out_fp32: bool = False,
              windowed: bool = False, check_cu: bool = False) -> int:
    return ((KDA_MODE_FP32_INTERMEDIATE if fp32_intermediate else 0)
            | (KDA_ACT_FP32 if act_fp32 else 0) | (KDA_OUT_FP32 if out_fp32 else 0)
            | (KDA_MODE_WINDOWED if windowed else 0) | (KDA_MODE_CHECK_CU if check_cu else 0))


def check_status(workspace) -> int:
    """The code a call with check_cu=True left in its workspace (read after
    the call has completed; this synchronises on the workspace's device):
    0 when cu_seqlens was valid, else bit 0 (cu_seqlens[0] != 0), bit 1 (a
    decrease), bit 2 (the last offset differs from the token count)."""
    return int(workspace[:4].view(__import__("torch").int32).item())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def chunk_fwd(q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, fp32_intermediate=False,
              out_fp32=False, out=None, workspace=None, stream=None, events=None,
              initial_state=None, final_state=None, return_final_state=False,
              conv_weight=None, conv_bias=None, conv_silu=True, noalloc=False,
              windowed=False, check_cu=False):
    """KDA chunked forward through libkda.

    q, k, v, f_raw: [T, H, 128] bfloat16 or float32 (one dtype for all);
    b_raw: [T, H] same dtype; A_log: [H] float32; dt_bias: [H, 128] float32;
    cu_seqlens: [N+1] int32.  All CUDA (HIP) tensors, contiguous.  Returns
    out [T, H, 128] (activation dtype, or float32 when out_fp32).
    A rectangular state (q, k, f_raw [T, H, dk], dt_bias [H, dk], v [T, H, dv],
    dk, dv <= 128, not both 128) selects kda_chunk_fwd_rect: out [T, H, dv],
    states [N, H, dk, dv].
    ``events``: optional list of num_stages(T, N, H, mode)+1 torch.cuda.Event
    objects recorded between the stages (kda_chunk_fwd_timed).
    ``windowed=True`` sets KDA_MODE_WINDOWED (schedule only: the pipeline of
    24-chunk windows whose workspace does not grow with the length).
    ``check_cu=True`` sets KDA_MODE_CHECK_CU: the device validates cu_seqlens
    first and, if invalid, touches no token data; pass a ``workspace`` and
    read the code with check_status(workspace) afterwards.
    ``initial_state``: optional [N, H, 128, 128] float32 start states (key,
    value); ``final_state`` (a tensor of that shape to fill, may be the
    initial_state tensor) or ``return_final_state=True`` (allocated) selects
    kda_chunk_fwd_state and makes the result (out, final_state).
    ``conv_weight`` [3, H, 128, 4] float32 (optional ``conv_bias`` [3, H, 128],
    ``conv_silu``) selects kda_chunk_fwd_conv: the short causal convolution on
    q, k, v fused in front of the core.
    ``noalloc=True`` selects kda_chunk_fwd_noalloc: no workspace is allocated
    or passed (the library's own device array serves), for shapes whose
    workspace fits NOALLOC_SCRATCH_BYTES; pass ``out`` to allocate nothing."""
    import torch

    lib = load_library()
    act_fp32 = q.dtype == torch.float32
    if not act_fp32 and q.dtype != torch.bfloat16:
        raise TypeError("activations must be bfloat16 or float32")
    for t in (k, v, f_raw, b_raw):
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, f_raw, b_raw must share one dtype")
    if A_log.dtype != torch.float32 or dt_bias.dtype != torch.float32:
        raise TypeError("A_log and dt_bias must be float32")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    T, H, d = q.shape
    dv = v.shape[2] if v.dim() == 3 else -1
    for t in (q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens):
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError("all tensors must be contiguous device tensors")
    if k.shape != q.shape or f_raw.shape != q.shape or v.shape != (T, H, dv):
        raise ValueError("q, k, f_raw must have one shape [T, H, dk] and v [T, H, dv]")
    if b_raw.shape != (T, H) or A_log.shape != (H,) or dt_bias.shape != (H, d):
        raise ValueError("b_raw [T,H], A_log [H], dt_bias [H,dk] expected")
    num_seqs = cu_seqlens.numel() - 1
    mode = make_mode(fp32_intermediate, act_fp32, out_fp32, windowed, check_cu)
    out_dtype = torch.float32 if (out_fp32 or act_fp32) else q.dtype
    if out is None:
        out = torch.empty((T, H, dv), dtype=out_dtype, device=q.device)
    elif out.dtype != out_dtype or out.shape != (T, H, dv) or not out.is_contiguous():
        raise ValueError("out has the wrong dtype, shape or layout")
    if (d, dv) != (128, 128):
        # rectangular state: kda_chunk_fwd_rect (workspace of the 128 x 128 call)
        if conv_weight is not None or events is not None or noalloc:
            raise ValueError("rectangular widths take no convolution, events or noalloc")
        sshape = (num_seqs, H, d, dv)
        for t in (initial_state, final_state):
            if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != sshape
                                  or not t.is_contiguous() or not t.is_cuda):
                raise ValueError("states must be contiguous float32 [N, H, dk, dv] device tensors")
        if final_state is None and return_final_state:
            final_state = torch.empty(sshape, dtype=torch.float32, device=q.device)
        m = mode & ~KDA_MODE_WINDOWED
        nbytes = workspace_bytes(T, max(num_seqs, 1), H, 128, m) if num_seqs >= 1 else 0
        if workspace is None:
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        st = lib.kda_chunk_fwd_rect(_ptr(q), _ptr(k), _ptr(v), _ptr(f_raw), _ptr(b_raw),
                                    _ptr(A_log), _ptr(dt_bias), _ptr(cu_seqlens), num_seqs, T, H,
                                    d, dv, m, _ptr(out), _ptr(workspace), workspace.numel(),
                                    _ptr(initial_state), _ptr(final_state),
                                    ctypes.c_void_p(stream.cuda_stream))
        if st != KDA_OK:
            raise KdaError(st, "kda_chunk_fwd_rect")
        return (out, final_state) if final_state is not None else out
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    sp = ctypes.c_void_p(stream.cuda_stream)
    if noalloc:
        if (workspace is not None or events is not None or conv_weight is not None
                or initial_state is not None or final_state is not None or return_final_state):
            raise ValueError("noalloc takes no workspace, events, states or convolution")
        st = lib.kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(f_raw), _ptr(b_raw),
                                       _ptr(A_log), _ptr(dt_bias), _ptr(cu_seqlens), num_seqs, T,
                                       H, d, mode, _ptr(out), sp)
        if st != KDA_OK:
            raise KdaError(st, "kda_chunk_fwd_noalloc")
        return out
    nbytes = workspace_bytes(T, max(num_seqs, 1), H, d, mode) if num_seqs >= 1 else 0
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(f_raw), _ptr(b_raw), _ptr(A_log), _ptr(dt_bias),
            _ptr(cu_seqlens), num_seqs, T, H, d, mode, _ptr(out), _ptr(workspace),
            workspace.numel(), sp)
    use_state = initial_state is not None or final_state is not None or return_final_state
    if conv_weight is not None:
        if events is not None:
            raise ValueError("events are not supported together with the convolution")
        if (conv_weight.dtype != torch.float32 or tuple(conv_weight.shape) != (3, H, d, 4)
                or not conv_weight.is_contiguous() or not conv_weight.is_cuda):
            raise ValueError("conv_weight must be a contiguous float32 [3, H, d, 4] device tensor")
        if conv_bias is not None and (conv_bias.dtype != torch.float32
                                      or tuple(conv_bias.shape) != (3, H, d)
                                      or not conv_bias.is_contiguous() or not conv_bias.is_cuda):
            raise ValueError("conv_bias must be a contiguous float32 [3, H, d] device tensor")
        sshape = (num_seqs, H, d, d)
        for t in (initial_state, final_state):
            if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != sshape
                                  or not t.is_contiguous() or not t.is_cuda):
                raise ValueError("states must be contiguous float32 [N, H, d, d] device tensors")
        if final_state is None and return_final_state:
            final_state = torch.empty(sshape, dtype=torch.float32, device=q.device)
        st = lib.kda_chunk_fwd_conv(*args[:13], _ptr(conv_weight), _ptr(conv_bias),
                                    int(bool(conv_silu)), *args[13:16], _ptr(initial_state),
                                    _ptr(final_state), sp)
        if st != KDA_OK:
            raise KdaError(st, "kda_chunk_fwd_conv")
        return (out, final_state) if final_state is not None else out
    if use_state:
        if events is not None:
            raise ValueError("events are not supported together with states")
        sshape = (num_seqs, H, d, d)
        for t in (initial_state, final_state):
            if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != sshape
                                  or not t.is_contiguous() or not t.is_cuda):
                raise ValueError("states must be contiguous float32 [N, H, d, d] device tensors")
        if final_state is None and return_final_state:
            final_state = torch.empty(sshape, dtype=torch.float32, device=q.device)
        st = lib.kda_chunk_fwd_state(*args[:-1], _ptr(initial_state), _ptr(final_state), sp)
        if st != KDA_OK:
            raise KdaError(st, "kda_chunk_fwd_state")
        return (out, final_state) if final_state is not None else out
    if events is None:
        st = lib.kda_chunk_fwd(*args)
        where = "kda_chunk_fwd"
    else:
        for e in events:  # torch creates the underlying hipEvent on first record
            if not e.cuda_event:
                e.record(stream)
        arr = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(e.cuda_event) for e in events])
        st = lib.kda_chunk_fwd_timed(*args, arr, len(events))
        where = "kda_chunk_fwd_timed"
    if st != KDA_OK:
        raise KdaError(st, where)
    return out


def recurrent_fwd(q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, out_fp32=False, out=None,
                  initial_state=None, final_state=None, return_final_state=False, stream=None):
    """Token-serial KDA forward through libkda (kda_recurrent_fwd): FP32 state,
    one token at a time; for decode steps and short sequences.  Tensors as for
    chunk_fwd; returns out, or (out, final_state) when a final state is asked
    for (``final_state`` tensor to fill, or ``return_final_state=True``).
    q, k, f_raw [T, H, dk] with v [T, H, dv], dv != dk, select
    kda_recurrent_fwd_rect (rectangular state [N, H, dk, dv])."""
    import torch

    lib = load_library()
    act_fp32 = q.dtype == torch.float32
    if not act_fp32 and q.dtype != torch.bfloat16:
        raise TypeError("activations must be bfloat16 or float32")
    for t in (k, v, f_raw, b_raw):
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, f_raw, b_raw must share one dtype")
    if A_log.dtype != torch.float32 or dt_bias.dtype != torch.float32:
        raise TypeError("A_log and dt_bias must be float32")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    T, H, dk = q.shape
    dv = v.shape[2]
    for t in (q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens):
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError("all tensors must be contiguous device tensors")
    if k.shape != q.shape or f_raw.shape != q.shape or v.shape != (T, H, dv):
        raise ValueError("q, k, f_raw must be [T, H, dk] and v [T, H, dv]")
    if b_raw.shape != (T, H) or A_log.shape != (H,) or dt_bias.shape != (H, dk):
        raise ValueError("b_raw [T,H], A_log [H], dt_bias [H,dk] expected")
    num_seqs = cu_seqlens.numel() - 1
    mode = make_mode(False, act_fp32, out_fp32)
    out_dtype = torch.float32 if (out_fp32 or act_fp32) else q.dtype
    if out is None:
        out = torch.empty((T, H, dv), dtype=out_dtype, device=q.device)
    elif out.dtype != out_dtype or out.shape != (T, H, dv) or not out.is_contiguous():
        raise ValueError("out has the wrong dtype, shape or layout")
    sshape = (num_seqs, H, dk, dv)
    for t in (initial_state, final_state):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != sshape
                              or not t.is_contiguous() or not t.is_cuda):
            raise ValueError("states must be contiguous float32 [N, H, d, d] device tensors")
    if final_state is None and return_final_state:
        final_state = torch.empty(sshape, dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    common = (_ptr(q), _ptr(k), _ptr(v), _ptr(f_raw), _ptr(b_raw), _ptr(A_log), _ptr(dt_bias),
              _ptr(cu_seqlens), num_seqs, T, H)
    tail = (mode, _ptr(out), _ptr(initial_state), _ptr(final_state),
            ctypes.c_void_p(stream.cuda_stream))
    if dk == dv:
        st, where = lib.kda_recurrent_fwd(*common, dk, *tail), "kda_recurrent_fwd"
    else:
        st, where = lib.kda_recurrent_fwd_rect(*common, dk, dv, *tail), "kda_recurrent_fwd_rect"
    if st != KDA_OK:
        raise KdaError(st, where)
    return (out, final_state) if final_state is not None else out


def bwd_workspace_bytes(total_tokens: int, num_seqs: int, H: int, d: int, mode: int) -> int:
    n = load_library().kda_chunk_bwd_workspace_bytes(int(total_tokens), int(num_seqs), int(H),
                                                     int(d), int(mode))
    if n == ctypes.c_size_t(-1).value:
        raise KdaError(KDA_ERR_INVALID_ARG, "kda_chunk_bwd_workspace_bytes")
    return int(n)


def bwd_conv_workspace_bytes(total_tokens: int, num_seqs: int, H: int, d: int, mode: int) -> int:
    n = load_library().kda_chunk_bwd_conv_workspace_bytes(int(total_tokens), int(num_seqs),
                                                          int(H), int(d), int(mode))
    if n == ctypes.c_size_t(-1).value:
        raise KdaError(KDA_ERR_INVALID_ARG, "kda_chunk_bwd_conv_workspace_bytes")
    return int(n)


def chunk_bwd(q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, dout, out_fp32=False,
              initial_state=None, dfinal_state=None, return_dinitial_state=False,
              conv_weight=None, conv_bias=None, conv_silu=True, workspace=None, stream=None,
              check_cu=False):
    """Backward (vector-Jacobian product) of the KDA chunked forward through
    libkda, recomputed in FP32 (kda_chunk_bwd; kda_chunk_bwd_conv when
    conv_weight is given).

    Inputs as for chunk_fwd, plus dout [T, H, 128] = dL/dout in the forward's
    output dtype (float32 when out_fp32 or float32 activations, else the
    activation dtype) and optionally dfinal_state [N, H, 128, 128] float32.
    Returns a dict: dq, dk, dv, df (= dL/df_raw), db (= dL/db_raw) in dout's
    dtype, dA_log [H] and ddt_bias [H, 128] float32, and dinit [N, H, 128,
    128] float32 when initial_state, dfinal_state or return_dinitial_state is
    given (the gradient of the start state; zero start if none was given).
    With conv_weight [3, H, 128, 4] (and optionally conv_bias [3, H, 128],
    conv_silu) the forward was chunk_fwd with that convolution: dq, dk, dv are
    then the gradients of the convolution's raw inputs, and the dict also
    holds dconv_weight [3, H, 128, 4] and dconv_bias [3, H, 128] (when
    conv_bias is given) in float32.  ``check_cu`` as for chunk_fwd."""
    import torch

    lib = load_library()
    act_fp32 = q.dtype == torch.float32
    if not act_fp32 and q.dtype != torch.bfloat16:
        raise TypeError("activations must be bfloat16 or float32")
    for t in (k, v, f_raw, b_raw):
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, f_raw, b_raw must share one dtype")
    if A_log.dtype != torch.float32 or dt_bias.dtype != torch.float32:
        raise TypeError("A_log and dt_bias must be float32")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    T, H, d = q.shape
    gdtype = torch.float32 if (out_fp32 or act_fp32) else q.dtype
    if dout.dtype != gdtype or tuple(dout.shape) != (T, H, d):
        raise ValueError("dout must have the forward output's dtype and shape")
    for t in (q, k, v, f_raw, b_raw, A_log, dt_bias, cu_seqlens, dout):
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError("all tensors must be contiguous device tensors")
    if k.shape != q.shape or v.shape != q.shape or f_raw.shape != q.shape:
        raise ValueError("q, k, v, f_raw must have one shape [T, H, d]")
    if b_raw.shape != (T, H) or A_log.shape != (H,) or dt_bias.shape != (H, d):
        raise ValueError("b_raw [T,H], A_log [H], dt_bias [H,d] expected")
    num_seqs = cu_seqlens.numel() - 1
    sshape = (num_seqs, H, d, d)
    for t in (initial_state, dfinal_state):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != sshape
                              or not t.is_contiguous() or not t.is_cuda):
            raise ValueError("states must be contiguous float32 [N, H, d, d] device tensors")
    if conv_weight is not None:
        if (conv_weight.dtype != torch.float32 or tuple(conv_weight.shape) != (3, H, d, 4)
                or not conv_weight.is_contiguous() or not conv_weight.is_cuda):
            raise ValueError("conv_weight must be a contiguous float32 [3, H, d, 4] device tensor")
        if conv_bias is not None and (conv_bias.dtype != torch.float32
                                      or tuple(conv_bias.shape) != (3, H, d)
                                      or not conv_bias.is_contiguous() or not conv_bias.is_cuda):
            raise ValueError("conv_bias must be a contiguous float32 [3, H, d] device tensor")
    elif conv_bias is not None:
        raise ValueError("conv_bias needs conv_weight")
    mode = make_mode(True, act_fp32, out_fp32, check_cu=check_cu)
    dev = q.device
    g = {"dq": torch.empty((T, H, d), dtype=gdtype, device=dev),
         "dk": torch.empty((T, H, d), dtype=gdtype, device=dev),
         "dv": torch.empty((T, H, d), dtype=gdtype, device=dev),
         "df": torch.empty((T, H, d), dtype=gdtype, device=dev),
         "db": torch.empty((T, H), dtype=gdtype, device=dev),
         "dA_log": torch.empty((H,), dtype=torch.float32, device=dev),
         "ddt_bias": torch.empty((H, d), dtype=torch.float32, device=dev)}
    want_dinit = initial_state is not None or dfinal_state is not None or return_dinitial_state
    if want_dinit:
        g["dinit"] = torch.empty(sshape, dtype=torch.float32, device=dev)
    wsq = bwd_conv_workspace_bytes if conv_weight is not None else bwd_workspace_bytes
    nbytes = wsq(T, max(num_seqs, 1), H, d, mode) if num_seqs >= 1 else 0
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    if conv_weight is not None:
        g["dconv_weight"] = torch.empty((3, H, d, 4), dtype=torch.float32, device=dev)
        if conv_bias is not None:
            g["dconv_bias"] = torch.empty((3, H, d), dtype=torch.float32, device=dev)
        st = lib.kda_chunk_bwd_conv(
            _ptr(q), _ptr(k), _ptr(v), _ptr(f_raw), _ptr(b_raw), _ptr(A_log), _ptr(dt_bias),
            _ptr(cu_seqlens), num_seqs, T, H, d, mode, _ptr(conv_weight), _ptr(conv_bias),
            1 if conv_silu else 0, _ptr(initial_state), _ptr(dout), _ptr(dfinal_state),
            _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["df"]), _ptr(g["db"]),
            _ptr(g["dA_log"]), _ptr(g["ddt_bias"]), _ptr(g.get("dinit")),
            _ptr(g["dconv_weight"]), _ptr(g.get("dconv_bias")), _ptr(workspace),
            workspace.numel(), ctypes.c_void_p(stream.cuda_stream))
        if st != KDA_OK:
            raise KdaError(st, "kda_chunk_bwd_conv")
        return g
    st = lib.kda_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(f_raw), _ptr(b_raw), _ptr(A_log),
                           _ptr(dt_bias), _ptr(cu_seqlens), num_seqs, T, H, d, mode,
                           _ptr(initial_state), _ptr(dout), _ptr(dfinal_state), _ptr(g["dq"]),
                           _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["df"]), _ptr(g["db"]),
                           _ptr(g["dA_log"]), _ptr(g["ddt_bias"]), _ptr(g.get("dinit")),
                           _ptr(workspace), workspace.numel(), ctypes.c_void_p(stream.cuda_stream))
    if st != KDA_OK:
        raise KdaError(st, "kda_chunk_bwd")
    return g
