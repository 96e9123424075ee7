#!/usr/bin/env python3
"""Benchmark of the KDA chunked forward (libkda) on one MI355X.

Workload: one sequence of 16384 tokens, 64 heads x 128 dims, bfloat16
activations, synthetic seeded inputs (the 16K-token operator timing of xtuner
PR #2301 "[Enhancement] Add opt-in FP32 KDA chunk computation", Validation).
One step = one kda_chunk_fwd call over the whole batch (every kernel of the
path).  The headline line times BF16-intermediate mode; FP32-intermediate mode
is timed on the same inputs and reported alongside.

Prints ONE JSON line.  --gpus above 1 is refused: the implementation runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA chunk fwd tokens/s @H=64,d=128,16K tok; % of FLOP/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_TFLOPS = 2500.0      # dense
MFMA_FP32_TFLOPS = 157.3
H200_CONTEXT_P50_US = {"bf16": 4050.976, "fp32": 7842.400}  # pages' H200 numbers (context only)

# Algorithmic counts per token-head (d = 128, chunk 64): what the method must
# read and write (its inputs and output) and the products it must form.
BYTES_IN_PER_TH = lambda s: (4 * 128 + 1) * s    # q, k, v, f_raw, b_raw
BYTES_OUT_PER_TH = lambda s: 128 * s             # out
FLOP_PER_TH = 139264                             # 3 d^2 + 1.5 C d + C d MACs, x2
# split by kernel: the intra-chunk blocks and solve (1.5 C d + C d MACs) and
# the state pass with the output (3 d^2 MACs: W S0, Qt S0, Kb^T D)
FLOP_INTRA_PER_TH = 2 * (3 * 64 * 128 // 2 + 64 * 128)   # 40,960
FLOP_STATE_PER_TH = 2 * 3 * 128 * 128                   # 98,304
# transcendentals per token-head on the path: the gate's softplus (exp, log)
# and decay (exp) per channel, beta's sigmoid (exp, reciprocal) and the two
# rsqrt of the norms; decay products inside a chunk are multiplications
TRANS_PER_TH = 3 * 128 + 2 + 2                          # 388
# quarter-rate transcendental VALU: 256 CUs x 4 SIMDs x 16 lanes / 4 x 2.4 GHz
VALU_TRANS_PER_S = 256 * 4 * 16 / 4 * 2.4e9             # 9.83e12
# the FP32-intermediate state pass forms every FP32 product from six bf16
# matrix-core products (three-piece split): its peak is the bf16 one / 6
SPLIT_PASSES = 6


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "chunked_gated_delta_07_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(name.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str, mode: str):
    """HBM traffic per launch measured by rocprofv3 counters (committed in
    profiles/), or None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"counters_{kernel}_{workload}_{mode}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(T: int, budget_s: float):
    """Time the FP64 oracle on the host cores on a bounded sample of the same
    workload (all 16384 tokens, a subset of heads), scaled to tokens/s at H=64."""
    import numpy as np

    import oracle
    from chunked_gated_delta_07_amd import synth

    H_total = 64
    probe = synth.make_inputs([0, 2048], H=1, d=128, act="bf16", seed=77)
    t0 = time.perf_counter()
    oracle.kda_forward(**probe.as_f64())
    rate = 2048 / max(time.perf_counter() - t0, 1e-6)  # token-heads/s on one head
    threads = oracle.num_threads()
    # pick heads so the timed run is about budget_s (parallel over heads)
    est_per_head = T / rate
    nh = int(max(1, min(H_total, budget_s * min(threads, H_total) / max(est_per_head, 1e-6))))
    inp = synth.make_inputs([0, T], H=nh, d=128, act="bf16", seed=1003)
    f64 = inp.as_f64()
    # repeat the sample until about budget_s of CPU work has been timed
    reps, dt = 0, 0.0
    while reps == 0 or dt < 0.66 * budget_s:
        t0 = time.perf_counter()
        oracle.kda_forward(**f64)
        dt += time.perf_counter() - t0
        reps += 1
    return {"value": T * nh * reps / H_total / dt, "unit": "tokens/s", "cores": min(threads, nh),
            "kind": "oracle",
            "sample": f"{T} tokens x {nh} of {H_total} heads (bf16 inputs, FP64 token-serial "
                      f"recurrence, OpenMP over heads) x {reps} runs, {dt:.1f} s; scaled to 64 heads"}


def copy_calibration(nbytes: int):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch

    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes}))


WIN_CHUNKS = 24  # chunks per window of the windowed schedule (libkda)


def stage_names(nst: int):
    """Stages kda_chunk_fwd_timed separates: the chunk table, then the
    intra-chunk and state-pass launches of each segment (two passes), or all
    launches of the windowed pipeline (each runs the intra-chunk work of one
    window and the state pass over the window before)."""
    if nst == 2:
        return ["chunk_table", "windows"]
    return ["chunk_table"] + [k for _ in range((nst - 1) // 2) for k in ("intra", "state_pass")]


def time_mode(args_dev, fp32: bool, steps: int, warmup: int, windowed: bool = False):
    import torch

    from chunked_gated_delta_07_amd import kda

    q = args_dev[0]
    T, H, d = q.shape
    N = args_dev[7].numel() - 1
    mode = kda.make_mode(fp32, False, False, windowed)
    ws = torch.empty(kda.workspace_bytes(T, N, H, d, mode), dtype=torch.uint8, device=q.device)
    out = torch.empty((T, H, d), dtype=q.dtype, device=q.device)
    stream = torch.cuda.current_stream()
    nst = kda.num_stages(T, N, H, mode)
    run = lambda ev=None: kda.chunk_fwd(*args_dev, fp32_intermediate=fp32, out=out, workspace=ws,
                                        events=ev, windowed=windowed)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(steps)]
    for e in evs:  # create the events outside the timed region
        for x in e:
            x.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        run(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step_us = [evs[i][0].elapsed_time(evs[i][nst]) * 1e3 for i in range(steps)]
    stage_us = [[evs[i][s].elapsed_time(evs[i][s + 1]) * 1e3 for i in range(steps)] for s in range(nst)]
    chunks = -(-T // 64)
    # per kernel: its launches' time per step (summed over segments) and count
    names, tot, launches = [], {}, {}
    for nm, su in zip(stage_names(nst), stage_us):
        if nm not in tot:
            names.append(nm)
            tot[nm], launches[nm] = 0.0, 0
        tot[nm] += sum(su) / len(su)
        launches[nm] += 1
    if nst == 2:
        launches["windows"] = -(-chunks // WIN_CHUNKS) + 1
    return {
        "ms_per_step": wall * 1e3 / steps,
        "p50_us": statistics.median(per_step_us),
        "max_us": max(per_step_us),
        "stage_avg_us": [tot[nm] for nm in names],
        "stage_names": names,
        "workspace_bytes": ws.numel(),
        "launches": launches,
    }


def time_decode(N: int, H: int, steps: int, warmup: int):
    """One decode step of the token-serial path: N sequences x 1 token x H
    heads, bf16 activations, FP32 states updated in place (kda_recurrent_fwd).
    Timed with HIP events on the launch stream.  Algorithmic bytes per step:
    the states read and written (2 x N H d^2 x 4 B) plus q, k, v, f_raw,
    b_raw read and out written (bf16)."""
    import numpy as np
    import torch

    from chunked_gated_delta_07_amd import kda, synth

    d = 128
    inp = synth.make_inputs(list(range(N + 1)), H=H, d=d, act="bf16", seed=4242)
    dev = torch.device("cuda:0")

    def t(a, bf16):
        x = torch.from_numpy(np.ascontiguousarray(a))
        return (x.view(torch.bfloat16) if bf16 else x).to(dev)

    args = [t(inp.q, True), t(inp.k, True), t(inp.v, True), t(inp.f_raw, True), t(inp.b_raw, True),
            t(inp.A_log, False), t(inp.dt_bias, False), t(inp.cu_seqlens, False)]
    S = 0.5 * torch.randn((N, H, d, d), generator=torch.Generator().manual_seed(4243)).to(dev)
    out = torch.empty((N, H, d), dtype=torch.bfloat16, device=dev)
    for _ in range(warmup):
        kda.recurrent_fwd(*args, out=out, initial_state=S, final_state=S)
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record(stream)
        kda.recurrent_fwd(*args, out=out, initial_state=S, final_state=S)
        b.record(stream)
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    p50 = statistics.median(us)
    nbytes = 2 * N * H * d * d * 4 + N * H * (5 * d + 1) * 2
    gbps = nbytes / (p50 * 1e-6) / 1e9
    return {"workload": f"decode {N} seq x 1 token, H={H}, d={d}, bf16 act, fp32 state in place",
            "entry_point": "kda_recurrent_fwd", "p50_us": round(p50, 2), "max_us": round(us[-1], 2),
            "tokens_per_s": round(N / (p50 * 1e-6), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBS, 4),
                         "bytes_per_step": nbytes}}


def time_graph(args_dev, fp32: bool, replays: int = 50, warmup: int = 10):
    """p50 / max of HIP-graph replays of one kda_chunk_fwd (the way the pages
    time their kernels), events on the replay stream."""
    import torch

    from chunked_gated_delta_07_amd import kda

    q = args_dev[0]
    T, H, d = q.shape
    mode = kda.make_mode(fp32, q.dtype == torch.float32, False)
    ws = torch.empty(kda.workspace_bytes(T, args_dev[7].numel() - 1, H, d, mode),
                     dtype=torch.uint8, device=q.device)
    out = torch.empty((T, H, d), dtype=q.dtype, device=q.device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kda.chunk_fwd(*args_dev, fp32_intermediate=fp32, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kda.chunk_fwd(*args_dev, fp32_intermediate=fp32, out=out, workspace=ws)
    for _ in range(warmup):
        g.replay()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(replays)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record(stream)
        g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    return {"replays": replays, "p50_us": round(statistics.median(us), 2), "max_us": round(us[-1], 2),
            "tokens_per_s": round(T / (statistics.median(us) * 1e-6), 1)}


def time_steps_graph(args_dev, fp32: bool, steps: int, warmup: int):
    """The headline timing: one step = one kda_chunk_fwd over the whole batch,
    captured once as a HIP graph and replayed; `warmup` untimed replays, then
    exactly `steps` replays bracketed by device synchronisation, wall clock."""
    import torch

    from chunked_gated_delta_07_amd import kda

    q = args_dev[0]
    T, H, d = q.shape
    mode = kda.make_mode(fp32, q.dtype == torch.float32, False)
    ws = torch.empty(kda.workspace_bytes(T, args_dev[7].numel() - 1, H, d, mode),
                     dtype=torch.uint8, device=q.device)
    out = torch.empty((T, H, d), dtype=q.dtype, device=q.device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kda.chunk_fwd(*args_dev, fp32_intermediate=fp32, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kda.chunk_fwd(*args_dev, fp32_intermediate=fp32, out=out, workspace=ws)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def time_conv(args_dev, steps: int, warmup: int):
    """kda_chunk_fwd_conv on the headline workload, BF16 intermediates: the
    width-4 causal convolution on q, k, v (bias, SiLU) fused into the intra
    kernel.  Step time from HIP events on the launch stream."""
    import numpy as np
    import torch

    from chunked_gated_delta_07_amd import kda

    q = args_dev[0]
    T, H, d = q.shape
    g = torch.Generator().manual_seed(4244)
    w = (0.5 * torch.randn((3, H, d, 4), generator=g)).to(q.device)
    b = (0.1 * torch.randn((3, H, d), generator=g)).to(q.device)
    mode = kda.make_mode(False, False, False)
    ws = torch.empty(kda.workspace_bytes(T, args_dev[7].numel() - 1, H, d, mode),
                     dtype=torch.uint8, device=q.device)
    out = torch.empty((T, H, d), dtype=q.dtype, device=q.device)
    for _ in range(warmup):
        kda.chunk_fwd(*args_dev, out=out, workspace=ws, conv_weight=w, conv_bias=b, conv_silu=True)
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    for a, e in evs:
        a.record(stream)
        kda.chunk_fwd(*args_dev, out=out, workspace=ws, conv_weight=w, conv_bias=b, conv_silu=True)
        e.record(stream)
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(e) * 1e3 for a, e in evs)
    p50 = statistics.median(us)
    return {"entry_point": "kda_chunk_fwd_conv", "workload": "headline + width-4 q/k/v conv, SiLU, bias",
            "intermediates": "bf16", "p50_us": round(p50, 2), "max_us": round(us[-1], 2),
            "tokens_per_s": round(T / (p50 * 1e-6), 1)}


def progress(msg: str):
    """One progress line on stderr (stdout carries only the result line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def time_bwd(args_dev, steps: int, warmup: int):
    """kda_chunk_bwd (and kda_chunk_bwd_conv, the q/k/v convolution in front)
    on the headline workload: the FP32-recomputed backward
    with bf16 activations, bf16 output gradient and bf16 input gradients
    (the pages' training path casts input gradients back to the activation
    dtype), a random dout.  Step time from HIP events on the launch stream."""
    import torch

    from chunked_gated_delta_07_amd import kda

    q = args_dev[0]
    T, H, d = q.shape
    g = torch.Generator().manual_seed(4245)
    dout = torch.randn((T, H, d), generator=g).to(torch.bfloat16).to(q.device)
    N = args_dev[7].numel() - 1
    mode = kda.make_mode(True)

    def timed(call):
        for _ in range(warmup):
            call()
        stream = torch.cuda.current_stream()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        torch.cuda.synchronize()
        for a, e in evs:
            a.record(stream)
            call()
            e.record(stream)
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(e) * 1e3 for a, e in evs)

    ws = torch.empty(kda.bwd_workspace_bytes(T, N, H, d, mode), dtype=torch.uint8, device=q.device)
    us = timed(lambda: kda.chunk_bwd(*args_dev, dout, workspace=ws))
    p50 = statistics.median(us)
    del ws
    # the same with the q/k/v short convolution in front (kda_chunk_bwd_conv)
    gw = torch.Generator().manual_seed(4244)
    cw = (0.5 * torch.randn((3, H, d, 4), generator=gw)).to(q.device)
    cb = (0.1 * torch.randn((3, H, d), generator=gw)).to(q.device)
    wsc = torch.empty(kda.bwd_conv_workspace_bytes(T, N, H, d, mode), dtype=torch.uint8,
                      device=q.device)
    usc = timed(lambda: kda.chunk_bwd(*args_dev, dout, conv_weight=cw, conv_bias=cb,
                                      conv_silu=True, workspace=wsc))
    conv = {"entry_point": "kda_chunk_bwd_conv", "p50_us": round(statistics.median(usc), 2),
            "max_us": round(usc[-1], 2), "workspace_bytes": wsc.numel()}
    del wsc
    # algorithmic FLOP of a vector-Jacobian product: twice the forward's
    # (every product of the forward has two adjoint products)
    flop = 2 * FLOP_PER_TH * T * H
    tflops = flop / (p50 * 1e-6) / 1e12
    return {"entry_point": "kda_chunk_bwd", "workload": "headline, dout bf16, gradients bf16",
            "intermediates": "fp32", "p50_us": round(p50, 2), "max_us": round(us[-1], 2),
            "tokens_per_s": round(T / (p50 * 1e-6), 1),
            "workspace_bytes": kda.bwd_workspace_bytes(T, N, H, d, mode),
            "with_conv": conv,
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_FP32_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / MFMA_FP32_TFLOPS, 4),
                         "flop_per_token_head": 2 * FLOP_PER_TH}}


def measured_peaks():
    """What this machine delivers against the datasheet peaks: a 1 GiB device copy
    (2 GiB moved; the faster of libkda_peaks' streaming copy kernel and torch's
    copy) and the matrix-core microbenchmarks of libkda_peaks."""
    import torch

    from chunked_gated_delta_07_amd import peaks

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    del src, dst
    torch_gbs = 2 * n / statistics.median(ts) / 1e9
    kernel_gbs = peaks.copy_gbs(n)
    out = {"hbm_copy_gbs": round(max(kernel_gbs, torch_gbs), 1),
           "hbm_copy_kernel_gbs": round(kernel_gbs, 1), "hbm_copy_torch_gbs": round(torch_gbs, 1)}
    out.update(peaks.measure())
    out["datasheet"] = {"hbm_gbs": HBM_PEAK_GBS, "mfma_bf16_tflops": MFMA_BF16_TFLOPS,
                        "mfma_fp32_tflops": MFMA_FP32_TFLOPS}
    out["measured_frac_of_datasheet"] = {
        "hbm": round(out["hbm_copy_gbs"] / HBM_PEAK_GBS, 4),
        "mfma_bf16": round(out["mfma_bf16_tflops"] / MFMA_BF16_TFLOPS, 4),
        "mfma_fp32": round(out["mfma_fp32_tflops"] / MFMA_FP32_TFLOPS, 4)}
    return out


def add_measured_fracs(roof: dict, mp: dict):
    """The roofline fraction against the measured peak as well (the datasheet
    one stays in `frac`)."""
    key = {"GB/s": "hbm_copy_gbs"}.get(roof["unit"])
    if key is None:
        key = "mfma_fp32_tflops" if roof["peak"] == MFMA_FP32_TFLOPS else "mfma_bf16_tflops"
    roof["measured_peak"] = mp[key]
    roof["frac_of_measured_peak"] = round(roof["achieved"] / mp[key], 4)


def roofline_for(mode_name: str, T: int, H: int, res: dict, workload: str):
    """Dominant kernel of the path (by measured time) against its roofline.

    BF16 intermediates (HBM-bound): achieved = the path's algorithmic bytes
    (1282 B per token-head: q, k, v, f_raw, b_raw read, out written, bf16)
    for the T x H token-heads of one launch, over the dominant kernel's average
    launch time.  FP32 intermediates (matrix-core bound): the dominant kernel's
    share of the algorithmic FLOP over its launch time, against the peak of
    the instructions it runs (intra: FP32 matrix cores and VALU, 157.3 TFLOP/s;
    state pass: six bf16 products per FP32 product, 2500 / 6 TFLOP/s); the
    whole step against the sum of both kernels' bounds (`path_frac`)."""
    names = res["stage_names"]
    st = res["stage_avg_us"]  # per step, each kernel's launches summed
    # the whole step: the headline's graph-replayed time when known, else the
    # event-instrumented launches' p50
    step_us = res["ms_per_step"] * 1e3 if res.get("graph_timed") else res["p50_us"]
    dom = max(range(len(st)), key=lambda i: st[i])
    nl = res["launches"][names[dom]]
    act = 2  # bf16 activations
    th = T * H
    # per launch: its share of the token-heads over its average duration,
    # i.e. the step's token-heads over the kernel's time per step
    t = st[dom] * 1e-6
    path_bytes = th * (BYTES_IN_PER_TH(act) + BYTES_OUT_PER_TH(act))
    if mode_name == "bf16":
        achieved = path_bytes / t / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "alg_bytes_per_launch": path_bytes, "alg_bytes_per_token_head": 1282}
        bound_us = path_bytes / (HBM_PEAK_GBS * 1e9) * 1e6
        roof["path_bound_us"] = round(bound_us, 1)
        roof["path_frac"] = round(bound_us / step_us, 4)
    else:
        peak_of = {"intra": MFMA_FP32_TFLOPS, "state_pass": MFMA_BF16_TFLOPS / SPLIT_PASSES}
        flop_of = {"intra": FLOP_INTRA_PER_TH, "state_pass": FLOP_STATE_PER_TH}
        dom = names[dom]
        kpeak = peak_of.get(dom, MFMA_FP32_TFLOPS)
        kfl = flop_of.get(dom, 0) * th / t / 1e12
        dom = names.index(dom)
        roof = {"bound": "mfma", "achieved": round(kfl, 2), "peak": round(kpeak, 1),
                "unit": "TFLOP/s", "frac": round(kfl / kpeak, 4),
                "alg_flop_per_launch": flop_of.get(names[dom], 0) * th // nl,
                "alg_flop_per_token_head": flop_of.get(names[dom], 0)}
        # split-aware bound of the whole step: each kernel's FLOP at the peak
        # of the instructions it runs
        b_intra = FLOP_INTRA_PER_TH * th / (MFMA_FP32_TFLOPS * 1e12) * 1e6
        b_state = FLOP_STATE_PER_TH * th / (MFMA_BF16_TFLOPS / SPLIT_PASSES * 1e12) * 1e6
        roof["path_bound_us"] = round(b_intra + b_state, 1)
        roof["path_bound_parts_us"] = {"intra_fp32": round(b_intra, 1),
                                       "state_pass_bf16x6": round(b_state, 1)}
        roof["path_frac"] = round((b_intra + b_state) / step_us, 4)
        sfl = FLOP_STATE_PER_TH * th / (st[names.index("state_pass")] * 1e-6) / 1e12
        speak = MFMA_BF16_TFLOPS / SPLIT_PASSES
        roof["state_pass_split"] = {"achieved": round(sfl, 2), "peak": round(speak, 1),
                                    "unit": "TFLOP/s", "frac": round(sfl / speak, 4),
                                    "passes": SPLIT_PASSES,
                                    "kernel_avg_us": round(st[names.index("state_pass")], 2)}
    if mode_name == "bf16":
        roof["alg_bytes_per_launch"] = path_bytes // nl
    roof["kernel"] = names[dom]
    roof["launches_per_step"] = nl
    roof["kernel_avg_us"] = round(st[dom] / nl, 2)  # per launch, as rocprofv3 averages
    roof["kernel_us_per_step"] = round(st[dom], 2)
    roof["traffic"] = load_traffic(names[dom], workload, mode_name)
    roof["traffic_source"] = (
        f"profiles/counters_{names[dom]}_{workload}_{mode_name}.json: rocprofv3 --pmc FETCH_SIZE "
        f"and WRITE_SIZE of this kernel, scaled by a device-copy calibration; replayed, not "
        f"measured in this run, and null when the kernel source differs from the counted one")
    # the path's lower bounds in time (whole step) and the step against the largest
    bounds = {"hbm": path_bytes / (HBM_PEAK_GBS * 1e9) * 1e6,
              "mfma_bf16": th * FLOP_PER_TH / (MFMA_BF16_TFLOPS * 1e12) * 1e6,
              "valu_transcendental": th * TRANS_PER_TH / VALU_TRANS_PER_S * 1e6}
    if mode_name == "fp32":
        bounds["mfma_split_aware"] = roof["path_bound_us"]
    roof["path_bounds_us"] = {k: round(v, 1) for k, v in bounds.items()}
    roof["path_frac_vs_max_bound"] = round(max(bounds.values()) / step_us, 4)
    return roof


# The pages' H200 forward p50 (CUDA-graph replay, one sequence), by token
# count and mode: context, not a target.
H200_P50_BY_TOKENS = {129: {"bf16": 71.712, "fp32": 112.096},
                      2048: {"bf16": 550.080, "fp32": 1039.648},
                      16384: {"bf16": 4050.976, "fp32": 7842.400}}


def cpu_oracle_timing(inp, heads, threads=None):
    """Wall-clock of the FP64 oracle on the given heads of a workload (after
    one warm-up call on a small piece), scaled to tokens/s at all heads."""
    import oracle

    f64 = inp.as_f64()
    sub = {k: (v[:, heads] if k in ("q", "k", "v", "f_raw", "b_raw") else
               v[heads] if k in ("A_log", "dt_bias") else v) for k, v in f64.items()}
    full_threads = oracle.num_threads()
    if threads:
        oracle.set_num_threads(threads)
    try:
        # the oracle parallelises over (sequence, head) pairs
        used = min(oracle.num_threads(), (len(inp.cu_seqlens) - 1) * len(heads))
        t0 = time.perf_counter()
        oracle.kda_forward(**sub)
        dt = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(full_threads)
    return {"tokens_per_s": round(inp.T * len(heads) / inp.H / dt, 1), "cores": used,
            "seconds": round(dt, 3),
            "sample": f"{inp.T} tokens x {len(heads)} of {inp.H} heads; scaled to {inp.H} heads"}


def time_configs(no_cpu: bool):
    """Every workload of the parity/timing set: HIP-graph replay p50 / max of
    one kda_chunk_fwd (10 warm-up, 50 timed replays, output in the activation
    dtype), in each listed precision mode, plus the oracle on the host cores
    (all cores; configs 0-2 also one core) on a bounded sample of heads."""
    import numpy as np
    import torch

    from chunked_gated_delta_07_amd import synth

    dev = torch.device("cuda:0")
    out = {}
    for i in range(5):
        c = synth.CONFIGS[i]
        inp = synth.config_inputs(i)
        bf = inp.act == "bf16"

        def t(a, is_act):
            x = torch.from_numpy(np.ascontiguousarray(a))
            return (x.view(torch.bfloat16) if (bf and is_act) else x).to(dev)

        args_dev = [t(inp.q, True), t(inp.k, True), t(inp.v, True), t(inp.f_raw, True),
                    t(inp.b_raw, True), t(inp.A_log, False), t(inp.dt_bias, False),
                    t(inp.cu_seqlens, False)]
        N = len(inp.cu_seqlens) - 1
        lens = np.diff(inp.cu_seqlens)
        rec = {"workload": c["name"], "tokens": inp.T, "sequences": N,
               "longest_sequence": int(lens.max()), "activations": inp.act, "modes": {}}
        for m in c["modes"] if i != 4 else ("bf16", "fp32"):
            g = time_graph(args_dev, m == "fp32")
            g["listed_mode"] = m in c["modes"]
            h200 = H200_P50_BY_TOKENS.get(inp.T, {}).get(m) if N == 1 else None
            if h200 is not None:
                g["context_h200_p50_us"] = h200
            rec["modes"][m] = g
        del args_dev
        torch.cuda.empty_cache()
        if not no_cpu:
            # enough heads that every (sequence, head) thread of the oracle has work
            nh = {0: 64, 1: 64, 2: 16, 3: 16, 4: 16}[i]
            heads = list(np.linspace(0, inp.H - 1, nh).astype(int))
            rec["cpu_oracle"] = cpu_oracle_timing(inp, heads)
            if i <= 2:
                nh1 = {0: 16, 1: 64, 2: 2}[i]
                rec["cpu_oracle_one_core"] = cpu_oracle_timing(
                    inp, list(np.linspace(0, inp.H - 1, nh1).astype(int)), threads=1)
        out[f"cfg{i}"] = rec
        print(json.dumps({"config_timed": f"cfg{i}", "modes": {
            m: v["p50_us"] for m, v in rec["modes"].items()}}), file=sys.stderr, flush=True)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-step measurement of the token-serial path")
    ap.add_argument("--no-bwd", action="store_true",
                    help="skip the backward (kda_chunk_bwd) measurement")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured-peak microbenchmarks (HBM copy, matrix cores)")
    ap.add_argument("--only-mode", choices=["bf16", "fp32"], default=None,
                    help="time one precision mode only (for profiling runs)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config graph-replay timings (configs 0-4)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="run only a device copy of BYTES bytes (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} requested; this implementation runs on one GPU only "
              f"(no multi-GPU path), use --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import torch

    from chunked_gated_delta_07_amd import kda, synth

    kda.load_library()
    cfg = synth.CONFIGS[3]
    inp = synth.config_inputs(3)
    T, H, d = inp.T, inp.H, inp.d
    dev = torch.device("cuda:0")

    def t(a, bf16):
        x = torch.from_numpy(a)
        return (x.view(torch.bfloat16) if bf16 else x).to(dev)

    args_dev = [t(inp.q, True), t(inp.k, True), t(inp.v, True), t(inp.f_raw, True),
                t(inp.b_raw, True), t(inp.A_log, False), t(inp.dt_bias, False),
                t(inp.cu_seqlens, False)]
    torch.cuda.synchronize()
    modes = ["bf16", "fp32"] if args.only_mode is None else [args.only_mode]
    res = {m: time_mode(args_dev, m == "fp32", args.steps, args.warmup) for m in modes}
    progress("launched steps timed")
    graph = {m: time_graph(args_dev, m == "fp32") for m in modes} if args.only_mode is None else {}
    # the headline ms_per_step: K graph-replayed steps (stage times above come
    # from the event-instrumented launches of time_mode)
    for m in modes:
        res[m]["ms_per_step_launched"] = res[m]["ms_per_step"]
        res[m]["ms_per_step"] = time_steps_graph(args_dev, m == "fp32", args.steps, args.warmup)
        res[m]["graph_timed"] = True
    progress("graph-replayed steps timed")
    head = modes[0]
    r = res[head]
    line = {
        "metric": METRIC,
        "value": round(T / (r["ms_per_step"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if head == "bf16" else "fp32",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "tokens": T, "sequences": 1, "heads": H, "head_dim": d,
                   "chunk": 64, "activations": "bf16",
                   "intermediates": "bf16" if head == "bf16" else "fp32", "seq_len": T,
                   "global_batch": 1, "parallelism": "none"},
        "timing": "ms_per_step: wall clock of K HIP-graph replays of one kda_chunk_fwd, "
                  "synchronised before and after; p50/max/stage times: the same call launched "
                  "directly with HIP events between its kernels",
        "ms_per_step_direct_launch": round(r["ms_per_step_launched"], 4),
        "p50_us": round(r["p50_us"], 2),
        "max_us": round(r["max_us"], 2),
        "stage_avg_us": {n: round(x, 2) for n, x in zip(r["stage_names"], r["stage_avg_us"])},
        "workspace_bytes": r["workspace_bytes"],
        "roofline": roofline_for(head, T, H, r, cfg["name"]),
    }
    if head in graph:
        line["graph_replay"] = graph[head]
    for m in modes[1:]:
        rm = res[m]
        line[f"{m}_mode"] = {
            "value": round(T / (rm["ms_per_step"] * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(rm["ms_per_step"], 4), "p50_us": round(rm["p50_us"], 2),
            "max_us": round(rm["max_us"], 2),
            "stage_avg_us": {n: round(x, 2) for n, x in zip(rm["stage_names"], rm["stage_avg_us"])},
            "workspace_bytes": rm["workspace_bytes"],
            "roofline": roofline_for(m, T, H, rm, cfg["name"]),
        }
        if m in graph:
            line[f"{m}_mode"]["graph_replay"] = graph[m]
    if args.only_mode in (None, "bf16"):
        # the same BF16-intermediate arithmetic in the windowed schedule
        # (KDA_MODE_WINDOWED: workspace independent of the length)
        tp = time_mode(args_dev, False, args.steps, args.warmup, windowed=True)
        line["bf16_windowed"] = {
            "value": round(T / (tp["ms_per_step"] * 1e-3), 1), "unit": "tokens/s",
            "p50_us": round(tp["p50_us"], 2), "workspace_bytes": tp["workspace_bytes"],
            "stage_avg_us": {n: round(x, 2) for n, x in zip(tp["stage_names"], tp["stage_avg_us"])}}
    if args.only_mode is None:
        line["conv_fused"] = time_conv(args_dev, max(args.steps, 10), max(args.warmup, 2))
        progress("fused convolution timed")
    if not args.no_bwd and args.only_mode is None:
        line["backward"] = time_bwd(args_dev, max(args.steps // 2, 5), max(args.warmup, 2))
        progress("backward timed")
    if not args.no_decode and args.only_mode is None:
        line["decode"] = time_decode(256, H, max(args.steps, 10), max(args.warmup, 2))
        progress("decode timed")
    if not args.no_peaks:
        mp = measured_peaks()
        line["measured_peaks"] = mp
        add_measured_fracs(line["roofline"], mp)
        for m in modes[1:]:
            add_measured_fracs(line[f"{m}_mode"]["roofline"], mp)
        for leg in ("backward", "decode"):
            if leg in line:
                add_measured_fracs(line[leg]["roofline"], mp)
    line["context_h200_p50_us"] = H200_CONTEXT_P50_US
    if not args.no_configs and args.only_mode is None:
        del args_dev
        torch.cuda.empty_cache()
        line["configs"] = time_configs(args.no_cpu_baseline)
    line["kernel_source_hash"] = kernel_source_hash()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(T, args.cpu_budget_s)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
