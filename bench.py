#!/usr/bin/env python3
"""Forward-pass throughput of log-linear Mamba-2 attention on one MI355X.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload NAME]

One step = one call of the C-ABI forward entry (the forward kernel, with a caller workspace
zero-filled once before the timed loop) over one batch of synthetic inputs already resident
in HBM. Prints ONE JSON line: tokens/s (B*T per call), the roofline of the
forward kernel (its average launch duration timed live by HIP events around the timed launches
on the launch stream), and the CPU oracle timed on a bounded sample of the same workload.

Only one GPU is used; --gpus N with N > 1 exits with a message.
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fwd tokens/sec, log-linear Mamba-2 T=8192 d=64 bf16; MFMA util % of peak"
HEADLINE = "b4h16_t8192_d64_bf16"

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3       # MI355X dense fp32 matrix


def algorithmic_per_token(w, chunk: int) -> tuple[float, float]:
    """(FLOP, bytes) per head-token.

    FLOP: dense masked intra-chunk block 2C(dk+dv), one decayed chunk state 2 dk dv, and
    the read-out of popcount(chunk index) Fenwick nodes, log2(T/C)/2 of them on average,
    2 dk dv each. Bytes: q, k, v, out once each in the element type, lambda (L levels)
    and log_a in float32.
    """
    import math
    e = 2 if w.dtype == "bf16" else 4
    n = max(1, w.T // chunk)
    pbar = math.log2(n) / 2 if n > 1 else 0.0
    flop = 2 * chunk * (w.dk + w.dv) + 2 * w.dk * w.dv * (1 + pbar)
    byts = (2 * w.dk + 2 * w.dv) * e + 4 * w.L + 4
    return flop, byts


def decode_measure(w, dev, stream, steps: int = 256, warmup: int = 32) -> dict:
    """Decoding steps (``loglinear_attn_decode_step``) at the workload's head shape, for the
    positions T-steps .. T-1 (decoding right after a prompt of ~T tokens).

    The cache holds finite random states (every level the steps read is live data), so the
    steps do exactly the work they do in use. Time per step = one launch each, back to back on
    one stream, between two events. Bytes per step (what the step must move): per head the
    live levels of t-1 (popcount(t-1) dk x dv fp32 states) read once, the merged level written,
    the level-0 factors and the log-scales read and written, the token's q, k, v, log_a and
    lambda read and its output written.
    """
    import torch
    import log_linear_attention_chunked_amd as lla
    B, H, dk, dv = w.B, w.H, w.dk, w.dv
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    e = 2 if w.dtype == "bf16" else 4
    Lc = max(w.L, 2)
    g = torch.Generator(device="cpu").manual_seed(1)
    state, log_scale = lla.new_decode_cache(B, H, dk, dv, Lc, device=dev)
    state.copy_(0.1 * torch.randn(state.shape, generator=g))
    log_scale.zero_()
    q = torch.randn((B, H, dk), generator=g).to(dev, dt)
    k = torch.randn((B, H, dk), generator=g).to(dev, dt)
    v = torch.randn((B, H, dv), generator=g).to(dev, dt)
    log_a = (-0.05 * torch.rand((B, H), generator=g)).to(dev)
    lam = torch.rand((B, H, Lc), generator=g).to(dev)
    out = torch.empty((B, H, dv), dtype=dt, device=dev)
    ts = list(range(max(w.T - steps, 1), w.T))     # positions the workload's cache covers
    steps = len(ts)
    for t in ts[:warmup]:
        lla.decode_step(q, k, v, log_a, lam, state, log_scale, t, out, stream=stream)
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for t in ts:
        lla.decode_step(q, k, v, log_a, lam, state, log_scale, t, out, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms_eager = e0.elapsed_time(e1) / steps
    # the same steps captured once in a HIP graph and replayed: launches without the Python
    # issue cost of each call (the eager loop above is bound by it)
    ms = ms_eager
    try:
        gs = torch.cuda.Stream(dev)
        gs.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gs):
            with torch.cuda.graph(graph, stream=gs):
                for t in ts:
                    lla.decode_step(q, k, v, log_a, lam, state, log_scale, t, out, stream=gs)
        stream.wait_stream(gs)
        graph.replay()
        torch.cuda.synchronize(dev)
        reps = 5
        e0.record(stream)
        for _ in range(reps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        ms = e0.elapsed_time(e1) / (reps * steps)
    except Exception as exc:  # pragma: no cover - report the eager figure alone
        print(f"decode graph capture failed ({exc}); reporting the eager loop", file=sys.stderr)
    # the hand-over from a prompt of the positions before the timed window (one call)
    from lla_synth import generate
    xp = generate(w.with_(T=ts[0]), seed=3)
    kp, vp, lap = (xp[n].to(dev) for n in ("k", "v", "log_a"))
    lla.decode_prefill(kp, vp, lap, state, log_scale, stream=stream)
    torch.cuda.synchronize(dev)
    reps_p = 5
    e0.record(stream)
    for _ in range(reps_p):
        lla.decode_prefill(kp, vp, lap, state, log_scale, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms_prefill = e0.elapsed_time(e1) / reps_p
    P = ts[0] - 1
    live = [l for l in range(1, Lc) if (P >> (l - 1)) & 1]
    # k and v of every live level's block (each read once), log_a, the live states written
    prefill_bytes = B * H * (sum(1 << (l - 1) for l in live) * (dk + dv) * e + ts[0] * 4
                             + len(live) * dk * dv * 4)
    per_head = 0
    for t in ts:
        live = bin(t - 1).count("1")
        per_head += (live + 1) * dk * dv * 4 + 4 * (dk + dv) * 4 + 4 * Lc * 4 \
            + (2 * dk + 2 * dv) * e + 4 + 4 * Lc
    byts = per_head * B * H / steps
    achieved = byts / (ms * 1e-3) / 1e9
    return {
        "kernel": "lla_decode_kernel",
        "config": {"B": B, "H": H, "dk": dk, "dv": dv, "levels": Lc, "positions": [ts[0], ts[-1]]},
        "ms_per_step": ms,
        "ms_per_step_eager_python": ms_eager,
        "timing": "HIP graph of the steps, replayed" if ms != ms_eager else "eager loop",
        "tokens_per_s": B / (ms * 1e-3),
        "prefill": {"prompt_tokens": ts[0], "ms": ms_prefill, "bytes": prefill_bytes,
                    "gbs": prefill_bytes / (ms_prefill * 1e-3) / 1e9},
        "algorithmic_bytes_per_step": byts,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS},
    }


def backward_algorithmic(w, chunk: int) -> tuple[float, float]:
    """(FLOP, bytes) per head-token of the backward pass.

    FLOP: the intra-chunk block's five products (scores and dO V^T, then dq, dk, dv),
    2C(3dk + 2dv); the chunk state 2 dk dv; popcount(chunk index) target-side partials and as
    many node read-outs for dq, 2 dk dv each, log2(T/C)/2 of each on average; the two read-outs
    of the combined right-sibling state for dk and dv, 2 dk dv each. Bytes: q, k, v, dO read and
    dq, dk, dv written once in the element type; log_a, lambda read and dlog_a, dlambda written
    once in float32.
    """
    import math
    e = 2 if w.dtype == "bf16" else 4
    n = max(1, -(-w.T // chunk))
    pbar = math.log2(n) / 2 if n > 1 else 0.0
    flop = 2 * chunk * (3 * w.dk + 2 * w.dv) + 2 * w.dk * w.dv * (3 + 2 * pbar)
    byts = (4 * w.dk + 3 * w.dv) * e + 8 * w.L + 8
    return flop, byts


def backward_measure(w, d, dev, stream, steps: int = 20, warmup: int = 5) -> dict:
    """The backward pass (``loglinear_attn_bwd``) on the workload's inputs and a seeded upstream
    gradient, with a caller workspace: time per call between events, per-stage times from the
    events the library records (chunk states + block decays + tree, gradient kernel, dlog_a
    scan), tokens/s and the roofline of the whole call against its algorithmic bytes."""
    import torch
    import log_linear_attention_chunked_amd as lla
    from lla_synth import grad_output
    do = grad_output(w, seed=0).to(dev)
    chunk = lla.bwd_default_chunk(w.dk, w.dv, w.dtype)
    ws = torch.empty(max(lla.bwd_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, chunk, w.dtype), 1),
                     dtype=torch.uint8, device=dev)
    outs = (torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"]),
            torch.empty_like(d["log_a"]), torch.empty_like(d["lam"]))

    def call(evs=None):
        lla.backward(d["q"], d["k"], d["v"], d["log_a"], d["lam"], do, chunk=chunk, workspace=ws,
                     stream=stream, stage_events=evs, out=outs)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps
    stages = {"states_tree": 0.0, "grads": 0.0, "dloga": 0.0}
    reps = 5
    for _ in range(reps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        for ev in evs:
            ev.record(stream)
        torch.cuda.synchronize(dev)
        call(evs)
        torch.cuda.synchronize(dev)
        stages["states_tree"] += evs[0].elapsed_time(evs[1]) / reps
        stages["grads"] += evs[1].elapsed_time(evs[2]) / reps
        stages["dloga"] += evs[2].elapsed_time(evs[3]) / reps
    flop_ht, byte_ht = backward_algorithmic(w, chunk)
    ht = w.B * w.H * w.T
    achieved = byte_ht * ht / (ms * 1e-3) / 1e9
    peak_flops = (BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS) * 1e12
    return {
        "config": {"chunk": chunk, "workspace_bytes": ws.numel()},
        "ms_per_call": ms,
        "stages_ms": stages,
        "tokens_per_s": w.B * w.T / (ms * 1e-3),
        "algorithmic_bytes_per_call": byte_ht * ht,
        "algorithmic_flop_per_call": flop_ht * ht,
        "mfma_util_algorithmic": flop_ht * ht / (ms * 1e-3) / peak_flops,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "scope": "whole backward call"},
    }


VARLEN_LENGTHS = [8192, 7000, 5000, 4096, 3000, 2500, 1500, 1000, 480]   # 32768 tokens per head


def varlen_measure(dev, stream, steps: int = 20, warmup: int = 5) -> dict:
    """The variable-length forward on 9 sequences of mixed lengths (longest 8192, 32768 tokens
    per head, the headline's count) packed along time, H=16, d=64, bf16, C=64: time per call
    between events (with a host copy of cu_seqlens, so one workgroup per sweep that exists;
    and without it, where the grid is sized for 9 sequences of 8192 tokens), tokens/s, and
    the roofline against the same algorithmic bytes per head-token as the dense forward
    (lambda rows of num_levels(8192) levels)."""
    import torch
    import log_linear_attention_chunked_amd as lla
    from lla_synth import custom, generate
    H, d, C = 16, 64, 64
    total, mx = sum(VARLEN_LENGTHS), max(VARLEN_LENGTHS)
    x = generate(custom(1, H, total, d, d, dtype="bf16"), seed=2)
    L = lla.num_levels(mx)
    q, k, v = (x[n][0].to(dev) for n in ("q", "k", "v"))
    log_a = x["log_a"][0].to(dev)
    lam = x["lam"][0, :, :, :L].contiguous().to(dev)
    cu_host = torch.tensor([0] + list(__import__("itertools").accumulate(VARLEN_LENGTHS)), dtype=torch.int32)
    cu = cu_host.to(dev)
    sweep = lla.default_sweep(len(VARLEN_LENGTHS), H, mx, d, d, C, "bf16")
    ws = torch.zeros(max(lla.workspace_bytes(len(VARLEN_LENGTHS), H, mx, d, d, C, sweep, "bf16"), 1),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(v)

    def timed(host):
        call = lambda: lla.forward_varlen(q, k, v, log_a, lam, cu, mx, out, chunk=C, sweep=sweep,
                                          workspace=ws, stream=stream, cu_seqlens_host=host)
        for _ in range(warmup):
            call()
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            call()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) / steps

    ms = timed(cu_host)
    ms_bounds = timed(None)
    byts = ((2 * d + 2 * d) * 2 + 4 * L + 4) * H * total
    return {
        "config": {"H": H, "dk": d, "dv": d, "chunk": C, "sweep": sweep, "lengths": VARLEN_LENGTHS},
        "ms_per_call": ms,
        "ms_per_call_without_host_copy": ms_bounds,
        "tokens_per_s": total / (ms * 1e-3),
        "algorithmic_bytes_per_call": byts,
        "roofline": {"bound": "hbm", "achieved": byts / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
    }


def lambda_bf16_measure(w, d, chunk, sweep, ws, dev, stream, steps: int) -> dict:
    """The same forward call with the level weights in bfloat16 (lambda_bf16 = 1, the same
    values rounded once): forward-kernel time between the library's events, tokens/s, and the
    roofline against the algorithmic bytes with 2L instead of 4L bytes of lambda per head-token."""
    import torch
    import log_linear_attention_chunked_amd as lla
    lam16 = d["lam"].to(torch.bfloat16).contiguous()
    out = torch.empty_like(d["v"])
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in evs:
        e.record(stream)
    call = lambda ev=None: lla.forward(d["q"], d["k"], d["v"], d["log_a"], lam16, out, chunk=chunk,
                                       sweep=sweep, workspace=ws, stream=stream,
                                       stage_events=None if ev is None else [None] + ev)
    for _ in range(3):
        call()
    torch.cuda.synchronize(dev)
    ms = 0.0
    for _ in range(steps):
        call(evs)
        torch.cuda.synchronize(dev)
        ms += evs[0].elapsed_time(evs[1]) / steps
    e = 2 if w.dtype == "bf16" else 4
    byts = ((2 * w.dk + 2 * w.dv) * e + 2 * w.L + 4) * w.B * w.H * w.T
    achieved = byts / (ms * 1e-3) / 1e9
    return {"kernel_ms": ms, "tokens_per_s": w.B * w.T / (ms * 1e-3),
            "algorithmic_bytes_per_launch": byts,
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS}}


def tune(names, steps: int = 20, warmup: int = 3) -> list:
    """Forward kernel time of every chunk size and sweep length that fits, per workload: the
    measurement behind the library's default chunk and sweep (one JSON line per workload).

    Each candidate runs with a caller workspace zero-filled once, timed between events over
    `steps` back-to-back calls after `warmup` calls."""
    import torch
    import log_linear_attention_chunked_amd as lla
    from lla_synth import WORKLOADS, generate
    from log_linear_attention_chunked_amd import _lib
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    rows = []
    from lla_synth import custom
    for name in names:
        if name.startswith("shape:"):      # shape:B,H,T,dk,dv,dtype
            B, H, T, dk, dv, dt = name.split(":", 1)[1].split(",")
            w = custom(int(B), int(H), int(T), int(dk), int(dv), dtype=dt)
            name = w.name
        else:
            w = WORKLOADS[name]
        x = generate(w, seed=0)
        d = {k: v.to(dev) for k, v in x.items()}
        out = torch.empty_like(d["v"])
        res = {}
        for C in (16, 32, 64, 128):
            for R in (1, 2):
                n = lla.workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, C, R, w.dtype)
                ws = torch.zeros(max(n, 1), dtype=torch.uint8, device=dev)
                call = lambda: lla.forward(d["q"], d["k"], d["v"], d["log_a"], d["lam"], out, chunk=C,
                                           sweep=R, workspace=ws if n else None, stream=stream)
                try:
                    call()
                except lla.LLAError as e:
                    if e.status != _lib.LLA_ERR_UNSUPPORTED:
                        raise
                    continue                  # does not fit shared memory
                for _ in range(warmup):
                    call()
                torch.cuda.synchronize(dev)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(steps):
                    call()
                e1.record(stream)
                torch.cuda.synchronize(dev)
                res[f"C{C}_R{R}"] = round(e0.elapsed_time(e1) / steps * 1e3, 2)
                del ws
        dc = lla.default_chunk(w.dk, w.dv, w.T, w.dtype)
        ds = lla.default_sweep(w.B, w.H, w.T, w.dk, w.dv, dc, w.dtype)
        best = min(res, key=res.get)
        row = {"workload": name, "us_per_call": res, "best": best, "default": f"C{dc}_R{ds}"}
        print(json.dumps(row), flush=True)
        rows.append(row)
    return rows


def gdn_algorithmic(w, chunk: int) -> tuple[float, float]:
    """(FLOP, bytes) per head-token of the chunkwise log-linear Gated DeltaNet forward.

    FLOP (2 per multiply-add): per chunk, K K^T and Q K^T (C dk each per token), the blockwise
    inverse of the C x C triangular matrix (~C^2/3 per token), W and U (C dk and C dv), the query
    rows' transport X0 (C dk), the in-chunk attention matrix (C^2) and its product with V (C dv),
    the leaf state and transition (dk dv and dk^2); then per Fenwick node read (log2(T/C)/2 on
    average) X N (dk dv) and, for all but the last, X Phi (dk^2); the up-sweep builds the n - 1
    nodes above the n chunks of a head, each Phi_R [N_L | Phi_L] (dk^2 (dv + dk)), spread over the
    head's T tokens. Bytes: q, k, v, out in the element type, log_a and beta and the L lambda
    levels in float32."""
    import math
    e = 2 if w.dtype == "bf16" else 4
    C, dk, dv = chunk, w.dk, w.dv
    n = max(1, -(-w.T // C))
    pbar = math.log2(n) / 2 if n > 1 else 0.0
    mac = (2 * C * dk + C * C / 3 + C * dk + C * dv + C * dk + C * C + C * dv + dk * dv + dk * dk
           + pbar * dk * dv + max(pbar - 1, 0) * dk * dk + (n - 1) * dk * dk * (dv + dk) / w.T)
    byts = (2 * dk + 2 * dv) * e + 8 + 4 * w.L
    return 2 * mac, byts


def gdn_measure(dev, stream, steps: int = 10, warmup: int = 2) -> dict:
    """Log-linear Gated DeltaNet (``loglinear_attn_gdn_fwd``) at the headline's shape (B=4, H=16,
    T=8192, d=64, bf16, keys L2-normalised, beta = sigmoid(N(0,1))): time per call between events,
    per-stage times from the library's events, tokens/s, and its roofline. Its chunk and up-sweep
    kernels multiply in float32 on the matrix cores (the query kernel in split bf16 for bf16
    inputs), so the bound is the float32 rate (157.3 TFLOP/s); the HBM fraction is reported
    beside it."""
    import torch
    import log_linear_attention_chunked_amd as lla
    from lla_synth import GDN_WORKLOADS, generate_gdn
    w = GDN_WORKLOADS["gdn_b4h16_t8192_d64_bf16"]
    x = generate_gdn(w, seed=0)
    d = {k: v.to(dev) for k, v in x.items()}
    chunk = lla.gdn_default_chunk(w.dk, w.dv, w.dtype)
    ws = torch.empty(lla.gdn_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, chunk, w.dtype),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(d["v"])
    call = lambda evs=None: lla.gdn_forward(d["q"], d["k"], d["v"], d["log_a"], d["beta"], d["lam"], out,
                                            chunk=chunk, workspace=ws, stream=stream, stage_events=evs)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for ev in evs:
        ev.record(stream)
    torch.cuda.synchronize(dev)
    call(evs)
    torch.cuda.synchronize(dev)
    stages = {"chunk": evs[0].elapsed_time(evs[1]), "upsweep": evs[1].elapsed_time(evs[2]),
              "query": evs[2].elapsed_time(evs[3])}
    flop_ht, byte_ht = gdn_algorithmic(w, chunk)
    ht = w.B * w.H * w.T
    tflops = flop_ht * ht / (ms * 1e-3) / 1e12
    return {
        "config": {"workload": w.name, "chunk": chunk, "workspace_bytes": ws.numel()},
        "ms_per_call": ms,
        "stages_ms": stages,
        "tokens_per_s": w.B * w.T / (ms * 1e-3),
        "algorithmic_flop_per_call": flop_ht * ht,
        "algorithmic_bytes_per_call": byte_ht * ht,
        "hbm_frac": byte_ht * ht / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "roofline": {"bound": "alu", "achieved": tflops, "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / FP32_PEAK_TFLOPS, "scope": "whole call, against the float32 rate (for bf16 inputs with dk >= 32 the up-sweep and query kernels multiply in split bf16, the chunk kernel its leaf products and the attention matrix times v; its other products in float32)"},
    }


def cpu_recurrent(w, x, heads: int) -> dict:
    """The oracle's O(T log T) recurrent form (one dk x dv state per level, carry merges) on
    `heads` heads of the workload, scaled to the whole call: the second CPU reference."""
    import oracle.loglinear as O
    heads = max(1, min(heads, w.H))
    sl = slice(0, heads)
    t = time.perf_counter()
    O.recurrent(x["q"][:1, sl], x["k"][:1, sl], x["v"][:1, sl], x["log_a"][:1, sl], x["lam"][:1, sl])
    dt = time.perf_counter() - t
    full = dt * w.B * w.H / heads
    return {"value": w.B * w.T / full, "unit": "tokens/s", "kind": "oracle (recurrent form)",
            "sample": f"recurrent form on {heads} of {w.B * w.H} heads, {dt:.2f} s measured, scaled "
                      f"x{w.B * w.H / heads:g}", "seconds_measured": dt}


def cpu_baseline(w, x, heads: int) -> dict:
    """The fp64 oracle as it stands, on `heads` heads of the workload, scaled to tokens/s."""
    import oracle.loglinear as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    heads = max(1, min(heads, w.H))
    sl = slice(0, heads)
    t = time.perf_counter()
    O.bruteforce(x["q"][:1, sl], x["k"][:1, sl], x["v"][:1, sl], x["log_a"][:1, sl], x["lam"][:1, sl])
    dt = time.perf_counter() - t
    # every head costs the same: the whole call (B*H heads) takes dt * B*H / heads
    full = dt * w.B * w.H / heads
    cpu = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": w.B * w.T / full,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"O(T^2) fp64 brute force on {heads} of {w.B * w.H} heads (b=0, h<{heads}), "
                   f"T={w.T}, {dt:.2f} s measured, scaled x{w.B * w.H / heads:g} to the full call"),
        "cpu_model": cpu or platform.processor(),
        "seconds_measured": dt,
    }


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--chunk", type=int, default=0, help="0: the workload's stated chunk size")
    ap.add_argument("--sweep", type=int, default=0, help="0: library default")
    ap.add_argument("--cpu-heads", type=int, default=12)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-only", action="store_true",
                    help="skip the cold-cache, copy-bandwidth and CPU legs (profiler runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 device copies of MIB MiB (hardware-counter calibration)")
    ap.add_argument("--no-decode", action="store_true", help="skip the decoding-step measurement")
    ap.add_argument("--no-varlen", action="store_true", help="skip the variable-length measurement")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass measurement")
    ap.add_argument("--no-gdn", action="store_true", help="skip the log-linear Gated DeltaNet measurement")
    ap.add_argument("--tune", nargs="*", metavar="WORKLOAD", default=None,
                    help="only time every chunk/sweep that fits, for these workloads (all if none; "
                         "shape:B,H,T,dk,dv,dtype for another shape)")
    ap.add_argument("--counters", default=os.path.join(ROOT, "profiles", "fwd_counters.json"),
                    help="forward-kernel counters per workload (rocprofv3: HBM traffic, MFMA busy cycles)")
    a = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {a.gpus}, WORLD_SIZE {world}); "
              "the heads of this method shard across GPUs with no communication, so the "
              "one-GPU figure is the per-GPU share.", file=sys.stderr)
        return 2

    import torch
    if a.copy_calibration:
        src = torch.ones(a.copy_calibration << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel(), "copies": 5}))
        return 0
    import log_linear_attention_chunked_amd as lla
    from lla_synth import WORKLOADS, generate
    from log_linear_attention_chunked_amd import _lib

    if a.tune is not None:
        tune(a.tune or list(WORKLOADS))
        return 0
    if not os.path.exists(_lib.LIB_PATH):
        from log_linear_attention_chunked_amd.build import build
        build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1

    w = WORKLOADS[a.workload]
    chunk = a.chunk or w.chunk
    dev = torch.device("cuda:0")
    x = generate(w, seed=0)
    d = {k: v.to(dev) for k, v in x.items()}
    out = torch.empty_like(d["v"])
    sweep = a.sweep or lla.default_sweep(w.B, w.H, w.T, w.dk, w.dv, chunk, w.dtype)
    nws = lla.workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, chunk, sweep, w.dtype)
    ws = torch.zeros(max(nws, 1), dtype=torch.uint8, device=dev)     # zero-filled once
    stream = torch.cuda.current_stream(dev)

    def new_events():
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for e in evs:
            e.record(stream)        # creates the underlying hipEvent_t
        return evs

    def step(evs=None):
        # only the events around the forward kernel: each recorded event costs a few
        # microseconds of queue time, and a caller workspace needs no fill kernel
        lla.forward(d["q"], d["k"], d["v"], d["log_a"], d["lam"], out, chunk=chunk, sweep=sweep,
                    workspace=ws, stream=stream, stage_events=None if evs is None else [None] + evs)

    # The timed region holds the K calls and nothing else (each call is one forward kernel
    # launch on this stream), bracketed by one pair of events (their interval over K: a launch
    # back to back with the next, the gap between them included). The kernel's own average
    # launch duration is then taken over K more launches with a pair of events around each (the
    # library's stage events on the launch stream), outside the timed region, whose step time
    # the extra event records would otherwise lengthen.
    region = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize(dev)
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    region[0].record(stream)
    for i in range(a.steps):
        step()
    region[1].record(stream)
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0
    back_to_back_ms = region[0].elapsed_time(region[1]) / a.steps

    evsets = [new_events() for _ in range(a.steps)]
    torch.cuda.synchronize(dev)
    for i in range(a.steps):
        step(evsets[i])
    torch.cuda.synchronize(dev)
    stage = {"forward": sum(e[0].elapsed_time(e[1]) for e in evsets) / a.steps}

    tokens = w.B * w.T
    ht = w.B * w.H * w.T
    flop_ht, byte_ht = algorithmic_per_token(w, chunk)
    ms_per_step = elapsed / a.steps * 1e3
    value = tokens * a.steps / elapsed

    t_out = stage["forward"] * 1e-3
    achieved = byte_ht * ht / t_out / 1e9
    # counters recorded by rocprofv3 for this workload and launch configuration, used only while
    # the forward kernel's sources are the ones they were taken from
    traffic = mfma_busy = None
    if os.path.exists(a.counters):
        try:
            rec = json.load(open(a.counters))["records"].get(w.name, {})
            if (rec.get("chunk") == chunk and rec.get("sweep") == sweep
                    and rec.get("kernel_source_sha") == _kernel_sha()):
                traffic = rec.get("hbm_bytes_per_launch")
                mfma_busy = rec.get("mfma_busy_frac")
        except (OSError, ValueError, KeyError):
            traffic = mfma_busy = None
    peak_flops = (BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS) * 1e12
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv,
                   "L": w.L, "chunk": chunk, "sweep": sweep, "parallelism": "single-gpu"},
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "kernel": "lla_fwd_kernel",
            "kernel_ms": stage["forward"],
            "kernel_ms_timing": "HIP events around each of K launches, right after the timed region",
            "ms_per_launch_back_to_back": back_to_back_ms,
            "algorithmic_bytes_per_launch": byte_ht * ht,
        },
        "stages_ms": stage,
        "path_hbm_frac": byte_ht * ht / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "mfma_util_algorithmic": flop_ht * ht / (ms_per_step * 1e-3) / peak_flops,
        "mfma_busy_counter": mfma_busy,
        "algorithmic_flop_per_step": flop_ht * ht,
    }

    if not a.no_decode:
        res["decode"] = decode_measure(w, dev, stream)
    if not a.no_varlen and not a.kernel_only:
        res["varlen"] = varlen_measure(dev, stream)
    if not a.no_backward:
        res["backward"] = backward_measure(w, d, dev, stream)
    if not a.kernel_only:
        res["lambda_bf16"] = lambda_bf16_measure(w, d, chunk, sweep, ws, dev, stream, a.steps)
    if not a.kernel_only and not a.no_gdn:
        res["gated_deltanet"] = gdn_measure(dev, stream)

    if not a.kernel_only:
        # cold caches: overwrite a 512 MiB buffer (outside the events) before each call
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cold = []
        for _ in range(max(5, min(a.steps, 20))):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            torch.cuda.synchronize(dev)
            cold.append(e0.elapsed_time(e1))
        cold.sort()
        res["cold_ms_per_step_median"] = cold[len(cold) // 2]
        del flush
        # achievable HBM reference: device-to-device copy of 1 GiB
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(5):
            dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize(dev)
        res["copy_gbs"] = 2 * 5 * (1 << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del src, dst

    if not a.kernel_only and not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, x, a.cpu_heads)
        res["cpu_baseline"]["recurrent_form"] = cpu_recurrent(w, x, 8)
        res["gpu_over_cpu"] = value / res["cpu_baseline"]["value"]

    print(json.dumps(res), flush=True)
    return 0


def _kernel_sha() -> str:
    """Hash of the forward kernel's sources (its kernels, instantiations and launch code), to tell
    whether recorded counters still apply."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "log_linear_attention_chunked_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")) and f.startswith(("lla_api", "lla_dispatch", "lla_inst", "lla_kernels")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    sys.exit(main())
