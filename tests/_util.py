"""Shared test helpers: build-on-demand, device runs, error metrics."""

from __future__ import annotations

import os

import numpy as np

from log_linear_attention_chunked_amd import _lib


def ensure_built():
    """Load what is built; build only when nothing is."""
    if not os.path.exists(_lib.LIB_PATH):
        from log_linear_attention_chunked_amd.build import build
        build()


def fits_smem(dtype: str, C: int, dk: int, dv: int, R: int) -> bool:
    """Whether R resident chunks fit the 160 KB of gfx950 shared memory (q, k, v images,
    24 lambda levels, decays and flag, P^T fragments per chunk, plus copies of up to 8 waves'
    node flags and the ticket)."""
    es = 2 if dtype == "bf16" else 4
    per = C * (2 * dk + dv) * es + C * 24 * 4 + 16 * C + 16 + (C // 16) * ((C + 31) // 32) * 512 * es
    return ((R * per + 256 + 16 + 255) & ~255) <= 160 * 1024


def host_threads() -> int:
    """Host cores this process may use (the GPU machine grants 16 per GPU), at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def per_head(fn, heads, workers: int | None = None) -> list:
    """[fn(b, h) for (b, h) in heads], evaluated by a thread pool with single-threaded BLAS.

    The oracle's work per head is numpy calls that release the GIL, so heads run in parallel
    on the host cores; results come back in the order of ``heads``. Only the scheduling lives
    here: what each call computes is the oracle's own code.
    """
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    heads = list(heads)
    workers = workers or host_threads()
    with threadpool_limits(1):
        with ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(lambda bh: fn(*bh), heads))


def rel_l2(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


def tol_for(dtype: str) -> float:
    """Relative-L2 bars: 1e-4 for float32 inputs, 2e-2 for bfloat16 inputs with float32
    accumulation."""
    return 1e-4 if dtype == "f32" else 2e-2


def to_device(x: dict):
    return {k: v.cuda() for k, v in x.items()}


def run_gpu(x: dict, **kw) -> np.ndarray:
    """Device forward pass on CPU inputs `x`; returns float64 numpy of the output."""
    import torch
    import log_linear_attention_chunked_amd as lla
    d = to_device(x)
    out = lla.forward(d["q"], d["k"], d["v"], d["log_a"], d["lam"], **kw)
    torch.cuda.synchronize()
    return out.double().cpu().numpy()
