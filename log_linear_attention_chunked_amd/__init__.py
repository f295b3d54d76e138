"""Log-linear Mamba-2 attention forward pass on MI355X (gfx950), behind a C ABI.

    from log_linear_attention_chunked_amd import forward, backward
    out = forward(q, k, v, log_a, lam)          # device tensors, [B,H,T,d] layout
    dq, dk, dv, dlog_a, dlam = backward(q, k, v, log_a, lam, dout)

Computes, per head, o_t = sum_{s<=t} lam[t, l(t,s)] * prod_{r=s+1..t} a_r * (q_t.k_s) v_s
with l(t,s) = bit_length(t XOR s) (Fenwick level) and a_r = exp(log_a[r]).
PyTorch supplies device memory and the current stream; every step of the computation
runs in the library's HIP kernels (``libloglinear_attn.so``).
"""

from __future__ import annotations

import ctypes

from . import _lib
from ._lib import LibraryNotBuilt  # noqa: F401

__all__ = ["forward", "forward_noalloc", "noalloc_scratch_bytes", "gdn_forward", "gdn_workspace_bytes",
           "gdn_default_chunk", "backward", "decode_prefill", "bwd_workspace_bytes", "bwd_default_chunk", "forward_varlen", "decode_step", "new_decode_cache", "num_levels", "workspace_bytes",
           "default_chunk", "default_sweep", "LLAError", "LibraryNotBuilt"]


class LLAError(RuntimeError):
    def __init__(self, status: int, where: str = "loglinear_attn_fwd_ex"):
        self.status = status
        super().__init__(f"{where} returned {status}: {_lib.status_string(status)}")


def num_levels(T: int) -> int:
    """Number of lambda levels for T tokens (bit_length(T-1) + 1)."""
    return _lib.lib().loglinear_attn_num_levels(int(T))


def _dtype_code(dtype) -> int:
    import torch
    if dtype in (torch.bfloat16, "bf16"):
        return _lib.LLA_DTYPE_BF16
    if dtype in (torch.float32, "f32"):
        return _lib.LLA_DTYPE_F32
    raise TypeError(f"unsupported q/k/v dtype {dtype}")


def workspace_bytes(B, H, T, dk, dv, chunk=0, sweep=0, dtype="bf16") -> int:
    return int(_lib.lib().loglinear_attn_workspace_bytes(
        int(B), int(H), int(T), int(dk), int(dv), int(chunk), int(sweep), _dtype_code(dtype)))


def default_chunk(dk, dv, T=0, dtype="bf16") -> int:
    return _lib.lib().loglinear_attn_default_chunk(int(dk), int(dv), int(T), _dtype_code(dtype))


def default_sweep(B, H, T, dk, dv, chunk=0, dtype="bf16") -> int:
    return _lib.lib().loglinear_attn_default_sweep(int(B), int(H), int(T), int(dk), int(dv),
                                                   int(chunk), _dtype_code(dtype))


def _check(t, name, dtype, shape):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_lam(lam, shape):
    """lambda: float32, or bfloat16 (the library widens it exactly)."""
    import torch
    _check(lam, "lam", torch.bfloat16 if getattr(lam, "dtype", None) == torch.bfloat16 else torch.float32,
           shape)


def make_args(q, k, v, log_a, lam, out, *, chunk=0, sweep=0, workspace=None,
              stage_events=None) -> _lib.FwdArgs:
    """Validate tensors and fill the C argument struct (no device work)."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, dk]")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    L = num_levels(T) if T > 0 else 0
    _check(q, "q", q.dtype, (B, H, T, dk))
    _check(k, "k", q.dtype, (B, H, T, dk))
    _check(v, "v", q.dtype, (B, H, T, dv))
    _check(log_a, "log_a", torch.float32, (B, H, T))
    _check_lam(lam, (B, H, T, L))
    _check(out, "out", q.dtype, (B, H, T, dv))
    a = _lib.FwdArgs()
    a.lambda_bf16 = int(lam.dtype == torch.bfloat16)
    a.q, a.k, a.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    a.log_a, a.lam, a.out = log_a.data_ptr(), lam.data_ptr(), out.data_ptr()
    a.B, a.H, a.T, a.dk, a.dv = int(B), int(H), int(T), int(dk), int(dv)
    a.dtype = _dtype_code(q.dtype)
    a.chunk, a.sweep = int(chunk), int(sweep)
    if workspace is not None:
        _check(workspace, "workspace", torch.uint8, (workspace.numel(),))
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    else:
        a.workspace, a.workspace_bytes = None, 0
    if stage_events is not None:
        for i, ev in enumerate(stage_events):
            a.stage_events[i] = ev.cuda_event if ev is not None else None
    return a


def forward(q, k, v, log_a, lam, out=None, *, chunk: int = 0, sweep: int = 0,
            workspace=None, stream=None, stage_events=None):
    """Forward pass on the current device and stream (or ``stream``).

    q, k: [B,H,T,dk]; v: [B,H,T,dv] (bfloat16 or float32, all the same);
    log_a: [B,H,T] float32; lam: [B,H,T,L] float32 (or bfloat16: half the bytes, read
    exactly) with L = num_levels(T). Returns out [B,H,T,dv] in q's dtype. ``chunk``/``sweep`` 0 = library default;
    ``workspace``: optional uint8 device tensor of >= workspace_bytes(...) bytes.
    ``stage_events``: optional recorded ``torch.cuda.Event`` objects (up to 4, or None)
    the library records around its kernels: before the fill kernel, before the forward
    kernel, after the forward kernel (the fourth is not used).
    """
    import torch
    if out is None:
        out = torch.empty(q.shape[:3] + (v.shape[-1],), dtype=q.dtype, device=q.device)
    a = make_args(q, k, v, log_a, lam, out, chunk=chunk, sweep=sweep, workspace=workspace,
                  stage_events=stage_events)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    st = _lib.lib().loglinear_attn_fwd_ex(ctypes.byref(a), ctypes.c_void_p(handle))
    if st != _lib.LLA_OK:
        raise LLAError(st)
    return out


def forward_noalloc(q, k, v, log_a, lam, out, *, chunk: int = 0, sweep: int = 0, stream=None,
                    stage_events=None):
    """``forward`` through ``loglinear_attn_fwd_noalloc``: the library allocates nothing (its
    workspace is a fixed per-device scratch of ``noalloc_scratch_bytes()`` bytes), and ``out``
    must be given, so the call allocates no device memory at all. Same output as ``forward``,
    bitwise. Calls on one device must not overlap in time (they share the scratch)."""
    import torch
    a = make_args(q, k, v, log_a, lam, out, chunk=chunk, sweep=sweep, workspace=None,
                  stage_events=stage_events)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    st = _lib.lib().loglinear_attn_fwd_noalloc(ctypes.byref(a), ctypes.c_void_p(handle))
    if st != _lib.LLA_OK:
        raise LLAError(st, "loglinear_attn_fwd_noalloc")
    return out


def noalloc_scratch_bytes() -> int:
    """Bytes of the fixed per-device scratch that ``forward_noalloc`` uses."""
    return int(_lib.lib().loglinear_attn_noalloc_scratch_bytes())


def gdn_workspace_bytes(B, H, T, dk, dv, chunk=0, dtype="bf16") -> int:
    return int(_lib.lib().loglinear_attn_gdn_workspace_bytes(
        int(B), int(H), int(T), int(dk), int(dv), int(chunk), _dtype_code(dtype)))


def gdn_default_chunk(dk, dv, dtype="bf16") -> int:
    return int(_lib.lib().loglinear_attn_gdn_default_chunk(int(dk), int(dv), _dtype_code(dtype)))


def gdn_forward(q, k, v, log_a, beta, lam, out=None, *, chunk: int = 0, workspace=None,
                stream=None, stage_events=None):
    """Log-linear Gated DeltaNet forward (``loglinear_attn_gdn_fwd``) on the current stream.

    q, k: [B,H,T,dk]; v: [B,H,T,dv] (bfloat16 or float32, all the same; keys L2-normalised by the
    caller); log_a, beta: [B,H,T] float32; lam: [B,H,T,L] float32 or bfloat16, L = num_levels(T).
    Returns out [B,H,T,dv] in q's dtype. ``chunk`` 0 = library default; ``workspace``: optional
    uint8 device tensor of >= gdn_workspace_bytes(...) bytes; ``stage_events``: up to 4 recorded
    ``torch.cuda.Event`` (before the chunk kernel, the up-sweep, the query kernel, after it).
    """
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, dk]")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    L = num_levels(T) if T > 0 else 0
    _check(q, "q", q.dtype, (B, H, T, dk))
    _check(k, "k", q.dtype, (B, H, T, dk))
    _check(v, "v", q.dtype, (B, H, T, dv))
    _check(log_a, "log_a", torch.float32, (B, H, T))
    _check(beta, "beta", torch.float32, (B, H, T))
    _check_lam(lam, (B, H, T, L))
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    _check(out, "out", q.dtype, (B, H, T, dv))
    a = _lib.GdnArgs()
    a.q, a.k, a.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    a.log_a, a.beta, a.lam, a.out = log_a.data_ptr(), beta.data_ptr(), lam.data_ptr(), out.data_ptr()
    a.lambda_bf16 = int(lam.dtype == torch.bfloat16)
    a.B, a.H, a.T, a.dk, a.dv = int(B), int(H), int(T), int(dk), int(dv)
    a.dtype = _dtype_code(q.dtype)
    a.chunk = int(chunk)
    if workspace is not None:
        _check(workspace, "workspace", torch.uint8, (workspace.numel(),))
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    else:
        a.workspace, a.workspace_bytes = None, 0
    if stage_events is not None:
        for i, ev in enumerate(stage_events):
            a.stage_events[i] = ev.cuda_event if ev is not None else None
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    st = _lib.lib().loglinear_attn_gdn_fwd(ctypes.byref(a), ctypes.c_void_p(handle))
    if st != _lib.LLA_OK:
        raise LLAError(st, "loglinear_attn_gdn_fwd")
    return out


def new_decode_cache(B, H, dk, dv, levels, device="cuda"):
    """An empty decoding cache: (state [B,H,levels,dk,dv], log_scale [B,H,2,levels]), float32.
    ``levels`` >= bit_length(t) + 1 for every position t it will see (<= 25)."""
    import torch
    state = torch.empty((B, H, levels, dk, dv), dtype=torch.float32, device=device)
    log_scale = torch.empty((B, H, 2, levels), dtype=torch.float32, device=device)
    return state, log_scale


def decode_prefill(k, v, log_a, state, log_scale, *, stream=None):
    """Fill a decoding cache from a prompt: afterwards ``decode_step`` continues at t = T.

    k: [B,H,T,dk], v: [B,H,T,dv] (bfloat16 or float32); log_a: [B,H,T] float32;
    state [B,H,Lc,dk,dv] and log_scale [B,H,2,Lc] float32 (``new_decode_cache`` with
    levels >= bit_length(T) + 1).
    """
    import torch
    if k.dim() != 4:
        raise ValueError("k must be [B, H, T, dk]")
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    Lc = state.shape[2] if state.dim() == 5 else -1
    _check(k, "k", k.dtype, (B, H, T, dk))
    _check(v, "v", k.dtype, (B, H, T, dv))
    _check(log_a, "log_a", torch.float32, (B, H, T))
    _check(state, "state", torch.float32, (B, H, Lc, dk, dv))
    _check(log_scale, "log_scale", torch.float32, (B, H, 2, Lc))
    a = _lib.PrefillArgs()
    a.k, a.v, a.log_a = k.data_ptr(), v.data_ptr(), log_a.data_ptr()
    a.state, a.log_scale = state.data_ptr(), log_scale.data_ptr()
    a.B, a.H, a.T, a.dk, a.dv, a.Lc = int(B), int(H), int(T), int(dk), int(dv), int(Lc)
    a.dtype = _dtype_code(k.dtype)
    if stream is None:
        stream = torch.cuda.current_stream(k.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    st = _lib.lib().loglinear_attn_decode_prefill(ctypes.byref(a), ctypes.c_void_p(handle))
    if st != _lib.LLA_OK:
        raise LLAError(st, "loglinear_attn_decode_prefill")
    return state, log_scale


def decode_step(q, k, v, log_a, lam, state, log_scale, t: int, out=None, *, stream=None,
                t_seq=None):
    """One decoding step at position ``t`` (the same for every (b, h)); updates the cache.

    q, k: [B,H,dk]; v: [B,H,dv] (bfloat16 or float32); log_a: [B,H] float32;
    lam: [B,H,Lc] float32 (the token's level weights); state [B,H,Lc,dk,dv] and
    log_scale [B,H,2,Lc] float32 (``new_decode_cache``). Returns out [B,H,dv] in q's dtype.
    Steps on one cache must be issued for t = 0, 1, 2, ... in order.
    ``t_seq``: optional int64 device tensor [B], one position per sequence (``t`` is then the
    largest of them); a negative entry skips that sequence (cache and out rows untouched).
    """
    import torch
    if q.dim() != 3:
        raise ValueError("q must be [B, H, dk]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    Lc = state.shape[2] if state.dim() == 5 else -1
    _check(q, "q", q.dtype, (B, H, dk))
    _check(k, "k", q.dtype, (B, H, dk))
    _check(v, "v", q.dtype, (B, H, dv))
    _check(log_a, "log_a", torch.float32, (B, H))
    _check(lam, "lam", torch.float32, (B, H, Lc))
    _check(state, "state", torch.float32, (B, H, Lc, dk, dv))
    _check(log_scale, "log_scale", torch.float32, (B, H, 2, Lc))
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    _check(out, "out", q.dtype, (B, H, dv))
    a = _lib.DecodeArgs()
    a.q, a.k, a.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    a.log_a, a.lam, a.out = log_a.data_ptr(), lam.data_ptr(), out.data_ptr()
    a.state, a.log_scale = state.data_ptr(), log_scale.data_ptr()
    a.B, a.H, a.dk, a.dv, a.Lc = int(B), int(H), int(dk), int(dv), int(Lc)
    a.dtype = _dtype_code(q.dtype)
    a.t = int(t)
    if t_seq is not None:
        _check(t_seq, "t_seq", torch.int64, (B,))
        a.t_seq = t_seq.data_ptr()
    else:
        a.t_seq = None
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    st = _lib.lib().loglinear_attn_decode_step(ctypes.byref(a), ctypes.c_void_p(handle))
    if st != _lib.LLA_OK:
        raise LLAError(st, "loglinear_attn_decode_step")
    return out


def forward_varlen(q, k, v, log_a, lam, cu_seqlens, max_T: int, out=None, *, chunk: int = 0,
                   sweep: int = 0, workspace=None, stream=None, cu_seqlens_host=None):
    """Forward pass over N sequences packed along time (variable-length batch).

    q, k: [H, total_T, dk]; v: [H, total_T, dv] (bfloat16 or float32); log_a: [H, total_T]
    float32; lam: [H, total_T, L] float32 with L = num_levels(max_T); cu_seqlens: int32
    device tensor [N+1] of sequence boundaries (0 = cu_seqlens[0] <= ... <= cu_seqlens[N] =
    total_T); max_T >= every sequence length. Each sequence's positions start at 0.
    cu_seqlens_host: optional host copy of the same values (CPU tensor or list): the launch then
    has one workgroup per sweep that exists instead of one per sweep of max_T tokens.
    Returns out [H, total_T, dv] in q's dtype (rows outside every sequence are untouched).
    """
    import torch
    if q.dim() != 3:
        raise ValueError("q must be [H, total_T, dk]")
    H, TT, dk = q.shape
    dv = v.shape[-1]
    L = num_levels(max_T) if max_T > 0 else 0
    N = cu_seqlens.numel() - 1
    _check(q, "q", q.dtype, (H, TT, dk))
    _check(k, "k", q.dtype, (H, TT, dk))
    _check(v, "v", q.dtype, (H, TT, dv))
    _check(log_a, "log_a", torch.float32, (H, TT))
    _check_lam(lam, (H, TT, L))
    _check(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,))
    if out is None:
        out = torch.empty((H, TT, dv), dtype=q.dtype, device=q.device)
    _check(out, "out", q.dtype, (H, TT, dv))
    a = _lib.VarlenArgs()
    a.q, a.k, a.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    a.log_a, a.lam, a.out = log_a.data_ptr(), lam.data_ptr(), out.data_ptr()
    a.lambda_bf16 = int(lam.dtype == torch.bfloat16)
    a.cu_seqlens = cu_seqlens.data_ptr()
    host = None
    if cu_seqlens_host is not None:
        host = torch.as_tensor(cu_seqlens_host, dtype=torch.int32, device="cpu").contiguous()
        if host.shape != (N + 1,):
            raise ValueError(f"cu_seqlens_host must hold {N + 1} values, got {tuple(host.shape)}")
    a.cu_seqlens_host = host.data_ptr() if host is not None else None
    a.N, a.H, a.total_T, a.max_T, a.dk, a.dv = int(N), int(H), int(TT), int(max_T), int(dk), int(dv)
    a.dtype = _dtype_code(q.dtype)
    a.chunk, a.sweep = int(chunk), int(sweep)
    if workspace is not None:
        _check(workspace, "workspace", torch.uint8, (workspace.numel(),))
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    else:
        a.workspace, a.workspace_bytes = None, 0
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    st = _lib.lib().loglinear_attn_fwd_varlen(ctypes.byref(a), ctypes.c_void_p(handle))
    if st != _lib.LLA_OK:
        raise LLAError(st, "loglinear_attn_fwd_varlen")
    return out


def bwd_workspace_bytes(B, H, T, dk, dv, chunk=0, dtype="bf16") -> int:
    return int(_lib.lib().loglinear_attn_bwd_workspace_bytes(
        int(B), int(H), int(T), int(dk), int(dv), int(chunk), _dtype_code(dtype)))


def bwd_default_chunk(dk, dv, dtype="bf16") -> int:
    return _lib.lib().loglinear_attn_bwd_default_chunk(int(dk), int(dv), _dtype_code(dtype))


def backward(q, k, v, log_a, lam, dout, *, chunk: int = 0, workspace=None, stream=None,
             stage_events=None, out=None):
    """Backward pass: gradients of ``sum(dout * forward(q, k, v, log_a, lam))``.

    Inputs as for ``forward`` plus ``dout`` [B,H,T,dv] in q's dtype. Returns
    ``(dq, dk, dv, dlog_a, dlam)``: dq, dk [B,H,T,dk] and dv [B,H,T,dv] in q's dtype,
    dlog_a [B,H,T] and dlam [B,H,T,L] float32. ``out``: optional tuple of those five
    tensors to write into. ``chunk`` 0 = library default (16, 32 or 64); ``workspace``:
    optional uint8 device tensor of >= bwd_workspace_bytes(...) bytes. ``stage_events``:
    up to 4 ``torch.cuda.Event`` (or None) recorded before the chunk states, before and
    after the gradient kernel, and after the log_a scan.
    """
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, dk]")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    L = num_levels(T) if T > 0 else 0
    _check(q, "q", q.dtype, (B, H, T, dk))
    _check(k, "k", q.dtype, (B, H, T, dk))
    _check(v, "v", q.dtype, (B, H, T, dv))
    _check(log_a, "log_a", torch.float32, (B, H, T))
    _check_lam(lam, (B, H, T, L))
    _check(dout, "dout", q.dtype, (B, H, T, dv))
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
               torch.empty_like(log_a), torch.empty(lam.shape, dtype=torch.float32, device=lam.device))
    gq, gk, gv, gla, glam = out
    _check(gq, "dq", q.dtype, (B, H, T, dk))
    _check(gk, "dk", q.dtype, (B, H, T, dk))
    _check(gv, "dv", q.dtype, (B, H, T, dv))
    _check(gla, "dlog_a", torch.float32, (B, H, T))
    _check(glam, "dlam", torch.float32, (B, H, T, L))
    a = _lib.BwdArgs()
    a.q, a.k, a.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    a.log_a, a.lam, a.grad_out = log_a.data_ptr(), lam.data_ptr(), dout.data_ptr()
    a.lambda_bf16 = int(lam.dtype == torch.bfloat16)
    a.grad_q, a.grad_k, a.grad_v = gq.data_ptr(), gk.data_ptr(), gv.data_ptr()
    a.grad_log_a, a.grad_lam = gla.data_ptr(), glam.data_ptr()
    a.B, a.H, a.T, a.dk, a.dv = int(B), int(H), int(T), int(dk), int(dv)
    a.dtype = _dtype_code(q.dtype)
    a.chunk = int(chunk)
    if workspace is not None:
        _check(workspace, "workspace", torch.uint8, (workspace.numel(),))
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    else:
        a.workspace, a.workspace_bytes = None, 0
    if stage_events is not None:
        for i, ev in enumerate(stage_events):
            a.stage_events[i] = ev.cuda_event if ev is not None else None
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    st = _lib.lib().loglinear_attn_bwd(ctypes.byref(a), ctypes.c_void_p(handle))
    if st != _lib.LLA_OK:
        raise LLAError(st, "loglinear_attn_bwd")
    return out
