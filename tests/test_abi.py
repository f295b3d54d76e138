"""The C-ABI library: it loads, exports what include/loglinear_attn.h declares, and its
host-side validation returns the documented codes without touching a device."""

import ctypes
import os
import re

import pytest

from log_linear_attention_chunked_amd import _lib
from tests._util import ensure_built

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "loglinear_attn.h")


@pytest.fixture(scope="module")
def L():
    ensure_built()
    return _lib.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(loglinear_attn_\w+)\s*\(", src)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_num_levels(L):
    assert [L.loglinear_attn_num_levels(T) for T in (0, 1, 2, 3, 4, 5, 256, 2048, 8192, 32768, 65536)] == \
        [0, 1, 2, 3, 3, 4, 9, 12, 14, 16, 17]


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, -5):
        s = _lib.status_string(code)
        assert s and s != "unknown status"
    assert _lib.status_string(-99) == "unknown status"


def test_defaults(L):
    # the measured rule (header): chunk 64, 128 for bf16 d = 128 at T >= 65536, 32 for small fp32
    assert L.loglinear_attn_default_chunk(16, 16, 256, 1) == 32
    assert L.loglinear_attn_default_chunk(16, 16, 4096, 0) == 64
    assert L.loglinear_attn_default_chunk(64, 64, 8192, 0) == 64
    assert L.loglinear_attn_default_chunk(128, 128, 32768, 0) == 64
    assert L.loglinear_attn_default_chunk(128, 128, 65536, 0) == 128
    assert L.loglinear_attn_default_chunk(128, 128, 65536, 1) == 64
    assert L.loglinear_attn_default_chunk(128, 64, 65536, 0) == 64
    assert L.loglinear_attn_default_chunk(48, 64, 8192, 0) == 0
    # headline shape: 64 heads x 128 chunks -> two resident chunks per workgroup
    assert L.loglinear_attn_default_sweep(4, 16, 8192, 64, 64, 64, 0) == 2
    assert L.loglinear_attn_default_sweep(2, 8, 2048, 64, 64, 64, 0) == 2      # 256 workgroups
    assert L.loglinear_attn_default_sweep(1, 1, 64, 64, 64, 64, 0) == 1        # one chunk
    assert L.loglinear_attn_default_sweep(1, 2, 2048, 64, 64, 64, 0) == 1      # too few workgroups
    assert L.loglinear_attn_default_sweep(64, 64, 65536, 128, 128, 64, 0) == 2
    assert L.loglinear_attn_default_sweep(1, 8, 65536, 128, 128, 0, 0) == 1   # chunk 128: shared memory
    assert L.loglinear_attn_default_sweep(64, 64, 65536, 64, 64, 64, 1) == 1   # float32
    assert L.loglinear_attn_default_sweep(1, 16, 4096, 16, 16, 0, 0) == 2      # d = 16 at chunk 64


def test_workspace_bytes(L):
    ws = L.loglinear_attn_workspace_bytes
    assert ws(1, 2, 32, 16, 16, 16, 2, 1) == 0              # one sweep covers T
    assert ws(1, 1, 64, 64, 64, 64, 1, 0) == 0              # one chunk
    assert ws(1, 2, 256, 16, 16, 16, 16, 1) == 0            # unsupported sweep -> 0
    n = ws(4, 16, 8192, 64, 64, 64, 2, 0)
    ns = 8192 // 64 // 2 - 1
    per = 64 * ns                   # (head, node) pairs; each node is kept per wave (dv/16 = 4)
    expect = per * 4 * 2 * 512 * 2 + 2 * per * 4 * 4 + 64 * 4   # bf16 fragments, decays, flags
    assert expect <= n <= expect + 3 * 256
    # dk = 16: a record still holds one full fragment per wave (features 16..31 zero)
    n16 = ws(1, 1, 4096, 16, 16, 64, 1, 0)
    per16 = 4096 // 64 - 1
    expect16 = per16 * 64 * 16 + 2 * per16 * 4 + 64 * 4
    assert expect16 <= n16 <= expect16 + 3 * 256
    assert ws(4, 16, 8192, 48, 64, 64, 2, 0) == 0           # invalid -> 0
    assert ws(1, 1, 1000, 64, 64, 64, 2, 0) > 0             # ragged T


def _args(**kw):
    a = _lib.FwdArgs()
    base = 1 << 40                 # fake, well-separated, aligned addresses: never dereferenced
    a.q, a.k, a.v = base, base + (1 << 32), base + (2 << 32)
    a.log_a, a.lam, a.out = base + (3 << 32), base + (4 << 32), base + (5 << 32)
    a.B, a.H, a.T, a.dk, a.dv = 1, 2, 4096, 64, 64
    a.dtype, a.chunk, a.sweep = 0, 64, 1
    a.workspace, a.workspace_bytes = None, 0
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


def _call(L, a):
    return L.loglinear_attn_fwd_ex(ctypes.byref(a), None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), _lib.LLA_ERR_INVALID_ARG),
    (dict(B=-1), _lib.LLA_ERR_INVALID_ARG),
    (dict(T=-5), _lib.LLA_ERR_INVALID_ARG),
    (dict(dk=48), _lib.LLA_ERR_UNSUPPORTED),
    (dict(dv=256), _lib.LLA_ERR_UNSUPPORTED),
    (dict(chunk=24), _lib.LLA_ERR_UNSUPPORTED),
    (dict(sweep=3), _lib.LLA_ERR_UNSUPPORTED),
    (dict(sweep=4), _lib.LLA_ERR_UNSUPPORTED),
    (dict(sweep=16), _lib.LLA_ERR_UNSUPPORTED),
    (dict(sweep=8), _lib.LLA_ERR_UNSUPPORTED),
    (dict(B=70000), _lib.LLA_ERR_UNSUPPORTED),
    (dict(q=None), _lib.LLA_ERR_INVALID_ARG),
    (dict(lam=None), _lib.LLA_ERR_INVALID_ARG),
    (dict(out=None), _lib.LLA_ERR_INVALID_ARG),
    (dict(q=(1 << 40) + 8), _lib.LLA_ERR_INVALID_ARG),           # misaligned
    (dict(log_a=(1 << 40) + (3 << 32) + 2), _lib.LLA_ERR_INVALID_ARG),
    (dict(out=(1 << 40) + 4096), _lib.LLA_ERR_INVALID_ARG),      # out overlaps q
    (dict(out=(1 << 40) + (4 << 32) + 256), _lib.LLA_ERR_INVALID_ARG),  # out overlaps lambda
    (dict(workspace=(1 << 44), workspace_bytes=1024), _lib.LLA_ERR_WORKSPACE),
    (dict(workspace=(1 << 44) + 16, workspace_bytes=1 << 30), _lib.LLA_ERR_INVALID_ARG),
])
def test_validation_codes(L, kw, code):
    assert _call(L, _args(**kw)) == code


def test_null_struct(L):
    assert L.loglinear_attn_fwd_ex(None, None) == _lib.LLA_ERR_INVALID_ARG


# float32 sweeps whose images exceed the 160 KB of shared memory of a compute unit: refused on
# the host, before any device call, with no workspace size either
FP32_TOO_BIG = [
    # chunk, dk, dv, sweep
    (128, 128, 128, 1), (128, 64, 64, 1), (128, 32, 128, 1), (128, 128, 16, 1),
    (128, 16, 16, 2), (64, 128, 128, 2), (64, 128, 16, 2), (64, 64, 128, 2),
]


@pytest.mark.parametrize("C,dk,dv,R", FP32_TOO_BIG)
def test_shared_memory_limits_are_host_checks(L, C, dk, dv, R):
    assert _call(L, _args(dtype=1, chunk=C, dk=dk, dv=dv, sweep=R)) == _lib.LLA_ERR_UNSUPPORTED
    assert L.loglinear_attn_workspace_bytes(1, 2, 4096, dk, dv, C, R, 1) == 0


@pytest.mark.parametrize("C,dk,dv,R", [(128, 64, 32, 1), (128, 16, 128, 1), (64, 128, 128, 1),
                                       (64, 64, 64, 2)])
def test_shared_memory_limits_largest_fp32_that_fit(L, C, dk, dv, R):
    assert L.loglinear_attn_workspace_bytes(1, 2, 4096, dk, dv, C, R, 1) > 0
    # defaults never pick a sweep that does not fit
    assert L.loglinear_attn_default_sweep(64, 64, 65536, dk, dv, C, 1) in (1, 2)


def test_lambda_dtype_validation(L):
    base = 1 << 40
    lam = base + (4 << 32)
    # bfloat16 lambda needs 2-byte alignment, float32 4-byte; other flag values are refused
    assert _call(L, _args(lambda_bf16=2)) == _lib.LLA_ERR_INVALID_ARG
    assert _call(L, _args(lambda_bf16=-1)) == _lib.LLA_ERR_INVALID_ARG
    assert _call(L, _args(lambda_bf16=1, lam=lam + 1)) == _lib.LLA_ERR_INVALID_ARG
    assert _call(L, _args(lambda_bf16=0, lam=lam + 2)) == _lib.LLA_ERR_INVALID_ARG
    # out overlapping the (half as long) bf16 lambda is still caught
    assert _call(L, _args(lambda_bf16=1, out=lam + 128)) == _lib.LLA_ERR_INVALID_ARG
    assert L.loglinear_attn_bwd(ctypes.byref(_bargs(lambda_bf16=3)), None) == _lib.LLA_ERR_INVALID_ARG
    assert L.loglinear_attn_bwd(ctypes.byref(_bargs(lambda_bf16=1, lam=lam + 1)), None) == _lib.LLA_ERR_INVALID_ARG
    assert L.loglinear_attn_bwd(ctypes.byref(_bargs(lambda_bf16=0, lam=lam + 2)), None) == _lib.LLA_ERR_INVALID_ARG
    # a 2-byte-aligned bf16 lambda passes validation (B = 0 keeps the call a no-op)
    assert _call(L, _args(B=0, lambda_bf16=1, lam=lam + 2)) == _lib.LLA_OK


def test_allocation_failure_returns_no_memory(L, monkeypatch):
    # the library takes the workspace itself (none given) and the allocation fails: the
    # documented status, before anything is launched
    monkeypatch.setenv("LLA_TEST_FAIL_ALLOC", "1")
    assert _call(L, _args()) == _lib.LLA_ERR_NO_MEMORY
    assert L.loglinear_attn_bwd(ctypes.byref(_bargs()), None) == _lib.LLA_ERR_NO_MEMORY
    # a caller workspace needs no allocation: validation still runs and reports its own codes
    assert _call(L, _args(workspace=(1 << 44), workspace_bytes=1024)) == _lib.LLA_ERR_WORKSPACE
    # one sweep covers the sequence: no workspace, so no allocation and nothing to fail (B = 0
    # keeps the call a no-op on a machine without a device)
    assert _call(L, _args(B=0)) == _lib.LLA_OK
    # the prefill's scratch for blocks longer than 256 positions (T = 1000: the 512-position
    # block of level 10 in two segments)
    assert L.loglinear_attn_decode_prefill(ctypes.byref(_pargs(T=1000, Lc=11)), None) == _lib.LLA_ERR_NO_MEMORY


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(T=0), dict(T=0, q=None, out=None)])
def test_empty_is_a_noop(L, kw):
    assert _call(L, _args(**kw)) == _lib.LLA_OK


def test_plain_entries_validate(L):
    vp = ctypes.c_void_p
    assert L.loglinear_attn_fwd(None, None, None, None, None, None, 1, 1, 8, 64, 64, None) == _lib.LLA_ERR_INVALID_ARG
    assert L.loglinear_attn_fwd_f32(None, None, None, None, None, None, 1, 1, 8, 20, 64, None) == _lib.LLA_ERR_UNSUPPORTED
    assert L.loglinear_attn_fwd(vp(16), vp(32), vp(48), vp(64), vp(80), vp(96), 0, 1, 8, 64, 64, None) == _lib.LLA_OK


def test_python_binding_requires_device_tensors():
    import torch
    import log_linear_attention_chunked_amd as lla
    ensure_built()
    x = torch.zeros(1, 1, 8, 16)
    with pytest.raises(ValueError):
        lla.forward(x, x, x, torch.zeros(1, 1, 8), torch.zeros(1, 1, 8, 4))


# ---------------------------------------------------------------------------------------
# decoding step: host-side validation only (every case returns before any launch)
# ---------------------------------------------------------------------------------------

def _dargs(**kw):
    a = _lib.DecodeArgs()
    base = 1 << 40                 # fake, well-separated, aligned addresses: never dereferenced
    a.q, a.k, a.v = base, base + (1 << 32), base + (2 << 32)
    a.log_a, a.lam, a.out = base + (3 << 32), base + (4 << 32), base + (5 << 32)
    a.state, a.log_scale = base + (6 << 32), base + (7 << 32)
    a.B, a.H, a.dk, a.dv, a.Lc, a.dtype, a.t = 1, 2, 64, 64, 14, 0, 100
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), _lib.LLA_ERR_UNSUPPORTED),
    (dict(B=-1), _lib.LLA_ERR_INVALID_ARG),
    (dict(t=-1), _lib.LLA_ERR_INVALID_ARG),
    (dict(Lc=0), _lib.LLA_ERR_INVALID_ARG),
    (dict(dk=48), _lib.LLA_ERR_UNSUPPORTED),
    (dict(dv=8), _lib.LLA_ERR_UNSUPPORTED),
    (dict(Lc=26), _lib.LLA_ERR_UNSUPPORTED),
    (dict(t=1 << 13, Lc=14), _lib.LLA_ERR_INVALID_ARG),     # needs bit_length(t)+1 = 15 levels
    (dict(q=None), _lib.LLA_ERR_INVALID_ARG),
    (dict(state=None), _lib.LLA_ERR_INVALID_ARG),
    (dict(log_scale=None), _lib.LLA_ERR_INVALID_ARG),
    (dict(q=(1 << 40) + 1), _lib.LLA_ERR_INVALID_ARG),     # misaligned bf16
    (dict(state=(1 << 40) + (6 << 32) + 2), _lib.LLA_ERR_INVALID_ARG),
    (dict(out=(1 << 40) + 64), _lib.LLA_ERR_INVALID_ARG),  # out overlaps q
    (dict(state=(1 << 40) + (7 << 32) - 1024), _lib.LLA_ERR_INVALID_ARG),  # state overlaps log_scale
    (dict(t_seq=(1 << 44) + 4), _lib.LLA_ERR_INVALID_ARG),                  # misaligned positions
])
def test_decode_validation_codes(L, kw, code):
    assert L.loglinear_attn_decode_step(ctypes.byref(_dargs(**kw)), None) == code


def test_decode_levels_boundary(L):
    # t = 2^13 - 1 needs 14 levels: accepted up to the launch, which a zero-head batch skips
    assert L.loglinear_attn_decode_step(ctypes.byref(_dargs(B=0, t=(1 << 13) - 1, Lc=14)), None) == _lib.LLA_OK
    assert L.loglinear_attn_decode_step(None, None) == _lib.LLA_ERR_INVALID_ARG


def test_decode_binding_requires_device_tensors():
    import torch
    import log_linear_attention_chunked_amd as lla
    ensure_built()
    x = torch.zeros(1, 1, 16)
    with pytest.raises(ValueError):
        lla.decode_step(x, x, x, torch.zeros(1, 1), torch.zeros(1, 1, 4),
                        torch.zeros(1, 1, 4, 16, 16), torch.zeros(1, 1, 2, 4), 0)


# ---------------------------------------------------------------------------------------
# variable-length forward: host-side validation only
# ---------------------------------------------------------------------------------------

def _vargs(**kw):
    a = _lib.VarlenArgs()
    base = 1 << 40                 # fake, well-separated, aligned addresses: never dereferenced
    a.q, a.k, a.v = base, base + (1 << 32), base + (2 << 32)
    a.log_a, a.lam, a.out = base + (3 << 32), base + (4 << 32), base + (5 << 32)
    a.cu_seqlens = base + (6 << 32)
    a.N, a.H, a.total_T, a.max_T, a.dk, a.dv = 3, 2, 700, 400, 64, 64
    a.dtype, a.chunk, a.sweep = 0, 64, 1
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(N=-1), _lib.LLA_ERR_INVALID_ARG),
    (dict(max_T=701), _lib.LLA_ERR_INVALID_ARG),        # longer than the packed rows
    (dict(dtype=5), _lib.LLA_ERR_INVALID_ARG),
    (dict(dk=24), _lib.LLA_ERR_UNSUPPORTED),
    (dict(cu_seqlens=None), _lib.LLA_ERR_INVALID_ARG),
    (dict(cu_seqlens=(1 << 40) + (6 << 32) + 2), _lib.LLA_ERR_INVALID_ARG),
    (dict(q=None), _lib.LLA_ERR_INVALID_ARG),
    (dict(out=(1 << 40) + 1024), _lib.LLA_ERR_INVALID_ARG),   # out overlaps q
    (dict(workspace=(1 << 44), workspace_bytes=64), _lib.LLA_ERR_WORKSPACE),
])
def test_varlen_validation_codes(L, kw, code):
    assert L.loglinear_attn_fwd_varlen(ctypes.byref(_vargs(**kw)), None) == code


@pytest.mark.parametrize("kw", [dict(N=0), dict(H=0), dict(max_T=0, total_T=0)])
def test_varlen_empty_is_a_noop(L, kw):
    assert L.loglinear_attn_fwd_varlen(ctypes.byref(_vargs(**kw)), None) == _lib.LLA_OK
    assert L.loglinear_attn_fwd_varlen(None, None) == _lib.LLA_ERR_INVALID_ARG


def test_varlen_host_copy_of_empty_sequences_launches_nothing(L):
    # a host copy whose sequences are all empty: nothing to compute, so no kernel is launched
    # (the fake device addresses are never touched)
    host = (ctypes.c_int * 4)(0, 0, 0, 0)
    a = _vargs()
    a.cu_seqlens_host = ctypes.cast(host, ctypes.c_void_p).value
    assert L.loglinear_attn_fwd_varlen(ctypes.byref(a), None) == _lib.LLA_OK


# ---- backward pass -------------------------------------------------------------------------

def _bargs(**kw):
    a = _lib.BwdArgs()
    base = 1 << 40                 # fake, well-separated, aligned addresses: never dereferenced
    names = ("q", "k", "v", "log_a", "lam", "grad_out", "grad_q", "grad_k", "grad_v",
             "grad_log_a", "grad_lam")
    for i, n in enumerate(names):
        setattr(a, n, base + (i << 32))
    a.B, a.H, a.T, a.dk, a.dv = 1, 2, 4096, 64, 64
    a.dtype, a.chunk = 0, 64
    a.workspace, a.workspace_bytes = None, 0
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), _lib.LLA_ERR_INVALID_ARG),
    (dict(H=-1), _lib.LLA_ERR_INVALID_ARG),
    (dict(dk=24), _lib.LLA_ERR_UNSUPPORTED),
    (dict(chunk=128), _lib.LLA_ERR_UNSUPPORTED),
    (dict(chunk=8), _lib.LLA_ERR_UNSUPPORTED),
    (dict(B=300, H=300), _lib.LLA_ERR_UNSUPPORTED),
    (dict(T=1 << 24), _lib.LLA_ERR_UNSUPPORTED),                     # 25 levels
    (dict(dtype=1, dk=128, dv=128, chunk=64), _lib.LLA_ERR_UNSUPPORTED),  # shared memory
    (dict(grad_out=None), _lib.LLA_ERR_INVALID_ARG),
    (dict(grad_lam=None), _lib.LLA_ERR_INVALID_ARG),
    (dict(grad_q=(1 << 40) + (6 << 32) + 8), _lib.LLA_ERR_INVALID_ARG),        # misaligned
    (dict(grad_log_a=(1 << 40) + (9 << 32) + 2), _lib.LLA_ERR_INVALID_ARG),
    (dict(grad_v=(1 << 40) + 4096), _lib.LLA_ERR_INVALID_ARG),                  # overlaps q
    (dict(grad_k=(1 << 40) + (6 << 32) + 4096), _lib.LLA_ERR_INVALID_ARG),      # overlaps grad_q
    (dict(workspace=(1 << 44), workspace_bytes=1024), _lib.LLA_ERR_WORKSPACE),
    (dict(workspace=(1 << 44) + 16, workspace_bytes=1 << 34), _lib.LLA_ERR_INVALID_ARG),
])
def test_bwd_validation_codes(L, kw, code):
    assert L.loglinear_attn_bwd(ctypes.byref(_bargs(**kw)), None) == code


def test_bwd_null_struct_and_empty(L):
    assert L.loglinear_attn_bwd(None, None) == _lib.LLA_ERR_INVALID_ARG
    for kw in (dict(B=0), dict(T=0), dict(T=0, q=None)):
        assert L.loglinear_attn_bwd(ctypes.byref(_bargs(**kw)), None) == _lib.LLA_OK


def test_bwd_defaults_and_workspace(L):
    assert L.loglinear_attn_bwd_default_chunk(16, 16, 1) == 16
    assert L.loglinear_attn_bwd_default_chunk(64, 64, 0) == 64
    assert L.loglinear_attn_bwd_default_chunk(128, 128, 0) == 64
    assert L.loglinear_attn_bwd_default_chunk(128, 128, 1) == 32   # float32 images need less C
    assert L.loglinear_attn_bwd_default_chunk(48, 64, 0) == 0
    ws = L.loglinear_attn_bwd_workspace_bytes
    # headline shape: N = 128 chunks, 7 chunk levels, 128 + 64 + ... + 2 = 254 tree slots per head
    n = ws(4, 16, 8192, 64, 64, 64, 0)
    sz = 64 * 64 * 4
    # fp32 chunk states/nodes, block decays, target-side sub-block states (64 + 32 + 16 + 4 x 8
    # = 144 per head), bf16 copies of the nodes and of each chunk's combined state, dA (the
    # tree's per-level values stay on chip at this size)
    sz2 = 64 * 64 * 2
    # (the bf16 copies twice: high and low parts)
    expect = (64 * 254 * sz + 64 * 254 * 4 + 64 * 144 * sz + 2 * (64 * 254 * sz2 + 64 * 128 * sz2)
              + 64 * 8192 * 4)
    assert expect <= n <= expect + 9 * 256
    # one chunk: only the per-position dA
    assert ws(1, 2, 64, 64, 64, 64, 0) == 2 * 64 * 4
    assert ws(1, 2, 64, 48, 64, 64, 0) == 0


def _pargs(**kw):
    a = _lib.PrefillArgs()
    base = 1 << 40
    a.k, a.v, a.log_a = base, base + (1 << 32), base + (2 << 32)
    a.state, a.log_scale = base + (3 << 32), base + (4 << 32)
    a.B, a.H, a.T, a.dk, a.dv, a.Lc, a.dtype = 1, 2, 100, 64, 64, 8, 0
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(T=0), _lib.LLA_ERR_INVALID_ARG),
    (dict(Lc=0), _lib.LLA_ERR_INVALID_ARG),
    (dict(dtype=5), _lib.LLA_ERR_UNSUPPORTED),
    (dict(dk=48), _lib.LLA_ERR_UNSUPPORTED),
    (dict(Lc=26), _lib.LLA_ERR_UNSUPPORTED),
    (dict(T=128, Lc=8), _lib.LLA_ERR_INVALID_ARG),      # t = 128 needs bit_length(128) + 1 = 9 levels
    (dict(k=None), _lib.LLA_ERR_INVALID_ARG),
    (dict(v=(1 << 40) + (1 << 32) + 8), _lib.LLA_ERR_INVALID_ARG),       # misaligned
    (dict(state=(1 << 40) + 4096), _lib.LLA_ERR_INVALID_ARG),            # overlaps k
    (dict(B=0), _lib.LLA_OK),
])
def test_prefill_validation_codes(L, kw, code):
    assert L.loglinear_attn_decode_prefill(ctypes.byref(_pargs(**kw)), None) == code


# ---- the forward entry point that allocates nothing ------------------------------------------

def test_noalloc_scratch_limit_and_arguments(L):
    scratch = L.loglinear_attn_noalloc_scratch_bytes()
    assert scratch == 64 << 20
    # the headline shape fits the scratch; the long d = 128 workloads do not
    assert L.loglinear_attn_workspace_bytes(4, 16, 8192, 64, 64, 64, 2, 0) <= scratch
    assert L.loglinear_attn_workspace_bytes(1, 16, 32768, 128, 128, 64, 0, 0) > scratch
    big = _args(B=1, H=16, T=32768, dk=128, dv=128, chunk=64, sweep=0)
    assert L.loglinear_attn_fwd_noalloc(ctypes.byref(big), None) == _lib.LLA_ERR_SCRATCH_LIMIT
    assert _lib.status_string(_lib.LLA_ERR_SCRATCH_LIMIT) != "unknown status"
    # a workspace argument is refused (the scratch replaces it); validation as in fwd_ex
    ws = _args(workspace=(1 << 44), workspace_bytes=1 << 30)
    assert L.loglinear_attn_fwd_noalloc(ctypes.byref(ws), None) == _lib.LLA_ERR_INVALID_ARG
    assert L.loglinear_attn_fwd_noalloc(None, None) == _lib.LLA_ERR_INVALID_ARG
    assert L.loglinear_attn_fwd_noalloc(ctypes.byref(_args(dk=48)), None) == _lib.LLA_ERR_UNSUPPORTED
    assert L.loglinear_attn_fwd_noalloc(ctypes.byref(_args(q=None)), None) == _lib.LLA_ERR_INVALID_ARG
    assert L.loglinear_attn_fwd_noalloc(ctypes.byref(_args(B=0)), None) == _lib.LLA_OK


# ---- log-linear Gated DeltaNet ------------------------------------------------------------------

def _gargs(**kw):
    a = _lib.GdnArgs()
    base = 1 << 40                 # fake, well-separated, aligned addresses: never dereferenced
    for i, n in enumerate(("q", "k", "v", "log_a", "beta", "lam", "out")):
        setattr(a, n, base + (i << 32))
    a.B, a.H, a.T, a.dk, a.dv = 1, 2, 4096, 64, 64
    a.dtype, a.chunk = 0, 0
    a.workspace, a.workspace_bytes = None, 0
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), _lib.LLA_ERR_INVALID_ARG),
    (dict(T=-1), _lib.LLA_ERR_INVALID_ARG),
    (dict(dk=48), _lib.LLA_ERR_UNSUPPORTED),
    (dict(chunk=128), _lib.LLA_ERR_UNSUPPORTED),
    (dict(chunk=8), _lib.LLA_ERR_UNSUPPORTED),
    (dict(dk=128, dv=128, chunk=64), _lib.LLA_ERR_UNSUPPORTED),     # shared memory
    (dict(B=300, H=300), _lib.LLA_ERR_UNSUPPORTED),
    (dict(T=1 << 24), _lib.LLA_ERR_UNSUPPORTED),
    (dict(beta=None), _lib.LLA_ERR_INVALID_ARG),
    (dict(out=None), _lib.LLA_ERR_INVALID_ARG),
    (dict(beta=(1 << 40) + (4 << 32) + 2), _lib.LLA_ERR_INVALID_ARG),   # misaligned
    (dict(out=(1 << 40) + (4 << 32) + 64), _lib.LLA_ERR_INVALID_ARG),   # out overlaps beta
    (dict(lambda_bf16=2), _lib.LLA_ERR_INVALID_ARG),
    (dict(workspace=(1 << 44), workspace_bytes=1024), _lib.LLA_ERR_WORKSPACE),
    (dict(workspace=(1 << 44) + 16, workspace_bytes=1 << 36), _lib.LLA_ERR_INVALID_ARG),
])
def test_gdn_validation_codes(L, kw, code):
    assert L.loglinear_attn_gdn_fwd(ctypes.byref(_gargs(**kw)), None) == code


def test_gdn_defaults_workspace_and_noop(L, monkeypatch):
    assert L.loglinear_attn_gdn_fwd(None, None) == _lib.LLA_ERR_INVALID_ARG
    for kw in (dict(B=0), dict(T=0), dict(T=0, q=None)):
        assert L.loglinear_attn_gdn_fwd(ctypes.byref(_gargs(**kw)), None) == _lib.LLA_OK
    # chunk 32 wherever it fits (every supported head size)
    assert L.loglinear_attn_gdn_default_chunk(64, 64, 0) == 32
    assert L.loglinear_attn_gdn_default_chunk(128, 128, 0) == 32
    assert L.loglinear_attn_gdn_default_chunk(128, 64, 1) == 32
    assert L.loglinear_attn_gdn_default_chunk(16, 16, 1) == 32
    assert L.loglinear_attn_gdn_default_chunk(48, 64, 0) == 0
    ws = L.loglinear_attn_gdn_workspace_bytes
    # B=4, H=16, T=8192, d=64, chunk 64: outputs and query rows in fp32; 128 chunks, whose
    # indices have bits 0..6, so tree levels 0..6: 128 + 64 + ... + 2 = 254 slots of a 64 x 64
    # state and a 64 x 64 transition per head
    n = ws(4, 16, 8192, 64, 64, 64, 0)
    expect = 64 * 8192 * (64 + 64) * 4 + 64 * 254 * (64 * 64 * 2) * 4
    assert expect <= n <= expect + 4 * 256
    # the default chunk 32: 256 chunks, levels 0..7, 256 + 128 + ... + 2 = 510 slots
    n = ws(4, 16, 8192, 64, 64, 0, 0)
    expect = 64 * 8192 * (64 + 64) * 4 + 64 * 510 * (64 * 64 * 2) * 4
    assert expect <= n <= expect + 4 * 256
    assert ws(1, 1, 64, 64, 64, 64, 0) > 0          # one chunk: a leaf, no levels above it
    assert ws(1, 1, 64, 64, 64, 128, 0) == 0         # unsupported -> 0
    monkeypatch.setenv("LLA_TEST_FAIL_ALLOC", "1")
    assert L.loglinear_attn_gdn_fwd(ctypes.byref(_gargs()), None) == _lib.LLA_ERR_NO_MEMORY
