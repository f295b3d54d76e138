"""ctypes binding of ``libloglinear_attn.so`` (argument marshalling only).

Every function here forwards to the C ABI declared in ``include/loglinear_attn.h``;
the computation happens in the library's HIP kernels. If the library has not been
built the first call raises ``LibraryNotBuilt``: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libloglinear_attn.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

LLA_OK = 0
LLA_ERR_INVALID_ARG = -1
LLA_ERR_UNSUPPORTED = -2
LLA_ERR_HIP = -3
LLA_ERR_NO_MEMORY = -4
LLA_ERR_WORKSPACE = -5
LLA_ERR_SCRATCH_LIMIT = -6

LLA_DTYPE_BF16 = 0
LLA_DTYPE_F32 = 1

# every exported symbol of include/loglinear_attn.h
EXPORTS = (
    "loglinear_attn_fwd",
    "loglinear_attn_fwd_f32",
    "loglinear_attn_fwd_ex",
    "loglinear_attn_workspace_bytes",
    "loglinear_attn_num_levels",
    "loglinear_attn_default_chunk",
    "loglinear_attn_default_sweep",
    "loglinear_attn_status_string",
    "loglinear_attn_decode_step",
    "loglinear_attn_fwd_varlen",
    "loglinear_attn_bwd",
    "loglinear_attn_bwd_workspace_bytes",
    "loglinear_attn_bwd_default_chunk",
    "loglinear_attn_decode_prefill",
    "loglinear_attn_fwd_noalloc",
    "loglinear_attn_noalloc_scratch_bytes",
    "loglinear_attn_gdn_fwd",
    "loglinear_attn_gdn_workspace_bytes",
    "loglinear_attn_gdn_default_chunk",
)


class LibraryNotBuilt(RuntimeError):
    pass


class FwdArgs(ctypes.Structure):
    """Mirror of ``lla_fwd_args``."""
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("log_a", ctypes.c_void_p),
        ("lam", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("B", ctypes.c_int),
        ("H", ctypes.c_int),
        ("T", ctypes.c_int),
        ("dk", ctypes.c_int),
        ("dv", ctypes.c_int),
        ("dtype", ctypes.c_int),
        ("chunk", ctypes.c_int),
        ("sweep", ctypes.c_int),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stage_events", ctypes.c_void_p * 4),
        ("lambda_bf16", ctypes.c_int),
    ]


class VarlenArgs(ctypes.Structure):
    """Mirror of ``lla_fwd_varlen_args``."""
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("log_a", ctypes.c_void_p),
        ("lam", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("cu_seqlens", ctypes.c_void_p),
        ("cu_seqlens_host", ctypes.c_void_p),
        ("N", ctypes.c_int),
        ("H", ctypes.c_int),
        ("total_T", ctypes.c_int),
        ("max_T", ctypes.c_int),
        ("dk", ctypes.c_int),
        ("dv", ctypes.c_int),
        ("dtype", ctypes.c_int),
        ("chunk", ctypes.c_int),
        ("sweep", ctypes.c_int),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("lambda_bf16", ctypes.c_int),
    ]


class DecodeArgs(ctypes.Structure):
    """Mirror of ``lla_decode_args``."""
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("log_a", ctypes.c_void_p),
        ("lam", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("state", ctypes.c_void_p),
        ("log_scale", ctypes.c_void_p),
        ("B", ctypes.c_int),
        ("H", ctypes.c_int),
        ("dk", ctypes.c_int),
        ("dv", ctypes.c_int),
        ("Lc", ctypes.c_int),
        ("dtype", ctypes.c_int),
        ("t", ctypes.c_longlong),
        ("t_seq", ctypes.c_void_p),
    ]


class BwdArgs(ctypes.Structure):
    """Mirror of ``lla_bwd_args``."""
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("log_a", ctypes.c_void_p),
        ("lam", ctypes.c_void_p),
        ("grad_out", ctypes.c_void_p),
        ("grad_q", ctypes.c_void_p),
        ("grad_k", ctypes.c_void_p),
        ("grad_v", ctypes.c_void_p),
        ("grad_log_a", ctypes.c_void_p),
        ("grad_lam", ctypes.c_void_p),
        ("B", ctypes.c_int),
        ("H", ctypes.c_int),
        ("T", ctypes.c_int),
        ("dk", ctypes.c_int),
        ("dv", ctypes.c_int),
        ("dtype", ctypes.c_int),
        ("chunk", ctypes.c_int),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stage_events", ctypes.c_void_p * 4),
        ("lambda_bf16", ctypes.c_int),
    ]


class PrefillArgs(ctypes.Structure):
    """Mirror of ``lla_prefill_args``."""
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("log_a", ctypes.c_void_p),
        ("state", ctypes.c_void_p),
        ("log_scale", ctypes.c_void_p),
        ("B", ctypes.c_int),
        ("H", ctypes.c_int),
        ("T", ctypes.c_int),
        ("dk", ctypes.c_int),
        ("dv", ctypes.c_int),
        ("Lc", ctypes.c_int),
        ("dtype", ctypes.c_int),
    ]


class GdnArgs(ctypes.Structure):
    """Mirror of ``lla_gdn_args``."""
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("log_a", ctypes.c_void_p),
        ("beta", ctypes.c_void_p),
        ("lam", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("B", ctypes.c_int),
        ("H", ctypes.c_int),
        ("T", ctypes.c_int),
        ("dk", ctypes.c_int),
        ("dv", ctypes.c_int),
        ("dtype", ctypes.c_int),
        ("chunk", ctypes.c_int),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stage_events", ctypes.c_void_p * 4),
        ("lambda_bf16", ctypes.c_int),
    ]


_lock = threading.Lock()
_lib = None


def _declare(lib):
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.loglinear_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.loglinear_attn_fwd.restype = i
    lib.loglinear_attn_fwd_f32.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.loglinear_attn_fwd_f32.restype = i
    lib.loglinear_attn_fwd_ex.argtypes = [ctypes.POINTER(FwdArgs), vp]
    lib.loglinear_attn_fwd_ex.restype = i
    lib.loglinear_attn_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i]
    lib.loglinear_attn_workspace_bytes.restype = sz
    lib.loglinear_attn_num_levels.argtypes = [i]
    lib.loglinear_attn_num_levels.restype = i
    lib.loglinear_attn_default_chunk.argtypes = [i, i, i, i]
    lib.loglinear_attn_default_chunk.restype = i
    lib.loglinear_attn_default_sweep.argtypes = [i, i, i, i, i, i, i]
    lib.loglinear_attn_default_sweep.restype = i
    lib.loglinear_attn_status_string.argtypes = [i]
    lib.loglinear_attn_status_string.restype = ctypes.c_char_p
    lib.loglinear_attn_decode_step.argtypes = [ctypes.POINTER(DecodeArgs), vp]
    lib.loglinear_attn_decode_step.restype = i
    lib.loglinear_attn_fwd_varlen.argtypes = [ctypes.POINTER(VarlenArgs), vp]
    lib.loglinear_attn_fwd_varlen.restype = i
    lib.loglinear_attn_bwd.argtypes = [ctypes.POINTER(BwdArgs), vp]
    lib.loglinear_attn_bwd.restype = i
    lib.loglinear_attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.loglinear_attn_bwd_workspace_bytes.restype = sz
    lib.loglinear_attn_bwd_default_chunk.argtypes = [i, i, i]
    lib.loglinear_attn_bwd_default_chunk.restype = i
    lib.loglinear_attn_decode_prefill.argtypes = [ctypes.POINTER(PrefillArgs), vp]
    lib.loglinear_attn_decode_prefill.restype = i
    lib.loglinear_attn_fwd_noalloc.argtypes = [ctypes.POINTER(FwdArgs), vp]
    lib.loglinear_attn_fwd_noalloc.restype = i
    lib.loglinear_attn_noalloc_scratch_bytes.argtypes = []
    lib.loglinear_attn_noalloc_scratch_bytes.restype = sz
    lib.loglinear_attn_gdn_fwd.argtypes = [ctypes.POINTER(GdnArgs), vp]
    lib.loglinear_attn_gdn_fwd.restype = i
    lib.loglinear_attn_gdn_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.loglinear_attn_gdn_workspace_bytes.restype = sz
    lib.loglinear_attn_gdn_default_chunk.argtypes = [i, i, i]
    lib.loglinear_attn_gdn_default_chunk.restype = i


def lib():
    """The loaded library (loaded once). Raises ``LibraryNotBuilt`` if absent."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                try:
                    # load torch's HIP runtime first so the library binds to the same one
                    # (one runtime per process: shared streams, events and allocations)
                    import torch  # noqa: F401
                except ImportError:
                    pass
                if not os.path.exists(LIB_PATH):
                    raise LibraryNotBuilt(
                        f"{LIB_PATH} is missing: build it with "
                        "`python -m log_linear_attention_chunked_amd.build` (hipcc, gfx950)")
                handle = ctypes.CDLL(LIB_PATH)
                _declare(handle)
                _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().loglinear_attn_status_string(int(status)).decode()
