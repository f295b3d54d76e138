"""The forward entry point that allocates nothing (loglinear_attn_fwd_noalloc), through the C ABI,
against the entry point it is a variant of (loglinear_attn_fwd_ex with a caller workspace):
bitwise the same output, on two calls in a row, the second with a smaller input, and on a
repeat of the first after it; the smaller one also against the oracle. (The scratch limit is a
host-side check, tested without a device in tests/test_abi.py.)
"""

import ctypes

import numpy as np
import pytest

import oracle.loglinear as O
from lla_synth import WORKLOADS, custom, generate
from tests._util import ensure_built, rel_l2, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    import torch
    ensure_built()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _call_noalloc(d, out, chunk, sweep):
    """loglinear_attn_fwd_noalloc straight through ctypes; returns the status."""
    import torch
    import log_linear_attention_chunked_amd as lla
    from log_linear_attention_chunked_amd import _lib
    a = lla.make_args(d["q"], d["k"], d["v"], d["log_a"], d["lam"], out, chunk=chunk, sweep=sweep)
    return _lib.lib().loglinear_attn_fwd_noalloc(
        ctypes.byref(a), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _reference(d, chunk, sweep):
    import torch
    import log_linear_attention_chunked_amd as lla
    B, H, T, dk = d["q"].shape
    dv = d["v"].shape[-1]
    dt = "bf16" if d["q"].dtype == torch.bfloat16 else "f32"
    n = lla.workspace_bytes(B, H, T, dk, dv, chunk, sweep, dt)
    ws = torch.zeros(max(n, 1), dtype=torch.uint8, device="cuda")
    return lla.forward(d["q"], d["k"], d["v"], d["log_a"], d["lam"], chunk=chunk, sweep=sweep,
                       workspace=ws if n else None)


def test_noalloc_matches_fwd_ex_two_calls_second_smaller():
    import torch
    import log_linear_attention_chunked_amd as lla
    from log_linear_attention_chunked_amd import _lib
    big = WORKLOADS["b4h16_t8192_d64_bf16"]            # 31.6 MiB of workspace: within the scratch
    small = custom(1, 3, 3000, 64, 32, dtype="bf16")     # ragged, dk != dv
    assert lla.workspace_bytes(big.B, big.H, big.T, big.dk, big.dv, 64, 2, "bf16") <= lla.noalloc_scratch_bytes()
    cases = [(big, generate(big, seed=40), 64, 2), (small, generate(small, seed=41, log_a_mode="lowdecay"), 64, 2),
             (big, generate(big, seed=42, log_a_mode="nodecay"), 64, 2)]
    for w, x, chunk, sweep in cases:
        print(f"[noalloc] {w.name} chunk={chunk} sweep={sweep}", flush=True)
        d = {k: v.cuda() for k, v in x.items()}
        out = torch.full_like(d["v"], float("nan"))
        st = _call_noalloc(d, out, chunk, sweep)
        assert st == _lib.LLA_OK, _lib.status_string(st)
        ref = _reference(d, chunk, sweep)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"noalloc differs from fwd_ex on {w.name}"
        if w is small:
            want = O.bruteforce(x["q"], x["k"], x["v"], x["log_a"], x["lam"])
            err = rel_l2(out.double().cpu().numpy(), want)
            print(f"[noalloc] {w.name}: rel_l2 vs oracle {err:.3e}", flush=True)
            assert err <= tol_for("bf16")


def test_noalloc_f32_and_one_sweep_shapes():
    import torch
    from log_linear_attention_chunked_amd import _lib
    for (B, H, T, dk, dv, chunk, sweep) in [(1, 2, 256, 16, 16, 16, 1), (2, 2, 40, 32, 32, 64, 1)]:
        x = generate(custom(B, H, T, dk, dv, dtype="f32"), seed=T)
        d = {k: v.cuda() for k, v in x.items()}
        out = torch.empty_like(d["v"])
        assert _call_noalloc(d, out, chunk, sweep) == _lib.LLA_OK
        ref = _reference(d, chunk, sweep)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
