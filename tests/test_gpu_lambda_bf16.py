"""bfloat16 level weights (lambda_bf16 = 1) through the C ABI.

lambda is rounded to bfloat16 once (round to nearest even); the oracle reads those bf16 values
exactly, so the bar is the usual one for the inputs' dtype. The library widens bf16 to float32
exactly, so the output (and every gradient) must also be bitwise the output of the float32 path
on a float32 lambda holding the same rounded values.
"""

import numpy as np
import pytest

import oracle.loglinear as O
from lla_synth import WORKLOADS, custom, generate, grad_output
from tests._util import ensure_built, rel_l2, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    import torch
    ensure_built()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bf16_lambda(x):
    import torch
    y = dict(x)
    y["lam"] = x["lam"].to(torch.bfloat16).contiguous()
    return y


SHAPES = [
    # B, H, T, dk, dv, dtype, chunk, sweep, mode
    (1, 2, 256, 16, 16, "f32", 16, 1, None),
    (2, 3, 999, 64, 64, "bf16", 64, 2, "lowdecay"),    # T*L odd: rows of later heads 2-byte aligned only
    (1, 2, 333, 64, 32, "bf16", 64, 1, None),
    (1, 2, 2048, 128, 128, "bf16", 128, 1, "nodecay"),
    (1, 1, 4160, 64, 64, "bf16", 64, 2, "lowdecay"),
    (1, 2, 1000, 32, 32, "f32", 32, 2, "strongdecay"),
]


@pytest.mark.parametrize("B,H,T,dk,dv,dtype,chunk,sweep,mode", SHAPES)
def test_forward_bf16_lambda(B, H, T, dk, dv, dtype, chunk, sweep, mode):
    import torch
    import log_linear_attention_chunked_amd as lla
    x = _bf16_lambda(generate(custom(B, H, T, dk, dv, dtype=dtype), seed=T + 3, log_a_mode=mode))
    d = {k: v.cuda() for k, v in x.items()}
    got = lla.forward(d["q"], d["k"], d["v"], d["log_a"], d["lam"], chunk=chunk, sweep=sweep)
    ref32 = lla.forward(d["q"], d["k"], d["v"], d["log_a"], d["lam"].float().contiguous(), chunk=chunk,
                        sweep=sweep)
    torch.cuda.synchronize()
    assert torch.equal(got, ref32), "bf16 lambda differs from float32 lambda of the same values"
    want = O.bruteforce(x["q"], x["k"], x["v"], x["log_a"], x["lam"])
    err = rel_l2(got.double().cpu().numpy(), want)
    print(f"bf16 lambda {B, H, T, dk, dv, dtype, chunk, sweep, mode}: rel_l2={err:.3e}", flush=True)
    assert err <= tol_for(dtype)


def test_forward_bf16_lambda_headline_sampled():
    # the headline shape with bf16 lambda: every head's sampled rows, and the float32 path bitwise
    import torch
    import log_linear_attention_chunked_amd as lla
    from tests._util import per_head
    from tests.test_gpu_fullsize import sample_rows
    w = WORKLOADS["b4h16_t8192_d64_bf16"]
    x = _bf16_lambda(generate(w, seed=0))
    d = {k: v.cuda() for k, v in x.items()}
    got = lla.forward(d["q"], d["k"], d["v"], d["log_a"], d["lam"], chunk=w.chunk)
    ref32 = lla.forward(d["q"], d["k"], d["v"], d["log_a"], d["lam"].float().contiguous(), chunk=w.chunk)
    torch.cuda.synchronize()
    assert torch.equal(got, ref32)
    got = got.double().cpu().numpy()
    rows = sample_rows(w.T, w.chunk, n_uniform=64)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    wants = per_head(lambda b, h: O.bruteforce_rows(x["q"], x["k"], x["v"], x["log_a"], x["lam"], b, h, rows),
                     heads)
    worst = max(rel_l2(got[b, h, rows], wt) for (b, h), wt in zip(heads, wants))
    print(f"bf16 lambda headline: worst head rel_l2={worst:.3e}", flush=True)
    assert worst <= tol_for(w.dtype)


def test_varlen_bf16_lambda():
    import torch
    import log_linear_attention_chunked_amd as lla
    lens = [700, 64, 1500, 33]
    H, d = 2, 64
    total, mx = sum(lens), max(lens)
    L = lla.num_levels(mx)
    x = generate(custom(1, H, total, d, d, dtype="bf16"), seed=5, log_a_mode="lowdecay")
    q, k, v = (x[n][0].cuda() for n in ("q", "k", "v"))
    log_a = x["log_a"][0].cuda()
    lam32 = x["lam"][0, :, :, :L].to(torch.bfloat16).float().contiguous().cuda()
    lam16 = lam32.to(torch.bfloat16).contiguous()
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    a = lla.forward_varlen(q, k, v, log_a, lam16, cu.cuda(), mx, chunk=64, sweep=2, cu_seqlens_host=cu)
    b = lla.forward_varlen(q, k, v, log_a, lam32, cu.cuda(), mx, chunk=64, sweep=2, cu_seqlens_host=cu)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("B,H,T,dk,dv,dtype,chunk", [(1, 2, 300, 64, 64, "bf16", 64),
                                                     (1, 2, 517, 32, 16, "f32", 32),
                                                     (1, 1, 2048, 64, 64, "bf16", 0)])
def test_backward_bf16_lambda(B, H, T, dk, dv, dtype, chunk):
    import torch
    import log_linear_attention_chunked_amd as lla
    w = custom(B, H, T, dk, dv, dtype)
    x = _bf16_lambda(generate(w, seed=T, log_a_mode="lowdecay"))
    do = grad_output(w, seed=T)
    d = {k: v.cuda() for k, v in x.items()}
    g16 = lla.backward(d["q"], d["k"], d["v"], d["log_a"], d["lam"], do.cuda(), chunk=chunk)
    g32 = lla.backward(d["q"], d["k"], d["v"], d["log_a"], d["lam"].float().contiguous(), do.cuda(), chunk=chunk)
    torch.cuda.synchronize()
    for a, b in zip(g16, g32):
        assert torch.equal(a, b)
    assert g16[4].dtype == torch.float32
    want = O.bruteforce_grad(**x, do=do)
    for n, t in zip(("dq", "dk", "dv", "dlog_a", "dlam"), g16):
        err = rel_l2(t.double().cpu().numpy(), want[n])
        assert err <= tol_for(dtype), (n, err)
