"""GPU parity of the variable-length forward: N sequences packed along time, each compared
with the fp64 oracle run on that sequence alone (its positions start at 0).

Bars (relative L2 per sequence): 1e-4 for float32 inputs, 2e-2 for bfloat16 inputs.
"""

import numpy as np
import pytest

import oracle.loglinear as O
from lla_synth import custom, generate
from tests._util import ensure_built, rel_l2, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    import torch
    ensure_built()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def packed_inputs(lengths, H, dk, dv, dtype, seed):
    """[H, total_T, .] tensors (CPU) for the given lengths, lambda with num_levels(max) levels."""
    total = sum(lengths)
    x = generate(custom(1, H, max(total, 1), dk, dv, dtype=dtype), seed=seed)
    Lmax = O.num_levels(max(max(lengths), 1))
    return {"q": x["q"][0, :, :total], "k": x["k"][0, :, :total], "v": x["v"][0, :, :total],
            "log_a": x["log_a"][0, :, :total], "lam": x["lam"][0, :, :total, :Lmax]}


def run_varlen(xp, lengths, **kw):
    import torch
    import log_linear_attention_chunked_amd as lla
    d = {k: v.contiguous().cuda() for k, v in xp.items()}
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device="cuda")
    out = torch.zeros_like(d["v"])
    lla.forward_varlen(d["q"], d["k"], d["v"], d["log_a"], d["lam"], cu, max(lengths), out, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


CASES = [
    # lengths, H, dk, dv, dtype, chunk, sweep
    ([100, 1, 257], 2, 64, 64, "bf16", 64, 2),
    ([0, 300, 0, 64], 2, 64, 32, "f32", 64, 2),
    ([640, 130, 999], 1, 64, 64, "bf16", 64, 2),     # several sweeps per sequence, ragged ends
    ([16, 48, 33], 2, 16, 16, "f32", 16, 1),
    ([500, 260], 1, 128, 64, "bf16", 64, 1),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "L{}_h{}_dk{}_dv{}_{}_c{}r{}".format(
    "-".join(map(str, c[0])), *c[1:]))
def test_varlen_matches_oracle_per_sequence(case):
    lengths, H, dk, dv, dtype, chunk, sweep = case
    xp = packed_inputs(lengths, H, dk, dv, dtype, seed=sum(lengths))
    got = run_varlen(xp, lengths, chunk=chunk, sweep=sweep)
    assert np.all(np.isfinite(got))
    s0 = 0
    for n, Tn in enumerate(lengths):
        if Tn:
            sl = slice(s0, s0 + Tn)
            Ln = O.num_levels(Tn)
            want = O.bruteforce(xp["q"][None, :, sl], xp["k"][None, :, sl], xp["v"][None, :, sl],
                                xp["log_a"][None, :, sl], xp["lam"][None, :, sl, :Ln])[0]
            err = rel_l2(got[:, sl], want)
            print(f"varlen {case} sequence {n} (T={Tn}): rel_l2={err:.3e}", flush=True)
            assert err <= tol_for(dtype), (n, err)
        s0 += Tn


def test_varlen_equal_lengths_is_the_batched_forward():
    # B sequences of one length packed along time give exactly the [B, H, T] forward's outputs
    import torch
    import log_linear_attention_chunked_amd as lla
    B, H, T, d = 3, 2, 512, 64
    x = generate(custom(B, H, T, d, d, dtype="bf16"), seed=5)
    dev = {k: v.cuda() for k, v in x.items()}
    ref = lla.forward(dev["q"], dev["k"], dev["v"], dev["log_a"], dev["lam"], chunk=64, sweep=2)
    pack = {k: v.transpose(0, 1).reshape((H, B * T) + tuple(v.shape[3:])).contiguous()
            for k, v in dev.items()}
    cu = torch.arange(0, (B + 1) * T, T, dtype=torch.int32, device="cuda")
    got = lla.forward_varlen(pack["q"], pack["k"], pack["v"], pack["log_a"], pack["lam"], cu, T,
                             chunk=64, sweep=2)
    torch.cuda.synchronize()
    assert torch.equal(got.reshape(H, B, T, d).transpose(0, 1), ref)


def test_varlen_reuses_a_caller_workspace():
    import torch
    import log_linear_attention_chunked_amd as lla
    lengths, H, d = [200, 330, 70], 2, 64
    xp = packed_inputs(lengths, H, d, d, "bf16", seed=8)
    nws = lla.workspace_bytes(len(lengths), H, max(lengths), d, d, 64, 2, "bf16")
    ws = torch.zeros(nws, dtype=torch.uint8, device="cuda")
    a = run_varlen(xp, lengths, chunk=64, sweep=2, workspace=ws)
    b = run_varlen(xp, lengths, chunk=64, sweep=2, workspace=ws)
    assert np.array_equal(a, b)
