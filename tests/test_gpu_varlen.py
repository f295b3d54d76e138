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


def run_varlen(xp, lengths, host=False, host_values=None, fill=0.0, **kw):
    """Packed forward; host=True also hands the library a host copy of cu_seqlens (host_values,
    if given, replaces that copy)."""
    import torch
    import log_linear_attention_chunked_amd as lla
    d = {k: v.contiguous().cuda() for k, v in xp.items()}
    cu_np = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    cu = torch.tensor(cu_np, device="cuda")
    out = torch.full_like(d["v"], fill)
    if host:
        kw["cu_seqlens_host"] = list(cu_np) if host_values is None else host_values
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


@pytest.mark.parametrize("host", [False, True], ids=["device_bounds", "host_copy"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "L{}_h{}_dk{}_dv{}_{}_c{}r{}".format(
    "-".join(map(str, c[0])), *c[1:]))
def test_varlen_matches_oracle_per_sequence(case, host):
    lengths, H, dk, dv, dtype, chunk, sweep = case
    xp = packed_inputs(lengths, H, dk, dv, dtype, seed=sum(lengths))
    got = run_varlen(xp, lengths, host=host, chunk=chunk, sweep=sweep)
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


def test_varlen_many_sequences_host_copy_changes_nothing():
    # more sequences than a wave has lanes, empty ones among them: the grid sized from a host
    # copy and the upper-bound grid give identical outputs; a sample is checked on the oracle
    rng = np.random.default_rng(21)
    lengths = [int(x) for x in rng.choice([0, 1, 63, 64, 65, 129, 200, 300, 511], size=150)]
    H = 2
    xp = packed_inputs(lengths, H, 64, 64, "bf16", seed=21)
    a = run_varlen(xp, lengths, host=False, chunk=64, sweep=2)
    b = run_varlen(xp, lengths, host=True, chunk=64, sweep=2)
    assert np.array_equal(a, b)
    starts = np.concatenate([[0], np.cumsum(lengths)])
    for n in (0, 63, 64, 100, 149):
        Tn = lengths[n]
        if Tn:
            sl = slice(starts[n], starts[n] + Tn)
            want = O.bruteforce(xp["q"][None, :, sl], xp["k"][None, :, sl], xp["v"][None, :, sl],
                                xp["log_a"][None, :, sl], xp["lam"][None, :, sl, :O.num_levels(Tn)])[0]
            assert rel_l2(b[:, sl], want) <= tol_for("bf16"), n


def test_varlen_host_copy_that_disagrees_writes_nothing():
    # a host copy that does not match the device array: every workgroup leaves before taking a
    # ticket, the outputs keep their contents, and the workspace still serves later calls
    import torch
    import log_linear_attention_chunked_amd as lla
    lengths, H, d = [300, 40, 257], 2, 64
    xp = packed_inputs(lengths, H, d, d, "bf16", seed=4)
    nws = lla.workspace_bytes(len(lengths), H, max(lengths), d, d, 64, 2, "bf16")
    ws = torch.zeros(nws, dtype=torch.uint8, device="cuda")
    wrong = [0, 300, 340, 341]                       # one sweep fewer than the device array
    got = run_varlen(xp, lengths, host=True, host_values=wrong, fill=7.0, chunk=64, sweep=2,
                     workspace=ws)
    assert np.all(got == 7.0)
    good = run_varlen(xp, lengths, host=True, chunk=64, sweep=2, workspace=ws)
    ref = run_varlen(xp, lengths, host=False, chunk=64, sweep=2)
    assert np.array_equal(good, ref)
