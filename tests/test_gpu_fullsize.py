"""GPU parity at full size, in the launch configurations the library and the benchmark use.

* b2h8_t2048_d64_bf16 and b4h16_t8192_d64_bf16: every element of every head against the O(T^2)
  fp64 definition (``oracle.bruteforce``, one head per call, heads spread over the host cores).
* b1h16_t32768_d128_bf16_knorm and b1h8_t65536_d128_bf16_coarse: every head, on sampled rows
  (the first two chunks, the last chunk, positions around every power of two, 256 uniform
  rows), as stated and with no decay (so that the coarse Fenwick levels carry weight).
* The benchmark's own path at the headline shape: one caller workspace zero-filled once, then
  back-to-back calls on different inputs (one with no decay) with nothing cleared in between,
  so every call after the first runs on the epoch hand-over of the one before; every head's
  sampled rows against the oracle, every output finite, and later calls on repeated inputs
  bitwise equal to the first.

Bars: relative L2 over the compared outputs, 2e-2 for bfloat16 inputs with float32
accumulation; the worst head is printed.
"""

import numpy as np
import pytest

import oracle.loglinear as O
from lla_synth import WORKLOADS, generate
from tests._util import ensure_built, per_head, rel_l2, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    import torch
    ensure_built()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def sample_rows(T, C, seed=1, n_uniform=256):
    """First two chunks, last chunk, t in {2^k - 1, 2^k, 2^k + 1}, chunk edges mC - 1 and mC for
    a few m, and n_uniform uniform rows."""
    rows = set(range(min(T, 2 * C))) | set(range(max(0, T - C), T))
    k = 1
    while k < T:
        rows |= {k - 1, k, k + 1}
        k <<= 1
    for m in (3, 5, 7, 9, 17, 33):
        rows |= {m * C - 1, m * C}
    rng = np.random.default_rng(seed)
    rows |= set(int(r) for r in rng.integers(0, T, n_uniform))
    return sorted(r for r in rows if 0 <= r < T)


def heads_of(w):
    return [(b, h) for b in range(w.B) for h in range(w.H)]


def run_default(x, **kw):
    """Forward pass through the library with its default chunk and sweep (or kw); float64."""
    import torch
    import log_linear_attention_chunked_amd as lla
    d = {k: v.cuda() for k, v in x.items()}
    out = lla.forward(d["q"], d["k"], d["v"], d["log_a"], d["lam"], **kw)
    torch.cuda.synchronize()
    return out.double().cpu().numpy()


def compare_every_element(w, x, got):
    def one(b, h):
        sl = slice(h, h + 1)
        want = O.bruteforce(x["q"][b:b + 1, sl], x["k"][b:b + 1, sl], x["v"][b:b + 1, sl],
                            x["log_a"][b:b + 1, sl], x["lam"][b:b + 1, sl])[0, 0]
        return want
    wants = per_head(one, heads_of(w))
    want = np.stack(wants).reshape(got.shape)
    per = [rel_l2(got[b, h], want[b, h]) for (b, h) in heads_of(w)]
    err = rel_l2(got, want)
    print(f"{w.name}: every element rel_l2={err:.3e}, worst head {max(per):.3e}", flush=True)
    assert np.all(np.isfinite(got))
    assert err <= tol_for(w.dtype) and max(per) <= tol_for(w.dtype), (err, max(per))


@pytest.mark.parametrize("variant", ["as_stated", "nodecay"])
def test_small_bf16_workload_every_element(variant):
    w = WORKLOADS["b2h8_t2048_d64_bf16"]
    x = generate(w, seed=0, **({} if variant == "as_stated" else dict(log_a_mode="nodecay")))
    got = run_default(x, chunk=w.chunk)
    compare_every_element(w, x, got)


def test_headline_workload_every_element():
    w = WORKLOADS["b4h16_t8192_d64_bf16"]
    x = generate(w, seed=0)
    print(f"[fullsize] {w.name}: GPU, then the oracle on all {w.B * w.H} heads", flush=True)
    got = run_default(x, chunk=w.chunk)
    compare_every_element(w, x, got)


def compare_sampled(w, x, got, rows, label):
    def one(b, h):
        return O.bruteforce_rows(x["q"], x["k"], x["v"], x["log_a"], x["lam"], b, h, rows)
    wants = per_head(one, heads_of(w))
    errs = [rel_l2(got[b, h, rows], want) for (b, h), want in zip(heads_of(w), wants)]
    tot = rel_l2(np.stack([got[b, h, rows] for (b, h) in heads_of(w)]), np.stack(wants))
    print(f"{label}: {len(rows)} rows x {len(errs)} heads, rel_l2={tot:.3e}, "
          f"worst head {max(errs):.3e}", flush=True)
    assert np.all(np.isfinite(got)), label
    assert max(errs) <= tol_for(w.dtype), (label, max(errs))
    return errs


@pytest.mark.parametrize("name", ["b1h16_t32768_d128_bf16_knorm", "b1h8_t65536_d128_bf16_coarse"])
@pytest.mark.parametrize("variant", ["as_stated", "nodecay"])
def test_long_workloads_every_head_sampled(name, variant):
    w = WORKLOADS[name]
    x = generate(w, seed=0, **({} if variant == "as_stated" else dict(log_a_mode="nodecay")))
    print(f"[fullsize] {name} {variant}", flush=True)
    got = run_default(x, chunk=w.chunk)
    compare_sampled(w, x, got, sample_rows(w.T, w.chunk), f"{name} {variant}")


def test_benchmark_path_epoch_reuse_headline():
    """The headline shape exactly as bench.py launches it: the workload's chunk, the library's
    sweep, one caller workspace zero-filled once; then three calls on different inputs (the
    second with no decay, the third with strong decay) back to back on one stream, then 20 more
    calls on the first input, nothing cleared or synchronised in between."""
    import torch
    import log_linear_attention_chunked_amd as lla
    w = WORKLOADS["b4h16_t8192_d64_bf16"]
    chunk = w.chunk
    sweep = lla.default_sweep(w.B, w.H, w.T, w.dk, w.dv, chunk, w.dtype)
    n = lla.workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, chunk, sweep, w.dtype)
    assert n > 0
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    modes = [None, "nodecay", "strongdecay"]
    xs = [generate(w, seed=10 + i, log_a_mode=m) for i, m in enumerate(modes)]
    ds = [{k: v.cuda() for k, v in x.items()} for x in xs]
    print(f"[fullsize] bench path chunk={chunk} sweep={sweep} workspace={n} bytes", flush=True)
    outs = [lla.forward(d["q"], d["k"], d["v"], d["log_a"], d["lam"], chunk=chunk, sweep=sweep,
                        workspace=ws) for d in ds]
    again = torch.empty_like(outs[0])
    d0 = ds[0]
    for _ in range(20):
        lla.forward(d0["q"], d0["k"], d0["v"], d0["log_a"], d0["lam"], again, chunk=chunk,
                    sweep=sweep, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(again, outs[0]), "repeated call on a reused workspace differs"
    rows = sample_rows(w.T, chunk)
    for x, o, m in zip(xs, outs, modes):
        got = o.double().cpu().numpy()
        compare_sampled(w, x, got, rows, f"bench path, log_a {m or 'as stated'}")


def test_unzeroed_workspace_counter_gives_nan_not_stale_output():
    """A caller workspace whose ticket counter holds a count at or past the number of sweeps (a
    workspace that was never zero-filled): the call still returns LLA_OK, and every output row
    is written as NaN rather than left holding what the buffer held before."""
    import torch
    import log_linear_attention_chunked_amd as lla
    B, H, T, d = 1, 3, 3000, 64
    from lla_synth import custom
    x = generate(custom(B, H, T, d, d), seed=5)
    dd = {k: v.cuda() for k, v in x.items()}
    n = lla.workspace_bytes(B, H, T, d, d, 64, 2, "bf16")
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    ws[:8].view(torch.int64)[0] = (7 << 32) | 0x7FFFFF00      # epoch 7, count far past the sweeps
    out = torch.zeros_like(dd["v"])
    lla.forward(dd["q"], dd["k"], dd["v"], dd["log_a"], dd["lam"], out, chunk=64, sweep=2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
