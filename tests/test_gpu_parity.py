"""GPU parity: the HIP path against the fp64 CPU oracle on identical seeded inputs.

Bars (relative L2 over all outputs): 1e-4 for float32 inputs, 2e-2 for bfloat16 inputs
with float32 accumulation. Shapes here compare every element with the O(T^2) oracle; the
full-size workloads are in tests/test_gpu_fullsize.py.
"""

import numpy as np
import pytest

import oracle.loglinear as O
from lla_synth import WORKLOADS, custom, generate
from tests._util import ensure_built, fits_smem, rel_l2, run_gpu, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    import torch
    ensure_built()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def check_full(x, dtype, **kw):
    got = run_gpu(x, **kw)
    want = O.bruteforce(x["q"], x["k"], x["v"], x["log_a"], x["lam"])
    err = rel_l2(got, want)
    print(f"rel_l2={err:.3e} kw={kw}", flush=True)
    assert np.all(np.isfinite(got))
    assert err <= tol_for(dtype), err
    return got, want


def expect_unsupported(x, **kw):
    """Shapes whose sweep images exceed the 160 KB of shared memory: the library refuses them
    with LLA_ERR_UNSUPPORTED (a host-side check) and writes nothing."""
    import torch
    import log_linear_attention_chunked_amd as lla
    from log_linear_attention_chunked_amd import _lib
    d = {k_: v_.cuda() for k_, v_ in x.items()}
    out = torch.full_like(d["v"], 7.0)
    with pytest.raises(lla.LLAError) as e:
        lla.forward(d["q"], d["k"], d["v"], d["log_a"], d["lam"], out, **kw)
    assert e.value.status == _lib.LLA_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


# --------------------------------------------------------------------------------------
# the small fp32 workload, every element
# --------------------------------------------------------------------------------------

def test_small_f32_workload_full():
    w = WORKLOADS["b1h2_t256_d16_f32"]
    x = generate(w, seed=0)
    check_full(x, "f32", chunk=w.chunk)


@pytest.mark.parametrize("chunk,sweep", [(16, 1), (16, 2), (32, 1), (32, 2), (64, 1), (64, 2), (128, 1), (128, 2)])
def test_small_f32_chunk_and_sweep_invariance(chunk, sweep):
    w = WORKLOADS["b1h2_t256_d16_f32"]
    x = generate(w, seed=0, log_a_mode="lowdecay")
    if not fits_smem("f32", chunk, w.dk, w.dv, sweep):
        expect_unsupported(x, chunk=chunk, sweep=sweep)   # documented: exceeds shared memory
        return
    check_full(x, "f32", chunk=chunk, sweep=sweep)


# --------------------------------------------------------------------------------------
# shapes: head dims, ragged T, degenerate sizes, both dtypes
# --------------------------------------------------------------------------------------

SHAPES = [
    # B, H, T, dk, dv, chunk, sweep
    (1, 1, 1, 16, 16, 16, 1),        # single token
    (1, 1, 16, 16, 16, 16, 1),       # T = C, one chunk
    (1, 2, 32, 32, 32, 16, 1),       # two chunks
    (2, 1, 100, 32, 64, 32, 2),      # ragged last chunk, dk != dv
    (1, 2, 333, 64, 32, 64, 2),      # ragged, dk > dv
    (1, 1, 1024, 64, 64, 64, 2),     # several sweeps
    (1, 2, 1000, 128, 128, 64, 2),   # d = 128, ragged
    (1, 1, 512, 128, 64, 128, 1),    # C = 128
    (2, 2, 768, 16, 128, 32, 2),     # dk = 16, dv = 128
    (1, 1, 4160, 64, 64, 64, 2),     # 65 chunks: many sweeps + a lone last chunk
    (1, 3, 999, 64, 64, 64, 2),      # T*L odd: lambda rows of heads 1, 2 not 16-byte aligned
    (1, 2, 8192, 32, 32, 16, 1),     # 512 sweeps per head: deep Fenwick tree over sweeps
    (1, 1, 2048, 128, 128, 128, 1),  # C = 128, d = 128
    # dv > dk with a lone last chunk (the output rows' staging reaches into its v image)
    (1, 2, 300, 32, 64, 64, 2),
    (2, 1, 600, 16, 128, 32, 2),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}h{}t{}dk{}dv{}c{}r{}".format(*s))
def test_shapes(shape, dtype):
    B, H, T, dk, dv, C, R = shape
    x = generate(custom(B, H, T, dk, dv, dtype=dtype), seed=T + dk)
    if not fits_smem(dtype, C, dk, dv, R):
        expect_unsupported(x, chunk=C, sweep=R)   # documented: exceeds shared memory
        return
    check_full(x, dtype, chunk=C, sweep=R)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_default_plan(dtype):
    x = generate(custom(2, 3, 1500, 64, 64, dtype=dtype), seed=11)
    check_full(x, dtype)


# --------------------------------------------------------------------------------------
# stress: no decay, so coarse Fenwick levels carry weight; one-hot levels isolate stages
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("lev", [0, 3, 6, 7, 8, 9, 10, 11, 12])
def test_onehot_levels_no_decay(lev, dtype):
    # T=4096 at C=64, sweep 2: levels 0..6 intra-chunk, 7 inside a sweep, 8..12 across sweeps
    x = generate(custom(1, 2, 4096, 64, 64, dtype=dtype), seed=lev,
                 log_a_mode="nodecay", lam_mode=f"onehot:{lev}")
    check_full(x, dtype, chunk=64, sweep=2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode", ["nodecay", "lowdecay"])
def test_low_decay_all_levels(mode, dtype):
    x = generate(custom(2, 2, 2048, 64, 64, dtype=dtype), seed=5, log_a_mode=mode)
    check_full(x, dtype, chunk=64, sweep=2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("chunk,sweep", [(64, 1), (64, 2), (128, 1), (128, 2)])
def test_strong_decay(chunk, sweep, dtype):
    # log_a = -U(0.5, 3) (strong Mamba-2-style gates): a chunk's local log decay passes -40 a few
    # positions in, so the score units take exp(A_i - A_s) directly instead of e^{A_i} e^{-A_s}
    # (whose factors would overflow); node decays underflow to exactly zero
    d = 64 if dtype == "bf16" else 32
    x = generate(custom(1, 2, 2048, d, d, dtype=dtype), seed=21, log_a_mode="strongdecay")
    if not fits_smem(dtype, chunk, d, d, sweep):
        expect_unsupported(x, chunk=chunk, sweep=sweep)
        return
    check_full(x, dtype, chunk=chunk, sweep=sweep)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("chunk,sweep", [(64, 2), (128, 1)])
def test_mixed_strong_and_no_decay(chunk, sweep, dtype):
    # strong gates over the first half of the sequence, none over the second: the first half
    # takes the direct-exponential path, the second keeps every Fenwick level visible, and the
    # nodes of the first half reach the second half decayed exactly to zero
    import torch
    d = 32
    w = custom(1, 2, 4096, d, d, dtype=dtype)
    x = generate(w, seed=22, log_a_mode="strongdecay")
    x["log_a"][..., 2048:] = 0.0
    x["log_a"][..., 1500:1520] = torch.tensor(-3.0)     # one burst of strong decay inside a chunk
    x["log_a"] = x["log_a"].contiguous()
    check_full(x, dtype, chunk=chunk, sweep=sweep)


def test_equal_lambda_reduces_to_mamba2_on_gpu():
    x = generate(custom(1, 2, 700, 32, 32, dtype="f32"), seed=9, lam_mode="equal")
    got = run_gpu(x, chunk=32, sweep=2)
    # c_t * (S_t^T q_t) with S_t = a_t S_{t-1} + k_t v_t^T, evaluated as the masked product
    q, k, v, la = (O.as_f64(x[n]) for n in ("q", "k", "v", "log_a"))
    c = O.as_f64(x["lam"])[..., 0]
    want = np.zeros_like(got)
    for h in range(2):
        A = np.cumsum(la[0, h])
        D = np.tril(np.exp(np.minimum(A[:, None] - A[None, :], 0.0)))
        want[0, h] = c[0, h][:, None] * ((q[0, h] @ k[0, h].T) * D) @ v[0, h]
    assert rel_l2(got, want) <= 1e-4


def test_zero_lambda_gives_zero():
    x = generate(custom(1, 2, 300, 64, 64), seed=1, lam_mode="zero")
    got = run_gpu(x, chunk=64, sweep=2)
    assert np.all(got == 0.0)


def test_causality():
    import torch
    w = custom(1, 2, 640, 64, 64)
    x = generate(w, seed=2)
    y = {k: v.clone() for k, v in x.items()}
    t0 = 300
    g = torch.Generator().manual_seed(3)
    for key in ("q", "k", "v"):
        y[key][:, :, t0:] = torch.randn(y[key][:, :, t0:].shape, generator=g).to(y[key].dtype)
    y["log_a"][:, :, t0:] = -torch.rand(y["log_a"][:, :, t0:].shape, generator=g)
    y["lam"][:, :, t0:] = torch.rand(y["lam"][:, :, t0:].shape, generator=g)
    a = run_gpu(x, chunk=64, sweep=2)
    b = run_gpu(y, chunk=64, sweep=2)
    assert np.array_equal(a[:, :, :t0], b[:, :, :t0])
    assert not np.array_equal(a[:, :, t0:], b[:, :, t0:])


def test_bitwise_deterministic():
    x = generate(custom(2, 4, 2048, 64, 64), seed=4)
    a = run_gpu(x, chunk=64, sweep=2)
    b = run_gpu(x, chunk=64, sweep=2)
    assert np.array_equal(a, b)


def test_caller_workspace_matches_library_workspace():
    import torch
    import log_linear_attention_chunked_amd as lla
    x = generate(custom(1, 4, 2048, 64, 64), seed=6)
    d = {k: v.cuda() for k, v in x.items()}
    n = lla.workspace_bytes(1, 4, 2048, 64, 64, 64, 2, "bf16")
    assert n > 0
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    a = lla.forward(d["q"], d["k"], d["v"], d["log_a"], d["lam"], chunk=64, sweep=2, workspace=ws)
    b = lla.forward(d["q"], d["k"], d["v"], d["log_a"], d["lam"], chunk=64, sweep=2)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def poison(ws, BH, T, chunk, sweep, dv):
    """0xFF over the whole workspace, then zeros over its counter-and-flags prefix (whose size
    the header documents)."""
    nsweep = -(-(-(-T // chunk)) // sweep)
    sync_bytes = (4 * (64 + BH * (nsweep - 1) * (dv // 16)) + 255) // 256 * 256
    ws.fill_(0xFF)
    ws[:sync_bytes].zero_()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("sweep", [1, 2])
def test_poisoned_workspace(dtype, sweep):
    """Nodes pass between workgroups through the workspace: node data filled with 0xFF bytes
    (NaN) before every call, the counter and flags zero-filled (the documented requirement),
    it must still give oracle parity, i.e. every node is read only after it was published."""
    import torch
    import log_linear_attention_chunked_amd as lla
    B, H, T = 2, 3, 3000
    n = lla.workspace_bytes(B, H, T, 64, 64, 64, sweep, dtype)
    assert n > 0
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    for seed in range(2):
        x = generate(custom(B, H, T, 64, 64, dtype=dtype), seed=100 + seed, log_a_mode="lowdecay")
        d = {k_: v_.cuda() for k_, v_ in x.items()}
        poison(ws, B * H, T, 64, sweep, 64)
        got = lla.forward(d["q"], d["k"], d["v"], d["log_a"], d["lam"], chunk=64, sweep=sweep, workspace=ws)
        torch.cuda.synchronize()
        got = got.double().cpu().numpy()
        want = O.bruteforce(x["q"], x["k"], x["v"], x["log_a"], x["lam"])
        err = rel_l2(got, want)
        print(f"poisoned workspace {dtype} sweep {sweep} seed {seed}: rel_l2={err:.3e}", flush=True)
        assert np.all(np.isfinite(got))
        assert err <= tol_for(dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_workspace_reused_across_inputs(dtype):
    """One workspace, several different inputs back to back with nothing in between: each
    call must match the oracle, so no node of an earlier call is ever read."""
    import torch
    import log_linear_attention_chunked_amd as lla
    B, H, T = 1, 4, 4096
    n = lla.workspace_bytes(B, H, T, 64, 64, 64, 2, dtype)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    outs, xs = [], []
    for seed in range(3):
        x = generate(custom(B, H, T, 64, 64, dtype=dtype), seed=300 + seed,
                     log_a_mode="nodecay" if seed == 2 else "lowdecay")
        d = {k_: v_.cuda() for k_, v_ in x.items()}
        outs.append(lla.forward(d["q"], d["k"], d["v"], d["log_a"], d["lam"], chunk=64, sweep=2, workspace=ws))
        xs.append(x)
    torch.cuda.synchronize()
    for seed, (x, o) in enumerate(zip(xs, outs)):
        got = o.double().cpu().numpy()
        want = O.bruteforce(x["q"], x["k"], x["v"], x["log_a"], x["lam"])
        err = rel_l2(got, want)
        print(f"reused workspace {dtype} call {seed}: rel_l2={err:.3e}", flush=True)
        assert np.all(np.isfinite(got))
        assert err <= tol_for(dtype)


def test_poisoned_workspace_headline_shape():
    """The same at the benchmark's shape and launch configuration, three calls in a row."""
    import torch
    import log_linear_attention_chunked_amd as lla
    w = WORKLOADS["b4h16_t8192_d64_bf16"]
    sweep = lla.default_sweep(w.B, w.H, w.T, w.dk, w.dv, w.chunk, w.dtype)
    n = lla.workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, w.chunk, sweep, w.dtype)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    rows = sample_rows(w.T, w.chunk)
    for seed in range(3):
        x = generate(w, seed=200 + seed, log_a_mode="nodecay" if seed == 1 else None)
        d = {k_: v_.cuda() for k_, v_ in x.items()}
        poison(ws, w.B * w.H, w.T, w.chunk, sweep, w.dv)
        got = lla.forward(d["q"], d["k"], d["v"], d["log_a"], d["lam"], chunk=w.chunk, sweep=sweep,
                          workspace=ws)
        torch.cuda.synchronize()
        got = got.double().cpu().numpy()
        assert np.all(np.isfinite(got))
        for (b, h) in [(0, 0), (w.B - 1, w.H - 1), (1, 7)]:
            want = O.bruteforce_rows(x["q"], x["k"], x["v"], x["log_a"], x["lam"], b, h, rows)
            err = rel_l2(got[b, h, rows], want)
            print(f"headline poisoned seed {seed} head ({b},{h}): rel_l2={err:.3e}", flush=True)
            assert err <= tol_for(w.dtype)


def test_plain_entry_points():
    import ctypes
    import torch
    from log_linear_attention_chunked_amd import _lib
    lib = _lib.lib()
    for dtype, fn in (("bf16", lib.loglinear_attn_fwd), ("f32", lib.loglinear_attn_fwd_f32)):
        x = generate(custom(1, 2, 1000, 64, 64, dtype=dtype), seed=8)
        d = {k: v.cuda() for k, v in x.items()}
        out = torch.empty_like(d["v"])
        st = fn(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), d["log_a"].data_ptr(),
                d["lam"].data_ptr(), out.data_ptr(), 1, 2, 1000, 64, 64,
                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0
        torch.cuda.synchronize()
        want = O.bruteforce(x["q"], x["k"], x["v"], x["log_a"], x["lam"])
        assert rel_l2(out.double().cpu().numpy(), want) <= tol_for(dtype)


# sampled rows for the full-size checks (every head of every full-size workload is checked in
# tests/test_gpu_fullsize.py)
def sample_rows(T, C, seed=1, n_uniform=48):
    rows = set(range(min(T, 2 * C))) | set(range(max(0, T - C), T))
    k = 1
    while k < T:
        rows |= {k - 1, k, min(T - 1, k + 1)}
        k <<= 1
    rng = np.random.default_rng(seed)
    rows |= set(int(r) for r in rng.integers(0, T, n_uniform))
    return sorted(r for r in rows if 0 <= r < T)
