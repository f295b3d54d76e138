"""GPU parity of log-linear Gated DeltaNet (loglinear_attn_gdn_fwd) against the fp64 oracle
(oracle.deltanet.gdn_bruteforce, the definition: every source carried through the delta-rule
transitions, then the hierarchical mask) on identical seeded inputs.

Bars (relative L2 over all compared outputs): 1e-4 for float32 inputs, 2e-2 for bfloat16.
Small shapes compare every element: several chunks and chunk levels, ragged tails, T = 1, T < C,
T = C, dk != dv, d = 128, each chunk size; one-hot lambda at every level kind with no decay
(intra-chunk, and each Fenwick level across chunks); equal lambda (Gated DeltaNet itself);
beta = 0; strong decay; bf16 lambda (bitwise the float32 path on the same values); bitwise
determinism; a caller workspace full of NaN bytes. Full size: every element of every head of
gdn_b2h8_t2048_d64_bf16 and of four heads of the 8192-token workloads.
"""

import numpy as np
import pytest

import oracle.deltanet as D
from lla_synth import GDN_WORKLOADS, custom, generate_gdn
from tests._util import ensure_built, per_head, rel_l2, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    import torch
    ensure_built()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_gdn(x, **kw):
    import torch
    import log_linear_attention_chunked_amd as lla
    d = {k: v.cuda() for k, v in x.items()}
    out = lla.gdn_forward(d["q"], d["k"], d["v"], d["log_a"], d["beta"], d["lam"], **kw)
    torch.cuda.synchronize()
    return out.double().cpu().numpy()


def check(x, dtype, label="", **kw):
    got = run_gdn(x, **kw)
    want = D.gdn_bruteforce(**x)
    err = rel_l2(got, want)
    print(f"[gdn] {label} {tuple(x['q'].shape)} dv={x['v'].shape[-1]} {dtype} {kw}: rel_l2={err:.3e}", flush=True)
    assert np.all(np.isfinite(got))
    assert err <= tol_for(dtype), err
    return got


def gdn_custom(B, H, T, dk, dv, dtype):
    return custom(B, H, T, dk, dv, dtype=dtype, k_l2norm=True)


SHAPES = [
    # B, H, T, dk, dv, dtype, chunk
    (1, 1, 1, 16, 16, "f32", 0),
    (1, 2, 16, 16, 16, "f32", 16),       # T = C
    (1, 2, 40, 32, 16, "f32", 64),       # T < C
    (2, 1, 300, 32, 64, "f32", 32),      # ragged, dk != dv
    (1, 2, 1000, 64, 64, "f32", 64),     # 16 chunks, 4 levels of nodes
    (1, 2, 256, 16, 16, "f32", 16),      # the small fp32 shape
    (1, 2, 333, 64, 32, "bf16", 64),
    (2, 2, 1024, 64, 64, "bf16", 0),
    (1, 2, 700, 128, 128, "bf16", 0),    # d = 128: chunk 32
    (1, 1, 513, 128, 64, "f32", 32),
    (1, 2, 2048, 16, 16, "bf16", 16),    # 128 chunks: 7 tree levels
    (1, 1, 999, 32, 128, "bf16", 32),
    # split-bf16 tree nodes: dk = 64 with dv = 128 (20 chunks, the two-level up-sweep's levels
    # 1-2 and 3-4), and dk = 32 over 94 chunks (odd node counts at levels 1, 2 and 5, levels
    # 1-2, 3-4 and 5-6 in pairs)
    (1, 2, 640, 64, 128, "bf16", 32),
    (2, 1, 1500, 32, 32, "bf16", 16),
    # 33 chunks at chunk 32 (an odd count: the two-level up-sweep's unpaired last node at level 1)
    (1, 2, 1050, 64, 64, "bf16", 32),
    # dk = 32, dv = 64: the query kernel's 64-wide node images with permuted windows hold a
    # 32 x 32 transition (27 chunks, a ragged tail)
    (2, 1, 850, 32, 64, "bf16", 32),
]


@pytest.mark.parametrize("B,H,T,dk,dv,dtype,chunk", SHAPES)
def test_gdn_shapes(B, H, T, dk, dv, dtype, chunk):
    x = generate_gdn(gdn_custom(B, H, T, dk, dv, dtype), seed=T + dk + dv, log_a_mode="lowdecay" if T > 500 else None)
    check(x, dtype, "shape", chunk=chunk)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("lev", [0, 2, 4, 5, 6, 7, 8, 9])
def test_gdn_onehot_levels_no_decay(lev, dtype):
    # T = 512 at chunk 16: levels 0..4 inside a chunk, 5..9 the Fenwick levels across chunks
    x = generate_gdn(gdn_custom(1, 2, 512, 32, 32, dtype), seed=lev, log_a_mode="nodecay",
                     lam_mode=f"onehot:{lev}")
    check(x, dtype, f"onehot:{lev}", chunk=16)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gdn_equal_lambda_is_gated_deltanet(dtype):
    # every level weight equal: Gated DeltaNet itself (the oracle is pinned to the textbook
    # recurrence in this case)
    x = generate_gdn(gdn_custom(1, 2, 600, 32, 32, dtype), seed=3, lam_mode="equal", log_a_mode="lowdecay")
    check(x, dtype, "equal lambda", chunk=32)


def test_gdn_zero_beta_gives_zero():
    x = generate_gdn(gdn_custom(1, 2, 300, 64, 64, "bf16"), seed=4, beta_mode="zero")
    got = run_gdn(x)
    assert np.all(got == 0.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gdn_strong_decay_and_beta_one(dtype):
    x = generate_gdn(gdn_custom(1, 2, 777, 32, 32, dtype), seed=5, log_a_mode="strongdecay")
    check(x, dtype, "strong decay", chunk=64)
    x = generate_gdn(gdn_custom(1, 2, 777, 32, 32, dtype), seed=6, beta_mode="ones", log_a_mode="nodecay")
    check(x, dtype, "beta = 1, no decay", chunk=32)


def test_gdn_bf16_lambda_bitwise_and_determinism_and_poisoned_workspace():
    import torch
    import log_linear_attention_chunked_amd as lla
    w = gdn_custom(2, 2, 1500, 64, 64, "bf16")
    x = generate_gdn(w, seed=7, log_a_mode="lowdecay")
    d = {k: v.cuda() for k, v in x.items()}
    lam16 = d["lam"].to(torch.bfloat16).contiguous()
    lam32 = lam16.float().contiguous()
    a = lla.gdn_forward(d["q"], d["k"], d["v"], d["log_a"], d["beta"], lam16)
    b = lla.gdn_forward(d["q"], d["k"], d["v"], d["log_a"], d["beta"], lam32)
    n = lla.gdn_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, 0, "bf16")
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")
    c = lla.gdn_forward(d["q"], d["k"], d["v"], d["log_a"], d["beta"], lam32, workspace=ws)
    e = lla.gdn_forward(d["q"], d["k"], d["v"], d["log_a"], d["beta"], lam32, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(b, c) and torch.equal(c, e)
    x16 = dict(x)
    x16["lam"] = lam16.cpu()
    want = D.gdn_bruteforce(**x16)
    assert rel_l2(a.double().cpu().numpy(), want) <= tol_for("bf16")


def test_gdn_chunk_invariance():
    # the same inputs at every chunk size agree with the oracle and with each other
    x = generate_gdn(gdn_custom(1, 2, 640, 32, 32, "f32"), seed=8, log_a_mode="lowdecay")
    outs = [check(x, "f32", f"chunk {C}", chunk=C) for C in (16, 32, 64)]
    assert rel_l2(outs[0], outs[2]) <= 1e-4


def _every_element(w, x, got, heads):
    def one(b, h):
        xs = {k: v[b:b + 1, h:h + 1] for k, v in x.items()}
        return D.gdn_bruteforce(**xs)[0, 0]
    wants = per_head(one, heads)
    errs = [rel_l2(got[b, h], want) for (b, h), want in zip(heads, wants)]
    print(f"[gdn] {w.name}: every element of {len(heads)} heads, worst head rel_l2={max(errs):.3e}", flush=True)
    assert np.all(np.isfinite(got))
    assert max(errs) <= tol_for(w.dtype)


def test_gdn_small_workload_every_head():
    w = GDN_WORKLOADS["gdn_b2h8_t2048_d64_bf16"]
    x = generate_gdn(w, seed=0)
    got = run_gdn(x)
    _every_element(w, x, got, [(b, h) for b in range(w.B) for h in range(w.H)])


@pytest.mark.parametrize("name", ["gdn_b4h16_t8192_d64_bf16", "gdn_b1h8_t8192_d128_bf16"])
def test_gdn_long_workloads_four_heads(name):
    w = GDN_WORKLOADS[name]
    x = generate_gdn(w, seed=0)
    print(f"[gdn] {name}: GPU, then the oracle on four heads", flush=True)
    got = run_gdn(x)
    heads = [(0, 0), (w.B - 1, w.H - 1), (w.B // 2, w.H // 2), (0, w.H - 1)]
    _every_element(w, x, got, heads)
