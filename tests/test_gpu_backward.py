"""GPU parity of the backward pass: gradients from the C ABI (loglinear_attn_bwd) against the
fp64 CPU oracle's gradients of the definition on identical seeded inputs and upstream gradient.

Every gradient (dq, dk, dv, dlog_a, dlambda) is compared element by element through the
relative L2 error over the whole tensor: 1e-4 for float32 inputs, 2e-2 for bfloat16 inputs
with float32 accumulation. Cases cover several chunks and chunk levels with a ragged tail,
dk != dv, the degenerate lengths (T = 1, T < C, T = C), one-hot lambda at every level with no
decay (so that coarse levels are not hidden by decay), strong decay, bitwise determinism, a
caller workspace full of NaN bytes, and every head of the headline and long workloads at full
size on sampled positions.
"""

import numpy as np
import pytest

import oracle.loglinear as O
from lla_synth import custom, generate, grad_output, workload
from tests._util import ensure_built, rel_l2, tol_for

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dlog_a", "dlam")


@pytest.fixture(scope="module", autouse=True)
def _built():
    import torch
    ensure_built()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_bwd(x, do, **kw):
    """Device backward pass on CPU inputs; returns the five gradients as float64 numpy."""
    import torch
    import log_linear_attention_chunked_amd as lla
    d = {k: v.cuda() for k, v in x.items()}
    g = lla.backward(d["q"], d["k"], d["v"], d["log_a"], d["lam"], do.cuda(), **kw)
    torch.cuda.synchronize()
    return {n: t.double().cpu().numpy() for n, t in zip(GRADS, g)}


def check(w, x, do, label, **kw):
    print(f"[bwd] {label} B={w.B} H={w.H} T={w.T} dk={w.dk} dv={w.dv} {w.dtype} {kw}", flush=True)
    got = run_bwd(x, do, **kw)
    want = O.bruteforce_grad(**x, do=do)
    tol = tol_for(w.dtype)
    errs = {n: rel_l2(got[n], want[n]) for n in GRADS}
    print(f"[bwd] {label}: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
    for n in GRADS:
        assert np.all(np.isfinite(got[n])), (label, n)
        assert errs[n] <= tol, (label, n, errs)
    return got


CASES = [
    # B, H, T, dk, dv, dtype, chunk
    (1, 2, 256, 16, 16, "f32", 0),      # the small fp32 workload's shape, default chunk 16
    (1, 2, 256, 16, 16, "f32", 32),
    (1, 2, 200, 32, 16, "f32", 16),     # ragged, dk != dv
    (2, 1, 333, 16, 32, "f32", 32),
    (1, 2, 130, 64, 64, "f32", 64),
    (1, 1, 100, 128, 16, "f32", 0),
    (1, 2, 300, 64, 64, "bf16", 64),
    (1, 2, 1000, 64, 64, "bf16", 0),
    (2, 2, 600, 64, 128, "bf16", 0),
    (1, 2, 520, 128, 32, "bf16", 32),
    (1, 1, 1024, 128, 128, "bf16", 0),
    (1, 2, 700, 32, 32, "bf16", 16),
    # d = 128 by columns of dq with a ragged last group of 8 chunks (21 and 22 chunks): the
    # gradient kernel forms U_c from the tree's group states in batches
    (1, 2, 1300, 128, 128, "bf16", 64),
    (1, 1, 700, 128, 128, "f32", 0),
]


@pytest.mark.parametrize("B,H,T,dk,dv,dtype,chunk", CASES)
def test_backward_matches_oracle(B, H, T, dk, dv, dtype, chunk):
    w = custom(B, H, T, dk, dv, dtype)
    x = generate(w, seed=T + dk)
    do = grad_output(w, seed=T + dk)
    check(w, x, do, "random", chunk=chunk)


@pytest.mark.parametrize("T,chunk", [(1, 16), (5, 16), (16, 16), (17, 16), (64, 64), (63, 64), (65, 64)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_degenerate_lengths(T, chunk, dtype):
    w = custom(1, 2, T, 32, 16, dtype)
    x = generate(w, seed=3)
    do = grad_output(w, seed=3)
    check(w, x, do, "short", chunk=chunk)


@pytest.mark.parametrize("level", list(range(10)))
def test_backward_onehot_levels_no_decay(level):
    # T = 512, C = 16: levels 0..4 inside a chunk, 5..9 across chunks (chunk levels 0..4)
    w = custom(1, 2, 512, 16, 16, "f32")
    x = generate(w, seed=11, log_a_mode="nodecay", lam_mode=f"onehot:{level}")
    do = grad_output(w, seed=11)
    check(w, x, do, f"onehot:{level}", chunk=16)


@pytest.mark.parametrize("mode", ["nodecay", "lowdecay"])
def test_backward_low_decay_bf16(mode):
    w = custom(1, 2, 2048, 64, 64, "bf16")
    x = generate(w, seed=5, log_a_mode=mode)
    do = grad_output(w, seed=5)
    check(w, x, do, mode, chunk=64)


@pytest.mark.parametrize("B,H,T,dk,dv,dtype,chunk", [
    (1, 2, 1000, 64, 64, "bf16", 64),
    (1, 2, 700, 32, 32, "bf16", 16),
    (1, 2, 600, 32, 16, "f32", 32),
    (1, 1, 513, 128, 128, "bf16", 0),
])
def test_backward_strong_decay(B, H, T, dk, dv, dtype, chunk):
    # log_a = -U(0.5, 3): decays inside a chunk span far more than e^-40 and across chunks
    # underflow to exactly zero; every gradient still matches the definition's
    w = custom(B, H, T, dk, dv, dtype)
    x = generate(w, seed=T + 5, log_a_mode="strongdecay")
    do = grad_output(w, seed=T + 5)
    check(w, x, do, "strongdecay", chunk=chunk)


def test_backward_mixed_strong_and_no_decay():
    # strong gates over the first half, none over the second (coarse levels visible there)
    w = custom(1, 2, 2048, 32, 32, "bf16")
    x = generate(w, seed=31, log_a_mode="strongdecay")
    x["log_a"][..., 1024:] = 0.0
    x["log_a"] = x["log_a"].contiguous()
    do = grad_output(w, seed=31)
    check(w, x, do, "mixed decay", chunk=32)


@pytest.mark.parametrize("level", [7, 9, 11])
def test_backward_coarse_onehot_bf16(level):
    w = custom(1, 1, 2048, 64, 64, "bf16")
    x = generate(w, seed=6, log_a_mode="lowdecay", lam_mode=f"onehot:{level}")
    do = grad_output(w, seed=6)
    check(w, x, do, f"onehot:{level}", chunk=64)


@pytest.mark.parametrize("T,dtype,mode", [(6000, "f32", "lowdecay"), (8192, "bf16", None)])
def test_backward_many_chunks(T, dtype, mode):
    # N = T/16 = 375 and 512 chunks, 9 chunk levels: the group tree with 4 groups per wave (a
    # ragged last run at 47 groups); one-hot-free random lambda, low decay so that the coarse
    # levels carry weight
    w = custom(1, 1, T, 16, 16, dtype)
    x = generate(w, seed=12, log_a_mode=mode)
    do = grad_output(w, seed=12)
    check(w, x, do, f"many chunks {mode}", chunk=16)


def test_backward_small_bf16_workload():
    w = workload("b2h8_t2048_d64_bf16")
    x = generate(w, seed=0)
    do = grad_output(w, seed=0)
    check(w, x, do, w.name, chunk=w.chunk)


def test_backward_equal_lambda_is_mamba2_gradient():
    # every level weight equal: the gradient of c_t x the Mamba-2 recurrence, here through the
    # oracle's definition; also checks that dlambda splits the row total across levels
    w = custom(1, 2, 400, 32, 32, "f32")
    x = generate(w, seed=8, lam_mode="equal")
    do = grad_output(w, seed=8)
    got = check(w, x, do, "equal", chunk=32)
    want = O.bruteforce_grad(**x, do=do)
    assert rel_l2(got["dlam"].sum(-1), want["dlam"].sum(-1)) <= 1e-4


def test_backward_deterministic_and_workspace_poison():
    import torch
    import log_linear_attention_chunked_amd as lla
    w = custom(2, 2, 1500, 64, 64, "bf16")
    x = {k: v.cuda() for k, v in generate(w, seed=9).items()}
    do = grad_output(w, seed=9).cuda()
    print("[bwd] determinism / poisoned workspace", flush=True)
    a = lla.backward(x["q"], x["k"], x["v"], x["log_a"], x["lam"], do)
    nbytes = lla.bwd_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, 0, "bf16")
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    b = lla.backward(x["q"], x["k"], x["v"], x["log_a"], x["lam"], do, workspace=ws)
    c = lla.backward(x["q"], x["k"], x["v"], x["log_a"], x["lam"], do, workspace=ws)
    torch.cuda.synchronize()
    for ta, tb, tc in zip(a, b, c):
        assert torch.equal(ta, tb) and torch.equal(ta, tc)


def _sample_rows(T, C, seed):
    rng = np.random.default_rng(seed)
    rows = set(range(0, C // 2)) | set(range(T - C // 2, T)) | {C - 1, C, 2 * C - 1, 2 * C}
    p = 1
    while p < T:
        rows |= {p - 1, p, p + 1}
        p <<= 1
    rows |= set(int(x) for x in rng.integers(0, T, 16))
    return sorted(r for r in rows if 0 <= r < T)


def check_sampled(label, x, do, got, heads, rows, tail=64):
    """Every gradient of the given heads at the sampled positions against the oracle computed
    position by position: dq, dk, dv, dlambda directly; dA_r = dlog_a[r] - dlog_a[r+1]
    (dlog_a[T] = 0) at the same positions; dlog_a itself over the last `tail` positions. Prints
    the worst head of each."""
    from tests._util import per_head
    T = x["q"].shape[2]
    refs = per_head(lambda b, h: O.bruteforce_grad_rows(**x, do=do, b=b, h=h, rows=rows, tail=tail),
                    heads)
    worst = {n: 0.0 for n in ("dq", "dk", "dv", "dlam", "dA", "dlog_a tail")}
    for (b, h), ref in zip(heads, refs):
        gh = {n: t[b, h].double().cpu().numpy() for n, t in got.items()}
        for n in ("dq", "dk", "dv", "dlam", "dlog_a"):
            assert np.all(np.isfinite(gh[n])), (label, b, h, n)
        for n in ("dq", "dk", "dv", "dlam"):
            worst[n] = max(worst[n], rel_l2(gh[n][rows], ref[n]))
        nxt = np.append(gh["dlog_a"][1:], 0.0)
        dA = (gh["dlog_a"] - nxt)[rows]
        worst["dA"] = max(worst["dA"], rel_l2(dA, ref["dA"]))
        worst["dlog_a tail"] = max(worst["dlog_a tail"], rel_l2(gh["dlog_a"][T - tail:], ref["dlog_a_tail"]))
    print(f"[bwd] {label}: {len(heads)} heads x {len(rows)} positions, worst rel_l2 " +
          ", ".join(f"{n} {e:.2e}" for n, e in worst.items()), flush=True)
    for n, e in worst.items():
        assert e <= 2e-2, (label, n, e)
    return worst


def _full_size(name, mode=None):
    import torch
    import log_linear_attention_chunked_amd as lla
    w = workload(name)
    x = generate(w, seed=0, log_a_mode=mode)
    do = grad_output(w, seed=0)
    print(f"[bwd] {name} {mode or 'as stated'} full size", flush=True)
    d = {k: v.cuda() for k, v in x.items()}
    g = lla.backward(d["q"], d["k"], d["v"], d["log_a"], d["lam"], do.cuda())
    torch.cuda.synchronize()
    got = {n: t for n, t in zip(GRADS, g)}
    C = lla.bwd_default_chunk(w.dk, w.dv, w.dtype)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    return w, x, do, got, heads, _sample_rows(w.T, C, seed=1)


@pytest.mark.parametrize("mode", [None, "nodecay"])
def test_backward_headline_every_head_sampled(mode):
    # the headline shape (B=4, H=16, T=8192, d=64, bf16) in the launch configuration the
    # benchmark times: all 64 heads at sampled positions
    w, x, do, got, heads, rows = _full_size("b4h16_t8192_d64_bf16", mode)
    check_sampled(f"{w.name} {mode or 'as stated'}", x, do, got, heads, rows)


@pytest.mark.parametrize("name", ["b1h16_t32768_d128_bf16_knorm", "b1h8_t65536_d128_bf16_coarse"])
def test_backward_long_workloads_sampled(name):
    # the two long workloads at full size, in the launch configuration the library picks: every
    # head at sampled positions (the first and last half chunk, chunk edges, around powers of
    # two, 16 uniform), dA there, and dlog_a over the last 64 positions
    w, x, do, got, heads, rows = _full_size(name)
    check_sampled(name, x, do, got, heads, rows)


def test_backward_group_tree_1000_chunks_sampled():
    # 1000 chunks per head (T = 16000, C = 16): the group tree at its largest tree, 125 groups in
    # runs of 8 per wave (the last run 5 groups), units of 2, 4 and 8 groups summed per right
    # block; sampled positions and a dlog_a tail, low decay so that the coarse levels carry weight
    import torch
    import log_linear_attention_chunked_amd as lla
    w = custom(1, 2, 16000, 16, 16, "bf16")
    x = generate(w, seed=14, log_a_mode="lowdecay")
    do = grad_output(w, seed=14)
    print("[bwd] T=16000 C=16 group tree, 1000 chunks", flush=True)
    d = {k: v.cuda() for k, v in x.items()}
    g = lla.backward(d["q"], d["k"], d["v"], d["log_a"], d["lam"], do.cuda(), chunk=16)
    torch.cuda.synchronize()
    got = {n: t for n, t in zip(GRADS, g)}
    check_sampled("T=16000 C=16 group tree", x, do, got, [(0, 0), (0, 1)], _sample_rows(w.T, 16, seed=3))


def test_backward_tree_in_workspace_sampled():
    # 2048 chunks per head (T = 32768, C = 16): the tree's levels no longer fit shared memory at
    # any width and stay in the workspace; sampled positions and a dlog_a tail, low decay so that
    # the coarse levels carry weight
    import torch
    import log_linear_attention_chunked_amd as lla
    w = custom(1, 1, 32768, 16, 16, "bf16")
    x = generate(w, seed=13, log_a_mode="lowdecay")
    do = grad_output(w, seed=13)
    print("[bwd] T=32768 C=16 tree in workspace", flush=True)
    d = {k: v.cuda() for k, v in x.items()}
    g = lla.backward(d["q"], d["k"], d["v"], d["log_a"], d["lam"], do.cuda(), chunk=16)
    torch.cuda.synchronize()
    got = {n: t for n, t in zip(GRADS, g)}
    check_sampled("T=32768 C=16 tree in workspace", x, do, got, [(0, 0)], _sample_rows(w.T, 16, seed=2))
