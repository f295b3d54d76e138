"""GPU parity of the decoding step: a cache advanced token by token through the C ABI
against the fp64 CPU oracle on identical seeded inputs.

Every output of a T-token run is compared with the O(T^2) definition (relative L2 over all
outputs: 1e-4 for float32 inputs, 2e-2 for bfloat16 inputs), the cache itself with the
oracle's recurrent states, and a cache full of NaN before t = 0 must change nothing.
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


def run_decode(x, levels=None, fill=None):
    """Decode every position of x (forward-pass inputs [B,H,T,..]) on a fresh cache; returns
    the outputs [B,H,T,dv] and the cache after the last step (all as numpy)."""
    import torch
    import log_linear_attention_chunked_amd as lla
    B, H, T, dk = x["q"].shape
    dv = x["v"].shape[-1]
    L = x["lam"].shape[-1]
    Lc = levels or L
    d = {k: v.cuda() for k, v in x.items()}
    state, log_scale = lla.new_decode_cache(B, H, dk, dv, Lc)
    if fill is not None:
        state.fill_(fill)
        log_scale.fill_(fill)
    lam = torch.zeros((B, H, T, Lc), dtype=torch.float32, device="cuda")
    lam[..., :L] = d["lam"]
    outs = []
    for t in range(T):
        o = lla.decode_step(d["q"][:, :, t].contiguous(), d["k"][:, :, t].contiguous(),
                            d["v"][:, :, t].contiguous(), d["log_a"][:, :, t].contiguous(),
                            lam[:, :, t].contiguous(), state, log_scale, t)
        outs.append(o)
    torch.cuda.synchronize()
    out = torch.stack(outs, dim=2).float().cpu().numpy().astype(np.float64)
    return out, state.cpu().numpy().astype(np.float64), log_scale.cpu().numpy().astype(np.float64)


CASES = [
    # B, H, T, dk, dv, dtype
    (2, 3, 300, 64, 64, "bf16"),
    (1, 2, 200, 16, 32, "f32"),
    (1, 1, 130, 128, 64, "bf16"),
    (2, 1, 257, 32, 128, "f32"),
    (1, 2, 64, 64, 16, "f32"),
    (1, 1, 1, 16, 16, "f32"),          # a single token: level 0 only
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}h{}t{}dk{}dv{}_{}".format(*c))
def test_decode_matches_oracle(case):
    B, H, T, dk, dv, dtype = case
    x = generate(custom(B, H, T, dk, dv, dtype=dtype), seed=T + dk + dv)
    got, _, _ = run_decode(x)
    want = O.bruteforce(x["q"], x["k"], x["v"], x["log_a"], x["lam"])
    err = rel_l2(got, want)
    print(f"decode {case}: rel_l2={err:.3e}", flush=True)
    assert np.all(np.isfinite(got))
    assert err <= tol_for(dtype), err


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_strong_decay(dtype):
    # log_a = -U(0.5, 3): per-level log-scales reach far below -40 and are reset on rewrite
    x = generate(custom(2, 2, 300, 64, 32, dtype=dtype), seed=17, log_a_mode="strongdecay")
    got, _, _ = run_decode(x)
    want = O.bruteforce(x["q"], x["k"], x["v"], x["log_a"], x["lam"])
    err = rel_l2(got, want)
    print(f"decode strong decay {dtype}: rel_l2={err:.3e}", flush=True)
    assert np.all(np.isfinite(got))
    assert err <= tol_for(dtype), err


def test_decode_cache_holds_the_level_states():
    # after the last step, every live level (times its scale) equals the oracle's state
    B, H, T, dk, dv = 1, 2, 77, 32, 16
    x = generate(custom(B, H, T, dk, dv, dtype="f32"), seed=3)
    _, state, log_scale = run_decode(x)
    L = x["lam"].shape[-1]
    xs = {k: O.as_f64(v) for k, v in x.items()}
    t = T - 1
    for h in range(H):
        S = np.zeros((L + 1, dk, dv))
        for s in range(T):
            O.recurrent_step(S, xs["q"][0, h, s], xs["k"][0, h, s], xs["v"][0, h, s],
                             xs["log_a"][0, h, s], xs["lam"][0, h, s, :L], s)
        par = t & 1
        k0 = state[0, h, 0].reshape(-1)[par * (dk + dv): par * (dk + dv) + dk]
        v0 = state[0, h, 0].reshape(-1)[par * (dk + dv) + dk: (par + 1) * (dk + dv)]
        assert rel_l2(np.outer(k0, v0), S[0]) <= 1e-6
        for lev in range(1, L):
            if (t >> (lev - 1)) & 1:
                got = state[0, h, lev] * np.exp(log_scale[0, h, par, lev])
                assert rel_l2(got, S[lev]) <= 1e-5, (h, lev)


def test_decode_never_reads_an_unwritten_cache():
    # NaN everywhere before t = 0: a level is read only after a step wrote it
    x = generate(custom(1, 2, 150, 64, 32, dtype="bf16"), seed=9)
    a, _, _ = run_decode(x)
    b, _, _ = run_decode(x, fill=float("nan"))
    assert np.all(np.isfinite(b))
    assert np.array_equal(a, b)


def test_decode_with_spare_levels():
    # a cache with more levels than the positions need
    x = generate(custom(1, 1, 100, 16, 16, dtype="f32"), seed=4)
    got, _, _ = run_decode(x, levels=20)
    want = O.bruteforce(x["q"], x["k"], x["v"], x["log_a"], x["lam"])
    assert rel_l2(got, want) <= tol_for("f32")


def test_decode_agrees_with_the_forward_pass():
    # the token-by-token path and the chunked path give the same outputs (up to rounding)
    import torch
    import log_linear_attention_chunked_amd as lla
    x = generate(custom(2, 2, 320, 64, 64, dtype="f32"), seed=12)
    got, _, _ = run_decode(x)
    d = {k: v.cuda() for k, v in x.items()}
    fwd = lla.forward(d["q"], d["k"], d["v"], d["log_a"], d["lam"], chunk=64, sweep=2)
    torch.cuda.synchronize()
    assert rel_l2(got, fwd.cpu().numpy().astype(np.float64)) <= 1e-5


PREFILL_CASES = [
    # B, H, prompt T, decoded tokens, dk, dv, dtype
    (2, 3, 300, 40, 64, 64, "bf16"),
    (1, 2, 1000, 33, 16, 32, "f32"),
    (1, 2, 1, 10, 64, 64, "f32"),
    (1, 2, 64, 65, 32, 32, "f32"),
    (1, 1, 4095, 20, 128, 128, "bf16"),
    (1, 2, 2048, 12, 64, 16, "bf16"),
]


@pytest.mark.parametrize("B,H,T,K,dk,dv,dtype,mode", [c + (None,) for c in PREFILL_CASES] + [
    (1, 2, 1000, 30, 64, 64, "bf16", "strongdecay"),
    (1, 2, 777, 20, 32, 16, "f32", "strongdecay"),
])
def test_prefill_then_decode(B, H, T, K, dk, dv, dtype, mode):
    # the cache filled from a prompt of T tokens in one call, then K decoding steps: their
    # outputs against the definition over the whole sequence
    import torch
    import log_linear_attention_chunked_amd as lla
    w = custom(B, H, T + K, dk, dv, dtype)
    x = generate(w, seed=T + K, log_a_mode=mode)
    print(f"[prefill] B={B} H={H} T={T} K={K} dk={dk} dv={dv} {dtype} {mode}", flush=True)
    d = {k: v.cuda() for k, v in x.items()}
    Lc = x["lam"].shape[-1]
    state, log_scale = lla.new_decode_cache(B, H, dk, dv, Lc)
    state.fill_(float("nan"))
    log_scale.fill_(float("nan"))
    lla.decode_prefill(d["k"][:, :, :T].contiguous(), d["v"][:, :, :T].contiguous(),
                       d["log_a"][:, :, :T].contiguous(), state, log_scale)
    outs = []
    for t in range(T, T + K):
        outs.append(lla.decode_step(d["q"][:, :, t].contiguous(), d["k"][:, :, t].contiguous(),
                                    d["v"][:, :, t].contiguous(), d["log_a"][:, :, t].contiguous(),
                                    d["lam"][:, :, t].contiguous(), state, log_scale, t))
    torch.cuda.synchronize()
    got = torch.stack(outs, dim=2).double().cpu().numpy()
    rows = list(range(T, T + K))
    want = np.stack([np.stack([O.bruteforce_rows(**x, b=b, h=h, rows=rows) for h in range(H)])
                     for b in range(B)])
    assert np.all(np.isfinite(got))
    assert rel_l2(got, want) <= tol_for(dtype), rel_l2(got, want)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_per_sequence_positions(dtype):
    # three sequences decoded together at their own positions: sequence b starts at global step
    # start[b] (skipped before that: negative position), so at step s it is at s - start[b];
    # each sequence's outputs against the definition on that sequence alone, and the skipped
    # steps leave its out rows and cache untouched
    import torch
    import log_linear_attention_chunked_amd as lla
    B, H, dk, dv = 3, 2, 32, 16
    start = [0, 37, 100]
    steps = 160
    x = generate(custom(B, H, steps, dk, dv, dtype=dtype), seed=23)
    d = {k: v.cuda() for k, v in x.items()}
    Lc = x["lam"].shape[-1]
    state, log_scale = lla.new_decode_cache(B, H, dk, dv, Lc)
    state.fill_(float("nan"))
    log_scale.fill_(float("nan"))
    got = torch.full((B, H, steps, dv), 7.0, dtype=d["q"].dtype, device="cuda")
    for s in range(steps):
        pos = [s - st for st in start]
        tq = torch.tensor(pos, dtype=torch.int64, device="cuda")
        # sequence b at position p reads token p of its own stream
        idx = [max(p, 0) for p in pos]
        sel = lambda t: torch.stack([t[b, :, idx[b]] for b in range(B)]).contiguous()
        out = torch.full((B, H, dv), 7.0, dtype=d["q"].dtype, device="cuda")
        lla.decode_step(sel(d["q"]), sel(d["k"]), sel(d["v"]), sel(d["log_a"]), sel(d["lam"]),
                        state, log_scale, max(pos), out, t_seq=tq)
        for b in range(B):
            if pos[b] >= 0:
                got[b, :, pos[b]] = out[b]
            else:
                assert torch.all(out[b] == 7.0)      # a skipped sequence's out rows untouched
    torch.cuda.synchronize()
    got = got.double().cpu().numpy()
    for b in range(B):
        n = steps - start[b]
        xb = {k_: v_[b:b + 1, :, :n] for k_, v_ in x.items()}
        want = O.bruteforce(xb["q"], xb["k"], xb["v"], xb["log_a"], xb["lam"][..., :O.num_levels(n)])
        err = rel_l2(got[b:b + 1, :, :n], want)
        print(f"decode per-sequence positions {dtype} seq {b} ({n} tokens): rel_l2={err:.3e}", flush=True)
        assert np.all(np.isfinite(got[b, :, :n]))
        assert err <= tol_for(dtype), (b, err)


def test_decode_position_past_the_declared_maximum_gives_nan():
    import torch
    import log_linear_attention_chunked_amd as lla
    B, H, dk, dv = 2, 1, 16, 16
    x = generate(custom(B, H, 8, dk, dv, dtype="f32"), seed=2)
    d = {k: v[:, :, 5].contiguous().cuda() for k, v in x.items()}
    state, log_scale = lla.new_decode_cache(B, H, dk, dv, 5)
    state.zero_()
    log_scale.zero_()
    before = state.clone()
    tq = torch.tensor([5, 9], dtype=torch.int64, device="cuda")       # the second is past t = 5
    lam = torch.rand((B, H, 5), dtype=torch.float32, device="cuda")
    out = lla.decode_step(d["q"], d["k"], d["v"], d["log_a"], lam, state, log_scale, 5, t_seq=tq)
    torch.cuda.synchronize()
    assert torch.all(torch.isnan(out[1])) and torch.all(torch.isfinite(out[0]))
    assert torch.equal(state[1], before[1])
