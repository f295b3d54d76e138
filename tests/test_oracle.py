"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

None of these checks re-types the oracle's own formula: each compares it with
an independent construction (the textbook Fenwick prefix decomposition, plain
causal linear attention, the Mamba-2 state recurrence, hand-worked examples,
the O(log T)-state recurrent form). ``test_planted_mistakes`` then plants
plausible errors in the oracle's helpers and checks that some pin catches each.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle.loglinear as O
from lla_synth import WORKLOADS, custom, generate

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# independent constructions used as pins
# ---------------------------------------------------------------------------

def fenwick_prefix_blocks(t):
    """Textbook binary-indexed-tree query for the prefix of length t (positions
    0..t-1): i = t; while i: block (i - lowbit(i), i]; i -= lowbit(i).
    Returned as 0-based half-open [start, end) ranges, most recent first."""
    out = []
    i = t
    while i > 0:
        low = i & -i
        out.append((i - low, i))
        i -= low
    return out


def oracle_level_row(t):
    """Levels l(t, s) for s = 0..t, from the oracle's level function."""
    return [O.level(t, s) for s in range(t + 1)]


def fenwick_buckets_from_oracle(t):
    lv = oracle_level_row(t)
    buckets = {}
    for s, l in enumerate(lv):
        buckets.setdefault(int(l), []).append(s)
    return buckets


def rand_case(rng, B, H, T, dk, dv, decay=True, L=None):
    L = L or O.num_levels(T)
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv))
    log_a = -rng.uniform(0.0, 0.5, (B, H, T)) if decay else np.zeros((B, H, T))
    lam = np.log1p(np.exp(rng.standard_normal((B, H, T, L))))
    return q, k, v, log_a, lam


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def causal_linear_attention(q, k, v):
    """tril(Q K^T) V with a library matmul (the plain linear attention output)."""
    out = np.zeros(q.shape[:3] + (v.shape[3],))
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            out[b, h] = np.tril(q[b, h] @ k[b, h].T) @ v[b, h]
    return out


def mamba2_ssd(q, k, v, log_a):
    """Gated state recurrence S_t = a_t S_{t-1} + k_t v_t^T, o_t = S_t^T q_t."""
    B, H, T, dk = q.shape
    dv = v.shape[3]
    out = np.zeros((B, H, T, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv))
            for t in range(T):
                S = math.exp(log_a[b, h, t]) * S + np.outer(k[b, h, t], v[b, h, t])
                out[b, h, t] = S.T @ q[b, h, t]
    return out


def onehot_reference(q, k, v, log_a, lev):
    """Only the bucket of level `lev`: {t} for lev 0, else the aligned block of
    2^(lev-1) positions [(t >> lev) << lev, +2^(lev-1)) when bit lev-1 of t is
    set (written from the textbook prefix decomposition, not from l(t, s))."""
    B, H, T, dk = q.shape
    out = np.zeros((B, H, T, v.shape[3]))
    for b in range(B):
        for h in range(H):
            for t in range(T):
                if lev == 0:
                    blk = [t]
                else:
                    size = 1 << (lev - 1)
                    blk = []
                    for (s0, s1) in fenwick_prefix_blocks(t):
                        if s1 - s0 == size:
                            blk = list(range(s0, s1))
                acc = np.zeros(v.shape[3])
                for s in blk:
                    d = math.exp(sum(log_a[b, h, s + 1: t + 1]))
                    acc += d * float(q[b, h, t] @ k[b, h, s]) * v[b, h, s]
                out[b, h, t] = acc
    return out


# ---------------------------------------------------------------------------
# pins on the level function
# ---------------------------------------------------------------------------

def load_levels_T8():
    rows = []
    with open(os.path.join(GOLDEN, "levels_T8.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    return rows


def test_level_matrix_T8_golden():
    want = load_levels_T8()
    got = O.level_matrix(8)
    for t, row in enumerate(want):
        assert list(got[t, : t + 1]) == row
        assert all(x == -1 for x in got[t, t + 1:])


@pytest.mark.parametrize("t", list(range(0, 300)) + [1023, 1024, 1025, 4095, 65535])
def test_levels_are_the_fenwick_prefix_decomposition(t):
    buckets = fenwick_buckets_from_oracle(t)
    assert buckets.pop(0) == [t]
    blocks = fenwick_prefix_blocks(t)
    # one bucket per set bit of t, plus the token itself
    assert len(buckets) == len(blocks) == bin(t).count("1")
    for (s0, s1) in blocks:
        size = s1 - s0
        lev = size.bit_length()          # size 2^(lev-1)
        assert buckets[lev] == list(range(s0, s1))
    # sizes sum to t + 1; recent positions sit in finer buckets
    assert sum(len(x) for x in buckets.values()) + 1 == t + 1
    lv = oracle_level_row(t)
    assert all(lv[i] >= lv[i + 1] for i in range(t))
    if t < 300:
        assert list(O.level_matrix(t + 1)[t, : t + 1]) == lv


def test_num_levels_matches_workloads():
    # level counts stated with the five workloads (T=256..65536)
    stated = {256: 9, 2048: 12, 8192: 14, 32768: 16, 65536: 17}
    for T, L in stated.items():
        assert O.num_levels(T) == L
    for w in WORKLOADS.values():
        assert O.num_levels(w.T) == w.L == stated[w.T]
    assert O.num_levels(1) == 1 and O.num_levels(2) == 2 and O.num_levels(3) == 3


def test_bit_length_integer_ops():
    xs = np.array([0, 1, 2, 3, 4, 7, 8, 255, 256, 2**31 - 1, 2**40])
    assert list(O.bit_length(xs)) == [int(x).bit_length() for x in xs]


# ---------------------------------------------------------------------------
# pins on the operator
# ---------------------------------------------------------------------------

def load_examples():
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("ex", load_examples(), ids=lambda e: e["name"])
def test_worked_examples(ex):
    q = np.array(ex["q"])[None, None]
    k = np.array(ex["k"])[None, None]
    v = np.array(ex["v"])[None, None]
    la = np.array(ex["log_a"])[None, None]
    lam = np.array(ex["lam"], dtype=np.float64)[None, None]
    want = np.array(ex["out"])
    np.testing.assert_allclose(O.bruteforce(q, k, v, la, lam)[0, 0], want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.recurrent(q, k, v, la, lam)[0, 0], want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("T", [1, 2, 3, 5, 8, 13, 16, 33, 64, 70])
@pytest.mark.parametrize("decay", [False, True])
def test_bruteforce_matches_recurrent(T, decay):
    rng = np.random.default_rng(1000 + T)
    case = rand_case(rng, 2, 1, T, 3, 5, decay=decay)
    a = O.bruteforce(*case, row_block=7)
    b = O.recurrent(*case)
    assert rel(a, b) <= 1e-12


def test_equal_lambda_no_decay_is_linear_attention():
    rng = np.random.default_rng(7)
    q, k, v, _, lam = rand_case(rng, 2, 2, 37, 4, 3)
    la = np.zeros(q.shape[:3])
    lam = np.ones_like(lam)
    assert rel(O.bruteforce(q, k, v, la, lam), causal_linear_attention(q, k, v)) <= 1e-12


def test_equal_lambda_is_scaled_mamba2():
    rng = np.random.default_rng(8)
    q, k, v, la, lam = rand_case(rng, 1, 2, 45, 3, 4)
    c = lam[..., :1]
    lam = np.broadcast_to(c, lam.shape).copy()
    want = c * mamba2_ssd(q, k, v, la)
    assert rel(O.bruteforce(q, k, v, la, lam), want) <= 1e-12
    assert rel(O.recurrent(q, k, v, la, lam), want) <= 1e-12


@pytest.mark.parametrize("lev", list(range(0, 7)))
def test_onehot_lambda_isolates_one_bucket(lev):
    rng = np.random.default_rng(9 + lev)
    T = 40
    q, k, v, la, lam = rand_case(rng, 1, 1, T, 3, 2)
    lam = np.zeros_like(lam)
    lam[..., lev] = 1.0
    want = onehot_reference(q, k, v, la, lev)
    got = O.bruteforce(q, k, v, la, lam)
    assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))
    if lev > 0:
        # bucket of level lev exists iff bit lev-1 of t is set
        for t in range(T):
            if not (t >> (lev - 1)) & 1:
                assert np.all(got[0, 0, t] == 0.0)


def test_linearity_in_lambda_and_v():
    rng = np.random.default_rng(11)
    q, k, v, la, lam = rand_case(rng, 1, 2, 29, 3, 3)
    L = lam.shape[-1]
    total = np.zeros(q.shape[:3] + (3,))
    for lev in range(L):
        oh = np.zeros_like(lam)
        oh[..., lev] = lam[..., lev]
        total += O.bruteforce(q, k, v, la, oh)
    assert rel(total, O.bruteforce(q, k, v, la, lam)) <= 1e-12
    v2 = rng.standard_normal(v.shape)
    lhs = O.bruteforce(q, k, 2.0 * v - 3.0 * v2, la, lam)
    rhs = 2.0 * O.bruteforce(q, k, v, la, lam) - 3.0 * O.bruteforce(q, k, v2, la, lam)
    assert rel(lhs, rhs) <= 1e-12


def test_zero_lambda_and_single_token():
    rng = np.random.default_rng(12)
    q, k, v, la, lam = rand_case(rng, 1, 1, 9, 2, 2)
    assert np.all(O.bruteforce(q, k, v, la, np.zeros_like(lam)) == 0.0)
    q1, k1, v1, la1, lam1 = rand_case(rng, 1, 1, 1, 3, 2)
    want = lam1[0, 0, 0, 0] * float(q1[0, 0, 0] @ k1[0, 0, 0]) * v1[0, 0, 0]
    np.testing.assert_allclose(O.bruteforce(q1, k1, v1, la1, lam1)[0, 0, 0], want, rtol=1e-14)
    np.testing.assert_allclose(O.recurrent(q1, k1, v1, la1, lam1)[0, 0, 0], want, rtol=1e-14)


def test_causality():
    rng = np.random.default_rng(13)
    q, k, v, la, lam = rand_case(rng, 1, 1, 50, 3, 3)
    base = O.bruteforce(q, k, v, la, lam)
    t0 = 21
    q2, k2, v2, la2, lam2 = (x.copy() for x in (q, k, v, la, lam))
    for x in (q2, k2, v2, la2, lam2):
        x[:, :, t0:] = rng.standard_normal(x[:, :, t0:].shape)
    pert = O.bruteforce(q2, k2, v2, la2, lam2)
    assert np.array_equal(pert[:, :, :t0], base[:, :, :t0])
    assert not np.allclose(pert[:, :, t0:], base[:, :, t0:])


def test_rows_match_full():
    rng = np.random.default_rng(14)
    q, k, v, la, lam = rand_case(rng, 2, 2, 100, 4, 3)
    full = O.bruteforce(q, k, v, la, lam, row_block=32)
    rows = [0, 1, 31, 32, 63, 64, 99]
    for b in range(2):
        for h in range(2):
            np.testing.assert_allclose(O.bruteforce_rows(q, k, v, la, lam, b, h, rows),
                                       full[b, h, rows], rtol=1e-13, atol=1e-13)


def test_inputs_from_generator_roundtrip_exactly():
    w = custom(1, 2, 48, 16, 8, dtype="bf16")
    x = generate(w, seed=3)
    # fp64 copies of bf16 inputs are exact (no rounding in the oracle's reads)
    qf = O.as_f64(x["q"])
    assert np.array_equal(qf.astype(np.float32), x["q"].float().numpy())
    a = O.bruteforce(x["q"], x["k"], x["v"], x["log_a"], x["lam"])
    b = O.recurrent(x["q"], x["k"], x["v"], x["log_a"], x["lam"])
    assert rel(a, b) <= 1e-12


# ---------------------------------------------------------------------------
# planted mistakes: every plausible slip in the oracle must fail some pin
# ---------------------------------------------------------------------------

def _pins_pass():
    """Run the oracle-side pins that do not depend on the recurrent form."""
    try:
        want = load_levels_T8()
        got = O.level_matrix(8)
        for t, row in enumerate(want):
            if list(got[t, : t + 1]) != row:
                return False
        for ex in load_examples():
            q = np.array(ex["q"])[None, None]
            k = np.array(ex["k"])[None, None]
            v = np.array(ex["v"])[None, None]
            la = np.array(ex["log_a"])[None, None]
            lam = np.array(ex["lam"], dtype=np.float64)[None, None]
            if not np.allclose(O.bruteforce(q, k, v, la, lam)[0, 0], np.array(ex["out"]), rtol=1e-12):
                return False
        rng = np.random.default_rng(99)
        q, k, v, la, lam = rand_case(rng, 1, 1, 24, 3, 2)
        c = lam[..., :1]
        lam_eq = np.broadcast_to(c, lam.shape).copy()
        if rel(O.bruteforce(q, k, v, la, lam_eq), c * mamba2_ssd(q, k, v, la)) > 1e-12:
            return False
        if rel(O.bruteforce(q, k, v, np.zeros_like(la), np.ones_like(lam)),
               causal_linear_attention(q, k, v)) > 1e-12:
            return False
        for lev in range(4):
            oh = np.zeros_like(lam)
            oh[..., lev] = 1.0
            ref = onehot_reference(q, k, v, la, lev)
            if np.max(np.abs(O.bruteforce(q, k, v, la, oh) - ref)) > 1e-12 * max(1, np.max(np.abs(ref))):
                return False
        return True
    except (IndexError, ValueError):
        return False


def test_pins_pass_on_the_real_oracle():
    assert _pins_pass()


MISTAKES = {
    "level_off_by_one": ("_levels", lambda orig: (lambda ts, ss: O.bit_length(ts[:, None] ^ ss[None, :]) + 1)),
    "one_based_positions": ("_levels", lambda orig: (lambda ts, ss: O.bit_length((ts[:, None] + 1) ^ (ss[None, :] + 1)))),
    "level_from_distance": ("_levels", lambda orig: (lambda ts, ss: O.bit_length(np.abs(ts[:, None] - ss[None, :])))),
    "decay_includes_a_s": ("_pair_log_decay", lambda orig: (lambda A, ts, ss: A[ts][:, None] - A[ss][None, :] + np.diff(np.concatenate([[0.0], A]))[ss][None, :])),
    "decay_wrong_sign": ("_pair_log_decay", lambda orig: (lambda A, ts, ss: -(A[ts][:, None] - A[ss][None, :]))),
    "exclusive_prefix": ("_prefix_log_decay", lambda orig: (lambda la: np.concatenate([[0.0], np.cumsum(la)[:-1]]))),
    "strict_causal": ("_causal", lambda orig: (lambda ts, ss: ss[None, :] < ts[:, None])),
    "query_key_swapped": ("_scores", lambda orig: (lambda q, k, ts, ss: k[ts] @ q[ss].T)),
}


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_planted_mistakes(name, monkeypatch):
    attr, make = MISTAKES[name]
    monkeypatch.setattr(O, attr, make(getattr(O, attr)))
    assert not _pins_pass(), f"planted mistake {name!r} passed every pin"


def test_planted_mistake_in_recurrent_carry(monkeypatch):
    # merging one level too few into the carry must break agreement with brute force
    rng = np.random.default_rng(5)
    case = rand_case(rng, 1, 1, 20, 2, 2)
    good = O.recurrent(*case)
    monkeypatch.setattr(O, "_ctz", lambda t: max(0, ((t & -t).bit_length() - 1) - 1))
    bad = O.recurrent(*case)
    assert rel(good, O.bruteforce(*case)) <= 1e-12
    assert rel(bad, O.bruteforce(*case)) > 1e-6


def test_planted_mistake_in_recurrent_step(monkeypatch):
    # a_t also applied to the new level-0 state k_t v_t^T (the decay of k_s must start after s)
    rng = np.random.default_rng(6)
    case = rand_case(rng, 1, 1, 24, 3, 2)
    good = O.recurrent(*case)

    def wrong_step(S, q_t, k_t, v_t, log_a_t, lam_t, t):
        if t > 0:
            c = O._ctz(t)
            merged = S[: c + 1].sum(axis=0)
            S[1: c + 1] = 0.0
            S[c + 1] = merged
        S[0] = np.outer(k_t, v_t)
        if t > 0:
            S *= np.exp(log_a_t)
        return np.einsum("l,lkv,k->v", np.asarray(lam_t, dtype=np.float64), S[:len(lam_t)], q_t)

    monkeypatch.setattr(O, "recurrent_step", wrong_step)
    bad = O.recurrent(*case)
    assert rel(good, O.bruteforce(*case)) <= 1e-12
    assert rel(bad, O.bruteforce(*case)) > 1e-6


def test_recurrent_step_state_blocks():
    # after step t the live states are exactly: level 0 = k_t v_t^T, and for each set bit j of t
    # the decayed sum of k_s v_s^T over the aligned block of 2^j positions below the lower bits
    rng = np.random.default_rng(7)
    T, dk, dv = 45, 3, 2
    q, k, v, la, lam = (np.asarray(x)[0, 0] for x in rand_case(rng, 1, 1, T, dk, dv))
    L = O.num_levels(T)
    S = np.zeros((L + 1, dk, dv))
    A = np.cumsum(la)
    for t in range(T):
        O.recurrent_step(S, q[t], k[t], v[t], la[t], lam[t, :L], t)
    t = T - 1
    want = np.zeros_like(S)
    want[0] = np.outer(k[t], v[t])
    hi = t
    for j in range(t.bit_length()):
        if (t >> j) & 1:
            lo = hi - (1 << j)
            for s in range(lo, hi):
                want[j + 1] += np.exp(A[t] - A[s]) * np.outer(k[s], v[s])
            hi = lo
    np.testing.assert_allclose(S, want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# the backward pass: gradients of sum(do * o)
# ---------------------------------------------------------------------------

def _tiny_grad_case(seed, B=1, H=1, T=11, dk=3, dv=2):
    rng = np.random.default_rng(seed)
    L = O.num_levels(T)
    return dict(q=rng.normal(size=(B, H, T, dk)), k=rng.normal(size=(B, H, T, dk)),
                v=rng.normal(size=(B, H, T, dv)), log_a=-rng.uniform(0.05, 0.6, size=(B, H, T)),
                lam=rng.uniform(0.2, 1.5, size=(B, H, T, L))), rng.normal(size=(B, H, T, dv))


def test_grad_matches_central_differences():
    # every input element: d/dx sum(do * bruteforce(x)) by central differences of the
    # forward definition, which is pinned on its own above
    x, do = _tiny_grad_case(1)
    g = O.bruteforce_grad(**x, do=do)
    loss = lambda xx: float(np.sum(do * O.bruteforce(**xx)))
    eps = 1e-6
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("log_a", "dlog_a"), ("lam", "dlam")):
        fd = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            xp = {n: a.copy() for n, a in x.items()}
            xm = {n: a.copy() for n, a in x.items()}
            xp[name][idx] += eps
            xm[name][idx] -= eps
            fd[idx] = (loss(xp) - loss(xm)) / (2 * eps)
        err = np.abs(fd - g[key]).max() / max(np.abs(fd).max(), 1e-30)
        assert err < 1e-7, (name, err)


def test_grad_matches_autograd_of_a_dense_formula():
    # CPU float64 autograd through the definition built pair by pair (a Python loop over
    # (t, s), no helper of the oracle), at a size with several levels and two heads
    import torch
    x, do = _tiny_grad_case(2, B=1, H=2, T=37, dk=4, dv=3)
    tx = {n: torch.tensor(a, dtype=torch.float64, requires_grad=True) for n, a in x.items()}
    T = x["q"].shape[2]
    A = torch.cumsum(tx["log_a"], dim=-1)
    outs = []
    for t in range(T):
        acc = 0.0
        for s in range(t + 1):
            lev = (t ^ s).bit_length()
            w = tx["lam"][..., t, lev] * torch.exp(A[..., t] - A[..., s])
            qk = (tx["q"][..., t, :] * tx["k"][..., s, :]).sum(-1)
            acc = acc + (w * qk)[..., None] * tx["v"][..., s, :]
        outs.append(acc)
    o = torch.stack(outs, dim=-2)
    (o * torch.tensor(do)).sum().backward()
    g = O.bruteforce_grad(**x, do=do)
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("log_a", "dlog_a"), ("lam", "dlam")):
        ref = tx[name].grad.numpy()
        assert np.allclose(g[key], ref, rtol=1e-10, atol=1e-12), name


def test_grad_structural_zeros():
    # log_a[0] shifts every A_t alike, so no decay depends on it: its gradient is 0;
    # lambda[t, l] for a level that t never reaches (l > 0 with bit l-1 of t clear) gets 0
    x, do = _tiny_grad_case(3, B=2, H=1, T=70, dk=5, dv=4)
    g = O.bruteforce_grad(**x, do=do)
    scale = np.abs(g["dlog_a"]).max()
    assert np.all(np.abs(g["dlog_a"][..., 0]) <= 1e-12 * scale)
    T, L = 70, x["lam"].shape[-1]
    for t in range(T):
        for lev in range(1, L):
            if not (t >> (lev - 1)) & 1:
                assert np.all(g["dlam"][:, :, t, lev] == 0.0), (t, lev)
    assert np.all(g["dlam"][..., 0] != 0.0)


def test_grad_of_plain_causal_linear_attention():
    # lambda = 1 on every level and no decay: o = causal (Q K^T) V, whose gradients are
    # the textbook ones, written here with the lower-triangular mask
    x, do = _tiny_grad_case(4, T=29, dk=3, dv=5)
    x["lam"][:] = 1.0
    x["log_a"][:] = 0.0
    g = O.bruteforce_grad(**x, do=do)
    q, k, v, d = x["q"][0, 0], x["k"][0, 0], x["v"][0, 0], do[0, 0]
    Mc = np.tril(np.ones((29, 29)))
    assert np.allclose(g["dq"][0, 0], (Mc * (d @ v.T)) @ k)
    assert np.allclose(g["dk"][0, 0], (Mc * (d @ v.T)).T @ q)
    assert np.allclose(g["dv"][0, 0], (Mc * (q @ k.T)).T @ d)


def test_grad_rows_match_dense_gradients():
    # the per-position form against the dense matrices, on rows spread over every level,
    # a dlog_a tail, and a second head
    x, do = _tiny_grad_case(5, B=2, H=2, T=70, dk=5, dv=4)
    g = O.bruteforce_grad(**x, do=do)
    rows = [0, 1, 2, 7, 8, 31, 32, 33, 63, 64, 69]
    for b, h in ((0, 0), (1, 1)):
        r = O.bruteforce_grad_rows(**x, do=do, b=b, h=h, rows=rows, tail=20)
        for key in ("dq", "dk", "dv", "dlam"):
            np.testing.assert_allclose(r[key], g[key][b, h][rows], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(r["dlog_a_tail"], g["dlog_a"][b, h][50:], rtol=1e-11, atol=1e-12)
        # dA from the dense gradients: q . dq - k . dk
        dA = np.einsum("td,td->t", x["q"][b, h], g["dq"][b, h]) - np.einsum("td,td->t", x["k"][b, h], g["dk"][b, h])
        np.testing.assert_allclose(r["dA"], dA[rows], rtol=1e-10, atol=1e-12)
