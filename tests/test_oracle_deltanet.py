"""Pins of the log-linear Gated DeltaNet oracle (CPU only).

Each pin checks the oracle against something other than itself: hand-derived values
(tests/golden/gdn_worked_examples.json), the textbook single-state Gated DeltaNet recurrence and
the closed form of its parallel (UT-transform) solution when every level weight is equal, the
independent level-state recurrent form, the reduction to log-linear Mamba-2 when the keys are
orthogonal, one-hot level weights against the Fenwick bucket written out, linearity, causality,
and planted mistakes that must each fail at least one of these.
"""

import json
import os

import numpy as np
import pytest
from scipy.linalg import solve_triangular

import oracle.deltanet as D
import oracle.loglinear as O

HERE = os.path.dirname(os.path.abspath(__file__))


def rand_inputs(T, dk, dv, seed, decay=True, l2=True, L=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 1, T, dk)) / np.sqrt(dk)
    k = rng.standard_normal((1, 1, T, dk))
    k = k / np.linalg.norm(k, axis=-1, keepdims=True) if l2 else k / np.sqrt(dk)
    v = rng.standard_normal((1, 1, T, dv))
    log_a = -rng.uniform(0.0, 0.3, (1, 1, T)) if decay else np.zeros((1, 1, T))
    beta = 1 / (1 + np.exp(-rng.standard_normal((1, 1, T))))
    L = L or O.num_levels(T)
    lam = np.log1p(np.exp(rng.standard_normal((1, 1, T, L))))
    return q, k, v, log_a, beta, lam


def rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# ---- hand-derived values ----------------------------------------------------------------------

def _golden():
    return json.load(open(os.path.join(HERE, "golden", "gdn_worked_examples.json")))["examples"]


@pytest.mark.parametrize("idx", range(3))
def test_worked_examples(idx):
    e = _golden()[idx]
    f = lambda n: np.array(e[n], dtype=float)[None, None]
    for fn in (D.gdn_bruteforce, D.gdn_recurrent):
        o = fn(f("q"), f("k"), f("v"), f("log_a"), f("beta"), f("lam"))[0, 0]
        if "out" in e:
            np.testing.assert_allclose(o, np.array(e["out"]), atol=1e-12)
        else:
            np.testing.assert_allclose(o[2], np.array(e["out_row2"]), atol=1e-12)


# ---- equal lambda: Gated DeltaNet itself -------------------------------------------------------

def textbook_gdn(q, k, v, log_a, beta):
    """S_t = a_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T, o_t = S_t^T q_t (one head)."""
    T, dk = q.shape
    S = np.zeros((dk, v.shape[1]))
    out = np.zeros((T, v.shape[1]))
    for t in range(T):
        S = np.exp(log_a[t]) * (np.eye(dk) - beta[t] * np.outer(k[t], k[t])) @ S + beta[t] * np.outer(k[t], v[t])
        out[t] = S.T @ q[t]
    return out


def ut_closed_form(q, k, v, log_a, beta):
    """The parallel solution of the same recurrence: pseudo-values U solve
    (I + strict_lower(diag(beta) (K K^T * Gam))) U = diag(beta) V, then O = ((Q K^T * Gam) on s <= t) U,
    Gam[t,s] = exp(A_t - A_s) (a library triangular solve)."""
    A = np.cumsum(log_a)
    Gam = np.exp(np.minimum(A[:, None] - A[None, :], 0.0))
    Tm = np.eye(len(A)) + np.tril(beta[:, None] * (k @ k.T) * Gam, -1)
    U = solve_triangular(Tm, beta[:, None] * v, lower=True, unit_diagonal=True)
    return np.tril((q @ k.T) * Gam) @ U


@pytest.mark.parametrize("T,dk,dv,seed", [(1, 4, 4, 0), (7, 4, 3, 1), (33, 8, 5, 2), (64, 16, 16, 3), (70, 6, 9, 4)])
def test_equal_lambda_is_gated_deltanet(T, dk, dv, seed):
    q, k, v, log_a, beta, lam = rand_inputs(T, dk, dv, seed)
    c = lam[..., :1]
    lam_eq = np.broadcast_to(c, lam.shape).copy()
    got = D.gdn_bruteforce(q, k, v, log_a, beta, lam_eq)[0, 0]
    ref = textbook_gdn(q[0, 0], k[0, 0], v[0, 0], log_a[0, 0], beta[0, 0]) * c[0, 0]
    assert rel(got, ref) <= 1e-12
    ref_ut = ut_closed_form(q[0, 0], k[0, 0], v[0, 0], log_a[0, 0], beta[0, 0]) * c[0, 0]
    assert rel(got, ref_ut) <= 1e-10


# ---- the two oracle forms agree -----------------------------------------------------------------

@pytest.mark.parametrize("T,dk,dv,seed,decay,l2", [
    (1, 3, 2, 0, True, True), (2, 4, 4, 1, True, True), (5, 4, 6, 2, False, True),
    (8, 8, 8, 3, True, False), (13, 5, 3, 4, True, True), (16, 16, 8, 5, False, False),
    (33, 8, 8, 6, True, True), (47, 12, 7, 7, True, True), (70, 16, 16, 8, True, True),
])
def test_bruteforce_equals_level_state_recurrence(T, dk, dv, seed, decay, l2):
    x = rand_inputs(T, dk, dv, seed, decay=decay, l2=l2)
    assert rel(D.gdn_bruteforce(*x), D.gdn_recurrent(*x)) <= 1e-12


# ---- special cases ---------------------------------------------------------------------------

def test_zero_beta_gives_zero():
    q, k, v, log_a, beta, lam = rand_inputs(40, 8, 8, 9)
    assert np.all(D.gdn_bruteforce(q, k, v, log_a, np.zeros_like(beta), lam) == 0.0)


@pytest.mark.parametrize("T,seed", [(5, 0), (16, 1), (32, 2)])
def test_orthogonal_keys_reduce_to_loglinear_mamba2(T, seed):
    # orthonormal keys: A_r k_s = a_r k_s for r != s, so G[t,s] = beta_s exp(A_t - A_s) q_t.k_s and
    # the operator is log-linear Mamba-2 on (q, k, beta v)
    rng = np.random.default_rng(seed)
    dk, dv = 32, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:T][None, None]
    q, _, v, log_a, beta, lam = rand_inputs(T, dk, dv, seed + 10)
    got = D.gdn_bruteforce(q, k, v, log_a, beta, lam)
    want = O.bruteforce(q, k, beta[..., None] * v, log_a, lam)
    assert rel(got, want) <= 1e-12


def _bucket(t, lev):
    """Positions s <= t with bit_length(t XOR s) = lev, from the Fenwick (BIT) decomposition:
    level 0 is t itself; level lev >= 1 is the aligned block of 2^(lev-1) positions starting at
    (t >> lev) << lev, present only when bit lev-1 of t is set."""
    if lev == 0:
        return [t]
    if not (t >> (lev - 1)) & 1:
        return []
    start = (t >> lev) << lev
    return list(range(start, start + (1 << (lev - 1))))


@pytest.mark.parametrize("lev", [0, 1, 2, 3, 4, 5])
def test_onehot_lambda_is_one_bucket(lev):
    T = 40
    q, k, v, log_a, beta, lam = rand_inputs(T, 8, 5, 20 + lev)
    oh = np.zeros_like(lam)
    oh[..., lev] = 1.0
    got = D.gdn_bruteforce(q, k, v, log_a, beta, oh)[0, 0]
    G = D.gdn_attention(q[0, 0], k[0, 0], log_a[0, 0], beta[0, 0])
    want = np.zeros_like(got)
    for t in range(T):
        for s in _bucket(t, lev):
            want[t] += G[t, s] * v[0, 0, s]
    assert rel(got, want) <= 1e-12 or (np.all(want == 0) and np.all(got == 0))


def test_linear_in_lambda_and_causal():
    T = 37
    q, k, v, log_a, beta, lam = rand_inputs(T, 6, 4, 31)
    L = lam.shape[-1]
    total = sum(D.gdn_bruteforce(q, k, v, log_a, beta, np.eye(L)[lev][None, None, None].repeat(T, 2))
                for lev in range(L))
    ones = D.gdn_bruteforce(q, k, v, log_a, beta, np.ones_like(lam))
    assert rel(total, ones) <= 1e-12
    t0 = 20
    y = [a.copy() for a in (q, k, v, log_a, beta, lam)]
    rng = np.random.default_rng(5)
    for a in y:
        a[0, 0, t0:] = rng.standard_normal(a[0, 0, t0:].shape)
    y[3] = -np.abs(y[3])
    a0 = D.gdn_bruteforce(q, k, v, log_a, beta, lam)
    a1 = D.gdn_bruteforce(*y)
    np.testing.assert_array_equal(a0[0, 0, :t0], a1[0, 0, :t0])


# ---- planted mistakes: each must fail a pin ------------------------------------------------------

def _attention_variant(q, k, log_a, beta, mistake):
    q, k, log_a, beta = (np.asarray(x, dtype=float) for x in (q, k, log_a, beta))
    T, dk = q.shape
    G = np.zeros((T, T))
    Wm = np.zeros((dk, T))
    for t in range(T):
        a = 1.0 if mistake == "no_gate" else np.exp(log_a[t])
        bt = beta[t]
        Wm[:, t] = bt * k[t] if mistake != "beta_on_target" else k[t]
        upto = t + 1 if mistake == "own_transition" else t
        if t > 0 or mistake == "own_transition":
            cols = Wm[:, :upto]
            cols -= bt * np.outer(k[t], k[t] @ cols)
            cols *= a
        G[t, : t + 1] = q[t] @ Wm[:, : t + 1] * (bt if mistake == "beta_on_target" else 1.0)
    return G


def _bruteforce_variant(x, mistake):
    q, k, v, log_a, beta, lam = (np.asarray(a, dtype=float) for a in x)
    T = q.shape[2]
    lv = O.level_matrix(T)
    if mistake == "mask_on_qk_only":
        # the other reading: the hierarchical mask on (Q K^T * Gam) only, pseudo-values unmasked
        qh, kh, vh = q[0, 0], k[0, 0], v[0, 0]
        A = np.cumsum(log_a[0, 0])
        Gam = np.exp(np.minimum(A[:, None] - A[None, :], 0.0))
        Tm = np.eye(T) + np.tril(beta[0, 0][:, None] * (kh @ kh.T) * Gam, -1)
        U = solve_triangular(Tm, beta[0, 0][:, None] * vh, lower=True, unit_diagonal=True)
        Lam = np.where(lv >= 0, lam[0, 0][np.arange(T)[:, None], np.maximum(lv, 0)], 0.0)
        return ((np.tril((qh @ kh.T) * Gam) * Lam) @ U)[None, None]
    G = _attention_variant(q[0, 0], k[0, 0], log_a[0, 0], beta[0, 0], mistake)
    Lam = np.where(lv >= 0, lam[0, 0][np.arange(T)[:, None], np.maximum(lv, 0)], 0.0)
    return ((G * Lam) @ v[0, 0])[None, None]


@pytest.mark.parametrize("mistake", ["no_gate", "own_transition", "beta_on_target", "mask_on_qk_only"])
def test_planted_mistakes_fail_a_pin(mistake):
    failed = []
    for e in _golden():
        f = lambda n: np.array(e[n], dtype=float)[None, None]
        x = (f("q"), f("k"), f("v"), f("log_a"), f("beta"), f("lam"))
        o = _bruteforce_variant(x, mistake)[0, 0]
        want = np.array(e["out"]) if "out" in e else None
        if want is not None and not np.allclose(o, want, atol=1e-9):
            failed.append(e["name"])
        if want is None and not np.allclose(o[2], np.array(e["out_row2"]), atol=1e-9):
            failed.append(e["name"])
    x = rand_inputs(24, 6, 4, 77)
    if rel(_bruteforce_variant(x, mistake), D.gdn_recurrent(*x)) > 1e-6:
        failed.append("level-state recurrence")
    assert failed, f"planted mistake {mistake} passed every pin"
    # and the unplanted copy passes them all
    assert rel(_bruteforce_variant(x, None), D.gdn_recurrent(*x)) <= 1e-12
