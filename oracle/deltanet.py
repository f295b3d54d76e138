"""CPU oracle (fp64) for the forward pass of log-linear Gated DeltaNet.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this module. It shares no code with the HIP library and imports
nothing from it.

What is computed. The pages apply the same lifting to Gated DeltaNet as to Mamba-2: the
model's temporal (semiseparable) mask is composed with the Fenwick hierarchical mask,
``M = M^S * M^H``, keeping the model's transition (study notes, dimensionstp.github.io,
section 3-5); every variant is written ``O = (A * M) V`` with the output a lambda-weighted sum
of per-level recurrent states, ``o_t = sum_l lambda_t^(l) q_t^T S_t^(l)`` (gist.science de
technical summary, "Kernidee"), and for Gated DeltaNet the delta rule is combined with the
hierarchical structure (same page, "Anwendung auf bestehende Modelle", item 2; gist.science zh
technical summary, section 2.4, replaces its mask by the hierarchical one). The pages print no
formula for the delta rule; the reading taken (the Gated DeltaNet recurrence, which the
textbook chapter's gated-update form generalises, with a matrix gate):

    A_r    = a_r (I - beta_r k_r k_r^T)           transition of token r (dk x dk), a_r = exp(log_a_r)
    Phi(s,t] = A_t A_{t-1} ... A_{s+1}              (identity for s = t)
    G[t,s] = beta_s q_t^T Phi(s,t] k_s             Gated DeltaNet's attention matrix (s <= t)
    o_t    = sum_{s <= t} lambda[t, l(t,s)] G[t,s] v_s,     l(t,s) = bit_length(t XOR s)

i.e. every level state is carried by the delta-rule transition, and new tokens enter level 0 as
beta_t k_t v_t^T. With every lambda equal this is exactly Gated DeltaNet,
``S_t = a_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T``, ``o_t = S_t^T q_t``.

Functions:

* ``gdn_attention``   G for one head, by carrying every source vector beta_s k_s through the
  transitions one token at a time (all sources at once, as the columns of a matrix).
* ``gdn_bruteforce``  the definition above: (G * Lambda) V per head, Lambda[t,s] = lambda[t, l(t,s)].
* ``gdn_recurrent``   the level-state form: one dk x dv state per level, merged like a carry
  when a lower level fills (as for Mamba-2), every state multiplied by A_t at each step. It
  shares no helper with ``gdn_bruteforce``.
"""

from __future__ import annotations

import numpy as np

from .loglinear import as_f64, level_matrix, num_levels

__all__ = ["gdn_attention", "gdn_bruteforce", "gdn_recurrent", "gdn_recurrent_step"]


def _check(q, k, v, log_a, beta, lam):
    B, H, T, dk = q.shape
    if k.shape != (B, H, T, dk) or v.shape[:3] != (B, H, T):
        raise ValueError("q, k, v shapes disagree")
    if log_a.shape != (B, H, T) or beta.shape != (B, H, T):
        raise ValueError("log_a and beta must be [B, H, T]")
    if lam.shape[:3] != (B, H, T) or (T > 0 and lam.shape[3] < num_levels(T)):
        raise ValueError("lambda too small")
    return B, H, T, dk, v.shape[3]


def gdn_attention(q, k, log_a, beta) -> np.ndarray:
    """G[t, s] = beta_s q_t^T A_t ... A_{s+1} k_s for s <= t (0 above the diagonal), one head.

    q, k [T, dk]; log_a, beta [T]. Column s of ``Wm`` holds the source vector beta_s k_s carried
    to the current position t: each step applies A_t = a_t (I - beta_t k_t k_t^T) to every
    earlier column, then adds the new column beta_t k_t (a token's own transition does not act
    on it); row t of G is q_t^T Wm.
    """
    q, k, log_a, beta = (as_f64(x) for x in (q, k, log_a, beta))
    T, dk = q.shape
    G = np.zeros((T, T), dtype=np.float64)
    Wm = np.zeros((dk, T), dtype=np.float64)
    for t in range(T):
        if t > 0:
            cols = Wm[:, :t]
            cols -= beta[t] * np.outer(k[t], k[t] @ cols)
            cols *= np.exp(log_a[t])
        Wm[:, t] = beta[t] * k[t]
        G[t, : t + 1] = q[t] @ Wm[:, : t + 1]
    return G


def gdn_bruteforce(q, k, v, log_a, beta, lam) -> np.ndarray:
    """The O(T^2) definition, fp64: o = (G * Lambda) V per head (see the module docstring).

    ``q, k [B,H,T,dk]``, ``v [B,H,T,dv]``, ``log_a, beta [B,H,T]``, ``lam [B,H,T,L]``;
    returns ``[B,H,T,dv]`` float64."""
    q, k, v, log_a, beta, lam = (as_f64(x) for x in (q, k, v, log_a, beta, lam))
    B, H, T, dk, dv = _check(q, k, v, log_a, beta, lam)
    out = np.zeros((B, H, T, dv), dtype=np.float64)
    t = np.arange(T)
    lv = level_matrix(T)                     # l(t, s) for s <= t, -1 above the diagonal
    causal = lv >= 0
    for b in range(B):
        for h in range(H):
            G = gdn_attention(q[b, h], k[b, h], log_a[b, h], beta[b, h])
            Lam = np.where(causal, lam[b, h][t[:, None], np.where(causal, lv, 0)], 0.0)
            out[b, h] = (G * Lam) @ v[b, h]
    return out


def _ctz(t: int) -> int:
    return (t & -t).bit_length() - 1


def gdn_recurrent_step(S: np.ndarray, q_t, k_t, v_t, log_a_t: float, beta_t: float, lam_t,
                       t: int) -> np.ndarray:
    """One step of the level-state form for one head, in place on ``S`` [Ls, dk, dv].

    For t > 0, with c = ctz(t): levels 0..c of t-1 merge into level c+1 (a carry: the lower
    drawers are full, study notes section 3-6) and levels 1..c empty; then every state is
    multiplied by the transition A_t = a_t (I - beta_t k_t k_t^T); then level 0 becomes
    beta_t k_t v_t^T and o_t = sum_l lambda[t, l] S_l^T q_t is returned.
    """
    if t > 0:
        c = _ctz(t)
        merged = S[: c + 1].sum(axis=0)
        S[1: c + 1] = 0.0
        S[c + 1] = merged
        a = np.exp(log_a_t)
        for lev in range(S.shape[0]):
            S[lev] = a * (S[lev] - beta_t * np.outer(k_t, k_t @ S[lev]))
    S[0] = beta_t * np.outer(k_t, v_t)
    n = len(lam_t)
    return np.einsum("l,lkv,k->v", np.asarray(lam_t, dtype=np.float64), S[:n], q_t)


def gdn_recurrent(q, k, v, log_a, beta, lam) -> np.ndarray:
    """The level-state (decoding) form over a whole sequence: ``gdn_recurrent_step`` for
    t = 0 .. T-1 on a fresh set of states. O(T L dk (dk + dv)) per head: an independent
    algorithm for the same operator, used to cross-check ``gdn_bruteforce``."""
    q, k, v, log_a, beta, lam = (as_f64(x) for x in (q, k, v, log_a, beta, lam))
    B, H, T, dk, dv = _check(q, k, v, log_a, beta, lam)
    out = np.zeros((B, H, T, dv), dtype=np.float64)
    if T == 0:
        return out
    L = num_levels(T)
    for b in range(B):
        for h in range(H):
            S = np.zeros((L + 1, dk, dv), dtype=np.float64)
            for t in range(T):
                out[b, h, t] = gdn_recurrent_step(S, q[b, h, t], k[b, h, t], v[b, h, t],
                                                  log_a[b, h, t], beta[b, h, t], lam[b, h, t, :L], t)
    return out
