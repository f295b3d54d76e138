"""CPU oracle for the forward pass of log-linear Mamba-2 attention (fp64).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The HIP library
and its Python binding never import, call or link anything under ``oracle/``,
and this module imports nothing from them; the only thing both sides share is
the seeded input generator in ``lla_synth`` (random draws, no method
arithmetic).

What is computed (sources are the five web pages on "Log-Linear Attention",
arXiv 2506.04761):

* The output is a level-weighted sum of per-level state read-outs,
  ``o_t = sum_l lambda_t^(l) q_t^T S_t^(l)`` with non-negative, input-dependent
  ``lambda`` (study notes, dimensionstp.github.io, sections 2-2 and 3-3;
  gist.science zh technical summary, section 2.2).
* The levels come from a Fenwick-tree (binary indexed tree) partition of the
  prefix into power-of-two buckets, fine for recent and coarse for distant
  tokens (study notes, sections 2-2 and 3-2). The level of a pair is
  ``l(t, s) = bit_length(t XOR s)`` on 0-based positions: 0 for s == t,
  otherwise floor(log2(t XOR s)) + 1.
* Parallel form ``O = (Q K^T * M) V`` with the hierarchical mask composed with
  Mamba-2's semiseparable decay mask, ``M = M^S * M^H`` (study notes, sections
  3-4 and 3-5), giving, per head,

      o_t = sum_{s <= t} lambda[t, l(t,s)] * prod_{r=s+1..t} a_r * (q_t . k_s) * v_s

  with ``a_r = exp(log_a[r])``, so the decay factor is ``exp(A_t - A_s)`` for
  the inclusive prefix sum ``A_t = sum_{r<=t} log_a[r]``.

Functions:

* ``bruteforce``        the O(T^2) definition above, row-blocked, fp64.
* ``bruteforce_rows``   the same definition for selected query rows of one head.
* ``recurrent``         the O(log T)-state recurrent form: one state per level,
  merged like a carry when a lower level fills (study notes, section 3-6; zh
  lay summary, "drawer" merging). It shares no helper with ``bruteforce``.
* ``recurrent_step``    one step of that form (the decoding step): the states
  after t-1 and token t give the states after t and o_t.
* ``bruteforce_grad_rows``  the same gradients for selected positions of one head (one row or
  column of the pair matrices at a time), for sequences too long for the dense matrices.
* ``bruteforce_grad``   the gradients of ``sum(do * o)`` with respect to q, k, v,
  log_a and lambda: the derivative of the definition above, written out on the
  dense O(T^2) matrices (the pages name the backward pass, and the lambda
  gradient in particular, as the hard part of training: study notes, sections
  3-5 and 4-5, and the discussion's point on engineering cost).

Readings taken where the pages are silent, stated at the functions that depend on
them: 0-based positions, the bucket of s == t is
level 0 and is included (the sum runs over s <= t), ``a_s`` itself is not in
the decay of k_s, no scale/normaliser/gate inside the operator.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bit_length", "level", "num_levels", "level_matrix", "as_f64",
    "bruteforce", "bruteforce_rows", "recurrent", "recurrent_step", "bruteforce_grad",
    "bruteforce_grad_rows",
]


# ----------------------------------------------------------------------------
# Levels
# ----------------------------------------------------------------------------

def bit_length(x) -> np.ndarray:
    """Elementwise bit length of non-negative integers, integer ops only."""
    y = np.array(x, dtype=np.int64, copy=True)
    if np.any(y < 0):
        raise ValueError("bit_length of a negative integer")
    out = np.zeros_like(y)
    while np.any(y):
        nz = y > 0
        out += nz
        y >>= 1
    return out


def level(t: int, s: int) -> int:
    """Fenwick level of position s seen from query position t (s <= t)."""
    return int(t ^ s).bit_length()


def num_levels(T: int) -> int:
    """Number of lambda levels for T tokens: the largest level of any pair in
    [0, T) is bit_length(T-1), so there are bit_length(T-1) + 1 of them."""
    if T < 1:
        raise ValueError("T must be >= 1")
    return int(T - 1).bit_length() + 1


def _levels(ts: np.ndarray, ss: np.ndarray) -> np.ndarray:
    """Level matrix block, rows ts (query positions), columns ss (key positions)."""
    return bit_length(ts[:, None] ^ ss[None, :])


def level_matrix(T: int) -> np.ndarray:
    """T x T matrix of levels l(t, s) for s <= t, -1 above the diagonal."""
    t = np.arange(T)
    lv = _levels(t, t)
    lv[t[:, None] < t[None, :]] = -1
    return lv


# ----------------------------------------------------------------------------
# Helpers of the parallel (masked) form
# ----------------------------------------------------------------------------

def as_f64(x) -> np.ndarray:
    """Exact float64 copy of a numpy array or a (CPU or device) torch tensor."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def _prefix_log_decay(log_a_row: np.ndarray) -> np.ndarray:
    """A_t = sum_{r <= t} log_a[r] (inclusive), so A_t - A_s = log prod_{r=s+1..t} a_r."""
    return np.cumsum(log_a_row)


def _pair_log_decay(A: np.ndarray, ts: np.ndarray, ss: np.ndarray) -> np.ndarray:
    """log of prod_{r=s+1..t} a_r for every (t, s) in the block."""
    return A[ts][:, None] - A[ss][None, :]


def _causal(ts: np.ndarray, ss: np.ndarray) -> np.ndarray:
    """Keys visible to each query: s <= t (the bucket of s == t is included)."""
    return ss[None, :] <= ts[:, None]


def _scores(q: np.ndarray, k: np.ndarray, ts: np.ndarray, ss: np.ndarray) -> np.ndarray:
    """q_t . k_s for the block."""
    return q[ts] @ k[ss].T


def _mask_block(lam: np.ndarray, A: np.ndarray, ts: np.ndarray, ss: np.ndarray) -> np.ndarray:
    """M[t, s] = lambda[t, l(t,s)] * exp(A_t - A_s) where s <= t, else 0."""
    vis = _causal(ts, ss)
    lv = _levels(ts, ss)
    lv = np.where(vis, lv, 0)              # index only; masked out below
    lam_ts = lam[ts[:, None], lv]
    logd = np.where(vis, _pair_log_decay(A, ts, ss), -np.inf)
    return np.where(vis, lam_ts * np.exp(logd), 0.0)


def _check_shapes(q, k, v, log_a, lam):
    B, H, T, dk = q.shape
    if k.shape != (B, H, T, dk):
        raise ValueError(f"k shape {k.shape} != {(B, H, T, dk)}")
    if v.shape[:3] != (B, H, T):
        raise ValueError(f"v shape {v.shape} does not start with {(B, H, T)}")
    if log_a.shape != (B, H, T):
        raise ValueError(f"log_a shape {log_a.shape} != {(B, H, T)}")
    if lam.shape[:3] != (B, H, T) or (T > 0 and lam.shape[3] < num_levels(T)):
        raise ValueError(f"lambda shape {lam.shape} too small for T={T}")
    return B, H, T, dk, v.shape[3]


def bruteforce(q, k, v, log_a, lam, row_block: int = 512) -> np.ndarray:
    """The O(T^2) definition, in fp64, for every (b, h, t).

    ``q, k [B,H,T,dk]``, ``v [B,H,T,dv]``, ``log_a [B,H,T]``,
    ``lam [B,H,T,L]``; returns ``[B,H,T,dv]`` float64. Row blocks of queries
    only bound memory: each block builds its own mask and applies two library
    matmuls, ``(scores * mask) @ V``.
    """
    q, k, v, log_a, lam = (as_f64(x) for x in (q, k, v, log_a, lam))
    B, H, T, dk, dv = _check_shapes(q, k, v, log_a, lam)
    out = np.zeros((B, H, T, dv), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            A = _prefix_log_decay(log_a[b, h])
            for t0 in range(0, T, row_block):
                ts = np.arange(t0, min(T, t0 + row_block))
                ss = np.arange(0, ts[-1] + 1)
                P = _scores(q[b, h], k[b, h], ts, ss) * _mask_block(lam[b, h], A, ts, ss)
                out[b, h, ts] = P @ v[b, h][ss]
    return out


def bruteforce_rows(q, k, v, log_a, lam, b: int, h: int, rows) -> np.ndarray:
    """The same definition for query rows ``rows`` of head (b, h) only.

    Returns ``[len(rows), dv]`` float64. Lets large sequences be checked on a
    sample of outputs at O(t d) cost per row.
    """
    qh, kh, vh = (as_f64(x[b, h]) for x in (q, k, v))
    la, lm = as_f64(log_a[b, h]), as_f64(lam[b, h])
    A = _prefix_log_decay(la)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), vh.shape[1]), dtype=np.float64)
    for i, t in enumerate(rows):
        ts = np.array([t])
        ss = np.arange(0, t + 1)
        P = _scores(qh, kh, ts, ss) * _mask_block(lm, A, ts, ss)
        out[i] = (P @ vh[ss])[0]
    return out


# ----------------------------------------------------------------------------
# Recurrent form with O(log T) states
# ----------------------------------------------------------------------------

def _ctz(t: int) -> int:
    """Number of trailing zero bits of t > 0."""
    return (t & -t).bit_length() - 1


def recurrent_step(S: np.ndarray, q_t, k_t, v_t, log_a_t: float, lam_t, t: int) -> np.ndarray:
    """One step of the recurrent form for one head, in place on the level states.

    ``S`` [Ls, dk, dv] holds the states after position t-1 (any contents for t = 0);
    on return it holds them after position t, and the output o_t [dv] is returned.
    With c = ctz(t) for t > 0: levels 0..c of t-1 are merged into level c+1 (the lower
    drawers are full and spill into the next one, study notes section 3-6; zh lay
    summary, "drawer" merging), levels 1..c empty, every state is multiplied by a_t;
    then level 0 becomes k_t v_t^T (a_t is not in the decay of k_t) and
    o_t = sum_l lambda[t, l] S_l^T q_t over the levels lam_t covers.
    """
    if t > 0:
        c = _ctz(t)
        merged = S[: c + 1].sum(axis=0)
        S[1: c + 1] = 0.0
        S[c + 1] = merged
        S *= np.exp(log_a_t)
    S[0] = np.outer(k_t, v_t)
    n = len(lam_t)
    return np.einsum("l,lkv,k->v", np.asarray(lam_t, dtype=np.float64), S[:n], q_t)


def recurrent(q, k, v, log_a, lam) -> np.ndarray:
    """The recurrent (decoding) form: one dk x dv state per level.

    At step t the live states are level 0 = {t} and, for each set bit j of t,
    level j+1 holding the aligned block of 2^j positions just before the
    blocks of the lower set bits; ``recurrent_step`` moves from t-1 to t.

    Cost O(T L dk dv) per head: a second, independent algorithm for the same
    operator, used to cross-check ``bruteforce``.
    """
    q, k, v, log_a, lam = (as_f64(x) for x in (q, k, v, log_a, lam))
    B, H, T, dk, dv = _check_shapes(q, k, v, log_a, lam)
    out = np.zeros((B, H, T, dv), dtype=np.float64)
    if T == 0:
        return out
    L = num_levels(T)
    for b in range(B):
        for h in range(H):
            S = np.zeros((L + 1, dk, dv), dtype=np.float64)
            for t in range(T):
                out[b, h, t] = recurrent_step(S, q[b, h, t], k[b, h, t], v[b, h, t],
                                              log_a[b, h, t], lam[b, h, t, :L], t)
    return out


# ----------------------------------------------------------------------------
# Gradients of the definition (the backward pass)
# ----------------------------------------------------------------------------

def bruteforce_grad(q, k, v, log_a, lam, do):
    """Gradients of ``sum(do * o)`` for ``o = bruteforce(q, k, v, log_a, lam)``, fp64.

    Per head, with ``D[t,s] = exp(A_t - A_s)`` (s <= t, else 0), the level
    weights ``Lam[t,s] = lam[t, l(t,s)]``, the mask ``M = Lam * D``, the scores
    ``S = Q K^T`` and ``W = dO V^T`` (so that ``o = (M * S) V``):

        dq = (M * W) K          dk = (M * W)^T Q          dv = (M * S)^T dO
        dlam[t, l] = sum over s with l(t,s) = l of D[t,s] S[t,s] W[t,s]
        dA_t = sum_s G[t,s] - sum_t' G[t',t],  G = M * S * W
        dlog_a[r] = sum_{t >= r} dA_t          (A_t = sum_{r <= t} log_a[r])

    ``dA_t`` collects A_t's two roles in the decay: it is the later end of
    every pair (t, s) and the earlier end of every pair (t', t). Levels that no
    pair of a row reaches get 0. Returns ``dict(dq, dk, dv, dlog_a, dlam)``
    shaped like the inputs. Builds T x T matrices: meant for T up to a few
    thousand.
    """
    q, k, v, log_a, lam, do = (as_f64(x) for x in (q, k, v, log_a, lam, do))
    B, H, T, dk, dv = _check_shapes(q, k, v, log_a, lam)
    if do.shape != (B, H, T, dv):
        raise ValueError(f"do shape {do.shape} != {(B, H, T, dv)}")
    L = lam.shape[3]
    g = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v),
         "dlog_a": np.zeros_like(log_a), "dlam": np.zeros_like(lam)}
    if T == 0:
        return g
    ts = np.arange(T)
    vis = _causal(ts, ts)
    lv = np.where(vis, _levels(ts, ts), 0)
    for b in range(B):
        for h in range(H):
            A = _prefix_log_decay(log_a[b, h])
            D = np.where(vis, np.exp(np.where(vis, _pair_log_decay(A, ts, ts), -np.inf)), 0.0)
            M = _mask_block(lam[b, h], A, ts, ts)
            S = _scores(q[b, h], k[b, h], ts, ts)
            W = do[b, h] @ v[b, h].T
            g["dq"][b, h] = (M * W) @ k[b, h]
            g["dk"][b, h] = (M * W).T @ q[b, h]
            g["dv"][b, h] = (M * S).T @ do[b, h]
            U = D * S * W                      # the lambda-free part of G, zero above the diagonal
            for lev in range(L):
                g["dlam"][b, h, :, lev] = np.where(lv == lev, U, 0.0).sum(axis=1)
            G = M * S * W
            dA = G.sum(axis=1) - G.sum(axis=0)
            g["dlog_a"][b, h] = np.cumsum(dA[::-1])[::-1]
    return g


def bruteforce_grad_rows(q, k, v, log_a, lam, do, b: int, h: int, rows, tail: int = 0):
    """The gradients of ``bruteforce_grad`` for selected positions of head (b, h).

    For each position p in ``rows``: dq[p] and dlam[p] from row p of the pair matrices
    (targets t = p, sources s <= p), dk[p] and dv[p] from column p (sources s = p, targets
    t >= p), and dA[p] = (row sum of G at p) - (column sum of G at p), G = M * S * W.
    ``tail`` > 0 also returns dlog_a[r] = sum_{t >= r} dA_t for the last ``tail`` positions,
    from dA at every one of them. Returns dict(rows, dq, dk, dv, dlam, dA, tail_start,
    dlog_a_tail) as float64 arrays. Cost O(T (dk + dv)) per position.
    """
    qh, kh, vh, oh = (as_f64(x[b, h]) for x in (q, k, v, do))
    la, lm = as_f64(log_a[b, h]), as_f64(lam[b, h])
    T, L = qh.shape[0], lm.shape[1]
    A = _prefix_log_decay(la)

    def row(t):
        ss = np.arange(0, t + 1)
        ts = np.array([t])
        lv = _levels(ts, ss)[0]
        D = np.exp(_pair_log_decay(A, ts, ss)[0])
        Sr = kh[ss] @ qh[t]
        Wr = vh[ss] @ oh[t]
        Mr = lm[t, lv] * D
        dq = (Mr * Wr) @ kh[ss]
        dl = np.zeros(L)
        np.add.at(dl, lv, D * Sr * Wr)
        return dq, dl, float(np.sum(Mr * Sr * Wr))

    def col(s):
        ts = np.arange(s, T)
        ss = np.array([s])
        lv = _levels(ts, ss)[:, 0]
        D = np.exp(_pair_log_decay(A, ts, ss)[:, 0])
        Sc = qh[ts] @ kh[s]
        Wc = oh[ts] @ vh[s]
        Mc = lm[ts, lv] * D
        dk = (Mc * Wc) @ qh[ts]
        dv = (Mc * Sc) @ oh[ts]
        return dk, dv, float(np.sum(Mc * Sc * Wc))

    rows = np.asarray(rows, dtype=np.int64)
    out = {"rows": rows, "dq": [], "dk": [], "dv": [], "dlam": [], "dA": []}
    for p in rows:
        dq, dl, rs = row(int(p))
        dk, dv, cs = col(int(p))
        out["dq"].append(dq)
        out["dlam"].append(dl)
        out["dk"].append(dk)
        out["dv"].append(dv)
        out["dA"].append(rs - cs)
    for key in ("dq", "dk", "dv", "dlam", "dA"):
        out[key] = np.array(out[key])
    out["tail_start"] = T - tail
    if tail > 0:
        dA = np.array([row(t)[2] - col(t)[2] for t in range(T - tail, T)])
        out["dlog_a_tail"] = np.cumsum(dA[::-1])[::-1]
    return out
