"""Seeded synthetic inputs for the log-linear Mamba-2 forward pass.

This module only draws random numbers and shapes them; it holds none of the
method's arithmetic (no levels, no decays, no contractions). Both the CPU
oracle's tests and the GPU path's tests/bench take their inputs from here, so
the two sides see bit-identical tensors.

Recipe (one ``torch.Generator('cpu')`` seeded with ``seed``), drawn in this
fixed order, all in float32:

1. ``q  ~ N(0,1)``  shape ``[B,H,T,dk]``
2. ``k  ~ N(0,1)``  shape ``[B,H,T,dk]``
3. ``v  ~ N(0,1)``  shape ``[B,H,T,dv]``
4. ``u  ~ U(0,1)``  shape ``[B,H,T]``   -> ``log_a = -(lo + (hi-lo) u)``
5. ``n  ~ N(0,1)``  shape ``[B,H,T,L]`` -> ``lambda = softplus(n + shift[level])``

then ``q /= sqrt(dk)``; ``k /= sqrt(dk)`` (or ``k = k/||k||_2`` per token for
the long-range workload); q, k, v are rounded to bfloat16 (round to nearest
even) for bf16 workloads. ``log_a`` and ``lambda`` stay float32. The value
distributions follow the workloads' statements: per-token decays in
``(lo, hi)``, non-negative per-level weights from a softplus of a normal.

Variants (parity stress cases; never timed) replace one drawn tensor after the
draw so that every other tensor stays identical:

* ``log_a_mode``: ``"nodecay"`` (all zero), ``"lowdecay"`` (``-1e-4 u``),
  ``"strongdecay"`` (``-(0.5 + 2.5 u)``, i.e. per-token decays a = exp(-U(0.5, 3)), strong
  Mamba-2-style gates: a chunk's local log decay then reaches well past -40).
* ``lam_mode``: ``"onehot:<l>"``, ``"zero"``, ``"ones"``,
  ``"equal"`` (one weight per token shared by all levels).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch

__all__ = ["Workload", "WORKLOADS", "GDN_WORKLOADS", "num_levels_for", "generate", "generate_gdn",
           "workload", "grad_output"]


def num_levels_for(T: int) -> int:
    """Level count for a sequence of T tokens: bit length of T-1, plus one.

    Pure integer bookkeeping used to size the lambda tensor (the 0-based
    Fenwick level of any pair of positions in [0, T) is at most
    bit_length(T-1)); T=1 needs a single level.
    """
    if T < 1:
        raise ValueError("T must be >= 1")
    return (T - 1).bit_length() + 1


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    dtype: str            # "bf16" or "f32" for q, k, v, out
    chunk: int            # chunk size the workload is stated at
    loga_lo: float = 0.001
    loga_hi: float = 0.1
    k_l2norm: bool = False
    lam_split: int | None = None   # levels >= split get N(1,1), below N(-1,1)

    @property
    def L(self) -> int:
        return num_levels_for(self.T)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads, by shape. The first is the small fp32 case, the third the
# headline shape (B=4, H=16, T=8192, d=64, bf16).
WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("b1h2_t256_d16_f32", 1, 2, 256, 16, 16, "f32", 16),
        Workload("b2h8_t2048_d64_bf16", 2, 8, 2048, 64, 64, "bf16", 64),
        Workload("b4h16_t8192_d64_bf16", 4, 16, 8192, 64, 64, "bf16", 64),
        Workload("b1h16_t32768_d128_bf16_knorm", 1, 16, 32768, 128, 128, "bf16", 64,
                 loga_lo=0.0001, loga_hi=0.05, k_l2norm=True),
        Workload("b1h8_t65536_d128_bf16_coarse", 1, 8, 65536, 128, 128, "bf16", 128,
                 lam_split=8),
    ]
}

HEADLINE = "b4h16_t8192_d64_bf16"


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _softplus(x: torch.Tensor) -> torch.Tensor:
    return torch.nn.functional.softplus(x)


def generate(w: Workload, seed: int = 0, *, log_a_mode: str | None = None,
             lam_mode: str | None = None) -> dict:
    """Draw one batch of inputs for workload ``w`` (CPU tensors).

    Returns ``dict(q, k, v, log_a, lam)``; q/k/v in bfloat16 or float32 per
    ``w.dtype``, log_a ``[B,H,T]`` and lam ``[B,H,T,L]`` in float32, all
    contiguous.
    """
    B, H, T, dk, dv, L = w.B, w.H, w.T, w.dk, w.dv, w.L
    g = torch.Generator("cpu").manual_seed(int(seed))
    q = torch.randn((B, H, T, dk), generator=g, dtype=torch.float32)
    k = torch.randn((B, H, T, dk), generator=g, dtype=torch.float32)
    v = torch.randn((B, H, T, dv), generator=g, dtype=torch.float32)
    u = torch.rand((B, H, T), generator=g, dtype=torch.float32)
    n = torch.randn((B, H, T, L), generator=g, dtype=torch.float32)

    q = q / math.sqrt(dk)
    if w.k_l2norm:
        k = k / k.norm(dim=-1, keepdim=True)
    else:
        k = k / math.sqrt(dk)
    log_a = -(w.loga_lo + (w.loga_hi - w.loga_lo) * u)
    if w.lam_split is None:
        lam = _softplus(n)
    else:
        shift = torch.where(torch.arange(L) >= w.lam_split, 1.0, -1.0).to(torch.float32)
        lam = _softplus(n + shift)

    if log_a_mode is not None:
        if log_a_mode == "nodecay":
            log_a = torch.zeros_like(log_a)
        elif log_a_mode == "lowdecay":
            log_a = -1e-4 * u
        elif log_a_mode == "strongdecay":
            log_a = -(0.5 + 2.5 * u)
        else:
            raise ValueError(f"unknown log_a_mode {log_a_mode!r}")
    if lam_mode is not None:
        if lam_mode.startswith("onehot:"):
            lev = int(lam_mode.split(":", 1)[1])
            if not 0 <= lev < L:
                raise ValueError(f"one-hot level {lev} outside [0, {L})")
            lam = torch.zeros_like(lam)
            lam[..., lev] = 1.0
        elif lam_mode == "zero":
            lam = torch.zeros_like(lam)
        elif lam_mode == "ones":
            lam = torch.ones_like(lam)
        elif lam_mode == "equal":
            lam = lam[..., :1].expand_as(lam).contiguous()
        else:
            raise ValueError(f"unknown lam_mode {lam_mode!r}")

    if w.dtype == "bf16":
        q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    elif w.dtype != "f32":
        raise ValueError(f"unknown dtype {w.dtype!r}")
    return dict(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(),
                log_a=log_a.contiguous(), lam=lam.contiguous())


# Log-linear Gated DeltaNet: the same shapes, keys L2-normalised per token (the delta rule's
# transition I - beta k k^T is then a contraction for beta in (0, 1)), plus beta.
GDN_WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("gdn_b1h2_t256_d16_f32", 1, 2, 256, 16, 16, "f32", 16, k_l2norm=True),
        Workload("gdn_b2h8_t2048_d64_bf16", 2, 8, 2048, 64, 64, "bf16", 64, k_l2norm=True),
        Workload("gdn_b4h16_t8192_d64_bf16", 4, 16, 8192, 64, 64, "bf16", 64, k_l2norm=True),
        Workload("gdn_b1h8_t8192_d128_bf16", 1, 8, 8192, 128, 128, "bf16", 32, k_l2norm=True),
    ]
}


def generate_gdn(w: Workload, seed: int = 0, *, log_a_mode: str | None = None,
                 lam_mode: str | None = None, beta_mode: str | None = None) -> dict:
    """Inputs of log-linear Gated DeltaNet: ``generate(w, seed, ...)`` (so q, k, v, log_a and
    lambda are bit-identical to it) plus ``beta [B,H,T]`` float32 = sigmoid(N(0,1)), drawn from
    a second generator seeded with ``seed + 104729``. ``beta_mode``: ``"zero"``, ``"ones"``
    (parity stress cases)."""
    x = generate(w, seed, log_a_mode=log_a_mode, lam_mode=lam_mode)
    g = torch.Generator("cpu").manual_seed(int(seed) + 104729)
    beta = torch.sigmoid(torch.randn((w.B, w.H, w.T), generator=g, dtype=torch.float32))
    if beta_mode == "zero":
        beta = torch.zeros_like(beta)
    elif beta_mode == "ones":
        beta = torch.ones_like(beta)
    elif beta_mode is not None:
        raise ValueError(f"unknown beta_mode {beta_mode!r}")
    x["beta"] = beta.contiguous()
    return x


def grad_output(w: Workload, seed: int = 0):
    """A seeded upstream gradient dO ``[B,H,T,dv]`` for the backward pass: standard normal
    entries, in q/k/v's dtype (CPU tensor)."""
    g = torch.Generator("cpu").manual_seed(int(seed) + 7919)
    do = torch.randn((w.B, w.H, w.T, w.dv), generator=g, dtype=torch.float32)
    return do.to(torch.bfloat16 if w.dtype == "bf16" else torch.float32).contiguous()


def custom(B: int, H: int, T: int, dk: int, dv: int, dtype: str = "bf16",
           chunk: int = 64, **kw) -> Workload:
    """An ad-hoc workload (same value distributions as the small fp32 case)."""
    return Workload(f"b{B}h{H}_t{T}_dk{dk}_dv{dv}_{dtype}", B, H, T, dk, dv, dtype, chunk, **kw)
