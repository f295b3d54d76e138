"""The seeded input generator: deterministic, right shapes and distributions."""

import math

import numpy as np
import pytest
import torch

from lla_synth import WORKLOADS, custom, generate


def test_deterministic_and_seed_dependent():
    w = custom(1, 2, 64, 16, 32)
    a, b, c = generate(w, 5), generate(w, 5), generate(w, 6)
    for key in a:
        assert torch.equal(a[key], b[key])
    assert not torch.equal(a["q"], c["q"])


def test_shapes_and_dtypes():
    w = custom(2, 3, 100, 32, 16, dtype="bf16")
    x = generate(w)
    assert x["q"].shape == (2, 3, 100, 32) and x["q"].dtype == torch.bfloat16
    assert x["k"].shape == (2, 3, 100, 32)
    assert x["v"].shape == (2, 3, 100, 16)
    assert x["log_a"].shape == (2, 3, 100) and x["log_a"].dtype == torch.float32
    assert x["lam"].shape == (2, 3, 100, 8) and x["lam"].dtype == torch.float32
    assert all(t.is_contiguous() for t in x.values())


def test_distributions_small_workload():
    w = WORKLOADS["b1h2_t256_d16_f32"].with_(B=4, H=8)
    x = generate(w)
    q = x["q"].double().numpy() * math.sqrt(16)
    v = x["v"].double().numpy()
    assert abs(q.mean()) < 0.02 and abs(q.std() - 1) < 0.02
    assert abs(v.std() - 1) < 0.02
    la = x["log_a"].numpy()
    assert la.max() <= -0.001 and la.min() >= -0.1
    assert abs(la.mean() + 0.0505) < 0.002
    lam = x["lam"].numpy()
    assert lam.min() > 0
    # E[softplus(N(0,1))] ~= 0.806
    assert abs(lam.mean() - 0.806) < 0.01


def test_long_range_and_coarse_variants():
    w = WORKLOADS["b1h16_t32768_d128_bf16_knorm"].with_(T=512, H=2)
    x = generate(w)
    kn = x["k"].float().norm(dim=-1)
    assert torch.allclose(kn, torch.ones_like(kn), atol=1e-2)
    la = x["log_a"]
    assert la.max() <= -0.0001 and la.min() >= -0.05
    w4 = WORKLOADS["b1h8_t65536_d128_bf16_coarse"].with_(T=2048, H=2)
    lam = generate(w4)["lam"].double().numpy()
    assert lam.shape[-1] == 12
    # softplus(N(1,1)) ~ 1.4 for levels >= 8; softplus(N(-1,1)) ~ 0.40 below
    assert abs(lam[..., 8:].mean() - 1.39) < 0.05
    assert abs(lam[..., :8].mean() - 0.40) < 0.05


def test_variants_keep_other_tensors():
    w = custom(1, 1, 64, 16, 16)
    base = generate(w, 1)
    nd = generate(w, 1, log_a_mode="nodecay", lam_mode="onehot:3")
    assert torch.equal(base["q"], nd["q"]) and torch.equal(base["v"], nd["v"])
    assert torch.all(nd["log_a"] == 0)
    assert torch.all(nd["lam"].sum(-1) == 1) and torch.all(nd["lam"][..., 3] == 1)
    low = generate(w, 1, log_a_mode="lowdecay")
    assert low["log_a"].min() >= -1e-4
    strong = generate(w, 1, log_a_mode="strongdecay")
    assert strong["log_a"].max() <= -0.5 and strong["log_a"].min() >= -3.0
    assert torch.equal(base["k"], strong["k"]) and torch.equal(base["lam"], strong["lam"])
    # a 64-token chunk's local log decay then lies far past -40 (about -112 on average)
    assert strong["log_a"].sum(-1).max() < -40
    eq = generate(w, 1, lam_mode="equal")
    assert torch.all(eq["lam"] == eq["lam"][..., :1])
    with pytest.raises(ValueError):
        generate(w, 1, lam_mode="onehot:99")


def test_bf16_rounding_is_round_to_nearest_even():
    w32 = custom(1, 1, 32, 16, 16, dtype="f32")
    w16 = custom(1, 1, 32, 16, 16, dtype="bf16")
    a, b = generate(w32, 2), generate(w16, 2)
    assert torch.equal(a["q"].to(torch.bfloat16), b["q"])
    assert np.array_equal(a["lam"].numpy(), b["lam"].numpy())
