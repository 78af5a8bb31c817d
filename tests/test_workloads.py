"""Checks on the seeded input generators (shapes, distributions, planted structure)."""
import math

import numpy as np
import torch

import workloads as wl


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0], np.float32)])
    ours = wl.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(wl.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_progress_distribution_closed_form():
    """E[progress] = 1 + sum_{k=1}^{15} P(a >= k) for a = min(Poisson(5.09), 15) is ~6.09
    (DScale Fig. 2 mean; the accepted-length identity E[L] = 1 + sum_k P(prefix >= k) of the
    PixelML card's offline metric section)."""
    lam = 5.09
    pmf = [math.exp(-lam + t * math.log(lam) - math.lgamma(t + 1)) for t in range(200)]
    tail = [sum(pmf[t:]) for t in range(200)]
    closed = 1 + sum(tail[kk] for kk in range(1, 16))
    assert abs(closed - 6.09) < 0.01
    draws = np.minimum(np.random.default_rng(1).poisson(lam, 200000), 15)
    assert abs((1 + draws.mean()) - closed) < 0.02


def test_rescaled_lengths():
    for n, budget, seed in ((32, 256, 4), (60, 480, 5), (7, 56, 9)):
        k = wl.lengths_geometric_rescaled(np.random.default_rng(seed), n, budget)
        assert k.sum() == budget and k.min() >= 1 and k.max() <= 16


def test_config_shapes():
    c1 = wl.config1()
    assert c1["q"].shape == (7, 2, 64) and c1["k_pool"].shape[0] == 1 and c1["logits"].shape == (7, 1000)
    assert list(c1["k"]) == [3, 4] and list(c1["ctx_len"]) == [32, 48]
    s1, s2 = wl.config2()
    assert s1["k"].sum() == s2["k"].sum() == 24
    assert np.array_equal(s2["ctx_len"], s1["ctx_len"] + 1 + s1["planted_accepted"])
    assert np.all(s2["ctx_len"] + s2["k"] <= s1["ctx_len"] + 2 * 16)


def test_sentinel_variant_poisons_only_invisible_rows():
    c = wl.make_case(77, dtype="bf16", hq=2, hkv=1, d=8, k=[3, 2], ctx_len=[5, 4], m_bs=6)
    s = wl.sentinel_variant(c)
    for i in range(2):
        b, cx = int(c["kv_base"][i]), int(c["ctx_len"][i])
        assert np.array_equal(s["k_pool"][:, b:b + cx], c["k_pool"][:, b:b + cx])
        assert np.all(s["k_pool"][:, b + cx:b + cx + 16] == wl.BF16_NAN)
