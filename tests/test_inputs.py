"""Host checks of the seeded input generators (no GPU)."""

import numpy as np
import pytest
import torch

from workloads import gdn_inputs as gi


def test_bf16_rounding_matches_torch():
    r = np.random.Generator(np.random.PCG64(0))
    x = (r.standard_normal(100000) * np.exp(r.uniform(-20, 20, 100000))) \
        .astype(np.float32)
    # include exact ties between two bf16 neighbours
    ties = (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = gi.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours, ref)
    assert np.all(gi.round_bf16(ours) == ours)


def test_seeds_and_determinism():
    assert gi.seed_for(2) == 20260020 and gi.seed_for(3, 1) == 20260031
    a, b = gi.tiny(), gi.tiny()
    for f in ["q", "k", "v", "alpha", "beta"]:
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))


def test_tiny_distributions():
    x = gi.tiny()
    assert x.dims == dict(B=1, T=512, H=2, dk=64, dv=64) and x.dtype == "f32"
    np.testing.assert_allclose(np.linalg.norm(x.q, axis=-1), 1, atol=1e-6)
    np.testing.assert_allclose(np.linalg.norm(x.k, axis=-1), 1, atol=1e-6)
    la = -np.log(x.alpha.astype(np.float64))
    assert la.min() >= 0.001 - 1e-6 and la.max() <= 0.1 + 1e-6
    assert 0 < x.beta.min() and x.beta.max() < 1
    assert abs(np.median(x.beta) - 0.5) < 0.05
    assert x.S0 is None


def test_prefill_16k_shape_and_geometry():
    T = 2048                                      # same recipe, shorter
    x = gi.prefill_16k(T=T)
    d = x.dims
    assert (d["B"], d["H"], d["dk"], d["dv"]) == (1, 16, 128, 128)
    assert x.dtype == "bf16"
    assert np.all(gi.round_bf16(x.q) == x.q)      # bf16-exact values
    assert int(x.short_heads.sum()) == 10         # round(0.61 * 16)
    for h in range(16):
        m = gi.mean_key_norm(x.k[0, :, h])
        assert abs(m - 0.85) < 0.02, (h, m)
        la = -np.log(x.alpha[0, :, h].astype(np.float64))
        if x.short_heads[h]:
            assert la.min() >= 0.004 - 1e-6 and la.max() <= 0.1 + 1e-6
        else:
            assert la.min() >= 1e-4 - 1e-7 and la.max() <= 1e-3 + 1e-7
    # queries are not in the cone
    assert gi.mean_key_norm(x.q[0, :, 0]) < 0.2
    assert abs(x.sigma - 0.0548) < 0.002


def test_cone_sigma_hits_target():
    s = gi.cone_sigma(128)
    r = np.random.Generator(np.random.PCG64(5))
    mu = r.standard_normal(128)
    mu /= np.linalg.norm(mu)
    k = mu + s * r.standard_normal((20000, 128))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    assert abs(gi.mean_key_norm(k) - 0.85) < 0.005


def test_pruned_variant_reuses_raw_draws():
    full = gi.batched_prefill(B=1, T=64, dk=128)
    half = gi.batched_prefill(B=1, T=64, dk=64)
    np.testing.assert_array_equal(full.v, half.v)
    np.testing.assert_array_equal(full.alpha, half.alpha)
    np.testing.assert_array_equal(full.beta, half.beta)
    idx = half.channel_idx
    assert idx.shape == (16, 64)
    assert np.all(np.diff(idx, axis=1) > 0)       # sorted, distinct
    np.testing.assert_array_equal(idx, gi.pruning_subsets(4))
    # q64 = renormalised gather of the same raw vector as q128 (bf16 rounding)
    for h in [0, 7, 15]:
        g = full.q[0, :, h][:, idx[h]]
        g = g / np.linalg.norm(g, axis=-1, keepdims=True)
        np.testing.assert_allclose(half.q[0, :, h], g, atol=2e-2)
        np.testing.assert_allclose(np.linalg.norm(half.k[0, :, h], axis=-1),
                                   1, atol=1e-2)


def test_decode_prompt_and_steps_share_subsets():
    p = gi.decode_prompt(B=2, T=8, dk=64)
    s = gi.decode_steps(B=2, n_steps=4, dk=64)
    np.testing.assert_array_equal(p.channel_idx, s.channel_idx)
    assert p.seed != s.seed
    assert s.q.shape == (2, 4, 16, 64)


def test_slicing_helpers():
    x = gi.generic(3, 20, 2, 8, 4, 1, S0_scale=0.5)
    y = x.slice_time(5, 9)
    assert y.q.shape == (3, 4, 2, 8) and y.S0 is None
    z = x.slice_batch(1, 2)
    assert z.S0.shape == (1, 2, 4, 8)


def test_row_subsets_regenerate_identically():
    full = gi.batched_prefill(B=4, T=16, dk=64)
    part = gi.batched_prefill(B=4, T=16, dk=64, rows=[1, 3])
    for f in ["q", "k", "v", "alpha", "beta"]:
        np.testing.assert_array_equal(getattr(part, f), getattr(full, f)[[1, 3]])
