"""Pins of the oracle's input path (qk_transform and the *_qk recurrences).

The input path of a channel-pruned layer keeps a per-head subset of the
query/key coordinates and recomputes the L2 normalisation over the kept
coordinates ("On State Reduction in Linear Attention", paper Sec. 3.2-3.3); a query
scale, if any, multiplies the normalised query.  Each pin below checks a
worked value, an exact identity or an invariance, chosen so that a slip in
the oracle's input path (normalising before selecting, another head's
subset, the scale on the keys, a per-head instead of per-token norm) fails
at least one of them.
"""

import numpy as np
import pytest

from oracle import gdn_oracle as orc
from tests.test_oracle_pins import golden, rng


def subsets(r, H, dk_in, dk):
    return np.stack([np.sort(r.permutation(dk_in)[:dk]) for _ in range(H)])


def raw_inputs(r, B, T, H, dk_in, dv):
    mag = np.exp(0.5 * r.standard_normal((B, T, H, 1)))
    q = mag * r.standard_normal((B, T, H, dk_in))
    mag = np.exp(0.5 * r.standard_normal((B, T, H, 1)))
    k = mag * r.standard_normal((B, T, H, dk_in))
    v = r.standard_normal((B, T, H, dv))
    a = r.uniform(0.6, 1.0, size=(B, T, H))
    b = r.uniform(0.0, 1.0, size=(B, T, H))
    return q, k, v, a, b


def test_worked_example_kept_channels():
    g = golden("input_path_kept_channels")
    x = np.array(g["x"])[None, :]                       # one head
    np.testing.assert_allclose(orc.qk_transform(x, [[0, 2]])[0], g["keep_02"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(orc.qk_transform(x, None)[0], g["keep_all"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(orc.qk_transform(x, [[2, 0]])[0], g["keep_20"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(orc.qk_transform(x, [[0, 2]], scale=2.0)[0], g["keep_02_scale2"],
                               rtol=0, atol=1e-15)


def test_selection_indexes_per_head():
    # marker values 1000 h + c: without normalisation the selection must
    # return exactly head h's own coordinates channels[h]
    H, dk_in, dk = 5, 16, 6
    r = rng(11)
    ch = subsets(r, H, dk_in, dk)
    x = (1000.0 * np.arange(H)[:, None] + np.arange(dk_in)[None, :])[None, None]
    x = np.broadcast_to(x, (2, 3, H, dk_in))
    y = orc.qk_transform(x, ch, l2norm=False)
    want = 1000.0 * np.arange(H)[:, None] + ch
    assert y.shape == (2, 3, H, dk)
    assert np.array_equal(y, np.broadcast_to(want, y.shape))


def test_unit_norm_over_kept_and_direction():
    r = rng(12)
    H, dk_in, dk = 4, 32, 12
    ch = subsets(r, H, dk_in, dk)
    x = r.standard_normal((3, 7, H, dk_in)) * np.exp(r.standard_normal((3, 7, H, 1)))
    y = orc.qk_transform(x, ch)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), 1.0, rtol=0, atol=1e-14)
    sel = orc.qk_transform(x, ch, l2norm=False)
    cos = np.sum(y * sel, axis=-1) / np.linalg.norm(sel, axis=-1)
    np.testing.assert_allclose(cos, 1.0, rtol=0, atol=1e-14)


def test_norm_is_per_token_and_scale_invariant():
    # multiplying each raw token vector by its own positive factor leaves the
    # normalised vector unchanged
    r = rng(13)
    x = r.standard_normal((2, 9, 3, 8))
    c = np.exp(3 * r.standard_normal((2, 9, 3, 1)))
    np.testing.assert_allclose(orc.qk_transform(c * x), orc.qk_transform(x), rtol=0, atol=1e-14)


def test_zero_vector_maps_to_zero_and_only_decays_the_state():
    r = rng(14)
    x = np.zeros((1, 1, 1, 6))
    assert np.array_equal(orc.qk_transform(x, [[1, 4, 5]]), np.zeros((1, 1, 1, 3)))
    # a zero key writes nothing: S_1 = alpha S_0 exactly; a zero query reads 0
    S0 = r.standard_normal((1, 1, 4, 3))
    q = r.standard_normal((1, 1, 1, 6))
    v = r.standard_normal((1, 1, 1, 4))
    o, S = orc.gdn_prefill_qk(q, x, v, np.array([[[0.7]]]), np.array([[[0.9]]]), S0,
                              channels=[[1, 4, 5]])
    np.testing.assert_allclose(S, 0.7 * S0, rtol=1e-15, atol=0)
    o, _ = orc.gdn_prefill_qk(x, q, v, np.array([[[0.7]]]), np.array([[[0.9]]]), S0,
                              channels=[[1, 4, 5]])
    assert np.array_equal(o, np.zeros_like(o))


def test_query_scale_scales_outputs_only():
    # o_t = S_t q_t is linear in q and q never enters the state (paper Sec. 2.1,
    # Eq. (1)): a query scale s gives s times the outputs and the same state
    r = rng(15)
    B, T, H, dk_in, dk, dv = 1, 40, 2, 16, 8, 5
    ch = subsets(r, H, dk_in, dk)
    q, k, v, a, b = raw_inputs(r, B, T, H, dk_in, dv)
    o1, S1 = orc.gdn_prefill_qk(q, k, v, a, b, channels=ch)
    o2, S2 = orc.gdn_prefill_qk(q, k, v, a, b, channels=ch, q_scale=0.125)
    np.testing.assert_allclose(o2, 0.125 * o1, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(S2, S1, rtol=0, atol=0)


def test_zero_padding_embedding():
    # raw vectors that vanish outside the kept set: renormalising over the
    # kept coordinates equals normalising over all of them, so the pruned
    # head reproduces the full-width head with S^(full) = S^(kept) P_I
    # (State Reduction, paper Sec. 3.2-3.3; the unit-norm precondition)
    r = rng(16)
    B, T, H, dk_in, dk, dv = 1, 50, 2, 12, 5, 4
    ch = subsets(r, H, dk_in, dk)
    q, k, v, a, b = raw_inputs(r, B, T, H, dk_in, dv)
    mask = np.zeros((H, dk_in))
    for h in range(H):
        mask[h, ch[h]] = 1.0
    q, k = q * mask, k * mask
    o_p, S_p = orc.gdn_prefill_qk(q, k, v, a, b, channels=ch)
    o_f, S_f = orc.gdn_prefill_qk(q, k, v, a, b, channels=None)
    np.testing.assert_allclose(o_p, o_f, rtol=1e-12, atol=1e-13)
    for h in range(H):
        P = np.zeros((dk, dk_in))
        P[np.arange(dk), ch[h]] = 1.0
        np.testing.assert_allclose(S_f[0, h], S_p[0, h] @ P, rtol=1e-12, atol=1e-13)


def test_decode_step_qk_is_one_token_of_prefill_qk():
    r = rng(17)
    B, H, dk_in, dk, dv = 2, 3, 16, 8, 6
    ch = subsets(r, H, dk_in, dk)
    q, k, v, a, b = raw_inputs(r, B, 1, H, dk_in, dv)
    S0 = r.standard_normal((B, H, dv, dk))
    o1, S1 = orc.gdn_prefill_qk(q, k, v, a, b, S0, channels=ch, q_scale=0.5)
    o2, S2 = orc.gdn_decode_step_qk(q[:, 0], k[:, 0], v[:, 0], a[:, 0], b[:, 0], S0,
                                    channels=ch, q_scale=0.5)
    np.testing.assert_allclose(o2, o1[:, 0], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(S2, S1, rtol=1e-14, atol=1e-15)


def test_beta_one_write_stores_value_along_normalised_key():
    # with the key renormalised over the kept channels, a beta = 1 write
    # makes S_t k_t = v_t exactly (the delta rule's defining property,
    # Linear Attention Architectures, paper Sec. 3.2), which fails if the key the
    # recurrence uses is not unit-norm over the kept coordinates
    r = rng(18)
    H, dk_in, dk, dv = 2, 20, 7, 3
    ch = subsets(r, H, dk_in, dk)
    q, k, v, a, _ = raw_inputs(r, 1, 1, H, dk_in, dv)
    S0 = r.standard_normal((1, H, dv, dk))
    _, S1 = orc.gdn_prefill_qk(q, k, v, a, np.ones((1, 1, H)), S0, channels=ch)
    kn = orc.qk_transform(k, ch)
    for h in range(H):
        np.testing.assert_allclose(S1[0, h] @ kn[0, 0, h], v[0, 0, h], rtol=1e-13, atol=1e-13)
