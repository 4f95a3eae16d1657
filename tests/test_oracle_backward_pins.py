"""Pins of the oracle's backward pass (gdn_head_backward / gdn_backward): the
gradient of L = sum_t do_t . o_t + <dST, S_T> through the gated delta rule
with respect to q, k, v, alpha, beta and S_0.  The pages print no backward
pass, so the pins are the definition of a gradient (central finite
differences of the pinned forward oracle, whose error is O(h^2)), the closed
form of the beta = 0 case (a pure decay: o_t = (prod_{s<=t} alpha_s) S_0 q_t)
and linearity in (do, dST)."""

import numpy as np
import pytest

from oracle import gdn_oracle as orc
from tests.test_oracle_pins import rng


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def case(seed, T, dk, dv, with_s0=True, with_dst=True):
    r = rng(seed)
    q = r.standard_normal((T, dk))
    k = unit(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    a = r.uniform(0.5, 1.0, T)
    b = r.uniform(0.0, 1.0, T)
    S0 = r.standard_normal((dv, dk)) if with_s0 else None
    do = r.standard_normal((T, dv))
    dST = r.standard_normal((dv, dk)) if with_dst else None
    return q, k, v, a, b, S0, do, dST


def loss(q, k, v, a, b, S0, do, dST):
    o, ST = orc.gdn_head(q, k, v, a, b, S0)
    out = float(np.sum(o * do))
    if dST is not None:
        out += float(np.sum(ST * dST))
    return out


def finite_difference(args, i, do, dST, h=1e-6):
    x = args[i]
    g = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        p = [y.copy() for y in args]
        m = [y.copy() for y in args]
        p[i][idx] += h
        m[i][idx] -= h
        g[idx] = (loss(*p, do, dST) - loss(*m, do, dST)) / (2 * h)
    return g


@pytest.mark.parametrize("with_s0,with_dst", [(True, True), (False, True), (True, False)])
def test_matches_finite_differences(with_s0, with_dst):
    q, k, v, a, b, S0, do, dST = case(41, 6, 5, 4, with_s0, with_dst)
    got = orc.gdn_head_backward(q, k, v, a, b, S0, do, dST)
    S0x = S0 if S0 is not None else np.zeros((4, 5))
    args = [q, k, v, a, b, S0x]
    names = ["dq", "dk", "dv", "dalpha", "dbeta", "dS0"]
    for i, name in enumerate(names):
        fd = finite_difference(args, i, do, dST)
        err = np.max(np.abs(fd - got[i])) / np.max(np.abs(fd))
        assert err < 1e-7, (name, err)


def test_beta_zero_closed_form():
    # beta = 0: S_t = (prod_{s<=t} alpha_s) S_0, nothing is written
    q, k, v, a, b, S0, do, dST = case(42, 9, 6, 3)
    b = np.zeros_like(b)
    dq, dk, dv, da, db, dS0 = orc.gdn_head_backward(q, k, v, a, b, S0, do, dST)
    c = np.cumprod(a)
    np.testing.assert_allclose(dq, c[:, None] * (do @ S0), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dv, 0.0, atol=0)
    np.testing.assert_allclose(dk, 0.0, atol=1e-12)
    want = sum(c[t] * np.outer(do[t], q[t]) for t in range(len(a))) + c[-1] * dST
    np.testing.assert_allclose(dS0, want, rtol=1e-12, atol=1e-12)
    # dalpha_t = (1 / alpha_t) * sum over later readouts and S_T of their
    # sensitivity: d/d alpha_t of prod_{s<=t'} alpha_s = that product / alpha_t
    want_da = np.array([
        (sum(c[u] * do[u] @ S0 @ q[u] for u in range(t, len(a))) +
         c[-1] * np.sum(dST * S0)) / a[t] for t in range(len(a))])
    np.testing.assert_allclose(da, want_da, rtol=1e-12, atol=1e-12)
    # dbeta_t = (G_t k_t) . (v_t - S~_t k_t): the only term left
    assert np.all(np.isfinite(db))


def test_linear_in_cotangents():
    q, k, v, a, b, S0, do, dST = case(43, 8, 4, 5)
    g1 = orc.gdn_head_backward(q, k, v, a, b, S0, do, dST)
    g2 = orc.gdn_head_backward(q, k, v, a, b, S0, 2.5 * do, 2.5 * dST)
    for x, y in zip(g1, g2):
        np.testing.assert_allclose(2.5 * x, y, rtol=1e-12, atol=1e-12)
    gz = orc.gdn_head_backward(q, k, v, a, b, S0, np.zeros_like(do), None)
    for x in gz:
        np.testing.assert_allclose(x, 0.0, atol=0)


def test_batched_layout_matches_heads():
    r = rng(44)
    B, T, H, dk, dv = 2, 5, 3, 4, 3
    q = r.standard_normal((B, T, H, dk))
    k = unit(r.standard_normal((B, T, H, dk)))
    v = r.standard_normal((B, T, H, dv))
    a = r.uniform(0.5, 1, (B, T, H))
    b = r.uniform(0, 1, (B, T, H))
    S0 = r.standard_normal((B, H, dv, dk))
    do = r.standard_normal((B, T, H, dv))
    dST = r.standard_normal((B, H, dv, dk))
    full = orc.gdn_backward(q, k, v, a, b, S0, do, dST)
    for bb in range(B):
        for h in range(H):
            one = orc.gdn_head_backward(q[bb, :, h], k[bb, :, h], v[bb, :, h], a[bb, :, h],
                                        b[bb, :, h], S0[bb, h], do[bb, :, h], dST[bb, h])
            np.testing.assert_array_equal(full[0][bb, :, h], one[0])
            np.testing.assert_array_equal(full[5][bb, h], one[5])
            np.testing.assert_array_equal(full[3][bb, :, h], one[3])
