"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these re-types the oracle's loop: each checks a worked example the
pages print, a closed form of a special case, an exact invariance, or a
bound, chosen so that a plausible slip in the oracle (a dropped decay on the
prediction, a read of the old state, a sign, a transposed state) fails at
least one of them.
"""

import json
import os

import numpy as np
import pytest

from oracle import gdn_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def golden(name):
    with open(GOLDEN) as f:
        return json.load(f)[name]


def rng(seed=0):
    return np.random.Generator(np.random.PCG64(seed))


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def random_head(r, T, dk, dv, alpha_range=(0.5, 1.0)):
    q = unit(r.standard_normal((T, dk)))
    k = unit(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    a = r.uniform(*alpha_range, size=T)
    b = r.uniform(0.0, 1.0, size=T)
    return q, k, v, a, b


def run_steps(q, k, v, a, b, S0):
    """States after every token, obtained by chaining single-token calls."""
    S = S0
    out = []
    for t in range(len(a)):
        _, S = orc.gdn_head(q[t:t + 1], k[t:t + 1], v[t:t + 1], a[t:t + 1],
                            b[t:t + 1], S)
        out.append(S)
    return out


# --- P-a: the worked delta-rule example ------------------------------------

def test_worked_example_scalar():
    g = golden("delta_rule_unit_key")
    S0 = np.array([[g["prediction"]]])          # unit key k = 1 -> S0 k = 2
    o, S = orc.gdn_head(q=[[1.0]], k=[[1.0]], v=[[g["target"]]],
                        alpha=[g["alpha"]], beta=[g["beta"]], S0=S0)
    assert S[0, 0] == pytest.approx(g["expected_new_prediction"], abs=1e-15)
    assert o[0, 0] == pytest.approx(g["expected_new_prediction"], abs=1e-15)


def test_worked_example_embedded():
    """Same numbers with a random unit key in dk=4 (one value channel); a
    query orthogonal to the key reads the old state unchanged."""
    g = golden("delta_rule_unit_key")
    r = rng(1)
    k = unit(r.standard_normal(4))
    s = r.standard_normal(4)
    s += (g["prediction"] - s @ k) * k            # now s . k = 2
    u = r.standard_normal(4)
    u -= (u @ k) * k                              # u orthogonal to k
    o, S = orc.gdn_head(q=np.stack([k]), k=np.stack([k]), v=[[g["target"]]],
                        alpha=[1.0], beta=[g["beta"]], S0=s[None, :])
    assert float(S[0] @ k) == pytest.approx(g["expected_new_prediction"],
                                            abs=1e-13)
    assert float(o[0, 0]) == pytest.approx(g["expected_new_prediction"],
                                           abs=1e-13)
    assert float(S[0] @ u) == pytest.approx(float(s @ u), abs=1e-13)


def test_prediction_moves_toward_target_general():
    """With ||k|| = 1: S_t k = (1 - beta) alpha S_{t-1} k + beta v."""
    r = rng(2)
    dv, dk = 3, 5
    S0 = r.standard_normal((dv, dk))
    k = unit(r.standard_normal(dk))
    v = r.standard_normal(dv)
    for a, b in [(1.0, 0.3), (0.7, 0.5), (0.2, 0.9)]:
        _, S = orc.gdn_head(k[None], k[None], v[None], [a], [b], S0)
        np.testing.assert_allclose(S @ k, (1 - b) * a * (S0 @ k) + b * v,
                                   rtol=0, atol=1e-13)


# --- P-b: a full-strength write stores the value exactly -------------------

@pytest.mark.parametrize("alpha", [1.0, 0.9, 0.3])
def test_beta_one_write_is_exact(alpha):
    r = rng(3)
    dv, dk = 3, 7                                 # dv != dk catches transposes
    S0 = r.standard_normal((dv, dk))
    k = unit(r.standard_normal(dk))
    v = r.standard_normal(dv)
    q = np.stack([k])                             # read back along the key
    o, S = orc.gdn_head(q, k[None], v[None], [alpha], [1.0], S0)
    np.testing.assert_allclose(S @ k, v, atol=1e-13)
    np.testing.assert_allclose(o[0], v, atol=1e-13)   # output reads NEW state


# --- P-c: decay is applied before the error is formed ----------------------

def test_decay_before_error_two_tokens():
    r = rng(4)
    dv, dk = 4, 3
    e1 = np.eye(dk)[0]
    v1, v2 = r.standard_normal(dv), r.standard_normal(dv)
    a1, a2, b1, b2 = 0.8, 0.6, 0.7, 0.4
    _, S = orc.gdn_head(np.stack([e1, e1]), np.stack([e1, e1]),
                        np.stack([v1, v2]), [a1, a2], [b1, b2], None)
    expect = a2 * b1 * v1 - b2 * a2 * b1 * v1 + b2 * v2
    np.testing.assert_allclose(S @ e1, expect, atol=1e-14)
    # the variant that forms the error from the undecayed state differs by
    # b1 b2 (1 - a2) v1, which is far from zero here
    wrong = expect - b1 * b2 * (1 - a2) * v1
    assert np.linalg.norm(S @ e1 - wrong) > 1e-2


# --- P-d: reduction to additive memory -------------------------------------

def test_additive_memory_without_erase():
    """Erase term off, alpha = beta = 1: S_T = V K^T and o_t = S_t q_t."""
    r = rng(5)
    T, dk, dv = 9, 4, 6
    q, k, v = r.standard_normal((T, dk)), r.standard_normal((T, dk)), \
        r.standard_normal((T, dv))
    o, S = orc.gdn_head(q, k, v, np.ones(T), np.ones(T), None, erase=False)
    np.testing.assert_allclose(S, v.T @ k, atol=1e-12)
    for t in range(T):
        np.testing.assert_allclose(o[t], (v[:t + 1].T @ k[:t + 1]) @ q[t],
                                   atol=1e-12)


def test_orthonormal_keys_closed_form():
    """Orthonormal keys, S0 = 0: nothing is erased (S_{t-1} k_t = 0), so
    S_T = sum_t (prod_{s>t} alpha_s) beta_t v_t k_t^T."""
    r = rng(6)
    T, dk, dv = 6, 8, 5
    Qm, _ = np.linalg.qr(r.standard_normal((dk, dk)))
    k = Qm[:, :T].T                                # T orthonormal keys
    q = r.standard_normal((T, dk))
    v = r.standard_normal((T, dv))
    a = r.uniform(0.3, 1.0, T)
    b = r.uniform(0.1, 1.0, T)
    o, S = orc.gdn_head(q, k, v, a, b, None)
    for t in range(T):
        St = sum(np.prod(a[i + 1:t + 1]) * b[i] * np.outer(v[i], k[i])
                 for i in range(t + 1))
        np.testing.assert_allclose(o[t], St @ q[t], atol=1e-13)
    np.testing.assert_allclose(S, St, atol=1e-13)


# --- P-e: rank bound by brute force ----------------------------------------

@pytest.mark.parametrize("rk,rv", [(2, 5), (5, 2), (3, 3), (6, 6)])
def test_rank_bound_brute_force(rk, rv):
    r = rng(10 + rk * 7 + rv)
    T, d = 10, 8
    Bk = r.standard_normal((d, rk))
    Bv = r.standard_normal((d, rv))
    k = unit((Bk @ r.standard_normal((rk, T))).T)  # keys in a rk-dim space
    v = (Bv @ r.standard_normal((rv, T))).T        # values in a rv-dim space
    q = r.standard_normal((T, d))
    a = r.uniform(0.5, 1.0, T)
    b = r.uniform(0.1, 1.0, T)
    states = run_steps(q, k, v, a, b, None)
    for t, S in enumerate(states, start=1):
        rank_S = np.linalg.matrix_rank(S, tol=1e-9)
        rank_K = np.linalg.matrix_rank(k[:t], tol=1e-9)
        rank_V = np.linalg.matrix_rank(v[:t], tol=1e-9)
        assert rank_S <= min(rank_K, rank_V) <= t
        # row space of S within span(keys so far); columns within span(values)
        Pk = np.linalg.pinv(k[:t]) @ k[:t]
        Pv = v[:t].T @ np.linalg.pinv(v[:t].T)
        np.testing.assert_allclose(S @ Pk, S, atol=1e-9)
        np.testing.assert_allclose(Pv @ S, S, atol=1e-9)


# --- P-f: stable rank, utilisation, condition number -----------------------

def test_stable_rank_worked_example():
    g = golden("stable_rank_diag")
    S = np.array(g["S"])
    assert orc.stable_rank(S) == pytest.approx(g["er"], rel=1e-12)
    assert orc.utilisation(S) == pytest.approx(g["u"], rel=1e-12)
    assert orc.condition_number(S) == pytest.approx(g["kappa"], rel=1e-12)
    qs, eps = np.array(g["q_star"]), 1e-3 * np.array(g["noise_direction"])
    amp = (np.linalg.norm(S @ eps) / np.linalg.norm(S @ qs)) / \
        (np.linalg.norm(eps) / np.linalg.norm(qs))
    assert amp == pytest.approx(g["amplification"], rel=1e-12)
    assert g["amplification"] >= 1 / np.sqrt(g["u"])


def test_stable_rank_bounds():
    r = rng(7)
    cases = [r.standard_normal((8, 8)), r.standard_normal((5, 9)),
             np.outer(r.standard_normal(6), r.standard_normal(6)),
             r.standard_normal((7, 3)) @ r.standard_normal((3, 7)),
             np.eye(4), np.diag([3.0, 1.0, 0.0])]
    for S in cases:
        er = orc.stable_rank(S)
        rank = np.linalg.matrix_rank(S)
        assert 1 - 1e-12 <= er <= rank + 1e-12 <= min(S.shape) + 1e-12
    assert orc.stable_rank(np.eye(4)) == pytest.approx(4.0)
    assert orc.stable_rank(np.outer([1.0, 2, 3], [4.0, 5])) == pytest.approx(1.0)
    assert np.isnan(orc.stable_rank(np.zeros((3, 3))))


def test_entropy_and_numerical_rank():
    assert orc.entropy_erank(np.eye(128)) == pytest.approx(128.0, rel=1e-12)
    assert orc.entropy_erank(np.outer(np.ones(5), np.ones(5))) == \
        pytest.approx(1.0, abs=1e-6)
    # two equal singular values -> exp(log 2) = 2
    assert orc.entropy_erank(np.diag([2.0, 2.0, 0.0])) == pytest.approx(2.0)
    s = np.array([1.0, 1e-3, 1e-5, 1e-6])        # threshold 128 * 2^-23 ~ 1.5e-5
    assert orc.numerical_rank(np.diag(s)) == 2


# --- P-g: orthogonal invariance --------------------------------------------

def test_orthogonal_invariance():
    r = rng(8)
    T, dk, dv = 40, 6, 5
    q, k, v, a, b = random_head(r, T, dk, dv)
    S0 = r.standard_normal((dv, dk))
    Tm, _ = np.linalg.qr(r.standard_normal((dk, dk)))
    o1, S1 = orc.gdn_head(q, k, v, a, b, S0)
    o2, S2 = orc.gdn_head(q @ Tm.T, k @ Tm.T, v, a, b, S0 @ Tm.T)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(S2, S1 @ Tm.T, atol=1e-12)


# --- P-h: zero-padding embedding ties the pruned width to the full one -----

def test_zero_padding_embedding():
    r = rng(9)
    T, dk, dkp, dv = 50, 16, 8, 6
    idx = np.sort(r.permutation(dk)[:dkp])
    q, k, v, a, b = random_head(r, T, dkp, dv)
    S0p = r.standard_normal((dv, dkp))
    P = np.eye(dk)[idx]                           # P_I, [dk', dk]
    o_small, S_small = orc.gdn_head(q, k, v, a, b, S0p)
    o_big, S_big = orc.gdn_head(q @ P, k @ P, v, a, b, S0p @ P)
    np.testing.assert_allclose(o_big, o_small, atol=1e-12)
    np.testing.assert_allclose(S_big, S_small @ P, atol=1e-12)


# --- P-i: value channels evolve independently ------------------------------

def test_value_channel_permutation():
    r = rng(11)
    T, dk, dv = 30, 5, 7
    q, k, v, a, b = random_head(r, T, dk, dv)
    S0 = r.standard_normal((dv, dk))
    perm = r.permutation(dv)
    o1, S1 = orc.gdn_head(q, k, v, a, b, S0)
    o2, S2 = orc.gdn_head(q, k, v[:, perm], a, b, S0[perm])
    np.testing.assert_allclose(o2, o1[:, perm], atol=1e-13)
    np.testing.assert_allclose(S2, S1[perm], atol=1e-13)


# --- P-j: one gradient step on the online regression loss ------------------

def test_update_is_gradient_step_on_decayed_state():
    r = rng(12)
    dv, dk = 4, 5
    S0 = r.standard_normal((dv, dk))
    k = r.standard_normal(dk)                      # any k, not only unit
    v = r.standard_normal(dv)
    alpha, beta = 0.7, 0.35
    St = alpha * S0                                # the decayed state

    def loss(S):
        return 0.5 * np.sum((v - S @ k) ** 2)

    h = 1e-6
    grad = np.zeros_like(St)
    for i in range(dv):
        for j in range(dk):
            E = np.zeros_like(St)
            E[i, j] = h
            grad[i, j] = (loss(St + E) - loss(St - E)) / (2 * h)
    _, S1 = orc.gdn_head(np.zeros((1, dk)), k[None], v[None], [alpha], [beta],
                         S0)
    np.testing.assert_allclose(S1, St - beta * grad, atol=1e-7)


# --- P-k: chunk/segment consistency and decode == one-token prefill --------

def test_split_and_decode_consistency():
    r = rng(13)
    B, T, H, dk, dv = 2, 37, 3, 6, 4
    q = unit(r.standard_normal((B, T, H, dk)))
    k = unit(r.standard_normal((B, T, H, dk)))
    v = r.standard_normal((B, T, H, dv))
    a = r.uniform(0.5, 1, (B, T, H))
    b = r.uniform(0, 1, (B, T, H))
    S0 = r.standard_normal((B, H, dv, dk))
    o, S = orc.gdn_prefill(q, k, v, a, b, S0)
    T1 = 15
    o1, S1 = orc.gdn_prefill(q[:, :T1], k[:, :T1], v[:, :T1], a[:, :T1],
                             b[:, :T1], S0)
    o2, S2 = orc.gdn_prefill(q[:, T1:], k[:, T1:], v[:, T1:], a[:, T1:],
                             b[:, T1:], S1)
    np.testing.assert_allclose(np.concatenate([o1, o2], 1), o, atol=1e-12)
    np.testing.assert_allclose(S2, S, atol=1e-12)
    Sd = S0
    for t in range(T):
        od, Sd = orc.gdn_decode_step(q[:, t], k[:, t], v[:, t], a[:, t],
                                     b[:, t], Sd)
        np.testing.assert_allclose(od, o[:, t], atol=1e-12)
    np.testing.assert_allclose(Sd, S, atol=1e-12)


# --- P-l: truncation --------------------------------------------------------

def test_truncation_properties():
    r = rng(14)
    S = r.standard_normal((12, 12)) @ np.diag(np.logspace(0, -3, 12)) @ \
        r.standard_normal((12, 12))
    s = np.linalg.svd(S, compute_uv=False)
    for rr in [1, 3, 7]:
        P = orc.truncate_rank(S, rr)
        assert np.linalg.norm(S - P) ** 2 == pytest.approx(np.sum(s[rr:] ** 2),
                                                           rel=1e-10)
        np.testing.assert_allclose(orc.truncate_rank(P, rr), P, atol=1e-12)
        assert np.linalg.matrix_rank(P, tol=1e-10) <= rr
        assert orc.stable_rank(P) <= rr + 1e-12
    # rank-3 state: r >= 3 keeps it exactly
    L = r.standard_normal((12, 3)) @ r.standard_normal((3, 12))
    np.testing.assert_allclose(orc.truncate_rank(L, 3), L, atol=1e-10)
    g = golden("truncation_identity_rank")
    X = r.standard_normal((g["d"], g["d"]))
    np.testing.assert_array_equal(orc.truncate_rank(X, g["r_identity"]), X)


def test_truncation_boundaries():
    """Truncation at t = 256 m between segments only; r = full is a no-op."""
    r = rng(15)
    T, dk, dv = 600, 8, 8
    q, k, v, a, b = random_head(r, T, dk, dv, alpha_range=(0.95, 1.0))
    o, S = orc.gdn_head(q, k, v, a, b, None, trunc_r=2, trunc_every=256)
    # segment by segment, truncating the carried state between segments
    oa, Sa = orc.gdn_head(q[:256], k[:256], v[:256], a[:256], b[:256], None)
    Sa = orc.truncate_rank(Sa, 2)
    ob, Sb = orc.gdn_head(q[256:512], k[256:512], v[256:512], a[256:512],
                          b[256:512], Sa)
    Sb = orc.truncate_rank(Sb, 2)
    oc, Sc = orc.gdn_head(q[512:], k[512:], v[512:], a[512:], b[512:], Sb)
    np.testing.assert_allclose(o, np.concatenate([oa, ob, oc]), atol=1e-12)
    np.testing.assert_allclose(S, Sc, atol=1e-12)     # no truncation at T
    assert np.linalg.matrix_rank(S, tol=1e-9) > 2
    # T a multiple of the segment length: the state after the last token is
    # not truncated (there is no next segment to carry it into)
    o2, S2 = orc.gdn_head(q[:512], k[:512], v[:512], a[:512], b[:512], None,
                          trunc_r=2, trunc_every=256)
    np.testing.assert_allclose(S2, Sb_untrunc := orc.gdn_head(
        q[256:512], k[256:512], v[256:512], a[256:512], b[256:512], Sa)[1],
        atol=1e-12)
    assert np.linalg.matrix_rank(Sb_untrunc, tol=1e-9) > 2
    o_full, S_full = orc.gdn_head(q, k, v, a, b, None, trunc_r=dk)
    o_none, S_none = orc.gdn_head(q, k, v, a, b, None)
    np.testing.assert_allclose(o_full, o_none, atol=1e-11)
    np.testing.assert_allclose(S_full, S_none, atol=1e-11)


# --- P-m: the erase-write map is a contraction -----------------------------

def test_spectral_norm_bound():
    r = rng(16)
    T, dk, dv = 200, 6, 6
    q, k, v, a, b = random_head(r, T, dk, dv, alpha_range=(0.2, 1.0))
    states = run_steps(q, k, v, a, b, r.standard_normal((dv, dk)))
    prev = None
    for t, S in enumerate(states):
        if prev is not None:
            assert np.linalg.norm(S, 2) <= a[t] * np.linalg.norm(prev, 2) + \
                b[t] * np.linalg.norm(v[t]) + 1e-12
        prev = S


# --- the product form stated for the method (cross-form check) -------------

def test_product_form_matches():
    r = rng(17)
    T, dk, dv = 25, 5, 3
    q, k, v, a, b = random_head(r, T, dk, dv)
    S = r.standard_normal((dv, dk))
    o, ST = orc.gdn_head(q, k, v, a, b, S)
    for t in range(T):
        S = a[t] * S @ (np.eye(dk) - b[t] * np.outer(k[t], k[t])) + \
            b[t] * np.outer(v[t], k[t])
        np.testing.assert_allclose(o[t], S @ q[t], atol=1e-12)
    np.testing.assert_allclose(ST, S, atol=1e-12)
