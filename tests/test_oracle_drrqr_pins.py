"""Pins of the oracle's DRRQR channel selection (drrqr_select).

"On State Reduction in Linear Attention" (reading notes), paper Sec. 3.4 with
Algorithm 2 and App. B.2: a column-pivoted QR of the calibration matrix, then
strong-RRQR trades until every rho_ij <= f; at that point, with
c_f = sqrt(1 + f^2 k (n - k)), sigma_i(A_k) >= sigma_i(M) / c_f,
||C_k||_2 <= c_f sigma_{k+1}(M) and kappa(A_k) <= c_f sigma_1 / sigma_k.
The pins check those bounds from the returned channels alone, and check the
stopping rule by brute force on volumes: rho_ij is the factor by which
trading kept column i for dropped column j would grow the volume spanned by
the kept columns, so no such trade may grow it by more than f."""

import itertools

import numpy as np
import pytest

from oracle import gdn_oracle as orc
from tests.test_oracle_pins import rng


def volume(M, cols):
    X = M[:, list(cols)]
    return np.sqrt(abs(np.linalg.det(X.T @ X)))


def calib(r, rows, n, decay=0.25):
    """Correlated calibration samples with a decaying spectrum."""
    return (r.standard_normal((rows, n)) * np.exp(-decay * np.arange(n))) @ r.standard_normal((n, n))


def kahan(n, c=0.285):
    s = np.sqrt(1 - c * c)
    R = np.triu(-c * np.ones((n, n)), 1) + np.eye(n)
    R = np.diag(s ** np.arange(n)) @ R
    # tiny growing diagonal perturbation: column pivoting keeps the identity order
    return R + np.diag(1e-9 * np.arange(n, 0, -1))


def check_bounds(M, sel, k, f):
    n = M.shape[1]
    sv = np.linalg.svd(M, compute_uv=False)
    cf = np.sqrt(1 + f * f * k * (n - k))
    A_sv = np.linalg.svd(M[:, sel], compute_uv=False)       # = sigma(A_k)
    assert np.all(A_sv >= sv[:k] / cf * (1 - 1e-9))
    rest = [c for c in range(n) if c not in set(sel.tolist())]
    Qs, _ = np.linalg.qr(M[:, sel])
    Cres = M[:, rest] - Qs @ (Qs.T @ M[:, rest])             # [0; C_k] up to rotation
    assert np.linalg.norm(Cres, 2) <= cf * sv[k] * (1 + 1e-9)
    assert A_sv[0] / A_sv[-1] <= cf * sv[0] / sv[k - 1] * (1 + 1e-9)


def check_stopping(M, sel, f):
    n = M.shape[1]
    kept = list(sel)
    v0 = volume(M, kept)
    worst = 0.0
    for i, j in itertools.product(range(len(kept)), [c for c in range(n) if c not in kept]):
        trial = kept.copy()
        trial[i] = j
        worst = max(worst, volume(M, trial) / v0)
    assert worst <= f * (1 + 1e-9), worst
    return worst


@pytest.mark.parametrize("n,k,f", [(12, 5, 1.1), (16, 8, 1.5), (10, 3, 2.0)])
def test_bounds_and_stopping_rule_random(n, k, f):
    r = rng(31 + n)
    M = calib(r, 300, n)
    sel, swaps, rho = orc.drrqr_select(M, k, f)
    assert len(set(sel.tolist())) == k and rho <= f
    check_bounds(M, sel, k, f)
    worst = check_stopping(M, sel, f)
    np.testing.assert_allclose(worst, rho, rtol=1e-8)       # rho is the worst volume ratio


def test_kahan_matrix_needs_trades():
    # pivoted QR alone keeps the Kahan order; strong RRQR must trade columns
    n, k = 12, 11
    M = kahan(n)
    sel0, sw0, rho0 = orc.drrqr_select(M, k, f=1e9)          # no trades allowed in practice
    assert sw0 == 0 and sorted(sel0.tolist()) == list(range(k))
    sel, swaps, rho = orc.drrqr_select(M, k, f=1.05)
    assert swaps >= 1 and rho <= 1.05
    check_stopping(M, sel, 1.05)
    check_bounds(M, sel, k, 1.05)
    assert volume(M, sel) > 1.05 * volume(M, sel0)


def test_duplicate_channel_is_not_kept_twice():
    r = rng(33)
    M = calib(r, 200, 9, decay=0.05)
    M[:, 4] = M[:, 2]                                        # channel 4 repeats channel 2
    sel, _, _ = orc.drrqr_select(M, 5, 1.2)
    assert not {2, 4} <= set(sel.tolist())


def test_dominant_orthogonal_channels_are_the_unique_choice():
    r = rng(34)
    rows, n, k = 256, 10, 4
    Q, _ = np.linalg.qr(r.standard_normal((rows, n)))
    M = 1e-3 * Q @ r.standard_normal((n, n))
    big = [1, 4, 6, 9]
    for c, col in zip(big, range(k)):
        M[:, c] += 10.0 * Q[:, col]
    sel, _, _ = orc.drrqr_select(M, k, 1.5)
    assert sorted(sel.tolist()) == big
