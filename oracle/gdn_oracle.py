"""fp64 CPU oracle of the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path (the HIP library and its Python binding)
never calls it, and it shares no code with that path.

What it computes, token by token and head by head, in float64:

    S~_t = alpha_t * S_{t-1}                      decay first
    vhat = S~_t k_t                               prediction of the decayed state
    S_t  = S~_t + beta_t (v_t - vhat) k_t^T       delta write
    o_t  = S_t q_t                                readout of the new state

which equals S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T.

Sources (page titles as published; sections/equations as the pages give them):
  * DeltaNet write and readout, o_t = S_t q_t, S in R^{dv x dk}:
    "On State Reduction in Linear Attention" (reading notes), paper Sec. 2.1,
    Eqs. (1)-(2); gated variant adds a per-token scalar decay (same section)
    and the update is written alpha_t S_{t-1} + u_t k_t^T in the proof of the
    rank bound, Eq. (3).
  * Ordering "decay, then compare with the target using the decayed state,
    then write, then read the new state": "Linear Attention Architectures:
    Mechanisms, Trade-offs, and Cross-Layer Routing" (reading notes),
    paper Sec. 3.3 (GDN, Eqs. 15-17) and the per-token data flow of Eq. 8.
  * Stable rank er(S) = ||S||_F^2 / ||S||_2^2: "On State Reduction in Linear
    Attention", paper Sec. 2.2, Eq. (5); entropy effective rank and the numerical
    rank threshold sigma_max * 128 * eps: "How much of its state does Gated
    DeltaNet use?" (state-rank post), §1.
  * Segment truncation (project the carried state onto its top-r left
    singular directions at every 256-token boundary, r = 128 = no change):
    state-rank post, §3.

  * Backward pass (gdn_head_backward): the gradient of
    sum_t do_t . o_t + <dST, S_T> with respect to q, k, v, alpha, beta and
    S_0, by the chain rule over the tokens in reverse.  The pages train
    these layers but print no backward pass; it is pinned to central finite
    differences of gdn_head and to the closed form of the beta = 0 case.
  * Generalised gates (gdn2_head): a per-key-channel decay applied on the
    right of the state (Kimi Delta Attention) and split key-side erase /
    value-side write gates whose outer products keep k_t on the right
    (Gated DeltaNet-2): "Linear Attention Architectures" reading notes on
    the paper's Secs. 3.4-3.5 (Eqs. 18-24) and their mechanism table.
  * DRRQR channel selection (drrqr_select): a column-pivoted QR of the
    calibration matrix of key and query samples, then strong-RRQR swaps
    until every rho_ij <= f: "On State Reduction in Linear Attention",
    paper Sec. 3.4 (Algorithm 2, App. B.2).
  * Input path of a channel-pruned layer (qk_transform): keep a per-head
    subset of query/key coordinates and renormalise over the kept ones:
    "On State Reduction in Linear Attention", paper Sec. 3.2-3.3.

Readings where the pages leave a step open:
  * No query scale: o_t = S_t q_t exactly.
  * alpha is given (not log alpha), in (0, 1]; beta in [0, 1].
  * Truncation happens only at boundaries between segments (t = 256 m with
    t < T), never after the last token.
  * The input path selects, then normalises, then scales (queries only); a
    vector whose kept coordinates are all zero maps to zero.
"""

from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


# ---------------------------------------------------------------------------
# the recurrence
# ---------------------------------------------------------------------------

def gdn_head(q: np.ndarray, k: np.ndarray, v: np.ndarray,
             alpha: np.ndarray, beta: np.ndarray,
             S0: Optional[np.ndarray] = None, *, erase: bool = True,
             trunc_r: Optional[int] = None, trunc_every: int = 256
             ) -> Tuple[np.ndarray, np.ndarray]:
    """One head, one sequence.

    q, k [T, dk]; v [T, dv]; alpha, beta [T]; S0 [dv, dk] or None (zero).
    erase=False drops the erase term (S_t = alpha S_{t-1} + beta v k^T), used
    only to pin the additive special case.
    trunc_r: if set, after token t (1-based) with t % trunc_every == 0 and
    t < T, replace S by its projection onto its top-trunc_r left singular
    directions.
    Returns o [T, dv], S_T [dv, dk] (float64).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, np.float64)
    o = np.empty((T, dv))
    for t in range(T):
        S *= float(alpha[t])                       # decay first
        if erase:
            vhat = S @ k[t]                        # predict with decayed state
            S += float(beta[t]) * np.outer(v[t] - vhat, k[t])
        else:
            S += float(beta[t]) * np.outer(v[t], k[t])
        o[t] = S @ q[t]                            # read the new state
        if trunc_r is not None and (t + 1) % trunc_every == 0 and t + 1 < T:
            S = truncate_rank(S, trunc_r)
    return o, S


def gdn_prefill(q, k, v, alpha, beta, S0=None, *, erase=True, trunc_r=None,
                trunc_every=256, heads=None):
    """Batched layout: q, k [B, T, H, dk]; v [B, T, H, dv]; alpha, beta
    [B, T, H]; S0 [B, H, dv, dk] or None.  Returns o [B, T, H, dv] and
    S_T [B, H, dv, dk] (float64).  `heads`: optional list of (b, h) pairs to
    compute (others are left as NaN) -- for sampled checks at full size."""
    B, T, H, dk = np.shape(q)
    dv = np.shape(v)[-1]
    o = np.full((B, T, H, dv), np.nan)
    ST = np.full((B, H, dv, dk), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B)
                                            for h in range(H)]
    for b, h in todo:
        s0 = None if S0 is None else S0[b, h]
        o[b, :, h], ST[b, h] = gdn_head(
            q[b, :, h], k[b, :, h], v[b, :, h], alpha[b, :, h],
            beta[b, :, h], s0, erase=erase, trunc_r=trunc_r,
            trunc_every=trunc_every)
    return o, ST


def gdn_decode_step(q, k, v, alpha, beta, S):
    """One token for a batch of carried states: q, k [B, H, dk]; v [B, H, dv];
    alpha, beta [B, H]; S [B, H, dv, dk].  Returns o [B, H, dv], S' (fp64)."""
    B, H, dk = np.shape(q)
    dv = np.shape(v)[-1]
    o = np.empty((B, H, dv))
    S1 = np.empty((B, H, dv, dk))
    for b in range(B):
        for h in range(H):
            ob, Sb = gdn_head(np.asarray(q)[b, h][None], np.asarray(k)[b, h][None],
                              np.asarray(v)[b, h][None],
                              np.asarray(alpha)[b, h][None],
                              np.asarray(beta)[b, h][None], S[b, h])
            o[b, h], S1[b, h] = ob[0], Sb
    return o, S1


# ---------------------------------------------------------------------------
# backward pass: the exact gradient of the recurrence above
# ---------------------------------------------------------------------------

def gdn_head_backward(q, k, v, alpha, beta, S0, do, dST):
    """Gradients of L = sum_t do_t . o_t + <dST, S_T> through one head of
    gdn_head (erase on, no truncation), by the chain rule taken backwards
    over the tokens in float64.

    The pages train these layers end to end ("Linear Attention
    Architectures" reading notes, the training set-ups of its experiments;
    "On State Reduction in Linear Attention", recovery fine-tuning after
    pruning) but print no backward pass: this is the derivative of the
    forward definition and nothing more.  Per token, with S~ = alpha S_prev,
    w = v - S~ k, u = beta w and S = S~ + u k^T:
        G      = dS + do q^T              gradient reaching S_t
        dq     = S^T do
        du     = G k;   dk = G^T u - beta S~^T du
        dbeta  = du . w;   dv = beta du
        dS~    = G - beta du k^T
        dalpha = <dS~, S_prev>;   dS_prev = alpha dS~
    q, k [T, dk]; v, do [T, dv]; alpha, beta [T]; S0, dST [dv, dk] or None
    (zero).  Returns dq, dk [T, dk], dv [T, dv], dalpha, dbeta [T] and
    dS0 [dv, dk], all float64.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, np.float64)
    prev = np.empty((T, dv, dk))                   # S_{t-1} for every token
    for t in range(T):
        prev[t] = S
        S = float(alpha[t]) * S
        S = S + float(beta[t]) * np.outer(v[t] - S @ k[t], k[t])
    G = np.zeros((dv, dk)) if dST is None else np.array(dST, np.float64)
    dq = np.empty((T, dk))
    dkk = np.empty((T, dk))
    dvv = np.empty((T, dv))
    da = np.empty(T)
    db = np.empty(T)
    for t in range(T - 1, -1, -1):
        a, b = float(alpha[t]), float(beta[t])
        St = a * prev[t]                           # S~
        w = v[t] - St @ k[t]
        u = b * w
        Snew = St + np.outer(u, k[t])
        G = G + np.outer(do[t], q[t])
        dq[t] = Snew.T @ do[t]
        du = G @ k[t]
        dkk[t] = G.T @ u - b * (St.T @ du)
        db[t] = du @ w
        dvv[t] = b * du
        dSt = G - b * np.outer(du, k[t])
        da[t] = np.sum(dSt * prev[t])
        G = a * dSt
    return dq, dkk, dvv, da, db, G


def gdn_backward(q, k, v, alpha, beta, S0, do, dST=None, heads=None):
    """Batched layout of gdn_head_backward: q, k [B, T, H, dk]; v, do
    [B, T, H, dv]; alpha, beta [B, T, H]; S0, dST [B, H, dv, dk] or None.
    Returns dq, dk, dv, dalpha, dbeta, dS0 in the same layouts (float64;
    heads not in `heads`, when given, are NaN)."""
    B, T, H, dk = np.shape(q)
    dv = np.shape(v)[-1]
    dq = np.full((B, T, H, dk), np.nan)
    dkk = np.full((B, T, H, dk), np.nan)
    dvv = np.full((B, T, H, dv), np.nan)
    da = np.full((B, T, H), np.nan)
    db = np.full((B, T, H), np.nan)
    dS0 = np.full((B, H, dv, dk), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B)
                                            for h in range(H)]
    for b, h in todo:
        r = gdn_head_backward(
            q[b, :, h], k[b, :, h], v[b, :, h], alpha[b, :, h], beta[b, :, h],
            None if S0 is None else S0[b, h], do[b, :, h],
            None if dST is None else dST[b, h])
        dq[b, :, h], dkk[b, :, h], dvv[b, :, h] = r[0], r[1], r[2]
        da[b, :, h], db[b, :, h], dS0[b, h] = r[3], r[4], r[5]
    return dq, dkk, dvv, da, db, dS0


# ---------------------------------------------------------------------------
# generalised gates: per-key-channel decay (KDA), split erase/write (GDN2)
# ---------------------------------------------------------------------------

def gdn2_head(q, k, v, alpha, b, w, S0=None):
    """One head with the generalised gates, token by token in float64.

    q, k [T, dk]; v [T, dv]; alpha [T, dk] per-key-channel retention;
    b [T, dk] key-side erase gate; w [T, dv] value-side write gate;
    S0 [dv, dk] or None.  Per token ("Linear Attention Architectures"
    reading notes on paper Sec. 3.4 Kimi Delta Attention and paper Sec. 3.5 Gated
    DeltaNet-2):
        S~ = S_{t-1} diag(alpha_t)       decay on the key-feature side (right)
        e  = b_t * k_t                    the direction the erase reads
        z  = w_t * v_t                    the content written
        S_t = S~ (I - e k_t^T) + z k_t^T  erase and write both along k_t
        o_t = S_t q_t
    b = w = beta * 1 is Kimi Delta Attention; with alpha = a * 1 as well it
    is the gated delta rule of gdn_head.  Returns o [T, dv], S_T [dv, dk].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    alpha = np.asarray(alpha, np.float64)
    b = np.asarray(b, np.float64)
    w = np.asarray(w, np.float64)
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, np.float64)
    o = np.empty((T, dv))
    for t in range(T):
        S = S * alpha[t][None, :]                   # S diag(alpha): scales columns
        e = b[t] * k[t]
        z = w[t] * v[t]
        S = S - np.outer(S @ e, k[t]) + np.outer(z, k[t])
        o[t] = S @ q[t]
    return o, S


def gdn2_prefill(q, k, v, alpha, b, w, S0=None, heads=None):
    """Batched layout: q, k [B, T, H, dk]; v [B, T, H, dv]; alpha, b
    [B, T, H, dk]; w [B, T, H, dv]; S0 [B, H, dv, dk] or None.  Returns o
    [B, T, H, dv], S_T [B, H, dv, dk]; `heads` as in gdn_prefill."""
    B, T, H, dk = np.shape(q)
    dv = np.shape(v)[-1]
    o = np.full((B, T, H, dv), np.nan)
    ST = np.full((B, H, dv, dk), np.nan)
    todo = heads if heads is not None else [(bb, h) for bb in range(B) for h in range(H)]
    for bb, h in todo:
        s0 = None if S0 is None else S0[bb, h]
        o[bb, :, h], ST[bb, h] = gdn2_head(q[bb, :, h], k[bb, :, h], v[bb, :, h],
                                           alpha[bb, :, h], b[bb, :, h], w[bb, :, h], s0)
    return o, ST


# ---------------------------------------------------------------------------
# the input path of a channel-pruned layer
# ---------------------------------------------------------------------------

def qk_transform(x, channels=None, l2norm: bool = True, scale: float = 1.0):
    """Query/key vectors as the recurrence consumes them, from the raw
    projection output.

    x [..., H, dk_in] (any leading axes; the head axis is second to last).
    channels: None, or int [H, dk] -- head h keeps coordinates channels[h]
      of its dk_in-wide vector, in that order (the coordinate selection
      P_I of "On State Reduction in Linear Attention", paper Sec. 3.2-3.3, one
      subset per head).
    l2norm: divide each kept vector by its L2 norm, computed over the KEPT
      coordinates only (the same page: normalisation is recomputed on the
      retained channels).  A vector whose kept coordinates are all zero stays
      zero.
    scale: multiplies the result (a query scale; 1 for keys).
    Returns float64 [..., H, dk].
    """
    x = np.asarray(x, np.float64)
    if channels is not None:
        ch = np.asarray(channels)
        H = x.shape[-2]
        assert ch.ndim == 2 and ch.shape[0] == H
        x = np.stack([x[..., h, :][..., ch[h]] for h in range(H)], axis=-2)
    if l2norm:
        nrm = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        safe = np.where(nrm > 0.0, nrm, 1.0)
        x = np.where(nrm > 0.0, x / safe, 0.0)
    return x * float(scale)


def gdn_prefill_qk(q_raw, k_raw, v, alpha, beta, S0=None, *, channels=None,
                   l2norm=True, q_scale=1.0, heads=None):
    """The recurrence on transformed inputs: q = qk_transform(q_raw, ...,
    scale=q_scale), k = qk_transform(k_raw, ...) (no scale), then
    gdn_prefill.  q_raw, k_raw [B, T, H, dk_in]."""
    q = qk_transform(q_raw, channels, l2norm, q_scale)
    k = qk_transform(k_raw, channels, l2norm, 1.0)
    return gdn_prefill(q, k, v, alpha, beta, S0, heads=heads)


def gdn_decode_step_qk(q_raw, k_raw, v, alpha, beta, S, *, channels=None,
                       l2norm=True, q_scale=1.0):
    """One decode token on transformed inputs; q_raw, k_raw [B, H, dk_in]."""
    q = qk_transform(q_raw, channels, l2norm, q_scale)
    k = qk_transform(k_raw, channels, l2norm, 1.0)
    return gdn_decode_step(q, k, v, alpha, beta, S)


# ---------------------------------------------------------------------------
# DRRQR channel selection (strong rank-revealing QR on calibration samples)
# ---------------------------------------------------------------------------

def _qr_r(X):
    """R factor (n x n, upper triangular) of a tall X with rows >= n."""
    return np.linalg.qr(np.asarray(X, np.float64), mode="r")[: X.shape[1]]


def drrqr_select(M, k: int, f: float = 2.0, max_swaps: int = 10000):
    """Keep k of the n columns of the calibration matrix M = [K_cal; Q_cal]
    (2N x n, samples as rows, one column per key/query channel).

    "On State Reduction in Linear Attention" (reading notes), paper Sec. 3.4 and
    its Algorithm 2 / App. B.2: a QR with column pivoting gives an initial
    permutation, M P = Q [[A_k, B_k], [0, C_k]]; then, with
    U = A_k^{-1} B_k, omega_i = 1 / ||row i of A_k^{-1}||, gamma_j =
    ||column j of C_k|| and rho_ij = sqrt(U_ij^2 + (gamma_j / omega_i)^2),
    while the largest rho_ij exceeds f, selected column i and candidate
    column j trade places and the factor is re-triangularised.  Returns
    (the k kept original channel indices in permutation order, the number
    of swaps, the final max rho_ij).
    """
    M = np.asarray(M, np.float64)
    n = M.shape[1]
    assert M.shape[0] >= n and 1 <= k < n
    # column-pivoted QR by hand: at each step the remaining column of largest
    # norm (in the part below the rows already reduced) goes next
    perm = list(range(n))
    X = M.copy()
    for c in range(n):
        norms = np.linalg.norm(X[c:, c:], axis=0)
        j = c + int(np.argmax(norms))
        if j != c:
            X[:, [c, j]] = X[:, [j, c]]
            perm[c], perm[j] = perm[j], perm[c]
        # Householder reflection zeroing X[c+1:, c]
        x = X[c:, c]
        nx = np.linalg.norm(x)
        if nx == 0.0:
            continue
        v = x.copy()
        v[0] += np.copysign(nx, x[0]) if x[0] != 0 else nx
        v /= np.linalg.norm(v)
        X[c:, c:] -= 2.0 * np.outer(v, v @ X[c:, c:])
    R = np.triu(X[:n])
    swaps = 0
    while True:
        A, B, Cm = R[:k, :k], R[:k, k:], R[k:, k:]
        Ainv = np.linalg.inv(A)
        U = Ainv @ B
        omega = 1.0 / np.linalg.norm(Ainv, axis=1)
        gamma = np.linalg.norm(Cm, axis=0)
        rho = np.sqrt(U ** 2 + (gamma[None, :] / omega[:, None]) ** 2)
        i, j = np.unravel_index(int(np.argmax(rho)), rho.shape)
        if rho[i, j] <= f or swaps >= max_swaps:
            return np.array(perm[:k]), swaps, float(rho[i, j])
        a, b = int(i), k + int(j)
        R[:, [a, b]] = R[:, [b, a]]
        perm[a], perm[b] = perm[b], perm[a]
        R = _qr_r(R)
        swaps += 1


# ---------------------------------------------------------------------------
# spectral quantities and truncation
# ---------------------------------------------------------------------------

def singular_values(S: np.ndarray) -> np.ndarray:
    return np.linalg.svd(np.asarray(S, np.float64), compute_uv=False)


def stable_rank(S: np.ndarray) -> float:
    """er(S) = ||S||_F^2 / sigma_1^2 (NaN for S == 0, where it is undefined)."""
    s = singular_values(S)
    if s[0] == 0.0:
        return float("nan")
    return float(np.sum(s ** 2) / s[0] ** 2)


def utilisation(S: np.ndarray) -> float:
    """u(S) = er(S) / min(dv, dk)."""
    return stable_rank(S) / min(np.shape(S))


def condition_number(S: np.ndarray) -> float:
    """sigma_1 / sigma_min over the min(dv, dk) singular values."""
    s = singular_values(S)
    return float(s[0] / s[-1])


def entropy_erank(S: np.ndarray) -> float:
    """exp(-sum p_i log p_i), p_i = sigma_i / sum_j sigma_j (0 log 0 = 0)."""
    s = singular_values(S)
    p = s / np.sum(s)
    p = p[p > 0]
    return float(np.exp(-np.sum(p * np.log(p))))


def numerical_rank(S: np.ndarray, eps: float = 2.0 ** -23,
                   factor: float = 128.0) -> int:
    """Count of sigma_i > sigma_max * factor * eps (fp32 eps by default)."""
    s = singular_values(S)
    return int(np.sum(s > s[0] * factor * eps))


def truncate_rank(S: np.ndarray, r: int) -> np.ndarray:
    """U_r U_r^T S with U_r the top-r left singular vectors (fp64 SVD).
    r >= min(dv, dk) returns S unchanged."""
    S = np.asarray(S, np.float64)
    if r >= min(S.shape):
        return S.copy()
    U, _, _ = np.linalg.svd(S, full_matrices=False)
    Ur = U[:, :r]
    return Ur @ (Ur.T @ S)


# ---------------------------------------------------------------------------
# comparison metric
# ---------------------------------------------------------------------------

def rel_l2_per_head(x: np.ndarray, ref: np.ndarray, head_axes) -> np.ndarray:
    """||x - ref||_2 / ||ref||_2 per head.

    head_axes: the axes that index a head, e.g. (0, 2) for o [B, T, H, dv]
    and (0, 1) for S [B, H, dv, dk].  Returns an array over those axes."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    red = tuple(a for a in range(ref.ndim) if a not in head_axes)
    num = np.sqrt(np.sum((x - ref) ** 2, axis=red))
    den = np.sqrt(np.sum(ref ** 2, axis=red))
    return num / np.maximum(den, 1e-300)


def rel_err_per_token(x: np.ndarray, ref: np.ndarray, head_axes,
                      token_axis) -> np.ndarray:
    """||x_t - ref_t||_2 / rms_t ||ref_t||_2, per head and token.

    x_t is one token's slice of a head (the axes that are neither head axes
    nor the token axis, e.g. the dv values of o [B, T, H, dv] with
    head_axes (0, 2) and token_axis 1; a scalar per token for [B, T, H]).
    The denominator is the root mean square over the head's tokens of the
    reference token norms, so a token whose own output is small is judged
    on the scale of its head.  The mean of the squared result over a head's
    tokens is the square of rel_l2_per_head; its maximum sees one bad token
    that the per-head figure averages away.  Returns an array over the head
    axes and the token axis, in that axis order."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    keep = tuple(sorted(tuple(head_axes) + (token_axis,)))
    red = tuple(a for a in range(ref.ndim) if a not in keep)
    num = np.sqrt(np.sum((x - ref) ** 2, axis=red))
    tok_norm2 = np.sum(ref ** 2, axis=red)
    t_pos = keep.index(token_axis)
    rms = np.sqrt(np.mean(tok_norm2, axis=t_pos, keepdims=True))
    return num / np.maximum(rms, 1e-300)
