"""Helpers for the GPU parity tests: device upload of seeded inputs, the
oracle on the same values, and the comparisons.

Tolerance stated for this path (max over heads of ||x - x_ref||_2 /
||x_ref||_2 against the fp64 oracle): 1e-3 for tensors stored in fp32 (the
final state always, o when the output dtype is fp32) and 1e-2 for o stored
in bf16.

Every comparison also bounds each token on its own (each state row, for S):
||x_t - x_ref,t||_2 divided by the root-mean-square token norm of the
reference head must stay within TOKEN_FACTOR times the per-head tolerance.
The per-head figure is the root mean square of these per-token errors, so
at T = 16384 one wrong token moves it by only ~1/sqrt(T); the per-token
bound catches it.  The factor allows for the spread of per-token errors
around their mean: bf16 rounding of o alone is up to 2^-8 of a token's own
norm, and token norms in a head spread over a few times their rms.
Non-finite values fail outright.
"""

import numpy as np
import torch

from oracle import gdn_oracle as orc

TOL_F32 = 1e-3
TOL_BF16 = 1e-2
TOKEN_FACTOR = 3.0


def tdtype(name):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def to_dev(x, dev="cuda"):
    """GdnInputs -> dict of device tensors with the storage dtypes."""
    dt = tdtype(x.dtype)
    d = dict(q=torch.from_numpy(x.q).to(dev).to(dt).contiguous(),
             k=torch.from_numpy(x.k).to(dev).to(dt).contiguous(),
             v=torch.from_numpy(x.v).to(dev).to(dt).contiguous(),
             alpha=torch.from_numpy(x.alpha).to(dev).contiguous(),
             beta=torch.from_numpy(x.beta).to(dev).contiguous(),
             S0=None if x.S0 is None else torch.from_numpy(x.S0).to(dev).contiguous())
    return d


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def oracle_prefill(x, heads=None, S0=None, **kw):
    s0 = x.S0 if S0 is None else S0
    return orc.gdn_prefill(x.q, x.k, x.v, x.alpha, x.beta, s0, heads=heads, **kw)


def _select_heads(x, head_axes, token_axis, heads):
    """Move the head axes to the front and keep only `heads` (a list of
    index tuples over the head axes), stacked on one leading axis.
    Returns the array and the token axis' new position."""
    x = np.asarray(x, np.float64)
    front = tuple(range(len(head_axes)))
    xm = np.moveaxis(x, tuple(head_axes), front)
    rest = [a for a in range(x.ndim) if a not in head_axes]
    tpos = len(head_axes) + rest.index(token_axis)
    if heads is None:
        nh = int(np.prod([x.shape[a] for a in head_axes]))
        xs = xm.reshape((nh,) + xm.shape[len(head_axes):])
    else:
        xs = np.stack([xm[tuple(h)] for h in heads])
    return xs, tpos - len(head_axes) + 1


def check_tokens(name, x, ref, head_axes, token_axis, tol, heads=None,
                 token_tol=None):
    """Assert finiteness, the per-head relative L2 (<= tol) and the
    per-token bound (<= token_tol, default TOKEN_FACTOR * tol)."""
    token_tol = TOKEN_FACTOR * tol if token_tol is None else token_tol
    xs, tpos = _select_heads(x, head_axes, token_axis, heads)
    rs, _ = _select_heads(ref, head_axes, token_axis, heads)
    bad = int(np.size(xs) - np.count_nonzero(np.isfinite(xs)))
    assert bad == 0, f"{name}: {bad} non-finite values"
    assert np.all(np.isfinite(rs)), f"{name}: non-finite reference"
    ph = orc.rel_l2_per_head(xs, rs, (0,))
    pt = orc.rel_err_per_token(xs, rs, (0,), tpos)
    worst_h, worst_t = float(np.max(ph, initial=0.0)), float(np.max(pt, initial=0.0))
    print(f"  {name}: max per-head rel L2 = {worst_h:.3e} (tol {tol:.0e}); "
          f"max per-token = {worst_t:.3e} (tol {token_tol:.0e})", flush=True)
    assert worst_h <= tol, f"{name}: per-head {worst_h:.3e} > {tol:.0e}"
    if worst_t > token_tol:
        i = np.unravel_index(int(np.argmax(pt)), pt.shape)
        raise AssertionError(f"{name}: per-token {worst_t:.3e} > {token_tol:.0e} "
                             f"at (head #{i[0]}, token {i[1]})")


def check_o(name, o, o_ref, tol, heads=None, **kw):
    """o [B, T, H, dv]: per head (b, h) and per token t."""
    check_tokens(name, o, o_ref, (0, 2), 1, tol, heads, **kw)


def check_S(name, S, S_ref, tol, heads=None, **kw):
    """S [B, H, dv, dk]: per head (b, h) and per state row (value channel)."""
    check_tokens(name, S, S_ref, (0, 1), 2, tol, heads, **kw)


def check_step(name, o, o_ref, tol):
    """One decode step's o [B, H, dv]: a head holds a single token, so the
    finer check is per value element, on the scale of the head's rms
    element."""
    check_tokens(name, o, o_ref, (0, 1), 2, tol, token_tol=tol * TOKEN_FACTOR)


def assert_close(name, err, tol):
    """For scalar-per-head comparisons that have no token axis."""
    err = np.asarray(err, np.float64)
    assert np.all(np.isfinite(err)), f"{name}: non-finite error"
    worst = float(np.max(err))
    print(f"  {name}: max per-head rel L2 = {worst:.3e} (tol {tol:.0e})",
          flush=True)
    assert worst <= tol, f"{name}: {worst:.3e} > {tol:.0e}"
