"""Helpers for the GPU parity tests: device upload of seeded inputs, the
oracle on the same values, and the per-head relative-L2 comparison.

Tolerances (max over heads of ||x - x_ref||_2 / ||x_ref||_2 against the fp64
oracle): 1e-3 for tensors stored in fp32 (the final state always, o when the
output dtype is fp32) and 1e-2 for o stored in bf16.
"""

import numpy as np
import torch

from oracle import gdn_oracle as orc

TOL_F32 = 1e-3
TOL_BF16 = 1e-2


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


def errs_o(o, o_ref, heads=None):
    """Per-head relative L2 of o [B, T, H, dv] (restricted to `heads`)."""
    e = orc.rel_l2_per_head(np.nan_to_num(o), np.nan_to_num(o_ref), (0, 2))
    return e if heads is None else np.array([e[b, h] for b, h in heads])


def errs_S(S, S_ref, heads=None):
    e = orc.rel_l2_per_head(np.nan_to_num(S), np.nan_to_num(S_ref), (0, 1))
    return e if heads is None else np.array([e[b, h] for b, h in heads])


def assert_close(name, err, tol):
    worst = float(np.max(err))
    print(f"  {name}: max per-head rel L2 = {worst:.3e} (tol {tol:.0e})",
          flush=True)
    assert worst <= tol, f"{name}: {worst:.3e} > {tol:.0e}"
