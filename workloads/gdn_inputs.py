"""Seeded synthetic inputs for the gated delta rule.

This module draws the tensors that both the HIP path and the fp64 oracle
consume.  It holds none of the recurrence's arithmetic: it only draws random
numbers, normalises query/key vectors (a precondition of the method, not a
step of it), gathers kept key/query channels, and rounds to the storage type.

Shapes (contiguous, row-major):
    q, k   [B, T, H, dk]        v   [B, T, H, dv]
    alpha, beta  [B, T, H]      S0  [B, H, dv, dk] or None

Every array is returned as numpy float32 holding exactly the values the device
receives: for bf16 workloads q/k/v are rounded to bf16 (round-to-nearest-even)
and stored back in float32, so up-casting them to fp64 is exact.

Where the workloads come from
-----------------------------
* Per-token distributions (q, k ~ N(0, I) then unit L2 norm; v ~ N(0, I);
  beta = sigmoid(N(0, 1)); log alpha ~ -U(lo, hi)) follow the tiny single-layer
  case and are reused for the batched and decode workloads.
* Keys "in a narrow cone" model the long-horizon heads of the state-rank post
  ("How much of its state does Gated DeltaNet use?", §2): unit-norm keys whose
  mean has norm about 0.85.
* The 10-of-16 short-horizon head split stands for that post's finding that
  about 61 % of heads forget within 256 tokens (§2); round(0.61 * 16) = 10.
* The channel-pruned width dk' = dk/2 uses a per-head coordinate selection
  P_I shared by q and k, with normalisation recomputed over the kept
  coordinates ("On State Reduction in Linear Attention", paper Sec. 3.2-3.3, and the
  Rand selector of paper Sec. 3.4).
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

SEED_BASE = 20260000


def seed_for(config: int, variant: int = 0) -> int:
    """Seed of workload `config` (1-5), `variant` 0-9."""
    return SEED_BASE + 10 * config + variant


# ---------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------

def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); float32 out.

    Finite inputs only (the generators never produce inf/nan).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(x.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------
# building blocks
# ---------------------------------------------------------------------------

def _unit(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / np.maximum(n, 1e-30)).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def mean_key_norm(keys: np.ndarray) -> float:
    """Norm of the mean of a set of (unit) key vectors, keys [..., d]."""
    k = keys.reshape(-1, keys.shape[-1]).astype(np.float64)
    return float(np.linalg.norm(k.mean(axis=0)))


def cone_sigma(d: int, target: float = 0.85, n_keys: int = 20000,
               seed: int = SEED_BASE + 9) -> float:
    """Noise scale sigma such that keys normalise(mu + sigma z) have a mean of
    norm `target` (bisection on a fixed seeded sample of `n_keys` keys)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    mu = _unit(rng.standard_normal(d))
    z = rng.standard_normal((n_keys, d)).astype(np.float32)
    lo, hi = 1e-4, 1.0
    for _ in range(50):
        mid = 0.5 * (lo + hi)
        m = mean_key_norm(_unit(mu[None, :] + mid * z))
        if m > target:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def channel_subsets(rng: np.random.Generator, H: int, dk: int,
                    dk_keep: int) -> np.ndarray:
    """Per-head sorted random subsets I_h of `dk_keep` of `dk` channels
    (the Rand selector); int32 [H, dk_keep]."""
    idx = np.stack([np.sort(rng.permutation(dk)[:dk_keep]) for _ in range(H)])
    return idx.astype(np.int32)


def gather_channels(x_raw: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """x_raw [B, T, H, dk] -> [B, T, H, dk'] keeping channels idx[h] of head h."""
    H = x_raw.shape[2]
    out = np.empty(x_raw.shape[:3] + (idx.shape[1],), dtype=x_raw.dtype)
    for h in range(H):
        out[:, :, h, :] = x_raw[:, :, h, idx[h]]
    return out


# ---------------------------------------------------------------------------
# workload container
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class GdnInputs:
    """One batch of recurrence inputs (numpy float32, exact device values)."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray
    beta: np.ndarray
    S0: Optional[np.ndarray]
    dtype: str                 # storage type of q/k/v/o: "bf16" or "f32"
    seed: int
    name: str
    channel_idx: Optional[np.ndarray] = None   # [H, dk'] when channel-pruned

    @property
    def dims(self):
        B, T, H, dk = self.q.shape
        return dict(B=B, T=T, H=H, dk=dk, dv=self.v.shape[-1])

    def slice_time(self, t0: int, t1: int, S0=None) -> "GdnInputs":
        return dataclasses.replace(
            self, q=self.q[:, t0:t1].copy(), k=self.k[:, t0:t1].copy(),
            v=self.v[:, t0:t1].copy(), alpha=self.alpha[:, t0:t1].copy(),
            beta=self.beta[:, t0:t1].copy(), S0=S0,
            name=f"{self.name}[{t0}:{t1}]")

    def slice_batch(self, b0: int, b1: int) -> "GdnInputs":
        return dataclasses.replace(
            self, q=self.q[b0:b1].copy(), k=self.k[b0:b1].copy(),
            v=self.v[b0:b1].copy(), alpha=self.alpha[b0:b1].copy(),
            beta=self.beta[b0:b1].copy(),
            S0=None if self.S0 is None else self.S0[b0:b1].copy(),
            name=f"{self.name}[b{b0}:{b1}]")


def _finish(q, k, v, alpha, beta, S0, dtype, seed, name, idx=None):
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    elif dtype != "f32":
        raise ValueError(dtype)
    return GdnInputs(q=np.ascontiguousarray(q, np.float32),
                     k=np.ascontiguousarray(k, np.float32),
                     v=np.ascontiguousarray(v, np.float32),
                     alpha=np.ascontiguousarray(alpha, np.float32),
                     beta=np.ascontiguousarray(beta, np.float32),
                     S0=S0, dtype=dtype, seed=seed, name=name,
                     channel_idx=idx)


def _decay(rng, shape, lo, hi):
    """alpha = exp(-U(lo, hi)) drawn in fp64, stored once as fp32."""
    return np.exp(-rng.uniform(lo, hi, size=shape)).astype(np.float32)


# ---------------------------------------------------------------------------
# the workloads
# ---------------------------------------------------------------------------

def generic(B: int, T: int, H: int, dk: int, dv: int, seed: int,
            dtype: str = "f32", log_alpha_range=(0.001, 0.1),
            S0_scale: Optional[float] = None, name: str = "generic",
            channel_idx: Optional[np.ndarray] = None,
            rows: Optional[Sequence[int]] = None) -> GdnInputs:
    """Tiny-case distributions at any shape: q, k ~ N(0, I) normalised,
    v ~ N(0, I), beta = sigmoid(N(0, 1)), log alpha ~ -U(range).

    Batch row b is drawn from its own stream PCG64(seed).jumped(b), so any
    subset of rows can be regenerated alone: `rows` selects the batch rows to
    draw (the result then has len(rows) rows; default all B).
    S0_scale: if given, S0 ~ S0_scale * N(0, 1) (else S0 = None, a zero state).
    channel_idx: if given ([H, dk'] int), draw raw dk-wide q/k, keep channels
    channel_idx[h] of head h and normalise over the kept channels.
    """
    rows = list(range(B)) if rows is None else [int(r) for r in rows]
    idx = None if channel_idx is None else np.asarray(channel_idx, np.int32)
    dko = dk if idx is None else idx.shape[1]
    n = len(rows)
    q = np.empty((n, T, H, dko), np.float32)
    k = np.empty((n, T, H, dko), np.float32)
    v = np.empty((n, T, H, dv), np.float32)
    beta = np.empty((n, T, H), np.float32)
    alpha = np.empty((n, T, H), np.float32)
    S0 = None if S0_scale is None else np.empty((n, H, dv, dko), np.float32)
    for i, b in enumerate(rows):
        assert 0 <= b < B
        rng = np.random.Generator(np.random.PCG64(seed).jumped(b))
        qr = rng.standard_normal((1, T, H, dk), dtype=np.float32)
        kr = rng.standard_normal((1, T, H, dk), dtype=np.float32)
        v[i] = rng.standard_normal((T, H, dv), dtype=np.float32)
        beta[i] = _sigmoid(rng.standard_normal((T, H)))
        alpha[i] = _decay(rng, (T, H), *log_alpha_range)
        if S0 is not None:
            s0 = (S0_scale * rng.standard_normal((H, dv, dk))).astype(np.float32)
            S0[i] = s0 if idx is None else s0[..., :dko]
        if idx is not None:
            assert idx.shape[0] == H and idx.shape[1] <= dk
            qr, kr = gather_channels(qr, idx), gather_channels(kr, idx)
        q[i], k[i] = _unit(qr)[0], _unit(kr)[0]
    return _finish(q, k, v, alpha, beta, S0, dtype, seed, name, idx)


def raw_qk(B: int, T: int, H: int, dk_in: int, dv: int, seed: int,
           dtype: str = "bf16", channel_idx: Optional[np.ndarray] = None,
           log_alpha_range=(0.001, 0.1), S0_scale: Optional[float] = None,
           rows: Optional[Sequence[int]] = None,
           name: str = "raw-qk") -> GdnInputs:
    """Inputs of a layer whose query/key normalisation and channel selection
    are left to the recurrence's own input path: q and k are raw
    dk_in-wide projection outputs, NOT normalised and NOT gathered.

    q, k = N(0, I) directions times a per-token magnitude exp(N(0, 0.5^2)),
    so every token has its own norm; v ~ N(0, I); beta = sigmoid(N(0, 1));
    log alpha ~ -U(range); S0 ~ S0_scale * N(0, 1) of the kept width, or
    None.  channel_idx ([H, dk] int) is returned as .channel_idx and only
    sets the width of S0.  Row b is drawn from PCG64(seed).jumped(b).
    """
    rows = list(range(B)) if rows is None else [int(r) for r in rows]
    idx = None if channel_idx is None else np.asarray(channel_idx, np.int32)
    dk = dk_in if idx is None else idx.shape[1]
    n = len(rows)
    q = np.empty((n, T, H, dk_in), np.float32)
    k = np.empty((n, T, H, dk_in), np.float32)
    v = np.empty((n, T, H, dv), np.float32)
    beta = np.empty((n, T, H), np.float32)
    alpha = np.empty((n, T, H), np.float32)
    S0 = None if S0_scale is None else np.empty((n, H, dv, dk), np.float32)
    for i, b in enumerate(rows):
        assert 0 <= b < B
        rng = np.random.Generator(np.random.PCG64(seed).jumped(b))
        for x in (q, k):
            mag = np.exp(0.5 * rng.standard_normal((T, H, 1))).astype(np.float32)
            x[i] = mag * rng.standard_normal((T, H, dk_in), dtype=np.float32)
        v[i] = rng.standard_normal((T, H, dv), dtype=np.float32)
        beta[i] = _sigmoid(rng.standard_normal((T, H)))
        alpha[i] = _decay(rng, (T, H), *log_alpha_range)
        if S0 is not None:
            S0[i] = (S0_scale * rng.standard_normal((H, dv, dk))).astype(np.float32)
    return _finish(q, k, v, alpha, beta, S0, dtype, seed, name, idx)


def gate_vectors(B: int, T: int, H: int, dk: int, dv: int, seed: int,
                 log_alpha_range=(0.001, 0.1)):
    """Gates of the generalised recurrence, float32: a retention per key
    channel alpha = exp(-U(range)) [B, T, H, dk], an erase gate per key
    channel b = sigmoid(N(0, 1)) [B, T, H, dk] and a write gate per value
    channel w = sigmoid(N(0, 1)) [B, T, H, dv]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    alpha = _decay(rng, (B, T, H, dk), *log_alpha_range)
    b = _sigmoid(rng.standard_normal((B, T, H, dk)))
    w = _sigmoid(rng.standard_normal((B, T, H, dv)))
    return alpha, b, w


def cotangents(B: int, T: int, H: int, dk: int, dv: int, seed: int,
               dtype: str = "f32", rows: Optional[Sequence[int]] = None):
    """Gradients flowing into a layer's outputs, for the backward pass:
    d_o ~ N(0, 1) [B, T, H, dv] (rounded to bf16 when dtype is "bf16", the
    storage dtype of o) and dST ~ N(0, 1) [B, H, dv, dk] float32.  Batch row
    b from its own stream PCG64(seed).jumped(b), like generic()."""
    rows = list(range(B)) if rows is None else [int(r) for r in rows]
    d_o = np.empty((len(rows), T, H, dv), np.float32)
    dST = np.empty((len(rows), H, dv, dk), np.float32)
    for i, b in enumerate(rows):
        assert 0 <= b < B
        rng = np.random.Generator(np.random.PCG64(seed).jumped(b))
        d_o[i] = rng.standard_normal((T, H, dv), dtype=np.float32)
        dST[i] = rng.standard_normal((H, dv, dk), dtype=np.float32)
    if dtype == "bf16":
        d_o = round_bf16(d_o)
    elif dtype != "f32":
        raise ValueError(dtype)
    return np.ascontiguousarray(d_o, np.float32), dST


def pruning_subsets(config: int, H: int = 16, dk: int = 128,
                    dk_keep: int = 64) -> np.ndarray:
    """The fixed per-head channel subsets P_I of a channel-pruned layer
    (one draw per workload family, shared by all its inputs)."""
    rng = np.random.Generator(np.random.PCG64(seed_for(config, 9)))
    return channel_subsets(rng, H, dk, dk_keep)


def tiny(seed: Optional[int] = None) -> GdnInputs:
    """Tiny gated delta rule, single layer: B=1, H=2, T=512, dk=dv=64, fp32."""
    s = seed_for(1) if seed is None else seed
    return generic(1, 512, 2, 64, 64, s, "f32", name="tiny-fp32")


def prefill_16k(T: int = 16384, H: int = 16, d: int = 128,
                seed: Optional[int] = None, n_short: Optional[int] = None,
                sigma: Optional[float] = None) -> GdnInputs:
    """Qwen3.5-0.8B-shaped GDN layer prefill: B=1, H=16, T=16384,
    dk=dv=128, bf16 q/k/v, fp32 alpha/beta, zero initial state.

    Keys: per head a seeded unit mean direction mu_h plus N(0, sigma^2) noise,
    then unit-normalised; sigma is chosen so the mean key has norm ~0.85.
    Decay: round(0.61 H) short-horizon heads with log alpha ~ -U(0.004, 0.1),
    the rest long-horizon with -U(1e-4, 1e-3); heads chosen by a seeded
    permutation.  q ~ N(0, I) normalised, v ~ N(0, I), beta = sigmoid(N(0,1)).
    """
    s = seed_for(2) if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(s))
    if sigma is None:
        sigma = cone_sigma(d)
    if n_short is None:
        n_short = int(round(0.61 * H))
    perm = rng.permutation(H)
    short = np.zeros(H, dtype=bool)
    short[perm[:n_short]] = True
    mu = _unit(rng.standard_normal((H, d)))
    z = rng.standard_normal((1, T, H, d), dtype=np.float32)
    k = _unit(mu[None, None, :, :] + np.float32(sigma) * z)
    del z
    q = _unit(rng.standard_normal((1, T, H, d), dtype=np.float32))
    v = rng.standard_normal((1, T, H, d), dtype=np.float32)
    beta = _sigmoid(rng.standard_normal((1, T, H)))
    alpha = np.empty((1, T, H), dtype=np.float32)
    for h in range(H):
        lo, hi = (0.004, 0.1) if short[h] else (1e-4, 1e-3)
        alpha[0, :, h] = _decay(rng, (T,), lo, hi)
    out = _finish(q, k, v, alpha, beta, None, "bf16", s, f"prefill-T{T}")
    out.short_heads = short          # type: ignore[attr-defined]
    out.sigma = sigma                # type: ignore[attr-defined]
    return out


def batched_prefill(B: int = 8, T: int = 4096, H: int = 16, dk: int = 128,
                    dv: int = 128, seed: Optional[int] = None,
                    rows: Optional[Sequence[int]] = None) -> GdnInputs:
    """Batched prefill for the state-halving comparison: B=8, H=16, T=4096,
    dv=128, dk in {128, 64}, bf16 inputs, tiny-case distributions.  The
    dk=64 variant reuses the dk=128 raw draws through a per-head seeded
    channel subset (normalised over the kept channels)."""
    s = seed_for(4) if seed is None else seed
    idx = None if dk == 128 else pruning_subsets(4, H, 128, dk)
    return generic(B, T, H, 128, dv, s, "bf16", channel_idx=idx,
                   name=f"batched-prefill-dk{dk}", rows=rows)


def decode_prompt(B: int = 64, T: int = 2048, H: int = 16, dk: int = 128,
                  dv: int = 128, seed: Optional[int] = None,
                  rows: Optional[Sequence[int]] = None) -> GdnInputs:
    """Prompt whose prefill initialises the carried decode states
    (tiny-case distributions, bf16 inputs, dk=64 by channel subset)."""
    s = seed_for(3, 0) if seed is None else seed
    idx = None if dk == 128 else pruning_subsets(3, H, 128, dk)
    return generic(B, T, H, 128, dv, s, "bf16", channel_idx=idx,
                   name=f"decode-prompt-B{B}-dk{dk}", rows=rows)


def decode_steps(B: int = 64, n_steps: int = 512, H: int = 16, dk: int = 128,
                 dv: int = 128, seed: Optional[int] = None,
                 rows: Optional[Sequence[int]] = None) -> GdnInputs:
    """`n_steps` fresh single-token inputs for the decode loop, laid out as a
    [B, n_steps, H, *] sequence (step t is [:, t])."""
    s = seed_for(3, 1) if seed is None else seed
    idx = None if dk == 128 else pruning_subsets(3, H, 128, dk)
    return generic(B, n_steps, H, 128, dv, s, "bf16", channel_idx=idx,
                   name=f"decode-steps-B{B}-dk{dk}", rows=rows)


def truncated_prefill(T: int = 16384, H: int = 16, d: int = 128,
                      seed: Optional[int] = None) -> GdnInputs:
    """Segment-truncated prefill: B=1, H=16, T=16384, dk=dv=128, tiny-case
    distributions, bf16 inputs."""
    s = seed_for(5) if seed is None else seed
    return generic(1, T, H, d, d, s, "bf16", name=f"truncated-prefill-T{T}")
