"""GPU parity of rank-r truncation (gdn_truncate_rank) and of the
segment-truncated prefill against the fp64 oracle.

Where sigma_r > sigma_{r+1} the truncation U_r U_r^T S is unique and is
compared element-wise (per-head relative L2, fp32 tolerance).  Where the
relative gap (sigma_r - sigma_{r+1}) / sigma_1 is tiny, several results are
correct, so only what is unique is compared: the discarded energy
||S - P S||_F^2 = sum_{i>r} sigma_i^2, the rank bound and the stable rank.
"""

import numpy as np
import pytest
import torch

from gated_deltanet_recurrent_delta_amd import binding as gdn
from oracle import gdn_oracle as orc
from tests.gpu_util import (TOL_BF16, TOL_F32, assert_close, check_o, check_S, check_step,
                            host, oracle_prefill, to_dev)
from workloads import gdn_inputs as gi

pytestmark = pytest.mark.gpu

GAP_MIN = 1e-3          # element-wise comparison needs a unique subspace


def rel_gap(S, r):
    s = orc.singular_values(S)
    return 1.0 if r >= len(s) else (s[r - 1] - s[r]) / s[0]


def check_truncation(S_in, S_out, er, r, label):
    """S_in [n, dv, dk] fp32 values (as fp64), S_out the GPU result, er the
    GPU stable ranks; compare with the oracle head by head."""
    worst = 0.0
    n_elem = 0
    for h in range(S_in.shape[0]):
        ref = orc.truncate_rank(S_in[h], r)
        s = orc.singular_values(S_in[h])
        if s[0] == 0.0:
            assert np.all(S_out[h] == 0.0) and np.isnan(er[h])
            continue
        # discarded energy is unique even when singular values tie
        tail = float(np.sum(s[r:] ** 2))
        got_tail = float(np.sum((S_in[h] - S_out[h]) ** 2))
        assert abs(got_tail - tail) <= 1e-5 * s[0] ** 2 + 1e-4 * tail, \
            (label, h, got_tail, tail)
        er_ref = orc.stable_rank(ref)
        assert er[h] == pytest.approx(er_ref, rel=1e-4), (label, h)
        so = orc.singular_values(S_out[h])
        if r < len(so):
            assert so[r] <= 1e-5 * so[0], (label, h, so[r] / so[0])
        if rel_gap(S_in[h], r) > GAP_MIN:
            e = np.linalg.norm(S_out[h] - ref) / np.linalg.norm(ref)
            worst = max(worst, e)
            n_elem += 1
    print(f"  {label}: {n_elem}/{S_in.shape[0]} heads element-wise, "
          f"max rel L2 {worst:.2e}", flush=True)
    assert worst <= TOL_F32, (label, worst)
    return n_elem


def run_truncate(S_host, r):
    S = torch.from_numpy(S_host.astype(np.float32)).cuda()
    er = gdn.truncate_rank(S, r)
    torch.cuda.synchronize()
    return host(S), er.cpu().numpy().astype(np.float64)


def prefill_states(dk, dv, H, seed, T=512):
    """Final fp32 states of an oracle prefill of tiny-case inputs."""
    x = gi.generic(1, T, H, dk, dv, seed, "bf16")
    _, ST = oracle_prefill(x)
    return ST[0].astype(np.float32).astype(np.float64)


def designed(dv, dk, sigmas, seed):
    rng = np.random.default_rng(seed)
    Qa, _ = np.linalg.qr(rng.standard_normal((dv, dv)))
    Qb, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    D = np.zeros((dv, dk))
    n = len(sigmas)
    D[:n, :n] = np.diag(sigmas)
    return (Qa @ D @ Qb.T).astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
@pytest.mark.parametrize("r", [1, 4, 12, 32, 63])
def test_truncate_prefill_states(dk, dv, r):
    S = prefill_states(dk, dv, 6, 700 + dk + dv)
    S_out, er = run_truncate(S, r)
    n = check_truncation(S, S_out, er, r, f"dk={dk} dv={dv} r={r}")
    # deep in the spectrum's tail (r = 63) the gaps are mostly below the bar
    # and only the unique quantities are compared
    if r <= 32:
        assert n >= 3


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64)])
def test_full_rank_is_identity_and_reports_stable_rank(dk, dv):
    S = prefill_states(dk, dv, 4, 71)
    for r in (min(dk, dv), 128, 1000):
        S_out, er = run_truncate(S, r)
        np.testing.assert_array_equal(S_out, S)
        for h in range(4):
            assert er[h] == pytest.approx(orc.stable_rank(S[h]), rel=1e-4)


def test_designed_spectra():
    dv = dk = 128
    mats = [
        designed(dv, dk, np.logspace(0, -6, 128), 1),       # wide range
        designed(dv, dk, 0.9 ** np.arange(128), 2),          # slow decay
        designed(dv, dk, [5.0, 3.0, 1.0], 3),                # rank 3
        designed(dv, dk, np.linspace(2.0, 1.0, 40), 4),      # flat, rank 40
    ]
    S = np.stack(mats)
    for r in (1, 2, 3, 5, 16, 39, 40, 41, 100):
        S_out, er = run_truncate(S, r)
        check_truncation(S, S_out, er, r, f"designed r={r}")
    # r at or above the rank keeps a low-rank state (to fp32 rounding)
    S_out, _ = run_truncate(S[2:3], 5)
    assert np.linalg.norm(S_out[0] - S[2]) <= 1e-5 * np.linalg.norm(S[2])


def test_tied_singular_values():
    """sigma_2 == sigma_3: any 2-dimensional subspace of the tied pair is a
    correct answer; the unique quantities must still match."""
    S = np.stack([designed(128, 128, [3.0, 2.0, 2.0, 2.0, 1.0, 0.5], 7),
                  designed(128, 128, [1.0] * 10, 8)])
    for r in (2, 3, 5):
        S_out, er = run_truncate(S, r)
        check_truncation(S, S_out, er, r, f"ties r={r}")
        # truncating the result again changes nothing
        S_again, _ = run_truncate(S_out, r)
        assert np.max(np.abs(S_again - S_out)) <= 1e-5 * np.max(np.abs(S_out))


def test_zero_and_mixed_batch():
    S = prefill_states(128, 128, 3, 9)
    S[1] = 0.0
    S_out, er = run_truncate(S, 4)
    assert np.all(S_out[1] == 0.0) and np.isnan(er[1])
    check_truncation(S, S_out, er, 4, "mixed")


def test_truncate_is_deterministic():
    S = torch.from_numpy(prefill_states(128, 128, 4, 10).astype(np.float32)).cuda()
    a, b = S.clone(), S.clone()
    ea = gdn.truncate_rank(a, 12)
    eb = gdn.truncate_rank(b, 12)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(ea, eb)


# --- segment-truncated prefill ----------------------------------------------

def oracle_truncated(x, r, heads, gap_min, segment=256):
    """The oracle's truncated recurrence, and for each head the first token
    after which its result stops being unique: the end of the first
    segment whose boundary projection has a relative gap
    (sigma_r - sigma_{r+1}) / sigma_1 <= gap_min (T if there is none)."""
    o_ref, S_ref = oracle_prefill(x, heads=heads, trunc_r=r,
                                  trunc_every=segment)
    T = x.q.shape[1]
    valid_until, min_gap = {}, {}
    for b, h in heads:
        S = None if x.S0 is None else x.S0[b, h]
        until, g_min = T, 1.0
        for t0 in range(0, T, segment):
            t1 = min(T, t0 + segment)
            _, S = orc.gdn_head(x.q[b, t0:t1, h], x.k[b, t0:t1, h],
                                x.v[b, t0:t1, h], x.alpha[b, t0:t1, h],
                                x.beta[b, t0:t1, h], S)
            if t1 < T:
                g = rel_gap(S, r)
                g_min = min(g_min, g)
                if g <= gap_min and until == T:
                    until = t1
                S = orc.truncate_rank(S, r)
        valid_until[(b, h)] = until
        min_gap[(b, h)] = g_min
    return o_ref, S_ref, valid_until, min_gap


def check_truncated_prefill(x, r, heads, label, gap_min=1e-3):
    d = to_dev(x)
    o, ST, er = gdn.prefill_truncated(d["q"], d["k"], d["v"], d["alpha"],
                                      d["beta"], r, d["S0"])
    torch.cuda.synchronize()
    o_ref, S_ref, until, gaps = oracle_truncated(x, r, heads, gap_min)
    T = x.q.shape[1]
    print(f"  {label}: unique up to {[until[bh] for bh in heads]} of {T}, "
          f"min gaps {[f'{gaps[bh]:.1e}' for bh in heads]}", flush=True)
    oh = host(o)
    for b, h in heads:
        n = until[(b, h)]
        check_o(f"{label} o (b={b}, h={h}, {n} tokens)", oh[b:b + 1, :n, h:h + 1],
                o_ref[b:b + 1, :n, h:h + 1], TOL_BF16)
    full = [bh for bh in heads if until[bh] == T]
    if full:
        check_S(f"{label} S_T", host(ST), S_ref, TOL_F32, full)
        erh = er.cpu().numpy()
        for b, h in full:
            assert erh[b, h] == pytest.approx(orc.stable_rank(S_ref[b, h]),
                                              rel=1e-3)
    return full


@pytest.mark.parametrize("r", [1, 4, 12, 32])
def test_truncated_prefill_small(r):
    x = gi.generic(1, 1024 + 37, 4, 128, 128, 300 + r, "bf16")
    heads = [(0, h) for h in range(4)]
    check_truncated_prefill(x, r, heads, f"T=1061 r={r}")


def test_truncated_prefill_batched_with_state_dk64():
    x = gi.generic(2, 600, 3, 64, 128, 55, "bf16", S0_scale=0.3)
    heads = [(b, h) for b in range(2) for h in range(3)]
    check_truncated_prefill(x, 8, heads, "B=2 dk=64 r=8")


def test_truncated_prefill_full_rank_equals_prefill():
    x = gi.generic(1, 700, 2, 128, 128, 56, "bf16")
    d = to_dev(x)
    f32 = torch.float32
    o1, S1, _ = gdn.prefill_truncated(d["q"], d["k"], d["v"], d["alpha"],
                                      d["beta"], 128, out_dtype=f32)
    o2, S2 = gdn.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                         out_dtype=f32)
    torch.cuda.synchronize()
    check_o("o", host(o1), host(o2), 1e-5)
    check_S("S", host(S1), host(S2), 1e-5)


@pytest.mark.parametrize("r", [4, 32])
def test_truncated_prefill_full_length_sampled_heads(r):
    """B=1, H=16, T=16384, dk=dv=128, 63 boundaries; the oracle follows two
    heads."""
    x = gi.truncated_prefill()
    check_truncated_prefill(x, r, [(0, 3), (0, 11)], f"T=16384 r={r}")
