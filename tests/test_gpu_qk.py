"""GPU parity of the fused input path (gdn_prefill_qk, gdn_decode_step_qk)
against the oracle: per-head channel subset of the raw q/k rows, L2
renormalisation over the kept channels and a query scale ("On State
Reduction in Linear Attention", paper Sec. 3.2-3.3), then the recurrence."""

import numpy as np
import pytest
import torch

from gated_deltanet_recurrent_delta_amd import binding as gdn
from oracle import gdn_oracle as orc
from tests.gpu_util import (TOL_BF16, TOL_F32, assert_close, check_o, check_S, check_step,
                            host, tdtype, to_dev)
from workloads import gdn_inputs as gi

pytestmark = pytest.mark.gpu

QSCALE = float(1.0 / np.sqrt(128.0))


def subsets(seed, H, dk_in, dk, permute=False):
    """Per-head channel subsets; permute=True keeps them in a random order
    (the kernels must follow the given order, not sort it)."""
    r = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(H):
        ch = r.permutation(dk_in)[:dk]
        out.append(ch if permute else np.sort(ch))
    return np.stack(out).astype(np.int32)


def dev_channels(ch):
    return None if ch is None else torch.from_numpy(np.ascontiguousarray(ch)).to("cuda")


def run_prefill_qk(x, ch, l2norm, q_scale, out_dt):
    d = to_dev(x)
    o, ST = gdn.prefill_qk(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                           channels=dev_channels(ch), l2norm=l2norm, q_scale=q_scale,
                           out_dtype=tdtype(out_dt))
    torch.cuda.synchronize()
    return o, ST


def check_prefill_qk(x, ch, l2norm=True, q_scale=1.0, out_dt=None, label="", heads=None):
    out_dt = x.dtype if out_dt is None else out_dt
    print(f"  case {label}: {x.q.shape} dk={None if ch is None else ch.shape[1]} "
          f"l2norm={l2norm} q_scale={q_scale} out={out_dt}", flush=True)
    o, ST = run_prefill_qk(x, ch, l2norm, q_scale, out_dt)
    o_ref, S_ref = orc.gdn_prefill_qk(x.q, x.k, x.v, x.alpha, x.beta, x.S0,
                                      channels=ch, l2norm=l2norm, q_scale=q_scale,
                                      heads=heads)
    tol_o = TOL_F32 if out_dt == "f32" else TOL_BF16
    check_o(f"{label} o", host(o), o_ref, tol_o, heads)
    check_S(f"{label} S_T", host(ST), S_ref, TOL_F32, heads)


@pytest.mark.parametrize("T", [1, 63, 65, 200])
@pytest.mark.parametrize("dk_in,dk,dv", [(128, 64, 128), (128, 128, 64), (100, 64, 64)])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_prefill_qk_subset_norm_scale(T, dk_in, dk, dv, dt):
    """Raw rows of dk_in channels, per-token magnitudes; dk=128 of 128 is a
    per-head permutation, dk_in=100 an odd row width."""
    ch = subsets(3000 + T + dk_in + dk, 3, dk_in, dk, permute=(dk == dk_in))
    x = gi.raw_qk(2, T, 3, dk_in, dv, 4000 + T + dk + dv, dt, channel_idx=ch,
                  S0_scale=0.3)
    check_prefill_qk(x, ch, True, QSCALE, label=f"T={T}")


@pytest.mark.parametrize("dk", [128, 64])
@pytest.mark.parametrize("dt,out_dt", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32")])
def test_prefill_qk_norm_only(dk, dt, out_dt):
    """No channel subset: the kernels normalise the dk-wide rows in place."""
    x = gi.raw_qk(2, 300, 4, dk, 128, 4100 + dk, dt, S0_scale=0.3)
    check_prefill_qk(x, None, True, 0.5, out_dt, label="norm only")


def test_prefill_qk_subset_without_normalisation():
    ch = subsets(4200, 2, 128, 64)
    x = gi.raw_qk(1, 150, 2, 128, 128, 4201, "f32", channel_idx=ch, S0_scale=0.3)
    # without normalisation the keys are used as given: give each token's
    # kept channels a norm in [0.5, 1.2] (beta |k|^2 <= 2 keeps the
    # recurrence a contraction), the other channels stay raw
    r = np.random.Generator(np.random.PCG64(4202))
    for h in range(2):
        kh = x.k[0, :, h]                                        # [T, 128] view
        kept = kh[:, ch[h]].astype(np.float64)                    # [T, 64]
        want = r.uniform(0.5, 1.2, size=(kept.shape[0], 1))
        kh[:, ch[h]] = (kept / np.linalg.norm(kept, axis=1, keepdims=True)
                        * want).astype(np.float32)
    check_prefill_qk(x, ch, False, 1.0, label="subset, no norm")


@pytest.mark.parametrize("T,dk", [(2048, 64), (1500, 128)])
def test_prefill_qk_segmented(T, dk):
    """Few heads, long sequences: the segment-parallel scan reads the
    gathered copy; transition rows carry the folded key/query factors."""
    assert gdn.prefill_segments(1, T, 2, dk, 128)[0] > 1
    ch = subsets(4300 + T, 2, 128, dk, permute=True)
    x = gi.raw_qk(1, T, 2, 128, 128, 4301 + T, "bf16", channel_idx=ch, S0_scale=0.3)
    check_prefill_qk(x, ch, True, QSCALE, label=f"segmented T={T}")


def test_prefill_qk_zero_rows():
    """Tokens whose kept q or k channels are all zero: the normalised vector
    is zero (the key writes nothing, the query reads zero)."""
    ch = subsets(4400, 2, 128, 64)
    x = gi.raw_qk(1, 130, 2, 128, 128, 4401, "bf16", channel_idx=ch, S0_scale=0.3)
    for h in range(2):
        x.k[0, 5, h, ch[h]] = 0.0
        x.k[0, 64, h, ch[h]] = 0.0
        x.q[0, 7, h, ch[h]] = 0.0
        x.q[0, 129, h, ch[h]] = 0.0
    check_prefill_qk(x, ch, True, 1.0, "f32", label="zero rows")


@pytest.mark.parametrize("dt,out_dt,T", [("bf16", "bf16", 200), ("f32", "f32", 70),
                                         ("bf16", "bf16", 2048)])
def test_prefill_qk_identity_equals_prefill_bitwise(dt, out_dt, T):
    x = gi.generic(1, T, 2, 128, 128, 4500 + T, dt, S0_scale=0.3)
    d = to_dev(x)
    o1, S1 = gdn.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                         out_dtype=tdtype(out_dt))
    o2, S2 = gdn.prefill_qk(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                            channels=None, l2norm=False, q_scale=1.0,
                            out_dtype=tdtype(out_dt))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_prefill_qk_batched_full_size_sampled_heads():
    """The batched prefill's shape (B=8, H=16, T=4096, dv=128) at dk=64
    from 128-wide raw rows, in the benchmark's launch configuration; the
    oracle follows three (batch, head) pairs."""
    ch = gi.pruning_subsets(4, 16, 128, 64)
    x = gi.raw_qk(8, 4096, 16, 128, 128, gi.seed_for(4, 5), "bf16", channel_idx=ch)
    heads = [(0, 0), (3, 7), (7, 15)]
    check_prefill_qk(x, ch, True, QSCALE, label="B=8 T=4096 dk=64<-128", heads=heads)


# --- decode ----------------------------------------------------------------

def decode_inputs(B, H, dk_in, dk, dv, dt, seed, permute=False):
    ch = subsets(seed, H, dk_in, dk, permute) if dk_in != dk or permute else None
    x = gi.raw_qk(B, 1, H, dk_in, dv, seed + 1, dt, channel_idx=ch, S0_scale=0.5)
    return x, ch


@pytest.mark.parametrize("B,H", [(3, 4), (64, 16)])
@pytest.mark.parametrize("dk_in,dk,dv,permute", [(128, 64, 128, False), (128, 128, 128, True),
                                                 (100, 64, 64, False), (64, 64, 128, False)])
@pytest.mark.parametrize("in_dt,out_dt", [("bf16", "bf16"), ("f32", "f32")])
def test_decode_qk_matches_oracle(B, H, dk_in, dk, dv, permute, in_dt, out_dt):
    x, ch = decode_inputs(B, H, dk_in, dk, dv, in_dt, 5000 + B + dk_in + dk + dv, permute)
    d = to_dev(x)
    sq = lambda t: t[:, 0].contiguous()
    o, S1 = gdn.decode_step_qk(sq(d["q"]), sq(d["k"]), sq(d["v"]), sq(d["alpha"]),
                               sq(d["beta"]), d["S0"], channels=dev_channels(ch),
                               l2norm=True, q_scale=QSCALE, out_dtype=tdtype(out_dt))
    torch.cuda.synchronize()
    o_ref, S_ref = orc.gdn_decode_step_qk(x.q[:, 0], x.k[:, 0], x.v[:, 0], x.alpha[:, 0],
                                          x.beta[:, 0], x.S0, channels=ch, l2norm=True,
                                          q_scale=QSCALE)
    tol_o = TOL_F32 if out_dt == "f32" else TOL_BF16
    check_step("o", host(o), o_ref, tol_o)
    check_S("S'", host(S1), S_ref, TOL_F32)


@pytest.mark.parametrize("dk", [128, 64])
def test_decode_qk_identity_equals_decode_bitwise(dk):
    x = gi.generic(64, 1, 16, dk, 128, 5100 + dk, "bf16", S0_scale=0.5)
    d = to_dev(x)
    args = [d[n][:, 0].contiguous() for n in ("q", "k", "v", "alpha", "beta")]
    o1, S1 = gdn.decode_step(*args, d["S0"])
    o2, S2 = gdn.decode_step_qk(*args, d["S0"], channels=None, l2norm=False, q_scale=1.0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_decode_qk_chain_matches_prefill_qk():
    """A prompt by prefill_qk, then 40 decode_step_qk tokens in place, against
    the oracle's token-by-token run over the same raw inputs."""
    ch = subsets(5200, 4, 128, 64)
    x = gi.raw_qk(2, 300, 4, 128, 128, 5201, "bf16", channel_idx=ch)
    Tp = 260
    d = to_dev(x)
    chd = dev_channels(ch)
    sl = lambda t: t[:, :Tp].contiguous()
    o_p, S = gdn.prefill_qk(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["alpha"]),
                            sl(d["beta"]), channels=chd, q_scale=QSCALE)
    outs = []
    for t in range(Tp, 300):
        st = lambda n: d[n][:, t].contiguous()
        o_t, _ = gdn.decode_step_qk(st("q"), st("k"), st("v"), st("alpha"), st("beta"),
                                    S, S_out=S, channels=chd, q_scale=QSCALE)
        outs.append(o_t)
    torch.cuda.synchronize()
    o_ref, S_ref = orc.gdn_prefill_qk(x.q, x.k, x.v, x.alpha, x.beta, channels=ch,
                                      q_scale=QSCALE)
    o_dec = torch.stack(outs, dim=1)
    check_o("prompt o", host(o_p), o_ref[:, :Tp], TOL_BF16)
    check_o("decode o", host(o_dec), o_ref[:, Tp:], TOL_BF16)
    check_S("S", host(S), S_ref, TOL_F32)


@pytest.mark.parametrize("T", [0, 130, 1500])
def test_prefill_qk_in_place_state_and_empty(T):
    """ST aliasing S0 (segmented at T=1500), and T = 0 copying S0."""
    H = 2
    ch = subsets(4600 + T, H, 128, 64)
    x = gi.raw_qk(1, max(T, 1), H, 128, 128, 4601 + T, "bf16", channel_idx=ch, S0_scale=0.3)
    d = to_dev(x)
    if T == 0:
        d = {n: (t[:, :0].contiguous() if n in ("q", "k", "v", "alpha", "beta") else t)
             for n, t in d.items()}
    S = d["S0"].clone()
    o, ST = gdn.prefill_qk(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S, ST=S,
                           channels=dev_channels(ch), q_scale=QSCALE)
    torch.cuda.synchronize()
    assert ST.data_ptr() == S.data_ptr()
    if T == 0:
        assert torch.equal(ST, d["S0"])
        return
    o_ref, S_ref = orc.gdn_prefill_qk(x.q, x.k, x.v, x.alpha, x.beta, x.S0, channels=ch,
                                      q_scale=QSCALE)
    check_o("o", host(o), o_ref, TOL_BF16)
    check_S("S_T", host(ST), S_ref, TOL_F32)


def test_prefill_qk_zero_initial_state_and_decode_in_place():
    ch = subsets(4700, 4, 128, 64)
    x = gi.raw_qk(2, 90, 4, 128, 128, 4701, "bf16", channel_idx=ch)
    check_prefill_qk(x, ch, True, QSCALE, label="S0=None")
    y = gi.raw_qk(8, 1, 4, 128, 128, 4702, "bf16", channel_idx=ch, S0_scale=0.4)
    d = to_dev(y)
    sq = lambda t: t[:, 0].contiguous()
    S = d["S0"].clone()
    o, S1 = gdn.decode_step_qk(sq(d["q"]), sq(d["k"]), sq(d["v"]), sq(d["alpha"]),
                               sq(d["beta"]), S, S_out=S, channels=dev_channels(ch),
                               q_scale=QSCALE)
    torch.cuda.synchronize()
    assert S1.data_ptr() == S.data_ptr()
    o_ref, S_ref = orc.gdn_decode_step_qk(y.q[:, 0], y.k[:, 0], y.v[:, 0], y.alpha[:, 0],
                                          y.beta[:, 0], y.S0, channels=ch, q_scale=QSCALE)
    check_step("o", host(o), o_ref, TOL_BF16)
    check_S("S'", host(S1), S_ref, TOL_F32)


@pytest.mark.parametrize("dk_in,dk", [(128, 64), (128, 128)])
def test_prefill_qk_16k_segmented_sampled_heads(dk_in, dk):
    """The 16K-token layer shape (B=1, H=16, T=16384, dv=128) from raw rows:
    128 -> 64 through the channel subset, or 128 wide with normalisation
    only; the segmented path; the oracle follows two heads."""
    H, T = 16, 16384
    ch = gi.pruning_subsets(2, H, dk_in, dk) if dk != dk_in else None
    assert gdn.prefill_segments(1, T, H, dk, 128)[0] > 1
    x = gi.raw_qk(1, T, H, dk_in, 128, gi.seed_for(2, 5), "bf16", channel_idx=ch)
    check_prefill_qk(x, ch, True, QSCALE, label=f"16K {dk_in}->{dk}", heads=[(0, 3), (0, 12)])


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_out_of_range_channels_are_clamped(dt):
    """Channel indices outside [0, dk_in) are clamped into the row by the
    kernels (never read out of bounds): the results equal those of the
    clamped subset, bitwise, and match the oracle on it.  bf16 rows 128 wide
    take the prepare kernel's staged path, fp32 rows the element path."""
    H, dk_in, dk = 3, 128, 64
    ch = subsets(6100, H, dk_in, dk)
    bad = ch.copy()
    bad[0, 5], bad[1, 0], bad[2, 63], bad[2, 10] = -7, 1 << 20, dk_in, -(1 << 30)
    good = np.clip(bad, 0, dk_in - 1).astype(np.int32)
    x = gi.raw_qk(2, 150, H, dk_in, 128, 6101, dt, channel_idx=good, S0_scale=0.3)
    d = to_dev(x)
    res = []
    for c in (bad, good):
        res.append(gdn.prefill_qk(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                                  channels=dev_channels(c), q_scale=QSCALE,
                                  validate=False))
    sq = lambda t: t[:, 0].contiguous()
    for c in (bad, good):
        res.append(gdn.decode_step_qk(sq(d["q"]), sq(d["k"]), sq(d["v"]), sq(d["alpha"]),
                                      sq(d["beta"]), d["S0"], channels=dev_channels(c),
                                      q_scale=QSCALE, validate=False))
    torch.cuda.synchronize()
    for (o1, S1), (o2, S2) in ((res[0], res[1]), (res[2], res[3])):
        assert torch.equal(o1, o2) and torch.equal(S1, S2)
    o_ref, S_ref = orc.gdn_prefill_qk(x.q, x.k, x.v, x.alpha, x.beta, x.S0,
                                      channels=good, l2norm=True, q_scale=QSCALE)
    tol_o = TOL_F32 if dt == "f32" else TOL_BF16
    check_o("clamped o", host(res[0][0]), o_ref, tol_o)
    check_S("clamped S_T", host(res[0][1]), S_ref, TOL_F32)
