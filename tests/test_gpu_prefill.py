"""GPU parity of the chunked prefill (gdn_prefill) against the fp64 oracle."""

import numpy as np
import pytest
import torch

from gated_deltanet_recurrent_delta_amd import binding as gdn
from oracle import gdn_oracle as orc
from tests.gpu_util import (TOL_BF16, TOL_F32, assert_close, check_o, check_S, check_step,
                            host, oracle_prefill, tdtype, to_dev)
from workloads import gdn_inputs as gi

pytestmark = pytest.mark.gpu


def run(x, out_dtype=None, S0=None, **kw):
    d = to_dev(x)
    s0 = d["S0"] if S0 is None else S0
    o, ST = gdn.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], s0,
                        out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return o, ST


def check_full(x, out_dt=None, label=""):
    out_dt = x.dtype if out_dt is None else out_dt
    o, ST = run(x, out_dtype=tdtype(out_dt))
    o_ref, S_ref = oracle_prefill(x)
    tol_o = TOL_F32 if out_dt == "f32" else TOL_BF16
    check_o(f"{label} o", host(o), o_ref, tol_o)
    check_S(f"{label} S_T", host(ST), S_ref, TOL_F32)


def test_tiny_fp32_workload():
    """B=1, H=2, T=512, dk=dv=64, fp32 in/out, zero initial state."""
    check_full(gi.tiny(), "f32", "tiny")


@pytest.mark.parametrize("T", [1, 5, 63, 64, 65, 129, 200])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_ragged_lengths_with_initial_state(T, dk, dv, dt):
    x = gi.generic(2, T, 3, dk, dv, 500 + T + dk + dv, dt, S0_scale=0.3)
    check_full(x, label=f"T={T}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_bf16_inputs_fp32_output(dt):
    x = gi.generic(2, 300, 4, 128, 128, 41, dt, S0_scale=0.3)
    check_full(x, "f32", "fp32 out")


@pytest.mark.parametrize("case", ["beta0", "beta1", "alpha1", "alpha_small"])
def test_gate_edge_values(case):
    x = gi.generic(1, 200, 4, 128, 128, 77, "bf16", S0_scale=0.5)
    if case == "beta0":
        x.beta[:] = 0.0          # the state only decays; o reads the decayed S0
    elif case == "beta1":
        x.beta[:] = 1.0          # every write stores v_t exactly along k_t
    elif case == "alpha1":
        x.alpha[:] = 1.0         # DeltaNet (no decay)
    else:
        x.alpha[:] = np.float32(np.exp(-3.0))   # very short horizon
    check_full(x, "f32", case)


def test_qwen_shaped_prefill_short():
    """16 heads of 128x128, keys in a narrow cone, 10 short / 6 long horizon
    heads; T=2048 so the oracle covers every head."""
    check_full(gi.prefill_16k(T=2048), "bf16", "T=2048")


def test_qwen_shaped_prefill_full_length_sampled_heads():
    """The full T=16384 workload in the benchmark's launch configuration;
    the oracle follows two short- and two long-horizon heads."""
    x = gi.prefill_16k()
    short = np.flatnonzero(x.short_heads)
    long_ = np.flatnonzero(~x.short_heads)
    heads = [(0, int(h)) for h in list(short[:2]) + list(long_[:2])]
    o, ST = run(x)
    print(f"  oracle on heads {heads}", flush=True)
    o_ref, S_ref = oracle_prefill(x, heads=heads)
    check_o("o", host(o), o_ref, TOL_BF16, heads)
    check_S("S_T", host(ST), S_ref, TOL_F32, heads)
    # spectra of the final state: stable rank bounds hold on every head
    S = host(ST)[0]
    for h in range(16):
        er = orc.stable_rank(S[h])
        assert 1.0 <= er <= 128.0


@pytest.mark.parametrize("dk", [128, 64])
def test_batched_prefill_sampled_heads(dk):
    """B=8, H=16, T=4096, dv=128, dk in {128, 64}: sampled heads."""
    x = gi.batched_prefill(dk=dk)
    heads = [(0, 0), (0, 9), (3, 4), (7, 15)]
    o, ST = run(x)
    o_ref, S_ref = oracle_prefill(x, heads=heads)
    check_o("o", host(o), o_ref, TOL_BF16, heads)
    check_S("S_T", host(ST), S_ref, TOL_F32, heads)


def test_split_consistency_and_in_place_state():
    """prefill(T) == prefill(T - T1, S0 = prefill(T1).S_T); ST may alias S0."""
    x = gi.generic(2, 333, 4, 128, 128, 99, "bf16", S0_scale=0.2)
    o_all, S_all = run(x, out_dtype=torch.float32)
    d = to_dev(x)
    T1 = 130
    o1, S1 = gdn.prefill(d["q"][:, :T1].contiguous(), d["k"][:, :T1].contiguous(),
                         d["v"][:, :T1].contiguous(), d["alpha"][:, :T1].contiguous(),
                         d["beta"][:, :T1].contiguous(), d["S0"],
                         out_dtype=torch.float32)
    o2, S2 = gdn.prefill(d["q"][:, T1:].contiguous(), d["k"][:, T1:].contiguous(),
                         d["v"][:, T1:].contiguous(), d["alpha"][:, T1:].contiguous(),
                         d["beta"][:, T1:].contiguous(), S1, ST=S1,
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert S2.data_ptr() == S1.data_ptr()
    o_split = torch.cat([o1, o2], dim=1)
    check_o("o split", host(o_split), host(o_all), 1e-4)
    check_S("S split", host(S2), host(S_all), 1e-4)


def test_zero_padding_embedding_ties_dk64_to_dk128():
    """q, k zero outside the kept channels: the dk=128 kernel's state equals
    the dk=64 kernel's state scattered to those channels, and o matches."""
    x64 = gi.generic(2, 257, 4, 64, 128, 123, "bf16", S0_scale=0.3)
    idx = np.stack([np.sort(np.random.default_rng(h).permutation(128)[:64])
                    for h in range(4)])
    x128 = gi.generic(2, 257, 4, 128, 128, 123, "bf16", S0_scale=0.3)
    for name in ("q", "k"):
        big = np.zeros(x64.q.shape[:3] + (128,), np.float32)
        for h in range(4):
            big[:, :, h, idx[h]] = getattr(x64, name)[:, :, h]
        setattr(x128, name, big)
    x128.v, x128.alpha, x128.beta = x64.v, x64.alpha, x64.beta
    S0big = np.zeros((2, 4, 128, 128), np.float32)
    for h in range(4):
        S0big[:, h][:, :, idx[h]] = x64.S0[:, h]
    x128.S0 = S0big
    o64, S64 = run(x64, out_dtype=torch.float32)
    o128, S128 = run(x128, out_dtype=torch.float32)
    S64s = np.zeros((2, 4, 128, 128))
    for h in range(4):
        S64s[:, h][:, :, idx[h]] = host(S64)[:, h]
    check_o("o", host(o128), host(o64), 1e-4)
    check_S("S", host(S128), S64s, 1e-4)


def test_deterministic_bitwise():
    x = gi.generic(2, 250, 4, 128, 128, 5, "bf16", S0_scale=0.3)
    o1, S1 = run(x)
    o2, S2 = run(x)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_empty_sequence_copies_state():
    x = gi.generic(2, 4, 3, 128, 64, 8, "bf16", S0_scale=1.0)
    d = to_dev(x)
    q0 = d["q"][:, :0].contiguous()
    o, ST = gdn.prefill(q0, q0, d["v"][:, :0].contiguous(),
                        d["alpha"][:, :0].contiguous(),
                        d["beta"][:, :0].contiguous(), d["S0"])
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 3, 64)
    assert torch.equal(ST, d["S0"])
    o, ST = gdn.prefill(q0, q0, d["v"][:, :0].contiguous(),
                        d["alpha"][:, :0].contiguous(),
                        d["beta"][:, :0].contiguous(), None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(ST) == 0


@pytest.mark.parametrize("T,H,out_dt", [(300, 4, "bf16"), (300, 4, "f32"),
                                        (2048 + 37, 2, "bf16")])
def test_two_phase_entry_points_match_composite(T, H, out_dt):
    """prepare (told the output dtype) then scan == gdn_prefill, bit for bit,
    for fp32 outputs (which read the lo half of P), bf16 outputs, and the
    segmented path."""
    x = gi.generic(1, T, H, 128, 128, 21 + T, "bf16", S0_scale=0.3)
    d = to_dev(x)
    o_ref, S_ref = run(x, out_dtype=tdtype(out_dt))
    nb = gdn.prefill_workspace_bytes(1, T, H, 128, 128)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(o_ref)
    ST = torch.empty_like(S_ref)
    gdn.prefill_prepare(d["q"], d["k"], d["alpha"], d["beta"], 128, ws,
                        out_dtype=o.dtype)
    gdn.prefill_scan(d["q"], d["k"], d["v"], d["S0"], o, ST, ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(ST, S_ref)


# (T, dk, dv, segments): the combine chains the segments in steps of three
# (its loop is unrolled by three), so the cases cover 1 to 4 chaining steps
# (every remainder modulo 3), ragged last segments and chunks, and all four
# head-size pairs.
@pytest.mark.parametrize("T,dk,dv,nseg", [(2048, 128, 128, 4), (1024 + 37, 128, 128, 2),
                                          (1600, 128, 128, 3), (2600, 128, 128, 5),
                                          (1500, 64, 128, 3), (2048, 128, 64, 4),
                                          (3000, 64, 64, 5)])
def test_segmented_prefill_few_heads(T, dk, dv, nseg):
    """Few heads and long sequences take the segment-parallel path (bf16 in
    and out): transition rows, segment chaining and output correction."""
    assert gdn.prefill_segments(1, T, 2, dk, dv)[0] == nseg
    x = gi.generic(1, T, 2, dk, dv, 900 + T + dk + dv, "bf16", S0_scale=0.3)
    check_full(x, "bf16", f"segmented T={T}")


@pytest.mark.parametrize("case", ["beta0", "beta1", "alpha1", "alpha_small"])
def test_segmented_gate_edge_values(case):
    """Gate edge values on the segment-parallel path, whose scan forms the
    masked Q K^T tiles from per-token exponent rows (e^-3 per token spans
    about 277 powers of two inside a chunk)."""
    x = gi.generic(1, 1100, 2, 128, 128, 78, "bf16", S0_scale=0.5)
    assert gdn.prefill_segments(1, 1100, 2, 128, 128)[0] > 1
    if case == "beta0":
        x.beta[:] = 0.0
    elif case == "beta1":
        x.beta[:] = 1.0
    elif case == "alpha1":
        x.alpha[:] = 1.0
    else:
        x.alpha[:] = np.float32(np.exp(-3.0))
    check_full(x, "bf16", f"segmented {case}")


def test_segmented_prefill_in_place_state():
    x = gi.generic(1, 1300, 3, 128, 128, 31, "bf16", S0_scale=0.5)
    d = to_dev(x)
    S = d["S0"].clone()
    o, ST = gdn.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S, ST=S)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_prefill(x)
    assert ST.data_ptr() == S.data_ptr()
    check_o("o", host(o), o_ref, TOL_BF16)
    check_S("S_T", host(ST), S_ref, TOL_F32)
