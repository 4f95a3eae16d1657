"""GPU parity of the generalised gates (gdn_gated_recurrent: a retention per
key channel, a key-side erase gate and a value-side write gate) against the
oracle's gdn2_prefill, and its reductions to Kimi Delta Attention and to the
gated delta rule of gdn_prefill ("Linear Attention Architectures" reading
notes on paper Secs. 3.4-3.5)."""

import numpy as np
import pytest
import torch

from gated_deltanet_recurrent_delta_amd import binding as gdn
from oracle import gdn_oracle as orc
from tests.gpu_util import (TOL_BF16, TOL_F32, assert_close, check_o, check_S, check_step,
                            host, tdtype, to_dev)
from workloads import gdn_inputs as gi

pytestmark = pytest.mark.gpu


def dev32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda")


def run(x, al, b, w, out_dt, S0=None, ST=None):
    d = to_dev(x)
    s0 = d["S0"] if S0 is None else S0
    o, S = gdn.gated_recurrent(d["q"], d["k"], d["v"], dev32(al), dev32(b), dev32(w), s0,
                               out_dtype=tdtype(out_dt), ST=ST)
    torch.cuda.synchronize()
    return o, S


def check(x, al, b, w, out_dt=None, label="", heads=None):
    out_dt = x.dtype if out_dt is None else out_dt
    print(f"  case {label}: {x.q.shape} out={out_dt}", flush=True)
    o, S = run(x, al, b, w, out_dt)
    o_ref, S_ref = orc.gdn2_prefill(x.q, x.k, x.v, al, b, w, x.S0, heads=heads)
    tol_o = TOL_F32 if out_dt == "f32" else TOL_BF16
    check_o(f"{label} o", host(o), o_ref, tol_o, heads)
    check_S(f"{label} S_T", host(S), S_ref, TOL_F32, heads)


@pytest.mark.parametrize("T", [1, 5, 37])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_gated_matches_oracle(T, dk, dv, dt):
    x = gi.generic(2, T, 3, dk, dv, 6000 + T + dk + dv, dt, S0_scale=0.3)
    al, b, w = gi.gate_vectors(2, T, 3, dk, dv, 6100 + T + dk + dv)
    check(x, al, b, w, label=f"T={T}")


def test_gated_long_sequence_fp32_out():
    """Several ring turns and a ragged tail (T = 601 = 4 * 150 + 1)."""
    x = gi.generic(1, 601, 2, 128, 128, 6200, "bf16", S0_scale=0.3)
    al, b, w = gi.gate_vectors(1, 601, 2, 128, 128, 6201)
    check(x, al, b, w, "f32", label="T=601")


def test_gated_decode_batch64():
    """T = 1 over B=64, H=16 carried states: the decode step (8 rows per
    wave at dk=128; 32 rows per wave with paced stores at dk=64)."""
    for dk in (128, 64):
        x = gi.generic(64, 1, 16, dk, 128, 6300 + dk, "bf16", S0_scale=0.5)
        al, b, w = gi.gate_vectors(64, 1, 16, dk, 128, 6301 + dk)
        check(x, al, b, w, label=f"decode B=64 dk={dk}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_gated_decode_paced_dv64(dt):
    """The paced dk=64 decode layout with dv=64 (two 32-row slices per head,
    B=128) and, with dt f32, fp32 inputs and outputs."""
    x = gi.generic(128, 1, 16, 64, 64, 6350, dt, S0_scale=0.5)
    al, b, w = gi.gate_vectors(128, 1, 16, 64, 64, 6351)
    check(x, al, b, w, label=f"decode B=128 dk=64 dv=64 {dt}")


def test_kda_and_gdn_reductions_match_chunked_prefill():
    """b = w = beta broadcast is Kimi Delta Attention; with alpha broadcast
    from the scalar gate too, the result must match gdn_prefill's chunked
    kernels (and the oracle)."""
    B, T, H, dk, dv = 1, 300, 4, 128, 128
    x = gi.generic(B, T, H, dk, dv, 6400, "bf16", S0_scale=0.3)
    al = np.repeat(x.alpha[..., None], dk, -1)
    b = np.repeat(x.beta[..., None], dk, -1)
    w = np.repeat(x.beta[..., None], dv, -1)
    o_g, S_g = run(x, al, b, w, "f32")
    d = to_dev(x)
    o_c, S_c = gdn.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, S_ref = orc.gdn_prefill(x.q, x.k, x.v, x.alpha, x.beta, x.S0)
    check_o("gated o vs oracle", host(o_g), o_ref, TOL_F32)
    check_S("gated S vs oracle", host(S_g), S_ref, TOL_F32)
    check_o("gated o vs chunked", host(o_g), host(o_c), TOL_F32)
    check_S("gated S vs chunked", host(S_g), host(S_c), TOL_F32)


def test_gated_in_place_and_empty():
    x = gi.generic(2, 20, 3, 64, 128, 6500, "f32", S0_scale=0.3)
    al, b, w = gi.gate_vectors(2, 20, 3, 64, 128, 6501)
    d = to_dev(x)
    S = d["S0"].clone()
    o1, S1 = run(x, al, b, w, "f32")
    o2, S2 = run(x, al, b, w, "f32", S0=S, ST=S)
    assert S2.data_ptr() == S.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    # T = 0 copies the initial state
    e = torch.empty((2, 0, 3, 64), dtype=torch.float32, device="cuda")
    ev = torch.empty((2, 0, 3, 128), dtype=torch.float32, device="cuda")
    o0, S0c = gdn.gated_recurrent(e, e, ev, e, e, ev, d["S0"])
    torch.cuda.synchronize()
    assert o0.numel() == 0 and torch.equal(S0c, d["S0"])


@pytest.mark.parametrize("B,H,T,dk,dv", [(8, 16, 40, 64, 128), (4, 16, 33, 128, 128),
                                         (8, 16, 21, 128, 64)])
def test_gated_many_heads_row_groupings(B, H, T, dk, dv):
    """Enough heads for the sequence form to carry 16 (B=8, H=16, dv=128) or
    8 (B=4, H=16; B=8 with dv=64) rows per wave; every head against the
    oracle."""
    x = gi.generic(B, T, H, dk, dv, 6600 + B + T + dk + dv, "bf16", S0_scale=0.3)
    al, b, w = gi.gate_vectors(B, T, H, dk, dv, 6700 + B + T + dk + dv)
    check(x, al, b, w, "f32", label=f"B={B} H={H} T={T}")


@pytest.mark.parametrize("B,H,T", [(2, 3, 37), (8, 16, 20), (64, 16, 1)])
def test_gated_zero_initial_state(B, H, T):
    """S0 = None (the kernels' zero-state instance) at every row grouping."""
    x = gi.generic(B, T, H, 64, 128, 6800 + B + T, "bf16")
    assert x.S0 is None
    al, b, w = gi.gate_vectors(B, T, H, 64, 128, 6900 + B + T)
    check(x, al, b, w, "f32", label=f"S0=None B={B} T={T}")


# ---------------------------------------------------------------------------
# chunked form (gdn_gated_prefill, bf16 inputs)
# ---------------------------------------------------------------------------

def run_chunked(x, al, b, w, out_dt, S0=None, ST=None):
    d = to_dev(x)
    s0 = d["S0"] if S0 is None else S0
    o, S = gdn.gated_prefill(d["q"], d["k"], d["v"], dev32(al), dev32(b), dev32(w), s0,
                             out_dtype=tdtype(out_dt), ST=ST)
    torch.cuda.synchronize()
    return o, S


def check_chunked(x, al, b, w, out_dt=None, label="", heads=None):
    out_dt = x.dtype if out_dt is None else out_dt
    print(f"  case chunked {label}: {x.q.shape} out={out_dt}", flush=True)
    o, S = run_chunked(x, al, b, w, out_dt)
    o_ref, S_ref = orc.gdn2_prefill(x.q, x.k, x.v, al, b, w, x.S0, heads=heads)
    tol_o = TOL_F32 if out_dt == "f32" else TOL_BF16
    check_o(f"{label} o", host(o), o_ref, tol_o, heads)
    check_S(f"{label} S_T", host(S), S_ref, TOL_F32, heads)


@pytest.mark.parametrize("T", [1, 37, 63, 64, 65, 130, 200])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
@pytest.mark.parametrize("out_dt", ["bf16", "f32"])
def test_gated_chunked_matches_oracle(T, dk, dv, out_dt):
    """Ragged chunks and several chunk boundaries, every head size, both
    output dtypes."""
    x = gi.generic(2, T, 3, dk, dv, 6500 + T + dk + dv, "bf16", S0_scale=0.3)
    al, b, w = gi.gate_vectors(2, T, 3, dk, dv, 6600 + T + dk + dv)
    check_chunked(x, al, b, w, out_dt, label=f"T={T} dk={dk} dv={dv}")


@pytest.mark.parametrize("case", ["alpha1", "alpha_small", "alpha_mixed", "b0", "b1", "w0"])
def test_gated_chunked_gate_edges(case):
    """Retentions at 1 and down to e^-3 per token (several channels each way
    in one head), erase gates 0 and 1, write gate 0."""
    x = gi.generic(1, 150, 3, 128, 128, 6700, "bf16", S0_scale=0.5)
    al, b, w = gi.gate_vectors(1, 150, 3, 128, 128, 6701)
    if case == "alpha1":
        al[:] = 1.0
    elif case == "alpha_small":
        al[:] = np.float32(np.exp(-3.0))
    elif case == "alpha_mixed":
        al[..., ::2] = np.float32(np.exp(-3.0))
        al[..., 1::4] = 1.0
    elif case == "b0":
        b[:] = 0.0
    elif case == "b1":
        b[:] = 1.0
    else:
        w[:] = 0.0
    check_chunked(x, al, b, w, "f32", label=case)


def test_gated_chunked_reduces_to_gdn():
    """b = w = beta 1 and alpha = a 1: the chunked generalised form equals
    the chunked gated delta rule of gdn_prefill."""
    x = gi.generic(2, 200, 3, 128, 128, 6800, "bf16", S0_scale=0.3)
    rep = lambda a, n: np.ascontiguousarray(np.repeat(a[..., None], n, axis=-1), np.float32)
    al, b, w = rep(x.alpha, 128), rep(x.beta, 128), rep(x.beta, 128)
    o_g, S_g = run_chunked(x, al, b, w, "f32")
    d = to_dev(x)
    o_c, S_c = gdn.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, S_ref = orc.gdn_prefill(x.q, x.k, x.v, x.alpha, x.beta, x.S0)
    check_o("chunked gated o vs oracle", host(o_g), o_ref, TOL_F32)
    check_S("chunked gated S vs oracle", host(S_g), S_ref, TOL_F32)
    check_o("chunked gated o vs gdn_prefill", host(o_g), host(o_c), TOL_F32)
    check_S("chunked gated S vs gdn_prefill", host(S_g), host(S_c), TOL_F32)


def test_gated_chunked_batched_shape_sampled_heads():
    """B=8, T=4096, H=16, dk=64, dv=128 (the benchmark's shape): all heads
    on the GPU, the oracle on sampled heads."""
    B, T, H, dk, dv = 8, 4096, 16, 64, 128
    heads = [(0, 0), (3, 7), (7, 15)]
    rows = sorted({bb for bb, _ in heads})
    x = gi.generic(B, T, H, dk, dv, gi.seed_for(4, 11), "bf16")
    al, b, w = gi.gate_vectors(B, T, H, dk, dv, gi.seed_for(4, 12))
    o, S = run_chunked(x, al, b, w, "bf16")
    remap = {bb: i for i, bb in enumerate(rows)}
    local = [(remap[bb], h) for bb, h in heads]
    sl = lambda a: a[rows]
    o_ref, S_ref = orc.gdn2_prefill(sl(x.q), sl(x.k), sl(x.v), sl(al), sl(b), sl(w), None,
                                    heads=local)
    check_o("batched o", host(o)[rows], o_ref, TOL_BF16, local)
    check_S("batched S_T", host(S)[rows], S_ref, TOL_F32, local)


def test_gated_chunked_in_place_deterministic_and_fp32_path():
    x = gi.generic(2, 130, 3, 64, 128, 6900, "bf16", S0_scale=0.4)
    al, b, w = gi.gate_vectors(2, 130, 3, 64, 128, 6901)
    d = to_dev(x)
    o1, S1 = run_chunked(x, al, b, w, "bf16")
    o2, S2 = run_chunked(x, al, b, w, "bf16")
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    S = d["S0"].clone()
    o3, S3 = run_chunked(x, al, b, w, "bf16", S0=S, ST=S)
    assert S3.data_ptr() == S.data_ptr() and torch.equal(S3, S1) and torch.equal(o3, o1)
    # fp32 inputs take the recurrent form: equal to gdn_gated_recurrent bitwise
    xf = gi.generic(1, 40, 2, 128, 64, 6902, "f32", S0_scale=0.3)
    alf, bf, wf = gi.gate_vectors(1, 40, 2, 128, 64, 6903)
    of, Sf = run_chunked(xf, alf, bf, wf, "f32")
    orr, Srr = run(xf, alf, bf, wf, "f32")
    assert torch.equal(of, orr) and torch.equal(Sf, Srr)
