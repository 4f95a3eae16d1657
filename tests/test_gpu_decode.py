"""GPU parity of the decode step (gdn_decode_step) against the fp64 oracle."""

import numpy as np
import pytest
import torch

from gated_deltanet_recurrent_delta_amd import binding as gdn
from oracle import gdn_oracle as orc
from tests.gpu_util import (TOL_BF16, TOL_F32, assert_close, check_o, check_S, check_step, host,
                            tdtype, to_dev, oracle_prefill)
from workloads import gdn_inputs as gi

pytestmark = pytest.mark.gpu


def one_step_inputs(B, H, dk, dv, dtype, seed, S_scale=0.5):
    x = gi.generic(B, 1, H, dk, dv, seed, dtype, S0_scale=S_scale)
    return x


@pytest.mark.parametrize("B,H", [(3, 4), (64, 16)])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
@pytest.mark.parametrize("in_dt,out_dt", [("bf16", "bf16"), ("f32", "f32"),
                                          ("bf16", "f32")])
def test_decode_matches_oracle(B, H, dk, dv, in_dt, out_dt):
    """One step against the oracle.  At dk=64 the launch picks the rows per
    wave and the store order from the number of waves: B=3 runs 4-row waves,
    B=64 with dv=64 8-row waves and B=64 with dv=128 32-row waves with paced
    stores, so all three are covered."""
    x = one_step_inputs(B, H, dk, dv, in_dt, seed=1000 + dk + dv + B)
    d = to_dev(x)
    o, S1 = gdn.decode_step(d["q"][:, 0].contiguous(), d["k"][:, 0].contiguous(),
                            d["v"][:, 0].contiguous(), d["alpha"][:, 0].contiguous(),
                            d["beta"][:, 0].contiguous(), d["S0"],
                            out_dtype=tdtype(out_dt))
    torch.cuda.synchronize()
    o_ref, S_ref = orc.gdn_decode_step(x.q[:, 0], x.k[:, 0], x.v[:, 0],
                                       x.alpha[:, 0], x.beta[:, 0], x.S0)
    tol_o = TOL_F32 if out_dt == "f32" else TOL_BF16
    check_step("o", host(o), o_ref, tol_o)
    check_S("S'", host(S1), S_ref, TOL_F32)


@pytest.mark.parametrize("B,H,dv", [(96, 16, 128), (128, 16, 64), (40, 8, 128)])
@pytest.mark.parametrize("in_dt,out_dt", [("bf16", "bf16"), ("f32", "f32")])
def test_decode_dk64_layouts(B, H, dv, in_dt, out_dt):
    """dk=64 at the grid sizes around the paced 32-row layout: more paced
    waves than one per head slice of a B=64 step (B=96), the paced layout
    with dv=64 (B=128), and a smaller batch that takes 4-row waves (B=40,
    H=8: 1280 waves of 32 rows would be too few)."""
    x = one_step_inputs(B, H, 64, dv, in_dt, seed=2000 + B + dv)
    d = to_dev(x)
    o, S1 = gdn.decode_step(d["q"][:, 0].contiguous(), d["k"][:, 0].contiguous(),
                            d["v"][:, 0].contiguous(), d["alpha"][:, 0].contiguous(),
                            d["beta"][:, 0].contiguous(), d["S0"],
                            out_dtype=tdtype(out_dt))
    torch.cuda.synchronize()
    o_ref, S_ref = orc.gdn_decode_step(x.q[:, 0], x.k[:, 0], x.v[:, 0],
                                       x.alpha[:, 0], x.beta[:, 0], x.S0)
    tol_o = TOL_F32 if out_dt == "f32" else TOL_BF16
    check_step("o", host(o), o_ref, tol_o)
    check_S("S'", host(S1), S_ref, TOL_F32)


@pytest.mark.parametrize("dk", [128, 64])
def test_decode_in_place_is_bitwise_identical(dk):
    x = one_step_inputs(64, 16, dk, 128, "bf16", seed=7)
    d = to_dev(x)
    args = [d[n][:, 0].contiguous() for n in ("q", "k", "v", "alpha", "beta")]
    o1, S1 = gdn.decode_step(*args, d["S0"])
    S_inplace = d["S0"].clone()
    o2, S2 = gdn.decode_step(*args, S_inplace, S_out=S_inplace)
    torch.cuda.synchronize()
    assert S2.data_ptr() == S_inplace.data_ptr()
    assert torch.equal(S1, S2) and torch.equal(o1, o2)
    # and deterministic across runs
    o3, S3 = gdn.decode_step(*args, d["S0"])
    torch.cuda.synchronize()
    assert torch.equal(S1, S3) and torch.equal(o1, o3)


@pytest.mark.parametrize("dk", [128, 64])
def test_decode_chain_full_batch(dk):
    """Decode workload at full size: B=64, H=16, dv=128, 512 steps from
    states of a 2048-token prompt.  The GPU steps all 64 rows (the launch
    configuration the benchmark times); the oracle follows sampled rows.

    (i) isolated: the GPU starts from the oracle's prompt state (rounded to
        fp32) on the sampled rows;
    (ii) end to end: GPU prefill of the prompt, then GPU decode."""
    B, H, n_steps, rows = 64, 16, 512, [0, 37, 63]
    prompt = gi.decode_prompt(B=B, dk=dk, rows=rows)
    steps = gi.decode_steps(B=B, n_steps=n_steps, dk=dk)
    heads = [(b, h) for b in range(len(rows)) for h in range(H)]
    print(f"  oracle prompt prefill on {len(heads)} heads", flush=True)
    _, S_prompt = oracle_prefill(prompt)
    # oracle chain on the sampled rows
    o_ref = np.empty((len(rows), n_steps, H, 128))
    S_ref = S_prompt.copy()
    for t in range(n_steps):
        o_ref[:, t], S_ref = orc.gdn_decode_step(
            steps.q[rows, t], steps.k[rows, t], steps.v[rows, t],
            steps.alpha[rows, t], steps.beta[rows, t], S_ref)
    ds = to_dev(steps)

    def run_gpu(S_init):
        S = S_init.clone()
        o_rows = torch.empty((len(rows), n_steps, H, 128), device="cuda")
        for t in range(n_steps):
            o, _ = gdn.decode_step(ds["q"][:, t].contiguous(), ds["k"][:, t].contiguous(),
                                   ds["v"][:, t].contiguous(),
                                   ds["alpha"][:, t].contiguous(),
                                   ds["beta"][:, t].contiguous(), S, S_out=S)
            o_rows[:, t] = o[rows].float()
        torch.cuda.synchronize()
        return host(o_rows), host(S[rows])

    # (i) isolated
    g = torch.Generator(device="cpu").manual_seed(3)
    S_init = (0.3 * torch.randn((B, H, 128, dk), generator=g)).cuda()
    S_init[rows] = torch.from_numpy(S_prompt.astype(np.float32)).cuda()
    o_g, S_g = run_gpu(S_init)
    check_o("o (isolated)", o_g, o_ref, TOL_BF16)
    check_S("S_512 (isolated)", S_g, S_ref, TOL_F32)

    # (ii) end to end: GPU prefill of the sampled prompt rows
    dp = to_dev(prompt)
    _, S_p = gdn.prefill(dp["q"], dp["k"], dp["v"], dp["alpha"], dp["beta"])
    torch.cuda.synchronize()
    check_S("prompt state", host(S_p), S_prompt, TOL_F32)
    S_init2 = S_init.clone()
    S_init2[rows] = S_p
    o_g2, S_g2 = run_gpu(S_init2)
    check_o("o (end to end)", o_g2, o_ref, TOL_BF16)
    check_S("S_512 (end to end)", S_g2, S_ref, TOL_F32)


def test_decode_equals_one_token_prefill():
    x = gi.generic(4, 1, 8, 128, 128, 11, "bf16", S0_scale=0.4)
    d = to_dev(x)
    o_d, S_d = gdn.decode_step(d["q"][:, 0].contiguous(), d["k"][:, 0].contiguous(),
                               d["v"][:, 0].contiguous(), d["alpha"][:, 0].contiguous(),
                               d["beta"][:, 0].contiguous(), d["S0"],
                               out_dtype=torch.float32)
    o_p, S_p = gdn.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_step("o", host(o_p)[:, 0], host(o_d), 1e-4)
    check_S("S", host(S_p), host(S_d), 1e-4)
