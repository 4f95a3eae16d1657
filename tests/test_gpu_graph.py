"""HIP graph capture of the entry points.

A caller may capture a prefill step (prepare + scan) or a chain of decode
steps in a HIP graph and replay it.  Every replay must reproduce the eager
results bit for bit (the kernels use no atomics and the workspace carries
nothing from one call to the next), also when the outputs and the workspace
hold garbage before the replay and eager work runs between replays.
"""

import pytest
import torch

from gated_deltanet_recurrent_delta_amd import binding as gdn
from tests.gpu_util import (TOL_BF16, TOL_F32, assert_close, check_o, check_S, check_step,
                            host, oracle_prefill, tdtype, to_dev)
from workloads import gdn_inputs as gi

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _other_eager_work(dev):
    """Unrelated eager work between replays: a prefill with its own
    workspace and a torch reduction."""
    y = to_dev(gi.generic(1, 300, 2, 64, 64, seed=77, dtype="bf16"))
    gdn.prefill(y["q"], y["k"], y["v"], y["alpha"], y["beta"])
    torch.randn(1 << 20, device=dev).sum().item()


# segmented and unsegmented plans, both key widths, and fp32 outputs (the
# scan that also reads the lo part of P); the NaN-filled workspace also shows
# that no scan reads the chunk-tile blocks prepare leaves unwritten
@pytest.mark.parametrize("B,T,H,dk,dv,out_dt", [
    (1, 2085, 2, 128, 128, "bf16"), (2, 700, 8, 128, 128, "bf16"),
    (1, 2085, 2, 64, 128, "bf16"), (2, 700, 8, 64, 64, "bf16"),
    (1, 300, 4, 128, 128, "f32"), (1, 300, 4, 64, 128, "f32")])
def test_prefill_graph_replays_match_eager(B, T, H, dk, dv, out_dt):
    dev = torch.device("cuda")
    x = gi.generic(B, T, H, dk, dv, seed=4242 + T + dk, dtype="bf16", S0_scale=0.3)
    d = to_dev(x)
    nseg = gdn.prefill_segments(B, T, H, dk, dv, out_dtype=tdtype(out_dt))[0]
    print(f"  B={B} T={T} H={H} dk={dk} dv={dv} out={out_dt}: {nseg} segments", flush=True)
    ws = torch.empty(gdn.prefill_workspace_bytes(B, T, H, dk, dv),
                     dtype=torch.uint8, device=dev)
    ws.fill_(0xFF)
    o = torch.empty((B, T, H, dv), dtype=tdtype(out_dt), device=dev)
    ST = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)

    def step():
        gdn.prefill_prepare(d["q"], d["k"], d["alpha"], d["beta"], dv, ws,
                            out_dtype=o.dtype)
        gdn.prefill_scan(d["q"], d["k"], d["v"], d["S0"], o, ST, ws)

    step()
    torch.cuda.synchronize()
    o_ref, S_ref = o.clone(), ST.clone()
    assert torch.isfinite(o_ref.float()).all() and torch.isfinite(S_ref).all()
    # the eager result itself, from the NaN-filled workspace, against the oracle
    o_or, S_or = oracle_prefill(x)
    check_o("o (eager)", host(o_ref), o_or, TOL_F32 if out_dt == "f32" else TOL_BF16)
    check_S("S_T (eager)", host(S_ref), S_or, TOL_F32)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        o.fill_(float("nan"))
        ST.fill_(float("nan"))
        ws.fill_(0xFF)                  # every byte 0xFF: NaN in fp32 and bf16
        _other_eager_work(dev)
        g.replay()
        torch.cuda.synchronize()
        print(f"  replay {rep}: o equal {torch.equal(o, o_ref)}, "
              f"S_T equal {torch.equal(ST, S_ref)}", flush=True)
        assert torch.equal(o, o_ref), f"replay {rep}: o differs"
        assert torch.equal(ST, S_ref), f"replay {rep}: S_T differs"


@pytest.mark.parametrize("B,dk", [(64, 128), (64, 64), (1, 64)])
def test_decode_graph_replays_match_eager(B, dk):
    H, dv, n = 16, 128, 4
    dev = torch.device("cuda")
    x = gi.generic(B, n, H, dk, dv, seed=990 + B + dk, dtype="bf16", S0_scale=0.5)
    d = to_dev(x)
    steps = [tuple(d[name][:, t].contiguous()
                   for name in ("q", "k", "v", "alpha", "beta"))
             for t in range(n)]
    S = d["S0"].clone()
    outs = torch.empty((n, B, H, dv), dtype=torch.bfloat16, device=dev)

    def chain():
        for t in range(n):
            gdn.decode_step(*steps[t], S, S_out=S, o=outs[t])

    chain()
    torch.cuda.synchronize()
    o_ref, S_ref = outs.clone(), S.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        S.copy_(d["S0"])
        outs.fill_(float("nan"))
        _other_eager_work(dev)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs, o_ref), f"replay {rep}: o differs"
        assert torch.equal(S, S_ref), f"replay {rep}: S differs"


# --- the fused input path and the generalised gates --------------------------

@pytest.mark.parametrize("B,T,H", [(1, 2085, 2), (4, 300, 8)])
def test_prefill_qk_graph_replays_match_eager(B, T, H):
    """Channel subset 128 -> 64, normalisation and query scale inside the
    kernels (the gathered copy lives in the workspace), segmented and not."""
    dev = torch.device("cuda")
    r = __import__("numpy").random.Generator(__import__("numpy").random.PCG64(515 + T))
    ch_np = __import__("numpy").stack([__import__("numpy").sort(r.permutation(128)[:64])
                                       for _ in range(H)]).astype("int32")
    x = gi.raw_qk(B, T, H, 128, 128, 516 + T, "bf16", channel_idx=ch_np, S0_scale=0.3)
    d = to_dev(x)
    ch = torch.from_numpy(ch_np).to(dev)
    ws = torch.empty(gdn.prefill_qk_workspace_bytes(B, T, H, 64, 128, torch.bfloat16, True),
                     dtype=torch.uint8, device=dev)
    ws.fill_(0xFF)
    o = torch.empty((B, T, H, 128), dtype=torch.bfloat16, device=dev)
    ST = torch.empty((B, H, 128, 64), dtype=torch.float32, device=dev)

    def step():
        gdn.prefill_qk(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], channels=ch,
                       q_scale=0.125, o=o, ST=ST, workspace=ws, validate=False)

    step()
    torch.cuda.synchronize()
    o_ref, S_ref = o.clone(), ST.clone()
    assert torch.isfinite(o_ref.float()).all() and torch.isfinite(S_ref).all()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        o.fill_(float("nan"))
        ST.fill_(float("nan"))
        ws.fill_(0xFF)
        _other_eager_work(dev)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"replay {rep}: o differs"
        assert torch.equal(ST, S_ref), f"replay {rep}: S_T differs"


@pytest.mark.parametrize("kind", ["decode_qk", "gated_decode", "gated_prefill"])
def test_new_entry_points_graph_replays_match_eager(kind):
    import numpy as np
    dev = torch.device("cuda")
    B, H, dv, n = 64, 16, 128, 3
    S0 = (0.3 * torch.randn((B, H, dv, 64), generator=torch.Generator().manual_seed(9))).to(dev)
    S = S0.clone()
    if kind == "decode_qk":
        ch_np = gi.pruning_subsets(3, H, 128, 64)
        x = gi.raw_qk(B, n, H, 128, dv, 8100, "bf16", channel_idx=ch_np)
        d = to_dev(x)
        ch = torch.from_numpy(ch_np).to(dev)
        outs = torch.empty((n, B, H, dv), dtype=torch.bfloat16, device=dev)

        steps = [[d[nm][:, t].contiguous() for nm in ("q", "k", "v", "alpha", "beta")]
                 for t in range(n)]

        def run():
            for t in range(n):
                gdn.decode_step_qk(*steps[t], S, S_out=S, o=outs[t], channels=ch,
                                   q_scale=0.125, validate=False)
    else:
        T = 1 if kind == "gated_decode" else 37
        reps = n if kind == "gated_decode" else 1
        x = gi.generic(B if T == 1 else 2, T, H, 64, dv, 8200 + T, "bf16")
        al, bg, wg = (torch.from_numpy(z).to(dev) for z in
                      gi.gate_vectors(x.q.shape[0], T, H, 64, dv, 8300 + T))
        d = to_dev(x)
        if T > 1:
            S0 = S0[:2].contiguous()
            S = S0.clone()
        outs = torch.empty((reps,) + tuple(x.v.shape), dtype=torch.bfloat16, device=dev)

        def run():
            for t in range(reps):
                gdn.gated_recurrent(d["q"], d["k"], d["v"], al, bg, wg, S, o=outs[t], ST=S)
    run()
    torch.cuda.synchronize()
    o_ref, S_ref = outs.clone(), S.clone()
    assert torch.isfinite(o_ref.float()).all()
    g = torch.cuda.CUDAGraph()
    S.copy_(S0)
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        S.copy_(S0)
        outs.fill_(float("nan"))
        _other_eager_work(dev)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs, o_ref), f"replay {rep}: o differs"
        assert torch.equal(S, S_ref), f"replay {rep}: S differs"


@pytest.mark.parametrize("dk", [128, 64])
def test_backward_graph_replays_match_eager(dk):
    """gdn_backward captured once (T = 37: four checkpoint blocks and a
    ragged one) and replayed with its outputs NaN, its workspace filled with
    0xFF bytes (NaN floats) and dS0 written over dS_T; every replay equals
    the eager call bitwise."""
    dev = torch.device("cuda")
    B, T, H, dv = 2, 37, 4, 128
    x = gi.generic(B, T, H, dk, dv, 8400 + dk, "bf16", S0_scale=0.3)
    d_o, dST = gi.cotangents(B, T, H, dk, dv, 8401 + dk, "bf16")
    d = to_dev(x)
    d_o = torch.from_numpy(d_o).to(dev).to(torch.bfloat16).contiguous()
    dST0 = torch.from_numpy(dST).to(dev)
    g_st = dST0.clone()
    ws = torch.empty(gdn.backward_workspace_bytes(B, T, H, dk, dv), dtype=torch.uint8, device=dev)
    names = ("dq", "dk", "dv", "dalpha", "dbeta")
    out = {nm: torch.empty(sh, dtype=torch.float32, device=dev) for nm, sh in
           zip(names, [(B, T, H, dk), (B, T, H, dk), (B, T, H, dv), (B, T, H), (B, T, H)])}
    out["dS0"] = g_st

    def run():
        gdn.backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d_o, g_st,
                     out=out, workspace=ws)
    run()
    torch.cuda.synchronize()
    ref = {nm: t.clone() for nm, t in out.items()}
    assert all(torch.isfinite(t).all() for t in ref.values())
    g = torch.cuda.CUDAGraph()
    g_st.copy_(dST0)
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        g_st.copy_(dST0)
        for nm in names:
            out[nm].fill_(float("nan"))
        ws.fill_(255)
        _other_eager_work(dev)
        g.replay()
        torch.cuda.synchronize()
        for nm, t in out.items():
            assert torch.equal(t, ref[nm]), f"replay {rep}: {nm} differs"
