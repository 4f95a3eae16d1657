"""gdn_prefill_noalloc (the prefill with its workspace in the library's
static device scratch) against gdn_prefill with a caller workspace, on two
calls in a row, the second with a smaller input: bitwise equal, and within
the stated tolerance of the fp64 oracle."""

import numpy as np
import pytest
import torch

from gated_deltanet_recurrent_delta_amd import binding as gdn
from tests.gpu_util import (TOL_BF16, TOL_F32, check_o, check_S, host,
                            oracle_prefill, tdtype, to_dev)
from workloads import gdn_inputs as gi

pytestmark = pytest.mark.gpu


def both(x, out_dt, S0=None):
    """(o, ST) from gdn_prefill and from gdn_prefill_noalloc."""
    d = to_dev(x)
    s0 = d["S0"] if S0 is None else S0
    o_ref, S_ref = gdn.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], s0,
                               out_dtype=tdtype(out_dt))
    o = torch.full_like(o_ref, float("nan"))
    ST = torch.full_like(S_ref, float("nan"))
    gdn.prefill_noalloc(d["q"], d["k"], d["v"], d["alpha"], d["beta"], s0, o, ST)
    torch.cuda.synchronize()
    return (o_ref, S_ref), (o, ST)


def test_noalloc_two_calls_second_smaller():
    # 1: the 16-head, 16,384-token layer (segmented path; 236 MiB of scratch)
    x1 = gi.prefill_16k()
    print(f"  call 1: B=1 T=16384 H=16 d=128, needs "
          f"{gdn.prefill_workspace_bytes(1, 16384, 16, 128, 128) / 2**20:.0f} MiB", flush=True)
    (o_ref, S_ref), (o, ST) = both(x1, "bf16")
    assert torch.equal(o, o_ref) and torch.equal(ST, S_ref)
    heads = [(0, 0), (0, 15)]
    oo, So = oracle_prefill(x1, heads=heads)
    check_o("call 1 o", host(o), oo, TOL_BF16, heads)
    check_S("call 1 S_T", host(ST), So, TOL_F32, heads)

    # 2: smaller, other shape and dtypes, with an initial state (unsegmented)
    x2 = gi.generic(2, 300, 3, 64, 128, 4242, "bf16", S0_scale=0.3)
    print("  call 2: B=2 T=300 H=3 dk=64 dv=128, fp32 out", flush=True)
    (o_ref, S_ref), (o, ST) = both(x2, "f32")
    assert torch.equal(o, o_ref) and torch.equal(ST, S_ref)
    oo, So = oracle_prefill(x2)
    check_o("call 2 o", host(o), oo, TOL_F32)
    check_S("call 2 S_T", host(ST), So, TOL_F32)


def test_noalloc_in_place_state_and_empty_sequence():
    x = gi.generic(1, 1300, 3, 128, 128, 31, "bf16", S0_scale=0.5)
    d = to_dev(x)
    o_ref, S_ref = gdn.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"])
    S = d["S0"].clone()
    o = torch.empty_like(o_ref)
    gdn.prefill_noalloc(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S, o, S)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    # T = 0: the final state is the initial one
    q0 = d["q"][:, :0].contiguous()
    o0 = torch.empty((1, 0, 3, 128), dtype=torch.bfloat16, device="cuda")
    S1 = torch.full_like(S, float("nan"))
    gdn.prefill_noalloc(q0, q0, d["v"][:, :0].contiguous(), d["alpha"][:, :0].contiguous(),
                        d["beta"][:, :0].contiguous(), d["S0"], o0, S1)
    torch.cuda.synchronize()
    assert torch.equal(S1, d["S0"])


def test_noalloc_rejects_sizes_beyond_the_scratch():
    d = to_dev(gi.generic(8, 4096, 16, 128, 128, 5, "bf16"))
    o = torch.empty((8, 4096, 16, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gdn.GdnError) as e:
        gdn.prefill_noalloc(d["q"], d["k"], d["v"], d["alpha"], d["beta"], None, o, None)
    assert e.value.status == gdn.GDN_EWORKSPACE
