"""Element offsets beyond 2**31: the chunked prefill and the decode step at
sizes whose tensors hold more than 2**31 elements, so that any offset formed
in 32-bit arithmetic would wrap.  Sampled heads, among them the last ones
(whose elements all lie past 2**31), are checked against the fp64 oracle to
the usual per-head and per-token bars.

Inputs stay exact and distinct per head without drawing gigabytes on the
host: the prefill's batch entry b is a cyclic token shift, by 997 b tokens,
of one of two seeded rows of the generic workload (its initial state a shift
of the head axis); the decode's state of head i is a (row, column) cyclic
shift of one of 64 seeded states; the segmented prefill's sequence is 34
copies of one seeded 32768-token row, copy j shifted by 7919 j tokens; the
generalised-gate prefill and the backward pass shift two seeded rows like
the plain prefill.  The oracle receives the same shifted arrays, built with
numpy.
"""

import numpy as np
import pytest
import torch

from gated_deltanet_recurrent_delta_amd import binding as gdn
from oracle import gdn_oracle as orc
from tests.gpu_util import TOL_BF16, TOL_F32, check_o, check_S, check_step, host
from workloads import gdn_inputs as gi

pytestmark = pytest.mark.gpu


def test_prefill_offsets_past_2_31():
    """B=144, T=8192, H=16, dk=dv=128, bf16: q/k/v/o hold 2.42e9 elements."""
    dev = torch.device("cuda", 0)
    B, T, H, d = 144, 8192, 16, 128
    assert B * T * H * d > 2 ** 31
    x = gi.generic(2, T, H, d, d, gi.seed_for(2, 8), "bf16", S0_scale=0.3)
    shift = lambda b: (997 * b) % T

    def host_row(b):
        """Inputs of batch entry b as [1, ...] arrays (the device's values)."""
        r, s = b % 2, shift(b)
        return (np.roll(x.q[r], s, axis=0)[None], np.roll(x.k[r], s, axis=0)[None],
                np.roll(x.v[r], s, axis=0)[None], np.roll(x.alpha[r], s, axis=0)[None],
                np.roll(x.beta[r], s, axis=0)[None], np.roll(x.S0[r], b % H, axis=0)[None])

    base = {n: torch.from_numpy(getattr(x, n)).to(dev) for n in ("q", "k", "v", "alpha", "beta", "S0")}
    for n in ("q", "k", "v"):
        base[n] = base[n].to(torch.bfloat16)
    big = {n: torch.empty((B,) + tuple(t.shape[1:]), dtype=t.dtype, device=dev)
           for n, t in base.items()}
    for b in range(B):
        for n in ("q", "k", "v", "alpha", "beta"):
            big[n][b] = torch.roll(base[n][b % 2], shifts=shift(b), dims=0)
        big["S0"][b] = torch.roll(base["S0"][b % 2], shifts=b % H, dims=0)
    del base
    o, ST = gdn.prefill(big["q"], big["k"], big["v"], big["alpha"], big["beta"], big["S0"])
    torch.cuda.synchronize()
    print(f"  prefill B={B} T={T} H={H} d={d}: o holds {o.numel():.3e} elements", flush=True)
    for b, h in ((0, 0), (77, 6), (B - 1, H - 1)):
        q, k, v, al, be, s0 = host_row(b)
        o_ref, S_ref = orc.gdn_prefill(q, k, v, al, be, s0, heads=[(0, h)])
        check_o(f"o (b={b}, h={h})", host(o[b])[None], o_ref, TOL_BF16, heads=[(0, h)])
        check_S(f"S_T (b={b}, h={h})", host(ST[b])[None], S_ref, TOL_F32, heads=[(0, h)])
    del big, o, ST
    torch.cuda.empty_cache()


def test_decode_offsets_past_2_31():
    """B=8448, H=16, dk=dv=128, in place: the state holds 2.21e9 floats."""
    dev = torch.device("cuda", 0)
    B, H, d, NB = 8448, 16, 128, 64
    N = B * H
    assert N * d * d > 2 ** 31
    x = gi.generic(B, 1, H, d, d, gi.seed_for(3, 8), "bf16")
    rng = np.random.Generator(np.random.PCG64(gi.seed_for(3, 9)))
    Sb = (0.3 * rng.standard_normal((NB, d, d))).astype(np.float32)
    r1 = lambda i: (i // NB) % d
    r2 = lambda i: (i // (NB * d)) % d

    def host_state(i):
        return np.roll(np.roll(Sb[i % NB], r1(i), axis=0), r2(i), axis=1)

    Sb_dev = torch.from_numpy(Sb).to(dev)
    S = torch.empty((N, d, d), dtype=torch.float32, device=dev)
    ar = torch.arange(d, device=dev)
    for c0 in range(0, N, 8192):              # gather in slices of 8192 states
        i = torch.arange(c0, min(N, c0 + 8192), device=dev)
        rows = (ar[None, :, None] - ((i // NB) % d)[:, None, None]) % d
        cols = (ar[None, None, :] - ((i // (NB * d)) % d)[:, None, None]) % d
        S[c0:c0 + len(i)] = Sb_dev[(i % NB)[:, None, None], rows, cols]
    S = S.view(B, H, d, d)
    picks = (0, 70001, N - 1)
    S_in = {i: host_state(i) for i in picks}
    for i in picks:                           # the construction, checked on the host
        assert np.array_equal(S[i // H, i % H].cpu().numpy(), S_in[i])
    q = torch.from_numpy(x.q[:, 0]).to(dev).to(torch.bfloat16)
    k = torch.from_numpy(x.k[:, 0]).to(dev).to(torch.bfloat16)
    v = torch.from_numpy(x.v[:, 0]).to(dev).to(torch.bfloat16)
    al = torch.from_numpy(x.alpha[:, 0]).to(dev)
    be = torch.from_numpy(x.beta[:, 0]).to(dev)
    o, S1 = gdn.decode_step(q, k, v, al, be, S, S_out=S)
    torch.cuda.synchronize()
    print(f"  decode B={B} H={H} d={d}: the state holds {S.numel():.3e} floats", flush=True)
    for i in picks:
        b, h = i // H, i % H
        sl = lambda a: np.asarray(a[b, 0, h], np.float64)[None, None]
        o_ref, S_ref = orc.gdn_decode_step(sl(x.q), sl(x.k), sl(x.v), sl(x.alpha),
                                           sl(x.beta), S_in[i][None, None].astype(np.float64))
        check_step(f"o (head {i})", host(o[b, h])[None, None], o_ref, TOL_BF16)
        check_S(f"S' (head {i})", host(S1[b, h])[None, None], S_ref, TOL_F32)
    del S, S1, o
    torch.cuda.empty_cache()


def test_segmented_prefill_offsets_past_2_31():
    """B=1, T=1,114,112, H=16, d=128, bf16 (the segmented path, 16 segments
    per head): q, k, v, o and x^ hold 2.28e9 elements.

    With log alpha <= -0.05 per token, the state before the last W = 4096
    tokens reaches the end only through the product of the window's
    transitions alpha_t (I - beta_t k_t k_t^T), whose norm is at most
    prod alpha_t <= e^(-0.05 W); so the oracle run over the last W tokens
    from a zero state gives S_T, and the outputs of the last W/2 tokens,
    exactly up to e^(-102) of the state's scale."""
    dev = torch.device("cuda", 0)
    T0, NCOPY, H, d, W = 32768, 34, 16, 128, 4096
    T = T0 * NCOPY
    assert T * H * d > 2 ** 31
    x = gi.generic(1, T0, H, d, d, gi.seed_for(2, 9), "bf16", log_alpha_range=(0.05, 0.1))
    shift = lambda j: (7919 * j) % T0
    big = {}
    for n in ("q", "k", "v", "alpha", "beta"):
        src = torch.from_numpy(getattr(x, n)[0]).to(dev)
        if n in ("q", "k", "v"):
            src = src.to(torch.bfloat16)
        t = torch.empty((1, T) + tuple(src.shape[1:]), dtype=src.dtype, device=dev)
        for j in range(NCOPY):
            t[0, j * T0:(j + 1) * T0] = torch.roll(src, shifts=shift(j), dims=0)
        big[n] = t
        del src
    o, ST = gdn.prefill(big["q"], big["k"], big["v"], big["alpha"], big["beta"])
    torch.cuda.synchronize()
    print(f"  segmented prefill T={T} H={H} d={d}: o holds {o.numel():.3e} elements", flush=True)
    win = lambda a: np.roll(a[0], shift(NCOPY - 1), axis=0)[T0 - W:][None]
    o_ref, S_ref = orc.gdn_prefill(win(x.q), win(x.k), win(x.v), win(x.alpha), win(x.beta),
                                   heads=[(0, 0), (0, H - 1)])
    o_dev = host(o[0, T - W // 2:])[None]
    for h in (0, H - 1):
        check_o(f"o, last {W // 2} tokens (h={h})", o_dev, o_ref[:, W // 2:], TOL_BF16,
                heads=[(0, h)])
        check_S(f"S_T (h={h})", host(ST), S_ref, TOL_F32, heads=[(0, h)])
    del big, o, ST
    torch.cuda.empty_cache()


def test_gated_prefill_offsets_past_2_31():
    """The generalised gates in chunked form at B=136, T=8192, H=16, dk=64,
    dv=128, bf16: v, o and the fp32 write gate hold 2.28e9 elements (the
    per-key-channel gates 1.14e9 fp32, 4.6 GB each); batch entry b is a
    cyclic token shift, by 997 b, of one of two seeded rows."""
    dev = torch.device("cuda", 0)
    B, T, H, dk, dv = 136, 8192, 16, 64, 128
    assert B * T * H * dv > 2 ** 31
    x = gi.generic(2, T, H, dk, dv, gi.seed_for(4, 8), "bf16", S0_scale=0.3)
    al, bg, wg = gi.gate_vectors(2, T, H, dk, dv, gi.seed_for(4, 9))
    shift = lambda b: (997 * b) % T
    rows = {"q": x.q, "k": x.k, "v": x.v, "alpha": al, "b": bg, "w": wg}
    big = {}
    for n, a in rows.items():
        src = torch.from_numpy(a).to(dev)
        if n in ("q", "k", "v"):
            src = src.to(torch.bfloat16)
        t = torch.empty((B,) + tuple(src.shape[1:]), dtype=src.dtype, device=dev)
        for b in range(B):
            t[b] = torch.roll(src[b % 2], shifts=shift(b), dims=0)
        big[n] = t
        del src
    S0_dev = torch.from_numpy(x.S0).to(dev)
    S0 = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    for b in range(B):
        S0[b] = torch.roll(S0_dev[b % 2], shifts=b % H, dims=0)
    o, ST = gdn.gated_prefill(big["q"], big["k"], big["v"], big["alpha"], big["b"], big["w"], S0)
    torch.cuda.synchronize()
    print(f"  gated prefill B={B} T={T} H={H} dk={dk} dv={dv}: o holds {o.numel():.3e} elements",
          flush=True)
    for b, h in ((0, 0), (B - 1, H - 1)):
        r, s = b % 2, shift(b)
        one = lambda a: np.roll(a[r], s, axis=0)[None]
        o_ref, S_ref = orc.gdn2_prefill(one(x.q), one(x.k), one(x.v), one(al), one(bg), one(wg),
                                        np.roll(x.S0[r], b % H, axis=0)[None], heads=[(0, h)])
        check_o(f"o (b={b}, h={h})", host(o[b])[None], o_ref, TOL_BF16, heads=[(0, h)])
        check_S(f"S_T (b={b}, h={h})", host(ST[b])[None], S_ref, TOL_F32, heads=[(0, h)])
    del big, o, ST, S0
    torch.cuda.empty_cache()


def test_backward_offsets_past_2_31():
    """The chunked backward pass at B=136, T=8192, H=16, dk=dv=128, bf16
    inputs: dq, dk and dv hold 2.28e9 floats each; batch entry b (inputs and
    d_o) is a cyclic token shift, by 997 b, of one of two seeded rows, its
    S0 and dS_T shifts of the head axis."""
    from tests.test_gpu_backward import compare
    dev = torch.device("cuda", 0)
    B, T, H, d = 136, 8192, 16, 128
    assert B * T * H * d > 2 ** 31
    x = gi.generic(2, T, H, d, d, gi.seed_for(5, 8), "bf16", S0_scale=0.3)
    d_o, dST = gi.cotangents(2, T, H, d, d, gi.seed_for(5, 9), "bf16")
    shift = lambda b: (997 * b) % T
    toks = {"q": x.q, "k": x.k, "v": x.v, "alpha": x.alpha, "beta": x.beta, "d_o": d_o}
    states = {"S0": x.S0, "dST": dST}
    big = {}
    for n, a in list(toks.items()) + list(states.items()):
        src = torch.from_numpy(a).to(dev)
        if n in ("q", "k", "v", "d_o"):
            src = src.to(torch.bfloat16)
        t = torch.empty((B,) + tuple(src.shape[1:]), dtype=src.dtype, device=dev)
        for b in range(B):
            t[b] = torch.roll(src[b % 2], shifts=shift(b) if n in toks else b % H, dims=0)
        big[n] = t
        del src
    g = gdn.backward(big["q"], big["k"], big["v"], big["alpha"], big["beta"], big["S0"],
                     big["d_o"], big["dST"])
    torch.cuda.synchronize()
    print(f"  backward B={B} T={T} H={H} d={d}: dq holds {g['dq'].numel():.3e} floats", flush=True)
    del big
    for b, h in ((0, 0), (B - 1, H - 1)):
        r, s = b % 2, shift(b)
        tk = lambda a: np.roll(a[r], s, axis=0)[None]
        hd = lambda a: np.roll(a[r], b % H, axis=0)[None]
        ref = orc.gdn_backward(tk(x.q), tk(x.k), tk(x.v), tk(x.alpha), tk(x.beta), hd(x.S0),
                               tk(d_o), hd(dST), heads=[(0, h)])
        gs = {n: (None if g[n] is None else g[n][b:b + 1]) for n in g}
        compare(f"(b={b}, h={h})", gs, ref, [(0, h)])
    del g
    torch.cuda.empty_cache()
