"""CPU emulation of the segmented chunked prefill's bf16 split points (a
design study, not a test: pytest does not collect it).

    python tests/emulate_split_precision.py [heads]   (e.g. 0,2)

The chunked form of the gated delta rule (64-token chunks; A, T = (I+A)^-1,
P; Z = V - gamma K S^T, U = T diag(beta) Z, O = gamma Q S^T + P U,
S' = gamma_C S + (U * delta)^T K) is run in fp64, with bf16 rounding
applied exactly where the GPU kernels split an fp32 operand into bf16 hi +
lo parts.  It follows the segmented structure of the 16K launch:
16 segments of 16 chunks, transition rows from the identity for segments
>= 1, the combine S_end = S_in X + S_loc with split operands, and the
correction o += bf16(S_in) x^ with x^ and o rounded to bf16.

Dropping one product of a split (as a faster kernel would) shows up as
the final-state and output errors against the fp64 oracle, printed per
variant.  The kernels keep every split pass because each variant here
leaves less than a 10x margin on the 1e-3 final-state bar.
"""
import sys
import time

import numpy as np

sys.path.insert(0, __file__.rsplit("/tests/", 1)[0])
from oracle import gdn_oracle as orc            # noqa: E402
from workloads import gdn_inputs as gi          # noqa: E402

C = 64


def bf(x):
    return gi.round_bf16(np.asarray(x, np.float64).astype(np.float32)).astype(np.float64)


def split(x):
    h = bf(x)
    return h, bf(x - h)


def chunk_consts(K, Q, al, be):
    """Padded K, Q; T diag(beta); P; gamma, gamma_C and delta of one chunk."""
    n, dk = K.shape
    g = np.cumsum(np.log(al))
    Kp = np.zeros((C, dk)); Kp[:n] = K
    Qp = np.zeros((C, dk)); Qp[:n] = Q
    gp = np.full(C, g[-1]); gp[:n] = g
    bp = np.zeros(C); bp[:n] = be
    E = np.exp(gp[:, None] - gp[None, :])
    A = np.tril(bp[:, None] * E * (Kp @ Kp.T), -1)
    P = np.tril(E * (Qp @ Kp.T))
    Tb = np.linalg.inv(np.eye(C) + A) * bp[None, :]
    gam = np.exp(gp)
    return Kp, Qp, Tb, P, gam, gam[-1], np.exp(gp[-1] - gp)


def step(S, Kp, Qp, Vp, Tb, Ph, gam, gC, dec, opt):
    """One chunk for rows S [R, dk]: new S and O^T [R, C] before rounding."""
    Sh, Sl = split(S)
    Y = Kp @ (Sh + (Sl if opt["Ylo"] else 0)).T
    Zh, Zl = split(Vp - gam[:, None] * Y)
    Th, Tl = split(Tb)
    U = Th @ Zh
    if opt["ThZl"]:
        U += Th @ Zl
    if opt["TlZh"]:
        U += Tl @ Zh
    OT = (Sh @ Qp.T) * gam[None, :] + bf(U).T @ Ph.T
    Dh, Dl = split(U * dec[:, None])
    return gC * S + (Dh + (Dl if opt["Dlo"] else 0)).T @ Kp, OT


def run_head(x, h, opt, xopt, seg_chunks=16):
    q, k, v = (np.asarray(a[0, :, h], np.float64) for a in (x.q, x.k, x.v))
    al, be = (np.asarray(a[0, :, h], np.float64) for a in (x.alpha, x.beta))
    T, dk = q.shape
    dv = v.shape[1]
    nch = (T + C - 1) // C
    nseg = (nch + seg_chunks - 1) // seg_chunks
    o = np.zeros((T, dv))
    xhat = np.zeros((T, dk))
    S_loc, X_fin = [], []
    for s in range(nseg):
        S = np.zeros((dv, dk))
        X = np.eye(dk) if s > 0 else None
        for c in range(s * seg_chunks, min(nch, (s + 1) * seg_chunks)):
            t0 = c * C
            n = min(C, T - t0)
            Kp, Qp, Tb, P, gam, gC, dec = chunk_consts(k[t0:t0 + n], q[t0:t0 + n],
                                                       al[t0:t0 + n], be[t0:t0 + n])
            Vp = np.zeros((C, dv)); Vp[:n] = v[t0:t0 + n]
            Ph = bf(P)
            S, OT = step(S, Kp, Qp, Vp, Tb, Ph, gam, gC, dec, opt)
            o[t0:t0 + n] = bf(OT.T[:n])
            if X is not None:
                X, XT = step(X, Kp, Qp, np.zeros((C, dk)), Tb, Ph, gam, gC, dec, xopt)
                xhat[t0:t0 + n] = bf(XT.T[:n])
        S_loc.append(S)
        X_fin.append(X)
    S_end = S_loc[0]
    for s in range(1, nseg):
        S_in = S_end
        Sh, Sl = split(S_in)
        Xh, Xl = split(X_fin[s])
        S_end = Sh @ Xh + Sh @ Xl + Sl @ Xh + S_loc[s]
        t0, t1 = s * seg_chunks * C, min(T, (s + 1) * seg_chunks * C)
        o[t0:t1] = bf(o[t0:t1] + xhat[t0:t1] @ bf(S_in).T)
    return o, S_end


def errors(o, ST, o_ref, S_ref):
    """Per-head relative L2 and worst per-token (per-row) error, as the
    GPU parity tests measure them."""
    rms_t = np.sqrt(np.mean(np.sum(o_ref ** 2, 1)))
    rms_r = np.sqrt(np.mean(np.sum(S_ref ** 2, 1)))
    return (np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref),
            np.max(np.linalg.norm(o - o_ref, axis=1)) / rms_t,
            np.linalg.norm(ST - S_ref) / np.linalg.norm(S_ref),
            np.max(np.linalg.norm(ST - S_ref, axis=1)) / rms_r)


def main():
    x = gi.prefill_16k()
    short = x.short_heads
    if len(sys.argv) > 1:
        heads = [int(a) for a in sys.argv[1].split(",")]
    else:
        heads = [int(np.where(~short)[0][0]), int(np.where(short)[0][0])]
    full = dict(Ylo=True, ThZl=True, TlZh=True, Dlo=True)
    single = dict(Ylo=False, ThZl=False, TlZh=False, Dlo=False)
    variants = [
        ("as built", full, full),
        ("no lo of S in K S^T", dict(full, Ylo=False), dict(full, Ylo=False)),
        ("no lo of D in the update", dict(full, Dlo=False), dict(full, Dlo=False)),
        ("no T lo . Z hi", dict(full, TlZh=False), dict(full, TlZh=False)),
        ("no T hi . Z lo", dict(full, ThZl=False), dict(full, ThZl=False)),
        ("transition rows: no lo of S", full, dict(full, Ylo=False)),
        ("transition rows: single pass", full, single),
    ]
    for h in heads:
        t = time.time()
        o_ref, S_ref = orc.gdn_prefill(x.q, x.k, x.v, x.alpha, x.beta, None, heads=[(0, h)])
        o_ref, S_ref = o_ref[0, :, h], S_ref[0, h]
        kind = "short" if short[h] else "long"
        print(f"head {h} ({kind}-horizon), oracle {time.time() - t:.1f} s", flush=True)
        for name, opt, xopt in variants:
            eo, et, eS, er = errors(*run_head(x, h, opt, xopt), o_ref, S_ref)
            print(f"  {name:30s} o {eo:.2e} (token {et:.2e})   S_T {eS:.2e} (row {er:.2e})",
                  flush=True)


if __name__ == "__main__":
    main()
