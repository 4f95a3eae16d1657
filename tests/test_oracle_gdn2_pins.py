"""Pins of the oracle's generalised gates (gdn2_head / gdn2_prefill): a
per-key-channel decay on the right of the state (Kimi Delta Attention) and a
key-side erase gate b with a value-side write gate w (Gated DeltaNet-2),
"Linear Attention Architectures" reading notes on paper Secs. 3.4-3.5.  Each pin is a
hand-worked value, an exact reduction to the already pinned gated delta rule,
or an invariant, chosen so that a slip (decay on the wrong side, the erase
outer product along e instead of k, the gates swapped) fails one of them."""

import numpy as np
import pytest

from oracle import gdn_oracle as orc
from tests.test_oracle_pins import golden, rng


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def test_worked_one_token():
    g = golden("generalised_gates_one_token")
    arr = lambda n: np.array(g[n], dtype=np.float64)[None]
    o, S = orc.gdn2_head(arr("q"), arr("k"), arr("v"), arr("alpha"), arr("b"), arr("w"),
                         np.array(g["S0"]))
    np.testing.assert_allclose(S, g["S1"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[0], g["o"], rtol=0, atol=1e-14)


@pytest.mark.parametrize("dk,dv", [(8, 5), (6, 6)])
def test_reduces_to_gated_delta_rule(dk, dv):
    # alpha = a * 1 and b = w = beta * 1 give exactly the gated delta rule
    r = rng(21)
    T = 30
    q, k = unit(r.standard_normal((T, dk))), unit(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    a, be = r.uniform(0.5, 1.0, T), r.uniform(0, 1, T)
    S0 = r.standard_normal((dv, dk))
    o1, S1 = orc.gdn2_head(q, k, v, np.repeat(a[:, None], dk, 1), np.repeat(be[:, None], dk, 1),
                           np.repeat(be[:, None], dv, 1), S0)
    o2, S2 = orc.gdn_head(q, k, v, a, be, S0)
    np.testing.assert_allclose(S1, S2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-13)


def test_kda_write_stores_value_exactly():
    # b = w = 1 with a unit key: after the write S_t k_t = v_t whatever the
    # per-channel decay (the delta rule's defining property survives KDA)
    r = rng(22)
    dk, dv = 7, 4
    k = unit(r.standard_normal((1, dk)))
    v = r.standard_normal((1, dv))
    S0 = r.standard_normal((dv, dk))
    _, S = orc.gdn2_head(r.standard_normal((1, dk)), k, v, r.uniform(0.1, 1, (1, dk)),
                         np.ones((1, dk)), np.ones((1, dv)), S0)
    np.testing.assert_allclose(S @ k[0], v[0], rtol=1e-13, atol=1e-13)


def test_zero_gates_only_decay_per_channel():
    r = rng(23)
    dk, dv, T = 5, 3, 4
    S0 = r.standard_normal((dv, dk))
    al = r.uniform(0.2, 1.0, (T, dk))
    _, S = orc.gdn2_head(r.standard_normal((T, dk)), r.standard_normal((T, dk)),
                         r.standard_normal((T, dv)), al, np.zeros((T, dk)), np.zeros((T, dv)), S0)
    np.testing.assert_allclose(S, S0 * np.prod(al, axis=0)[None, :], rtol=1e-14, atol=0)


def test_unkeyed_channel_keeps_its_column():
    # a key channel that no key uses, with retention 1, is never read by the
    # erase nor written: its state column stays exactly as it was
    r = rng(24)
    dk, dv, T = 6, 4, 20
    k = r.standard_normal((T, dk))
    k[:, 2] = 0.0
    al = r.uniform(0.5, 1.0, (T, dk))
    al[:, 2] = 1.0
    S0 = r.standard_normal((dv, dk))
    _, S = orc.gdn2_head(r.standard_normal((T, dk)), k, r.standard_normal((T, dv)), al,
                         r.uniform(0, 1, (T, dk)), r.uniform(0, 1, (T, dv)), S0)
    assert np.array_equal(S[:, 2], S0[:, 2])


def test_write_gate_scales_value_rows_only():
    # w enters only as z = w * v: scaling the value channel i of both the
    # write gate's target (v) and its gate by reciprocal factors changes nothing
    r = rng(25)
    dk, dv, T = 5, 4, 15
    args = [r.standard_normal((T, dk)), unit(r.standard_normal((T, dk))),
            r.standard_normal((T, dv)), r.uniform(0.5, 1, (T, dk)), r.uniform(0, 1, (T, dk)),
            r.uniform(0.1, 1, (T, dv))]
    o1, S1 = orc.gdn2_head(*args)
    c = np.array([2.0, 0.5, 4.0, 0.25])
    args2 = list(args)
    args2[2] = args[2] * c
    args2[5] = args[5] / c
    o2, S2 = orc.gdn2_head(*args2)
    np.testing.assert_allclose(S2, S1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)


def test_batched_layout_matches_per_head():
    r = rng(26)
    B, T, H, dk, dv = 2, 9, 3, 4, 5
    q, k = r.standard_normal((B, T, H, dk)), unit(r.standard_normal((B, T, H, dk)))
    v = r.standard_normal((B, T, H, dv))
    al, b, w = r.uniform(0.5, 1, (B, T, H, dk)), r.uniform(0, 1, (B, T, H, dk)), r.uniform(0, 1, (B, T, H, dv))
    S0 = r.standard_normal((B, H, dv, dk))
    o, S = orc.gdn2_prefill(q, k, v, al, b, w, S0)
    o1, S1 = orc.gdn2_head(q[1, :, 2], k[1, :, 2], v[1, :, 2], al[1, :, 2], b[1, :, 2],
                           w[1, :, 2], S0[1, 2])
    np.testing.assert_array_equal(o[1, :, 2], o1)
    np.testing.assert_array_equal(S[1, 2], S1)
