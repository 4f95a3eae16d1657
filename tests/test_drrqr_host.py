"""The library's host DRRQR (gdn_drrqr_select) against the oracle's
drrqr_select: the same kept channels on calibration-like inputs, and the
strong-RRQR guarantees checked on the library's own output.  Host code: these
run without a GPU."""

import numpy as np
import pytest

from gated_deltanet_recurrent_delta_amd import binding as bd
from oracle import gdn_oracle as orc
from tests.test_oracle_drrqr_pins import calib, check_bounds, check_stopping, kahan
from workloads import gdn_inputs as gi


def calibration_head(h, n_tokens=1024, d=128):
    """M = [K_cal; Q_cal] for head h: raw (unnormalised) key and query
    projections of seeded synthetic tokens, as a pruned layer would collect
    them."""
    x = gi.raw_qk(1, n_tokens, 4, d, 8, gi.seed_for(4, 6))
    return np.concatenate([x.k[0, :, h], x.q[0, :, h]], axis=0).astype(np.float64)


@pytest.mark.parametrize("case", ["decaying", "kahan", "head0", "head3"])
def test_library_matches_oracle(case):
    if case == "decaying":
        M, k, f = calib(np.random.default_rng(41), 600, 24), 10, 1.2
    elif case == "kahan":
        M, k, f = kahan(12), 11, 1.05
    else:
        M, k, f = calibration_head(int(case[-1])), 64, 1.1
    sel_l, sw_l, rho_l = bd.drrqr_select(M, k, f)
    sel_o, sw_o, rho_o = orc.drrqr_select(M, k, f)
    print(f"  {case}: library {sw_l} trades, rho {rho_l:.4f}; oracle {sw_o} trades, rho {rho_o:.4f}")
    assert rho_l <= f
    assert set(sel_l.tolist()) == set(sel_o.tolist())
    assert sel_l.tolist() == sel_o.tolist()                    # the same factor order
    np.testing.assert_allclose(rho_l, rho_o, rtol=1e-9)
    if M.shape[1] <= 24:
        check_stopping(M, sel_l, f)
    check_bounds(M, sel_l, k, f)


def test_kahan_trades_happen_in_the_library():
    _, sw, rho = bd.drrqr_select(kahan(12), 11, 1.05)
    assert sw >= 1 and rho <= 1.05


@pytest.mark.parametrize("kw", [dict(k=0), dict(k=8), dict(f=0.5), dict(rows=7),
                                dict(max_swaps=-1)])
def test_argument_errors(kw):
    M = calib(np.random.default_rng(42), 40, 8)
    a = dict(k=3, f=1.5, rows=40, max_swaps=100)
    a.update(kw)
    sel = np.empty(8, np.int32)
    st = bd.lib.gdn_drrqr_select(M.ctypes.data_as(bd.ctypes.c_void_p), a["rows"], 8, a["k"],
                                 a["f"], a["max_swaps"], sel.ctypes.data_as(bd.ctypes.c_void_p),
                                 None, None)
    assert st == bd.GDN_EINVAL


def test_rank_deficient_input_is_rejected():
    M = np.zeros((50, 6))
    M[:, 0] = 1.0
    M[:, 3] = np.arange(50)
    with pytest.raises(bd.GdnError):
        bd.drrqr_select(M, 3)
