"""The pins must fail for plausible mistakes in the oracle.

Each mutant below is a copy of the per-head recurrence with one slip planted
(on the CPU, in this file only).  With the mutant swapped in for the oracle's
`gdn_head`, at least one pin of test_oracle_pins.py must fail.
"""

import numpy as np
import pytest

from oracle import gdn_oracle as orc
from tests import test_oracle_pins as pins


def _make(mutation):
    def head(q, k, v, alpha, beta, S0=None, *, erase=True, trunc_r=None,
             trunc_every=256):
        q = np.asarray(q, np.float64)
        k = np.asarray(k, np.float64)
        v = np.asarray(v, np.float64)
        T, dk = k.shape
        dv = v.shape[1]
        S = np.zeros((dv, dk)) if S0 is None else np.array(S0, np.float64)
        o = np.empty((T, dv))
        for t in range(T):
            a, b = float(alpha[t]), float(beta[t])
            Sprev = S.copy()
            if mutation == "decay_after_write":
                S = a * (S + b * np.outer(v[t] - S @ k[t], k[t]))
            else:
                S = a * S
                if mutation == "undecayed_prediction":
                    vhat = Sprev @ k[t]
                else:
                    vhat = S @ k[t]
                if not erase:
                    vhat = 0 * vhat
                if mutation == "sign":
                    S = S - b * np.outer(v[t] - vhat, k[t])
                elif mutation == "no_beta":
                    S = S + np.outer(v[t] - vhat, k[t])
                elif mutation == "beta_on_value_only":
                    S = S + np.outer(b * v[t] - vhat, k[t])
                elif mutation == "transposed_key_write":
                    S = S + b * np.outer(v[t] - vhat, k[t])[:, ::-1]
                else:
                    S = S + b * np.outer(v[t] - vhat, k[t])
            if mutation == "read_old_state":
                o[t] = Sprev @ q[t]
            elif mutation == "query_scale":
                o[t] = S @ q[t] / np.sqrt(dk)
            else:
                o[t] = S @ q[t]
            last = (t + 1 < T) if mutation != "truncate_at_end" else True
            if trunc_r is not None and (t + 1) % trunc_every == 0 and last:
                S = orc.truncate_rank(S, trunc_r)
        return o, S
    return head


MUTANTS = ["decay_after_write", "undecayed_prediction", "sign", "no_beta",
           "beta_on_value_only", "transposed_key_write", "read_old_state",
           "query_scale", "truncate_at_end"]

PIN_TESTS = [
    pins.test_worked_example_scalar,
    pins.test_worked_example_embedded,
    pins.test_prediction_moves_toward_target_general,
    lambda: pins.test_beta_one_write_is_exact(0.9),
    pins.test_decay_before_error_two_tokens,
    pins.test_orthonormal_keys_closed_form,
    pins.test_update_is_gradient_step_on_decayed_state,
    pins.test_truncation_boundaries,
    pins.test_zero_padding_embedding,
]


def test_unmutated_copy_passes(monkeypatch):
    monkeypatch.setattr(orc, "gdn_head", _make("none"))
    for t in PIN_TESTS:
        t()


@pytest.mark.parametrize("mutation", MUTANTS)
def test_mutant_is_caught(monkeypatch, mutation):
    monkeypatch.setattr(orc, "gdn_head", _make(mutation))
    failures = 0
    for t in PIN_TESTS:
        try:
            t()
        except (AssertionError, ValueError, IndexError):
            failures += 1
    assert failures > 0, f"no pin catches the '{mutation}' slip"


# --- the input path (qk_transform / gdn_prefill_qk / gdn_decode_step_qk) ---

from tests import test_oracle_qk_pins as qk_pins  # noqa: E402

QK_PIN_TESTS = [
    qk_pins.test_worked_example_kept_channels,
    qk_pins.test_selection_indexes_per_head,
    qk_pins.test_unit_norm_over_kept_and_direction,
    qk_pins.test_norm_is_per_token_and_scale_invariant,
    qk_pins.test_zero_vector_maps_to_zero_and_only_decays_the_state,
    qk_pins.test_query_scale_scales_outputs_only,
    qk_pins.test_zero_padding_embedding,
    qk_pins.test_decode_step_qk_is_one_token_of_prefill_qk,
    qk_pins.test_beta_one_write_stores_value_along_normalised_key,
]

QK_MUTANTS = ["normalise_before_select", "next_heads_subset", "scale_on_keys",
              "norm_over_tokens", "no_renormalisation"]


def _make_qk(mutation):
    def transform(x, channels=None, l2norm=True, scale=1.0):
        x = np.asarray(x, np.float64)
        if mutation == "normalise_before_select" and l2norm:
            x = x / np.linalg.norm(x, axis=-1, keepdims=True)
        if channels is not None:
            ch = np.asarray(channels)
            H = x.shape[-2]
            off = 1 if mutation == "next_heads_subset" else 0
            x = np.stack([x[..., h, :][..., ch[(h + off) % H]] for h in range(H)], axis=-2)
        if l2norm and mutation not in ("normalise_before_select", "no_renormalisation"):
            if mutation == "norm_over_tokens" and x.ndim >= 3:
                nrm = np.sqrt(np.mean(np.sum(x * x, axis=-1, keepdims=True), axis=-3,
                                      keepdims=True))
            else:
                nrm = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
            x = np.where(nrm > 0, x / np.where(nrm > 0, nrm, 1.0), 0.0)
        return x * float(scale)

    def prefill_qk(q_raw, k_raw, v, alpha, beta, S0=None, *, channels=None,
                   l2norm=True, q_scale=1.0, heads=None):
        ks = q_scale if mutation == "scale_on_keys" else 1.0
        q = transform(q_raw, channels, l2norm, q_scale)
        k = transform(k_raw, channels, l2norm, ks)
        return orc.gdn_prefill(q, k, v, alpha, beta, S0, heads=heads)

    def decode_qk(q_raw, k_raw, v, alpha, beta, S, *, channels=None,
                  l2norm=True, q_scale=1.0):
        ks = q_scale if mutation == "scale_on_keys" else 1.0
        q = transform(q_raw, channels, l2norm, q_scale)
        k = transform(k_raw, channels, l2norm, ks)
        return orc.gdn_decode_step(q, k, v, alpha, beta, S)

    return transform, prefill_qk, decode_qk


def _swap_qk(monkeypatch, mutation):
    t, p, d = _make_qk(mutation)
    monkeypatch.setattr(orc, "qk_transform", t)
    monkeypatch.setattr(orc, "gdn_prefill_qk", p)
    monkeypatch.setattr(orc, "gdn_decode_step_qk", d)


def test_unmutated_input_path_copy_passes(monkeypatch):
    _swap_qk(monkeypatch, "none")
    for t in QK_PIN_TESTS:
        t()


@pytest.mark.parametrize("mutation", QK_MUTANTS)
def test_input_path_mutant_is_caught(monkeypatch, mutation):
    _swap_qk(monkeypatch, mutation)
    failures = 0
    for t in QK_PIN_TESTS:
        try:
            t()
        except (AssertionError, ValueError, IndexError):
            failures += 1
    assert failures > 0, f"no pin catches the '{mutation}' slip"


# --- the generalised gates (gdn2_head) --------------------------------------

from tests import test_oracle_gdn2_pins as g2_pins  # noqa: E402

G2_PIN_TESTS = [
    g2_pins.test_worked_one_token,
    lambda: g2_pins.test_reduces_to_gated_delta_rule(8, 5),
    lambda: g2_pins.test_reduces_to_gated_delta_rule(6, 6),
    g2_pins.test_kda_write_stores_value_exactly,
    g2_pins.test_zero_gates_only_decay_per_channel,
    g2_pins.test_unkeyed_channel_keeps_its_column,
    g2_pins.test_write_gate_scales_value_rows_only,
]

G2_MUTANTS = ["decay_on_value_side", "erase_outer_along_e", "erase_read_along_k",
              "decay_after_erase", "write_gate_on_key"]


def _make_g2(mutation):
    def head(q, k, v, alpha, b, w, S0=None):
        q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
        alpha, b, w = (np.asarray(x, np.float64) for x in (alpha, b, w))
        T, dk = k.shape
        dv = v.shape[1]
        S = np.zeros((dv, dk)) if S0 is None else np.array(S0, np.float64)
        o = np.empty((T, dv))
        for t in range(T):
            e = b[t] * k[t]
            z = (w[t] * v[t]) if mutation != "write_gate_on_key" else (
                v[t] * np.resize(b[t], dv))
            if mutation == "decay_on_value_side" and dv == dk:
                S = alpha[t][:, None] * S
            elif mutation != "decay_after_erase":
                S = S * alpha[t][None, :]
            rd = S @ (k[t] if mutation == "erase_read_along_k" else e)
            S = S - np.outer(rd, e if mutation == "erase_outer_along_e" else k[t]) + np.outer(z, k[t])
            if mutation == "decay_after_erase":
                S = S * alpha[t][None, :]
            o[t] = S @ q[t]
        return o, S
    return head


@pytest.mark.parametrize("mutation", G2_MUTANTS)
def test_generalised_gate_mutant_is_caught(monkeypatch, mutation):
    monkeypatch.setattr(orc, "gdn2_head", _make_g2(mutation))
    failures = 0
    for t in G2_PIN_TESTS:
        try:
            t()
        except (AssertionError, ValueError, IndexError):
            failures += 1
    assert failures > 0, f"no pin catches the '{mutation}' slip"


def test_unmutated_generalised_gate_copy_passes(monkeypatch):
    monkeypatch.setattr(orc, "gdn2_head", _make_g2("none"))
    for t in G2_PIN_TESTS:
        t()


# --- backward pass ---------------------------------------------------------

def _make_backward(mutation):
    def backward(q, k, v, alpha, beta, S0, do, dST):
        q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
        T, dk = k.shape
        dv = v.shape[1]
        S = np.zeros((dv, dk)) if S0 is None else np.array(S0, np.float64)
        prev = []
        for t in range(T):
            prev.append(S)
            S = alpha[t] * S
            S = S + beta[t] * np.outer(v[t] - S @ k[t], k[t])
        G = np.zeros((dv, dk)) if dST is None else np.array(dST, np.float64)
        out = [np.empty((T, dk)), np.empty((T, dk)), np.empty((T, dv)), np.empty(T), np.empty(T)]
        for t in range(T - 1, -1, -1):
            a, b = float(alpha[t]), float(beta[t])
            St = a * prev[t]
            w = v[t] - St @ k[t]
            u = b * w
            Snew = St + np.outer(u, k[t])
            G = G + np.outer(do[t], q[t])
            out[0][t] = (prev[t] if mutation == "dq_old_state" else Snew).T @ do[t]
            du = G @ k[t]
            out[1][t] = G.T @ u - (0 if mutation == "dk_no_erase_term" else b * (St.T @ du))
            out[4][t] = du @ (u if mutation == "dbeta_times_beta" else w)
            out[2][t] = b * du
            dSt = G - b * np.outer(du, k[t])
            out[3][t] = np.sum(dSt * (St if mutation == "dalpha_decayed_state" else prev[t]))
            G = dSt if mutation == "state_grad_undecayed" else a * dSt
        return (*out, G)
    return backward


BACKWARD_MUTANTS = ["dq_old_state", "dk_no_erase_term", "dbeta_times_beta",
                    "dalpha_decayed_state", "state_grad_undecayed"]


def _backward_pins_fail():
    from tests import test_oracle_backward_pins as bp
    checks = [lambda: bp.test_matches_finite_differences(True, True),
              bp.test_beta_zero_closed_form, bp.test_linear_in_cotangents]
    failed = 0
    for c in checks:
        try:
            c()
        except AssertionError:
            failed += 1
    return failed


def test_unmutated_backward_copy_passes(monkeypatch):
    monkeypatch.setattr(orc, "gdn_head_backward", _make_backward(None))
    assert _backward_pins_fail() == 0


@pytest.mark.parametrize("mutation", BACKWARD_MUTANTS)
def test_backward_mutant_is_caught(monkeypatch, mutation):
    monkeypatch.setattr(orc, "gdn_head_backward", _make_backward(mutation))
    assert _backward_pins_fail() > 0
