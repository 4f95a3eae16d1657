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
