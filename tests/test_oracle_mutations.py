"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch each one.

Each mutation replaces one piece of ``oracle.recurrence`` or
``oracle.activations`` with a wrong variant; the pin tests of
tests/test_oracle_recurrence.py and tests/test_oracle_activations.py are
then run against the mutated oracle and at least one of them must fail.
"""
import numpy as np
import pytest

import oracle.activations as act
import oracle.recurrence as rec
import tests.test_oracle_activations as pins_act
import tests.test_oracle_recurrence as pins


def _order_write_then_decay(S, q_hat, k_hat, v, alpha, beta, state_qdq=None, readout_mode="working"):
    S = rec.delta_write(S, k_hat, v, beta)
    S = rec.decay(S, alpha)
    return rec.readout(S, q_hat), S


def _readout_before_write(S, q_hat, k_hat, v, alpha, beta, state_qdq=None, readout_mode="working"):
    S = rec.decay(S, alpha)
    o = rec.readout(S, q_hat)
    return o, rec.delta_write(S, k_hat, v, beta)


def _wrong_sign(S, k_hat, v, beta):
    v_old = np.einsum("hk,hkv->hv", k_hat, S)
    u = np.asarray(beta)[:, None] * (v_old - v)
    return S + np.einsum("hk,hv->hkv", k_hat, u)


def _no_beta(S, k_hat, v, beta):
    v_old = np.einsum("hk,hkv->hv", k_hat, S)
    return S + np.einsum("hk,hv->hkv", k_hat, v - v_old)


def _decay_columns(S, alpha):
    alpha = np.asarray(alpha)
    if alpha.ndim == 1:
        return alpha[:, None, None] * S
    return alpha[:, None, :] * S


def _no_decay(S, alpha):
    return S


def _transposed_read(S, k_hat, v, beta):
    v_old = np.einsum("hv,hkv->hk", k_hat, S)
    u = np.asarray(beta)[:, None] * (v - v_old)
    return S + np.einsum("hk,hv->hkv", k_hat, u)


def _softplus_wrong_sign(x):
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(-x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def _sigmoid_wrong_sign(x):
    return 1.0 / (1.0 + np.exp(np.asarray(x, dtype=np.float64)))


MUTATIONS = {
    "no_decay": [(rec, "decay", _no_decay)],
    "decay_after_write": [(rec, "gated_delta_step", _order_write_then_decay),
                          (pins, "gated_delta_step", _order_write_then_decay)],
    "readout_before_write": [(rec, "gated_delta_step", _readout_before_write),
                             (pins, "gated_delta_step", _readout_before_write)],
    "wrong_sign_in_u": [(rec, "delta_write", _wrong_sign)],
    "beta_dropped": [(rec, "delta_write", _no_beta)],
    "kda_decay_on_columns": [(rec, "decay", _decay_columns)],
    "transposed_read": [(rec, "delta_write", _transposed_read)],
    "softplus_sign": [(act, "softplus", _softplus_wrong_sign)],
    "sigmoid_sign": [(act, "sigmoid", _sigmoid_wrong_sign)],
}

PIN_TESTS = [
    lambda: pins.test_golden_worked_step("gated_scalar"),
    lambda: pins.test_golden_worked_step("kda_rows"),
    lambda: pins.test_golden_worked_step("forget_all"),
    pins.test_golden_activated_through_front_end,
    pins.test_beta0_gate0_leaves_state_bit_identical,
    lambda: pins.test_beta0_is_pure_decay(True),
    pins.test_alpha0_forgets_then_writes,
    lambda: pins.test_alpha1_beta1_orthonormal_keys_recover_values(False),
    lambda: pins.test_chunked_scan_matches_sequential(4, True),
    lambda: pins.test_unrolled_products_match_sequential(3, True),
    lambda: pins.test_exact_rationals_match_float64(True),
    pins_act.test_softplus_special_values_and_math_library,
    pins_act.test_sigmoid_special_values_and_math_library,
    pins_act.test_gate_formula_against_math_library,
]


def test_unmutated_oracle_passes_every_pin():
    for t in PIN_TESTS:
        t()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_each_planted_mistake_is_caught(name, monkeypatch):
    for mod, attr, fn in MUTATIONS[name]:
        monkeypatch.setattr(mod, attr, fn)
    caught = 0
    for t in PIN_TESTS:
        try:
            t()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught >= 1, f"mutation {name} passed every pin"
