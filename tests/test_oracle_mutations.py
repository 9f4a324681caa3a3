"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch each one.

Each mutation replaces one piece of ``oracle.recurrence``,
``oracle.activations`` or ``oracle.hadamard`` with a wrong variant; the pin
tests of tests/test_oracle_recurrence.py, tests/test_oracle_activations.py,
tests/test_oracle_hadamard.py and tests/test_oracle_qdq_placement.py are
then run against the mutated oracle and at least one of them must fail.
"""
import numpy as np
import pytest

import oracle.activations as act
import oracle.hadamard as had
import oracle.recurrence as rec
import tests.test_oracle_activations as pins_act
import tests.test_oracle_hadamard as pins_had
import tests.test_oracle_qdq_placement as pins_qdq
import tests.test_oracle_recurrence as pins

_true_hadamard = had.hadamard_matrix
_true_qdq = had.int8_hadamard32_qdq
_true_step = rec.gated_delta_step
_true_run = rec.run_suffix


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


def _hadamard_one_sign(n=32):
    H = _true_hadamard(n).copy()
    H[3, 7] = -H[3, 7]
    return H


def _butterfly_swapped(x, dtype=np.float64):
    y = np.array(x, dtype=dtype, copy=True)
    n = y.shape[-1]
    h = 1
    while h < n:
        y = y.reshape(y.shape[:-1] + (n // (2 * h), 2, h))
        a, b = y[..., 0, :].copy(), y[..., 1, :].copy()
        y[..., 0, :], y[..., 1, :] = a - b, a + b
        y = y.reshape(y.shape[:-3] + (n,))
        h *= 2
    return y


def _qdq_round_half_away(S, precision="float32"):
    S = np.asarray(S, dtype=np.float64)
    Hh, K, V = S.shape
    x = S.reshape(Hh, K, V // 32, 32)
    z = x @ _true_hadamard()
    amax = np.max(np.abs(z), axis=-1, keepdims=True)
    safe = np.where(amax > 0, amax, 1.0)
    t = z * 127 / safe
    code = np.sign(t) * np.floor(np.abs(t) + 0.5)
    out = np.where(amax > 0, (code @ _true_hadamard()) * (safe / 127 / 32), x)
    return out.reshape(Hh, K, V)


def _qdq_no_back_rotation(S, precision="float32"):
    S = np.asarray(S, dtype=np.float64)
    Hh, K, V = S.shape
    y = S.reshape(Hh, K, V // 32, 32) @ (_true_hadamard() / np.sqrt(32))
    s = np.max(np.abs(y), axis=-1, keepdims=True) / 127
    s = np.where(s > 0, s, 1.0)
    return (s * np.rint(y / s)).reshape(Hh, K, V)


# ---- where the state rounding sits (LinearAttentionDecodeConfig: readout, quantize_initial)

def _qdq_before_decay(S, q_hat, k_hat, v, alpha, beta, state_qdq=None, readout_mode="working"):
    if state_qdq is not None:
        S = state_qdq(S)
    return _true_step(S, q_hat, k_hat, v, alpha, beta)


def _readout_swapped(S, q_hat, k_hat, v, alpha, beta, state_qdq=None, readout_mode="working"):
    other = {"working": "stored", "stored": "working"}[readout_mode]
    return _true_step(S, q_hat, k_hat, v, alpha, beta, state_qdq=state_qdq, readout_mode=other)


def _quantize_initial_ignored(S0, q_hat, k_hat, v, alpha, beta, state_qdq=None, quantize_initial=False,
                              readout_mode="working", trace=None):
    return _true_run(S0, q_hat, k_hat, v, alpha, beta, state_qdq=state_qdq, quantize_initial=False,
                     readout_mode=readout_mode, trace=trace)


def _last_token_unrounded(S0, q_hat, k_hat, v, alpha, beta, state_qdq=None, quantize_initial=False,
                          readout_mode="working", trace=None):
    T = q_hat.shape[0]
    if T == 0:
        return _true_run(S0, q_hat, k_hat, v, alpha, beta, state_qdq=state_qdq,
                         quantize_initial=quantize_initial, readout_mode=readout_mode, trace=trace)
    o, S = _true_run(S0, q_hat[:-1], k_hat[:-1], v[:-1], alpha[:-1], beta[:-1], state_qdq=state_qdq,
                     quantize_initial=quantize_initial, readout_mode=readout_mode, trace=trace)
    S_in = S
    o_last, S = _true_step(S, q_hat[-1], k_hat[-1], v[-1], alpha[-1], beta[-1])
    if trace is not None:
        trace.append(dict(S_in=S_in, q_hat=q_hat[-1], k_hat=k_hat[-1], alpha=alpha[-1], beta=beta[-1], S_out=S))
    return np.concatenate([o, o_last[None]]), S


MUTATIONS = {
    "hadamard_entry_sign": [(had, "hadamard_matrix", _hadamard_one_sign)],
    "butterfly_swapped": [(had, "fwht_butterflies", _butterfly_swapped)],
    "int8_max_128": [(had, "INT8_MAX", 128.0)],
    "codec_round_half_away": [(had, "int8_hadamard32_qdq", _qdq_round_half_away)],
    "codec_no_back_rotation": [(had, "int8_hadamard32_qdq", _qdq_no_back_rotation)],
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
    "qdq_before_decay": [(rec, "gated_delta_step", _qdq_before_decay)],
    "readout_swapped": [(rec, "gated_delta_step", _readout_swapped)],
    "quantize_initial_ignored": [(rec, "run_suffix", _quantize_initial_ignored)],
    "qdq_skipped_on_last_token": [(rec, "run_suffix", _last_token_unrounded)],
}

# hand-worked QDQ tokens (tests/golden/qdq_steps.txt); each placement mistake must fail one of these,
# not only a property
GOLDEN_PLACEMENT_PINS = [
    lambda: pins_qdq.test_fp8_two_hand_worked_tokens("float64", "working", False),
    lambda: pins_qdq.test_fp8_two_hand_worked_tokens("float64", "stored", False),
    lambda: pins_qdq.test_fp8_two_hand_worked_tokens("float64", "working", True),
    lambda: pins_qdq.test_codec_hand_worked_token("float64", "working", True),
    lambda: pins_qdq.test_codec_hand_worked_token("float64", "stored", False),
]
PLACEMENT = ("qdq_before_decay", "readout_swapped", "quantize_initial_ignored", "qdq_skipped_on_last_token")

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
    pins_had.test_hadamard_is_orthonormal_symmetric_and_butterflies_equal_the_matrix,
    pins_had.test_folded_form_equals_the_normalised_definition,
    lambda: pins_had.test_half_code_grid_rounds_to_even_exactly("float64"),
    lambda: pins_had.test_half_code_grid_rounds_to_even_exactly("float32"),
    lambda: pins_had.test_code_points_round_trip("float32"),
    lambda: pins_had.test_error_within_half_step_per_rotated_coordinate("float64"),
    pins_had.test_a_spike_spreads_over_the_group_and_comes_back_exactly,
    *GOLDEN_PLACEMENT_PINS,
    lambda: pins_qdq.test_every_state_leaving_a_token_is_rounded("fp8", pins_qdq._fp8("float64", 4), 8, False, 3),
    lambda: pins_qdq.test_readouts_and_rounding_against_the_unrounded_step(
        "codec", pins_qdq._codec("float64"), 32, True),
    lambda: pins_qdq.test_quantize_initial_equals_starting_from_the_rounded_state(
        "fp8", pins_qdq._fp8("float64", 4), 8, "working", 4),
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


@pytest.mark.parametrize("name", PLACEMENT)
def test_placement_mistakes_fail_a_hand_worked_case(name, monkeypatch):
    for mod, attr, fn in MUTATIONS[name]:
        monkeypatch.setattr(mod, attr, fn)
    caught = 0
    for t in GOLDEN_PLACEMENT_PINS:
        try:
            t()
        except (AssertionError, ValueError, IndexError, TypeError):
            caught += 1
    assert caught >= 1, f"mutation {name} passed every hand-worked QDQ case"
