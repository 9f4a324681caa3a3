"""Pins of the oracle's activations against scalar ``math`` evaluations and special values."""
import math

import numpy as np
import pytest

from oracle import activations as act


def test_softplus_special_values_and_math_library():
    assert act.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    xs = np.linspace(-30, 30, 241)
    ref = np.array([math.log1p(math.exp(x)) if x < 30 else x + math.log1p(math.exp(-x)) for x in xs])
    np.testing.assert_allclose(act.softplus(xs), ref, rtol=1e-14, atol=1e-300)
    # no overflow far out, and the asymptote is x
    assert act.softplus(800.0) == pytest.approx(800.0, rel=1e-15)
    assert act.softplus(-800.0) == 0.0 or act.softplus(-800.0) < 1e-300


def test_sigmoid_special_values_and_math_library():
    assert act.sigmoid(0.0) == 0.5
    xs = np.linspace(-40, 40, 161)
    ref = np.array([1.0 / (1.0 + math.exp(-x)) for x in xs])
    np.testing.assert_allclose(act.sigmoid(xs), ref, rtol=1e-14)
    np.testing.assert_allclose(act.sigmoid(xs) + act.sigmoid(-xs), 1.0, rtol=1e-15)
    assert act.beta_from(0.3, "probability") == 0.3


def test_gate_formula_against_math_library():
    rng = np.random.default_rng(0)
    A_log = rng.uniform(0, math.log(16), 4)
    dt = rng.uniform(-1, 1, 4)
    a = rng.standard_normal((3, 4))
    g = act.gdn_log_gate(A_log, a, dt)
    for t in range(3):
        for h in range(4):
            ref = -math.exp(A_log[h]) * math.log1p(math.exp(a[t, h] + dt[h]))
            assert g[t, h] == pytest.approx(ref, rel=1e-14)
    assert np.all(g < 0)
    # A_log = 0 and a + dt_bias = 0 give alpha = exp(-ln 2) = 1/2
    assert np.exp(act.gdn_log_gate(np.zeros(1), np.zeros((1, 1)), np.zeros(1)))[0, 0] == pytest.approx(0.5, rel=1e-15)


def test_kda_gate_is_per_channel_with_per_head_rate():
    rng = np.random.default_rng(1)
    HV, K = 3, 5
    a_log = rng.uniform(0, math.log(16), HV)
    dt = rng.uniform(-1, 1, (HV, K))
    raw = rng.standard_normal((2, HV, K))
    g = act.kda_log_gate(a_log, raw, dt)
    for t in range(2):
        for h in range(HV):
            for c in range(K):
                ref = -math.exp(a_log[h]) * math.log1p(math.exp(raw[t, h, c] + dt[h, c]))
                assert g[t, h, c] == pytest.approx(ref, rel=1e-14)


def test_l2_normalisation_and_scale():
    rng = np.random.default_rng(2)
    K = 16
    q, k = rng.standard_normal((3, K)) * 7, rng.standard_normal((3, K)) * 0.1
    qh, kh = act.prepare_qk(q, k)
    # unit norm up to the epsilon: ||x|| / sqrt(||x||^2 + 1e-6)
    nk = np.linalg.norm(k, axis=-1)
    np.testing.assert_allclose(np.linalg.norm(kh, axis=-1), nk / np.sqrt(nk ** 2 + 1e-6), rtol=1e-14)
    np.testing.assert_allclose(np.linalg.norm(kh, axis=-1), 1.0, rtol=1e-4)
    np.testing.assert_allclose(np.linalg.norm(qh, axis=-1), 1.0 / math.sqrt(K), rtol=1e-6)
    # the epsilon reading: ||x|| = 5 gives 5 / sqrt(25 + 1e-6)
    x = np.array([3.0, 4.0])
    assert np.linalg.norm(act.l2_normalize(x)) == pytest.approx(5.0 / math.sqrt(25.0 + 1e-6), rel=1e-15)
    qh2, kh2 = act.prepare_qk(q, k, scale=2.0, use_qk_l2norm=False)
    np.testing.assert_array_equal(qh2, q * 2.0)
    np.testing.assert_array_equal(kh2, k)
