"""Pins of the float64 sequential recurrence against what the pages and the mathematics fix.

None of these compares the oracle with a retyped copy of itself: they use
hand-worked values (tests/golden/worked_steps.txt), closed forms, limiting
cases from the Circuit.LLM.Mixer page, invariances, and three independently
written forms (chunked WY scan, explicit transition products, exact
rationals).
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import activations as act
from oracle import chunked, exact, unrolled
from oracle import decode as odec
from oracle.recurrence import gated_delta_step, run_suffix
from tests.golden import load_cases

CASES = load_cases()


def _f(x):
    return np.array(x, dtype=np.float64)


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# ---------------------------------------------------------------- golden

@pytest.mark.parametrize("name", ["gated_scalar", "kda_rows", "forget_all"])
def test_golden_worked_step(name):
    c = CASES[name]
    S0 = _f(c["S0"])[None]
    alpha = _f([c["alpha"]]) if "alpha" in c else _f(c["alpha_vec"])[None]
    o, S1 = gated_delta_step(S0, _f(c["q"])[None], _f(c["k"])[None], _f(c["v"])[None],
                             alpha, _f([c["beta"]]))
    np.testing.assert_allclose(S1[0], _f(c["S1"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[0], _f(c["o"]), rtol=0, atol=1e-15)


def test_golden_activated_through_front_end():
    c = CASES["activated"]
    q = _f(c["q_raw"])[None, None]          # [T=1, HK=1, K=2]
    k = _f(c["k_raw"])[None, None]
    v = _f(c["v"])[None, None]
    a = _f([[c["a"]]])
    b = _f([[c["b"]]])
    pool = _f(c["S0"])[None, None]          # [slots=1, HV=1, K, V]
    out, written = odec.gdn_decode_pooled(q, k, v, a, b, _f([c["A_log"]]), _f([c["dt_bias"]]),
                                          None, [0], pool, scale=float(c["scale"]))
    np.testing.assert_allclose(written[0][0], _f(c["S1"]), rtol=1e-7, atol=0)
    np.testing.assert_allclose(out[0, 0], _f(c["o"]), rtol=1e-7, atol=0)


# ---------------------------------------------------------------- closed forms

def test_beta0_gate0_leaves_state_bit_identical():
    rng = _rng(1)
    H, K, V = 3, 8, 5
    S0 = rng.standard_normal((H, K, V))
    q, k = _unit(rng, (H, K)), _unit(rng, (H, K))
    v = rng.standard_normal((H, V))
    alpha = np.exp(np.zeros(H))                   # g = 0
    o, S1 = gated_delta_step(S0, q, k, v, alpha, np.zeros(H))
    assert np.array_equal(S1, S0)
    np.testing.assert_allclose(o, np.einsum("hk,hkv->hv", q, S0), rtol=1e-15, atol=1e-15)


@pytest.mark.parametrize("kda", [False, True])
def test_beta0_is_pure_decay(kda):
    rng = _rng(2)
    H, K, V = 2, 6, 4
    S0 = rng.standard_normal((H, K, V))
    alpha = rng.uniform(0.1, 0.9, (H, K) if kda else (H,))
    _, S1 = gated_delta_step(S0, _unit(rng, (H, K)), _unit(rng, (H, K)),
                             rng.standard_normal((H, V)), alpha, np.zeros(H))
    for h in range(H):
        for i in range(K):
            a = alpha[h, i] if kda else alpha[h]
            np.testing.assert_allclose(S1[h, i], a * S0[h, i], rtol=1e-15)


def test_alpha0_forgets_then_writes():
    rng = _rng(3)
    H, K, V = 2, 7, 5
    S0 = rng.standard_normal((H, K, V))
    q, k = _unit(rng, (H, K)), _unit(rng, (H, K))
    v = rng.standard_normal((H, V))
    beta = rng.uniform(0, 1, H)
    o, S1 = gated_delta_step(S0, q, k, v, np.zeros(H), beta)
    for h in range(H):
        np.testing.assert_allclose(S1[h], beta[h] * np.outer(k[h], v[h]), rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(o[h], beta[h] * (q[h] @ k[h]) * v[h], rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("zero_init", [True, False])
def test_alpha1_beta1_orthonormal_keys_recover_values(zero_init):
    rng = _rng(4)
    K, V, T = 8, 5, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((K, K)))
    keys = Qm.T[:T]                                 # orthonormal rows
    vals = rng.standard_normal((T, V))
    S = np.zeros((1, K, V)) if zero_init else rng.standard_normal((1, K, V))
    for t in range(T):
        _, S = gated_delta_step(S, keys[t][None], keys[t][None], vals[t][None], np.ones(1), np.ones(1))
    for t in range(T):
        np.testing.assert_allclose(keys[t] @ S[0], vals[t], rtol=1e-12, atol=1e-12)


def test_alpha1_beta1_signed_basis_keys_recover_bit_exactly():
    rng = _rng(5)
    K, V = 6, 4
    perm = rng.permutation(K)
    S = np.zeros((1, K, V))
    vals = rng.standard_normal((K, V))
    keys = []
    for t in range(K):
        kv = np.zeros(K)
        kv[perm[t]] = -1.0 if t % 2 else 1.0
        keys.append(kv)
        _, S = gated_delta_step(S, kv[None], kv[None], vals[t][None], np.ones(1), np.ones(1))
    for t in range(K):
        assert np.array_equal(keys[t] @ S[0], vals[t])


def test_scalar_gate_equals_kda_gate_with_equal_channels():
    rng = _rng(6)
    T, H, K, V = 5, 3, 8, 6
    S0 = rng.standard_normal((H, K, V))
    q, k = _unit(rng, (T, H, K)), _unit(rng, (T, H, K))
    v = rng.standard_normal((T, H, V))
    g = -rng.uniform(0.01, 3, (T, H))
    beta = rng.uniform(0, 1, (T, H))
    o1, S1 = run_suffix(S0, q, k, v, np.exp(g), beta)
    o2, S2 = run_suffix(S0, q, k, v, np.repeat(np.exp(g)[:, :, None], K, axis=2), beta)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
    # and through the activation front-ends: a KDA gate whose raw_gate and
    # dt_bias are equal across channels reproduces the GDN gate
    A_log = rng.uniform(0, np.log(16), H)
    a = rng.standard_normal((T, H))
    dt = rng.uniform(-1, 1, H)
    g_gdn = act.gdn_log_gate(A_log, a, dt)
    g_kda = act.kda_log_gate(A_log, np.repeat(a[:, :, None], K, axis=2), np.repeat(dt[:, None], K, axis=1))
    assert np.array_equal(np.repeat(g_gdn[:, :, None], K, axis=2), g_kda)


# ---------------------------------------------------------------- independent forms

def _random_suffix(seed, T, K, V, kda):
    rng = _rng(seed)
    S0 = rng.standard_normal((K, V)) * 0.5
    q = _unit(rng, (T, K)) / np.sqrt(K)
    k = _unit(rng, (T, K))
    v = rng.standard_normal((T, V))
    g = -rng.uniform(0.01, 2.0, (T, K) if kda else (T,))
    beta = rng.uniform(0.05, 1.0, T)
    return S0, q, k, v, g, beta


@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("C", [1, 2, 3, 4, 8, 64])
def test_chunked_scan_matches_sequential(C, kda):
    T, K, V = 21, 8, 5                         # 21 is not a multiple of 2, 4, 8, 64
    S0, q, k, v, g, beta = _random_suffix(100 + C, T, K, V, kda)
    o_seq, S_seq = run_suffix(S0[None], q[:, None], k[:, None], v[:, None],
                              np.exp(g)[:, None], beta[:, None])
    o_ch, S_ch = chunked.chunked_scan(S0, q, k, v, g, beta, chunk_size=C)
    np.testing.assert_allclose(o_ch, o_seq[:, 0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S_ch, S_seq[0], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("T", [1, 2, 3, 5])
def test_unrolled_products_match_sequential(T, kda):
    K, V = 6, 4
    S0, q, k, v, g, beta = _random_suffix(200 + T, T, K, V, kda)
    alpha = np.exp(g)
    o_seq, S_seq = run_suffix(S0[None], q[:, None], k[:, None], v[:, None], alpha[:, None], beta[:, None])
    o_un, S_un = unrolled.unrolled_scan(S0, q, k, v, alpha, beta)
    np.testing.assert_allclose(o_un, o_seq[:, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S_un, S_seq[0], rtol=1e-12, atol=1e-13)


def _pythagorean_key(K, i, j, sgn=1):
    k = [Fraction(0)] * K
    k[i] = Fraction(3, 5) * sgn
    k[j] = Fraction(4, 5)
    return k


@pytest.mark.parametrize("kda", [False, True])
def test_exact_rationals_match_float64(kda):
    rng = _rng(7)
    K, V, T = 5, 3, 4
    S0 = [[Fraction(int(rng.integers(-8, 9)), 8) for _ in range(V)] for _ in range(K)]
    keys = [_pythagorean_key(K, t % K, (t + 2) % K, 1 if t % 2 else -1) for t in range(T)]
    qs = [_pythagorean_key(K, (t + 1) % K, (t + 3) % K) for t in range(T)]
    vals = [[Fraction(int(rng.integers(-16, 17)), 4) for _ in range(V)] for _ in range(T)]
    if kda:
        alpha = [[Fraction(int(rng.integers(1, 8)), 8) for _ in range(K)] for _ in range(T)]
    else:
        alpha = [Fraction(int(rng.integers(1, 8)), 8) for _ in range(T)]
    beta = [Fraction(int(rng.integers(1, 5)), 4) for _ in range(T)]
    o_ex, S_ex = exact.exact_scan(S0, qs, keys, vals, alpha, beta)
    fl = lambda m: np.array([[float(x) for x in r] for r in m])
    al = np.array([[float(x) for x in a] for a in alpha]) if kda else np.array([float(a) for a in alpha])
    o_f, S_f = run_suffix(fl(S0)[None], fl(qs)[:, None], fl(keys)[:, None], fl(vals)[:, None],
                          al[:, None], np.array([float(b) for b in beta])[:, None])
    np.testing.assert_allclose(o_f[:, 0], fl(o_ex), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(S_f[0], fl(S_ex), rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- invariances of the front-ends

def _pooled_inputs(seed, B=3, HK=2, HV=4, K=8, V=6, lens=(2, 0, 3)):
    rng = _rng(seed)
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    d = dict(q=rng.standard_normal((T, HK, K)), k=rng.standard_normal((T, HK, K)),
             v=rng.standard_normal((T, HV, V)), a=rng.standard_normal((T, HV)),
             b=rng.standard_normal((T, HV)), A_log=rng.uniform(0, np.log(16), HV),
             dt_bias=rng.uniform(-1, 1, HV))
    pool = rng.standard_normal((5, HV, K, V)) * 0.05
    return d, cu, np.array([4, 1, 2]), pool


def test_layout_transpose_invariance():
    d, cu, si, pool = _pooled_inputs(10)
    o1, w1 = odec.gdn_decode_pooled(**d, cu_seqlens=cu, state_indices=si, pool=pool, state_layout="K_FIRST")
    o2, w2 = odec.gdn_decode_pooled(**d, cu_seqlens=cu, state_indices=si, pool=np.swapaxes(pool, -1, -2),
                                    state_layout="V_FIRST")
    assert np.array_equal(o1, o2, equal_nan=True)
    assert w1.keys() == w2.keys()
    for s in w1:
        assert np.array_equal(w1[s], np.swapaxes(w2[s], -1, -2))


def test_gqa_equals_repeated_keys():
    d, cu, si, pool = _pooled_inputs(11)
    o1, w1 = odec.gdn_decode_pooled(**d, cu_seqlens=cu, state_indices=si, pool=pool)
    d2 = dict(d)
    d2["q"] = np.repeat(d["q"], 2, axis=1)      # HK=2 -> 4: value head h uses key head h // 2
    d2["k"] = np.repeat(d["k"], 2, axis=1)
    o2, w2 = odec.gdn_decode_pooled(**d2, cu_seqlens=cu, state_indices=si, pool=pool)
    assert np.array_equal(o1, o2, equal_nan=True)
    for s in w1:
        assert np.array_equal(w1[s], w2[s])


def test_empty_suffix_writes_nothing():
    d, cu, si, pool = _pooled_inputs(12)
    _, w = odec.gdn_decode_pooled(**d, cu_seqlens=cu, state_indices=si, pool=pool,
                                  qdq="fp8_e4m3_tile", block_v=3, quantize_initial=True)
    assert set(w) == {4, 2}                      # sequence 1 (slot 1) has no tokens


def test_batch_permutation_invariance():
    d, cu, si, pool = _pooled_inputs(13)
    o1, w1 = odec.gdn_decode_pooled(**d, cu_seqlens=cu, state_indices=si, pool=pool)
    lens = np.diff(cu)
    perm = [2, 0, 1]
    rows = np.concatenate([np.arange(cu[p], cu[p + 1]) for p in perm]).astype(int)
    d2 = {kk: (vv[rows] if kk in ("q", "k", "v", "a", "b") else vv) for kk, vv in d.items()}
    cu2 = np.concatenate([[0], np.cumsum(lens[perm])])
    o2, w2 = odec.gdn_decode_pooled(**d2, cu_seqlens=cu2, state_indices=si[perm], pool=pool)
    assert np.array_equal(o1[rows], o2, equal_nan=True)
    for s in w1:
        assert np.array_equal(w1[s], w2[s])


def test_suffix_split_into_two_calls_equals_one_call():
    rng = _rng(14)
    HK, HV, K, V, T = 1, 2, 8, 4, 5
    d = dict(q=rng.standard_normal((T, HK, K)), k=rng.standard_normal((T, HK, K)),
             v=rng.standard_normal((T, HV, V)), a=rng.standard_normal((T, HV)),
             b=rng.standard_normal((T, HV)), A_log=rng.uniform(0, np.log(16), HV),
             dt_bias=rng.uniform(-1, 1, HV))
    pool = rng.standard_normal((2, HV, K, V))
    o_all, w_all = odec.gdn_decode_pooled(**d, cu_seqlens=np.array([0, T]), state_indices=[1], pool=pool)
    cut = 2
    first = {kk: (vv[:cut] if kk in ("q", "k", "v", "a", "b") else vv) for kk, vv in d.items()}
    second = {kk: (vv[cut:] if kk in ("q", "k", "v", "a", "b") else vv) for kk, vv in d.items()}
    o1, w1 = odec.gdn_decode_pooled(**first, cu_seqlens=np.array([0, cut]), state_indices=[1], pool=pool)
    pool2 = pool.copy()
    pool2[1] = w1[1]
    o2, w2 = odec.gdn_decode_pooled(**second, cu_seqlens=np.array([0, T - cut]), state_indices=[1], pool=pool2)
    np.testing.assert_allclose(np.concatenate([o1, o2]), o_all, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(w2[1], w_all[1], rtol=1e-14, atol=1e-15)
