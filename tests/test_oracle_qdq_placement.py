"""Pins of where the state rounding sits inside a token, and of the two decode-policy flags.

The pages fix (modelopt ... linear_attention.config, LinearAttentionConfig,
the state.block_v paragraph, and LinearAttentionDecodeConfig, readout and
quantize_initial; modelopt ... linear_attention.decode,
recurrent_decode_reference):
* the state is rounded after each token's whole update (decay, then the
  delta write), so every state leaving a token, the last one included, is
  on its tiles' grids;
* readout 'working' reads the output from the updated state before that
  rounding, 'stored' from the rounded state;
* quantize_initial rounds the state read from the pool once, before the
  first token (and a call with no tokens does not round at all).

Pinned here by hand-worked tokens (tests/golden/qdq_steps.txt: an fp8 tile
case over two tokens and an int8_hadamard32 case, every value worked out by
hand with the arithmetic shown) and by properties on random states that
hold for any correct placement: a rounded state is a fixed point of the
rounding, a stored-readout output is q_hat^T of the state the token leaves,
a working-readout output and the state before rounding are those of the
same token without rounding, and quantize_initial equals starting from the
rounded state.  tests/test_oracle_mutations.py plants the plausible wrong
placements (rounding before the decay, the readouts swapped,
quantize_initial ignored, the last token left unrounded) and checks that
these pins catch each one.
"""
import numpy as np
import pytest

import oracle.recurrence as rec
from oracle import e4m3
from oracle import hadamard as had
from tests.golden import load_cases

CASES = load_cases("qdq_steps.txt")


def _f(x):
    return np.array(x, dtype=np.float64)


def _alt(rows):
    """Rows written as their two alternating entries -> [rows, 32]."""
    r = _f(rows)
    r = r[None] if r.ndim == 1 else r
    return np.repeat(r[:, None, :], 16, axis=1).reshape(r.shape[0], 32)


def _tokens(c, n):
    """[T, H=1, ...] arrays of the case's per-token inputs (preactivated)."""
    alt = "v1_alt" in c
    q = _f([c[f"q{t}"] for t in range(1, n + 1)])[:, None]
    k = _f([c[f"k{t}"] for t in range(1, n + 1)])[:, None]
    v = np.stack([_alt(c[f"v{t}_alt"])[0] if alt else _f(c[f"v{t}"]) for t in range(1, n + 1)])[:, None]
    alpha = _f([[c[f"alpha{t}"]] for t in range(1, n + 1)])
    beta = _f([[c[f"beta{t}"]] for t in range(1, n + 1)])
    return q, k, v, alpha, beta


def _fp8(precision, block_v):
    return lambda S: e4m3.tile_qdq(S, block_v, precision)


def _codec(precision):
    return lambda S: had.int8_hadamard32_qdq(S, precision)


# ---------------------------------------------------------------- hand-worked fp8 tiles, two tokens

FP8 = CASES["fp8_two_tokens"]


@pytest.mark.parametrize("precision", ["float64", "float32"])
def test_fp8_tile_rounding_of_hand_worked_states(precision):
    bv = int(FP8["block_v"])
    for before, after in (("S1w", "S1"), ("S2w", "S2"), ("S0", "Q0"), ("S1w_qi", "S1")):
        got = e4m3.tile_qdq(_f(FP8[before])[None], bv, precision)[0]
        assert np.array_equal(got, _f(FP8[after])), (before, got)


@pytest.mark.parametrize("precision", ["float64", "float32"])
@pytest.mark.parametrize("readout", ["working", "stored"])
@pytest.mark.parametrize("qi", [False, True])
def test_fp8_two_hand_worked_tokens(precision, readout, qi):
    c = FP8
    q, k, v, alpha, beta = _tokens(c, 2)
    trace = []
    o, S = rec.run_suffix(_f(c["S0"])[None], q, k, v, alpha, beta, state_qdq=_fp8(precision, int(c["block_v"])),
                          quantize_initial=qi, readout_mode=readout, trace=trace)
    o1 = c["o1_working_qi"] if (qi and readout == "working") else c[f"o1_{readout}"]
    np.testing.assert_allclose(o[0, 0], _f(o1), rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[1, 0], _f(c[f"o2_{readout}"]), rtol=0, atol=1e-14)
    # the rounded states are dyadic and exact; so is the initial rounding
    assert np.array_equal(trace[0]["S_in"][0], _f(c["Q0"] if qi else c["S0"]))
    assert np.array_equal(trace[0]["S_out"][0], _f(c["S1"]))
    assert np.array_equal(S[0], _f(c["S2"]))


def test_fp8_single_step_places_the_rounding_after_the_update():
    c = FP8
    q, k, v, alpha, beta = _tokens(c, 1)
    qdq = _fp8("float64", int(c["block_v"]))
    S0 = _f(c["S0"])[None]
    o, S1w = rec.gated_delta_step(S0, q[0], k[0], v[0], alpha[0], beta[0])
    np.testing.assert_allclose(S1w[0], _f(c["S1w"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[0], _f(c["o1_working"]), rtol=0, atol=1e-14)
    for mode in ("working", "stored"):
        o, S1 = rec.gated_delta_step(S0, q[0], k[0], v[0], alpha[0], beta[0], state_qdq=qdq, readout_mode=mode)
        assert np.array_equal(S1[0], _f(c["S1"]))
        np.testing.assert_allclose(o[0], _f(c[f"o1_{mode}"]), rtol=0, atol=1e-14)


# ---------------------------------------------------------------- hand-worked int8_hadamard32, one token

CODEC = CASES["codec_one_token"]


@pytest.mark.parametrize("precision", ["float64", "float32"])
def test_codec_rounding_of_hand_worked_states(precision):
    tol = 1e-14 if precision == "float64" else 1e-6
    for before, after in (("S1w_alt", "S1_alt"), ("S0_alt", "Q0_alt"), ("S1w_qi_alt", "S1_alt")):
        got = had.int8_hadamard32_qdq(_alt(CODEC[before])[None], precision)[0]
        np.testing.assert_allclose(got, _alt(CODEC[after]), rtol=tol, atol=tol, err_msg=before)
    # an all-zero group is left as it is (row 0 of S0)
    assert np.array_equal(had.int8_hadamard32_qdq(_alt(CODEC["S0_alt"])[None], precision)[0, 0], np.zeros(32))


@pytest.mark.parametrize("precision", ["float64", "float32"])
@pytest.mark.parametrize("readout", ["working", "stored"])
@pytest.mark.parametrize("qi", [False, True])
def test_codec_hand_worked_token(precision, readout, qi):
    c = CODEC
    tol = 1e-13 if precision == "float64" else 1e-6
    q, k, v, alpha, beta = _tokens(c, 1)
    trace = []
    o, S = rec.run_suffix(_alt(c["S0_alt"])[None], q, k, v, alpha, beta, state_qdq=_codec(precision),
                          quantize_initial=qi, readout_mode=readout, trace=trace)
    o1 = c["o1_working_qi_alt"] if (qi and readout == "working") else c[f"o1_{readout}_alt"]
    np.testing.assert_allclose(o[0, 0], _alt(o1)[0], rtol=tol, atol=tol)
    np.testing.assert_allclose(trace[0]["S_in"][0], _alt(c["Q0_alt"] if qi else c["S0_alt"]), rtol=tol, atol=tol)
    np.testing.assert_allclose(S[0], _alt(c["S1_alt"]), rtol=tol, atol=tol)


# ---------------------------------------------------------------- properties on random states

def _random_suffix(seed, T, kda, H=2, K=8, V=8):
    rng = np.random.default_rng(seed)
    S0 = rng.standard_normal((H, K, V))
    q = rng.standard_normal((T, H, K)) / np.sqrt(K)
    k = rng.standard_normal((T, H, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, V))
    alpha = rng.uniform(0.6, 1.0, (T, H, K) if kda else (T, H))
    beta = rng.uniform(0.1, 0.9, (T, H))
    return S0, q, k, v, alpha, beta


def _kinds():
    return [("fp8", _fp8("float64", 4), 8), ("codec", _codec("float64"), 32)]


@pytest.mark.parametrize("kind,qdq,V", _kinds())
@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("T", [1, 3])
def test_every_state_leaving_a_token_is_rounded(kind, qdq, V, kda, T):
    """Rounding is idempotent (a grid value maps to itself), so the state after each token -- the
    last one included -- must be a fixed point of the rounding, and (with random states) the
    state before the rounding must not be."""
    S0, q, k, v, alpha, beta = _random_suffix(61, T, kda, V=V)
    trace = []
    _, S = rec.run_suffix(S0, q, k, v, alpha, beta, state_qdq=qdq, trace=trace)
    assert len(trace) == T
    for rec_t in trace:
        np.testing.assert_allclose(qdq(rec_t["S_out"]), rec_t["S_out"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(qdq(S), S, rtol=1e-12, atol=1e-15)
    assert not np.allclose(qdq(S0), S0, rtol=1e-6, atol=0)


@pytest.mark.parametrize("kind,qdq,V", _kinds())
@pytest.mark.parametrize("kda", [False, True])
def test_readouts_and_rounding_against_the_unrounded_step(kind, qdq, V, kda):
    """Per token, from the state entering it: the unrounded step gives the working-readout output
    and the state before rounding S'; the state leaving the token is the rounding of S'; the
    stored-readout output is q_hat^T of that state; and the two outputs differ by
    q_hat^T (QDQ(S') - S')."""
    T = 3
    S0, q, k, v, alpha, beta = _random_suffix(62, T, kda, V=V)
    trace = []
    o_work, _ = rec.run_suffix(S0, q, k, v, alpha, beta, state_qdq=qdq, readout_mode="working", trace=trace)
    o_stor, _ = rec.run_suffix(S0, q, k, v, alpha, beta, state_qdq=qdq, readout_mode="stored")
    for t, r in enumerate(trace):
        o_plain, S_upd = rec.gated_delta_step(r["S_in"], q[t], k[t], v[t], alpha[t], beta[t])
        np.testing.assert_allclose(o_work[t], o_plain, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(r["S_out"], qdq(S_upd), rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(o_stor[t], np.einsum("hk,hkv->hv", q[t], r["S_out"]), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(o_stor[t] - o_work[t], np.einsum("hk,hkv->hv", q[t], qdq(S_upd) - S_upd),
                                   rtol=1e-9, atol=1e-13)
    assert not np.allclose(o_stor, o_work, rtol=1e-6, atol=0)


@pytest.mark.parametrize("kind,qdq,V", _kinds())
@pytest.mark.parametrize("readout", ["working", "stored"])
@pytest.mark.parametrize("T", [1, 4])
def test_quantize_initial_equals_starting_from_the_rounded_state(kind, qdq, V, readout, T):
    S0, q, k, v, alpha, beta = _random_suffix(63, T, False, V=V)
    o_qi, S_qi = rec.run_suffix(S0, q, k, v, alpha, beta, state_qdq=qdq, quantize_initial=True, readout_mode=readout)
    o_ref, S_ref = rec.run_suffix(qdq(S0), q, k, v, alpha, beta, state_qdq=qdq, quantize_initial=False,
                                  readout_mode=readout)
    assert np.array_equal(o_qi, o_ref) and np.array_equal(S_qi, S_ref)
    o_no, _ = rec.run_suffix(S0, q, k, v, alpha, beta, state_qdq=qdq, quantize_initial=False, readout_mode=readout)
    if readout == "working":
        assert not np.allclose(o_qi[0], o_no[0], rtol=1e-9, atol=0)


@pytest.mark.parametrize("kind,qdq,V", _kinds())
def test_empty_suffix_rounds_nothing(kind, qdq, V):
    S0, q, k, v, alpha, beta = _random_suffix(64, 0, False, V=V)
    o, S = rec.run_suffix(S0, q, k, v, alpha, beta, state_qdq=qdq, quantize_initial=True)
    assert o.shape[0] == 0 and np.array_equal(S, S0)
