"""Pins of the int8_hadamard32 codec against the algebra of the Hadamard transform."""
import numpy as np
import pytest

from oracle import hadamard as hd


def test_hadamard_is_orthonormal_symmetric_and_butterflies_equal_the_matrix():
    H = hd.hadamard_matrix() / np.sqrt(32)
    np.testing.assert_allclose(H @ H.T, np.eye(32), atol=1e-15)
    assert np.array_equal(H, H.T)
    assert np.array_equal(np.abs(hd.hadamard_matrix()), np.ones((32, 32)))
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 32))
    np.testing.assert_allclose(hd.fwht_butterflies(x), x @ hd.hadamard_matrix(), rtol=1e-14, atol=1e-13)


def test_folded_form_equals_the_normalised_definition():
    rng = np.random.default_rng(5)
    S = rng.standard_normal((2, 5, 96)) * 0.3
    Hn = hd.hadamard_matrix() / np.sqrt(32)
    y = S.reshape(2, 5, 3, 32) @ Hn
    s = np.max(np.abs(y), axis=-1, keepdims=True) / 127
    direct = ((s * np.clip(np.rint(y / s), -127, 127)) @ Hn).reshape(2, 5, 96)
    np.testing.assert_allclose(hd.int8_hadamard32_qdq(S, "float64"), direct, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("precision", ["float64", "float32"])
def test_half_code_grid_rounds_to_even_exactly(precision):
    """Rotated values z = (n + f) 2^k with amax|z| = 127 2^k: the codes are rint(n + f) exactly,
    ties to even, and the result is (code H) 2^k / 32 exactly."""
    rng = np.random.default_rng(6)
    k = -3
    n = rng.integers(-126, 126, (4, 6, 2, 32)).astype(np.float64)
    f = rng.choice([0.0, 0.5, 0.25, 0.75, -0.5], n.shape)
    z = (n + f) * 2.0 ** k
    z[..., 0] = 127 * 2.0 ** k
    z[..., 1, 3] = -127 * 2.0 ** k
    x = (z @ hd.hadamard_matrix()) / 32                  # x H = z exactly (dyadic values)
    assert np.array_equal(x.astype(np.float32).astype(np.float64), x)
    code = np.rint(z * 2.0 ** -k)                        # numpy rint: ties to even
    expect = ((code @ hd.hadamard_matrix()) * 2.0 ** (k - 5)).reshape(4, 6, 64)
    got = hd.int8_hadamard32_qdq(x.reshape(4, 6, 64), precision)
    assert np.array_equal(got, expect)
    assert np.sum(np.abs(f) == 0.5) > 100                # ties were exercised


@pytest.mark.parametrize("precision", ["float64", "float32"])
def test_code_points_round_trip(precision):
    rng = np.random.default_rng(1)
    codes = rng.integers(-127, 128, (2, 3, 64)).astype(np.float64)
    codes[..., 0] = 127.0                   # every group reaches the top code
    codes[..., 32] = -127.0
    s = 0.01
    x = (s * codes).reshape(2, 3, 2, 32) @ hd.hadamard_matrix() / np.sqrt(32)
    x = x.reshape(2, 3, 64)
    if precision == "float32":
        x = x.astype(np.float32).astype(np.float64)
    out = hd.int8_hadamard32_qdq(x, precision)
    # a wrong code would move some entry by at least s / sqrt(32) ~ 1.8e-3; rounding noise stays far below
    np.testing.assert_allclose(out, x, rtol=0, atol=1e-13 if precision == "float64" else 4e-6)


@pytest.mark.parametrize("precision", ["float64", "float32"])
def test_error_within_half_step_per_rotated_coordinate(precision):
    rng = np.random.default_rng(2)
    S = rng.standard_normal((3, 8, 64)) * 0.05
    out = hd.int8_hadamard32_qdq(S, precision)
    H = hd.hadamard_matrix() / np.sqrt(32)
    y = S.reshape(3, 8, 2, 32) @ H
    yo = out.reshape(3, 8, 2, 32) @ H
    step = np.max(np.abs(y), axis=-1, keepdims=True) / 127
    assert np.all(np.abs(yo - y) <= step / 2 * (1 + 1e-5) + 1e-7)
    # and the state error norm equals the rotated error norm (orthonormal transform)
    np.testing.assert_allclose(np.linalg.norm(out - S), np.linalg.norm(yo - y), rtol=1e-6)


def test_groups_and_key_rows_are_independent():
    rng = np.random.default_rng(3)
    S = rng.standard_normal((1, 4, 64))
    base = hd.int8_hadamard32_qdq(S, "float64")
    S2 = S.copy()
    S2[0, 1, 32:] *= 1024.0                 # one (key row, group): exact power-of-two scaling
    S2[0, 2, :] += 100.0 * (np.arange(64) == 5)   # a spike in another key row's first group
    out = hd.int8_hadamard32_qdq(S2, "float64")
    np.testing.assert_allclose(out[0, 1, 32:], base[0, 1, 32:] * 1024.0, rtol=1e-14)
    for r, cols in ((0, slice(None)), (3, slice(None)), (1, slice(0, 32)), (2, slice(32, 64))):
        assert np.array_equal(out[0, r, cols], base[0, r, cols])


def test_a_spike_spreads_over_the_group_and_comes_back_exactly():
    S = np.zeros((1, 1, 32))
    S[0, 0, 7] = 3.0
    y = S[0, 0] @ hd.hadamard_matrix() / np.sqrt(32)
    assert np.allclose(np.abs(y), 3.0 / np.sqrt(32))   # equal magnitude everywhere: all codes +-127
    np.testing.assert_allclose(hd.int8_hadamard32_qdq(S, "float64"), S, atol=1e-15)


def test_zero_group_unchanged_and_float32_agrees_with_float64():
    rng = np.random.default_rng(4)
    S = (rng.standard_normal((4, 8, 64)) * 0.05).astype(np.float32).astype(np.float64)
    S[1, 3, :32] = 0.0
    a = hd.int8_hadamard32_qdq(S, "float64")
    b = hd.int8_hadamard32_qdq(S, "float32")
    assert np.array_equal(b[1, 3, :32], np.zeros(32))
    H = hd.hadamard_matrix() / np.sqrt(32)
    step = np.max(np.abs(S.reshape(4, 8, 2, 32) @ H), axis=-1, keepdims=True) / 127
    diff = np.abs((a - b).reshape(4, 8, 2, 32) @ H)
    assert np.all(diff <= step * (1 + 1e-4) + 1e-7)      # at most one code step apart
    assert np.mean(diff > 0.5 * step) < 0.02            # code flips are rare ties


# ---------------------------------------------------------------- packed storage (codes + scales)

@pytest.mark.parametrize("precision", ["float64", "float32"])
def test_decode_of_encode_is_the_qdq(precision):
    rng = np.random.default_rng(21)
    S = rng.standard_normal((3, 5, 96)) * 0.05
    S[1, 2, 32:64] = 0.0                                   # an all-zero group
    code, scale = hd.int8_hadamard32_encode(S, precision)
    assert code.dtype == np.int8 and np.abs(code.astype(int)).max() == 127
    assert np.all(scale[1, 2, 1] == 0) and np.all(code[1, 2, 32:64] == 0)
    tol = 0 if precision == "float64" else 1e-7 * np.abs(S).max()
    np.testing.assert_allclose(hd.int8_hadamard32_decode(code, scale), hd.int8_hadamard32_qdq(S, precision),
                               rtol=0, atol=tol + 1e-17)


def test_encode_of_decode_returns_the_codes_and_scales():
    """A stored state re-encodes to the same codes (every group holds +-127) and the same scales."""
    rng = np.random.default_rng(22)
    code = rng.integers(-127, 128, (2, 4, 64)).astype(np.int8)
    code[..., 5] = 127
    code[..., 40] = -127
    scale = rng.uniform(1e-4, 1e-1, (2, 4, 2))
    for precision in ("float64", "float32"):
        c2, s2 = hd.int8_hadamard32_encode(hd.int8_hadamard32_decode(code, scale), precision)
        assert np.array_equal(c2, code)
        np.testing.assert_allclose(s2, scale, rtol=1e-6 if precision == "float32" else 1e-13)


def test_scale_is_amax_over_127_in_the_pm1_basis():
    """A single 1 in a group rotates to a row of H: every |z| = 1, scale = 1/127, codes = 127 H[j]."""
    S = np.zeros((1, 1, 32))
    S[0, 0, 9] = 1.0
    code, scale = hd.int8_hadamard32_encode(S, "float64")
    assert scale[0, 0, 0] == 1.0 / 127
    assert np.array_equal(code[0, 0], (127 * hd.hadamard_matrix()[9]).astype(np.int8))


def test_pack_layout_and_round_trip():
    rng = np.random.default_rng(23)
    code = rng.integers(-127, 128, (3, 2, 4, 64)).astype(np.int8)
    scale = rng.uniform(0, 1, (3, 2, 4, 2))
    t = hd.pack_tiles(code, scale)
    assert t.shape == (3, 2, hd.packed_tile_bytes(4, 64)) == (3, 2, 4 * 64 + 4 * 4 * 2)
    # codes first in [V / 32][K][32] order; then the float32 scales in [V / 32][K] order
    assert t[1, 0, 1 * 32 + 7] == np.uint8(code[1, 0, 1, 7].view(np.uint8))            # group 0, row 1
    assert t[1, 0, 4 * 32 + 2 * 32 + 5] == np.uint8(code[1, 0, 2, 37].view(np.uint8))   # group 1, row 2
    assert t[2, 1, 256:260].view(np.float32)[0] == np.float32(scale[2, 1, 0, 0])
    assert t[2, 1, 256 + 4 * (4 + 1):256 + 4 * (4 + 2)].view(np.float32)[0] == np.float32(scale[2, 1, 1, 1])
    c2, s2 = hd.unpack_tiles(t, 4, 64)
    assert np.array_equal(c2, code)
    assert np.array_equal(s2, scale.astype(np.float32).astype(np.float64))
