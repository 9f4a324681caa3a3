"""Pins of the E4M3 rounding and of the per-tile quantise/dequantise.

The format is fixed by the OCP 8-bit floating point specification (the
pages only name ``fp8_e4m3``); PyTorch's CPU ``float8_e4m3fn`` is an
independent implementation of the same format and is used as a cross-check.
"""
import numpy as np
import pytest
import torch

from oracle import e4m3


def test_code_table_matches_torch_decode():
    ours = e4m3.e4m3_table()
    theirs = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(theirs))
    fin = ~np.isnan(ours)
    assert np.array_equal(ours[fin], theirs[fin])
    assert np.nanmax(ours) == 448.0
    assert np.isnan(ours).sum() == 2            # S.1111.111 only
    assert ours[1] == 2.0 ** -9                  # smallest subnormal


def _positive_grid():
    t = e4m3.e4m3_table()[:128]
    return np.sort(t[~np.isnan(t)])


def test_every_finite_code_is_a_fixed_point():
    t = e4m3.e4m3_table()
    fin = t[~np.isnan(t)]
    assert np.array_equal(e4m3.e4m3_round(fin), fin)


def test_midpoints_round_to_even_code_and_neighbours_to_nearest():
    g = _positive_grid()
    codes = {float(v): c for c, v in enumerate(e4m3.e4m3_table()[:128]) if not np.isnan(v)}
    for lo, hi in zip(g[:-1], g[1:]):
        mid = (lo + hi) / 2
        want = lo if codes[float(lo)] % 2 == 0 else hi
        assert e4m3.e4m3_round(mid) == want
        assert e4m3.e4m3_round(-mid) == -want
        eps = (hi - lo) * 1e-6
        assert e4m3.e4m3_round(mid - eps) == lo
        assert e4m3.e4m3_round(mid + eps) == hi


def test_saturation_above_448():
    assert e4m3.e4m3_round(463.9) == 448.0
    assert e4m3.e4m3_round(464.0) == 448.0      # tie between 448 and (absent) 480 -> even code 448
    assert e4m3.e4m3_round(1e6) == 448.0
    assert e4m3.e4m3_round(-1e6) == -448.0
    assert np.isnan(e4m3.e4m3_round(np.nan))


def test_random_values_match_torch_cast_inside_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(-448, 448, 20000),
                        rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 8, 20000)])
    x = x[np.abs(x) <= 448]
    ours = e4m3.e4m3_round(x)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ours, theirs)


@pytest.mark.parametrize("precision", ["float64", "float32"])
def test_tile_qdq_extreme_maps_to_amax_and_error_is_half_step(precision):
    rng = np.random.default_rng(1)
    H, K, V, bv = 2, 16, 8, 4
    S = rng.standard_normal((H, K, V)) * 0.05
    if precision == "float32":
        S = S.astype(np.float32).astype(np.float64)
    tol = 1e-15 if precision == "float64" else 2e-7
    Q = e4m3.tile_qdq(S, bv, precision)
    s = e4m3.tile_scales(S, bv)
    for h in range(H):
        for j in range(V // bv):
            tile, qt = S[h, :, j * bv:(j + 1) * bv], Q[h, :, j * bv:(j + 1) * bv]
            np.testing.assert_allclose(np.max(np.abs(qt)), np.max(np.abs(tile)), rtol=tol)
            step = s[h, j] * e4m3.e4m3_spacing(tile / s[h, j])
            assert np.all(np.abs(qt - tile) <= step / 2 * (1 + 1e-6) + tol * np.abs(tile))
            codes = qt / s[h, j]
            assert np.allclose(e4m3.e4m3_round(codes), codes, rtol=4 * tol, atol=0)


@pytest.mark.parametrize("precision", ["float64", "float32"])
def test_tile_qdq_idempotent_and_zero_tile_untouched(precision):
    rng = np.random.default_rng(2)
    S = rng.standard_normal((3, 8, 12))
    S[1, :, 4:8] = 0.0
    Q = e4m3.tile_qdq(S, 4, precision)
    np.testing.assert_allclose(e4m3.tile_qdq(Q, 4, precision), Q, rtol=1e-15 if precision == "float64" else 3e-7,
                               atol=0)
    assert np.array_equal(Q[1, :, 4:8], np.zeros((8, 4)))


def test_float32_decision_agrees_with_float64_rule_away_from_ties():
    rng = np.random.default_rng(4)
    S = (rng.standard_normal((4, 16, 8)) * 0.05).astype(np.float32).astype(np.float64)
    a = e4m3.tile_qdq(S, 4, "float64")
    b = e4m3.tile_qdq(S, 4, "float32")
    s = np.repeat(e4m3.tile_scales(S, 4), 4, axis=1)[:, None, :]
    step = s * e4m3.e4m3_spacing(S / s)
    # the two precisions may pick neighbouring codes only for values within
    # float32 rounding of a midpoint: never more than one step apart, and rarely
    assert np.all(np.abs(a - b) <= step * (1 + 1e-6))
    assert np.mean(np.abs(a - b) > 1e-6 * np.abs(a)) < 0.01


def test_float32_decision_is_exact_when_amax_is_448():
    # with amax = 448 the scale and its inverse are exactly 1, so the code of a
    # float32 value is e4m3_round of that value itself
    rng = np.random.default_rng(5)
    x = rng.uniform(-448, 448, (1, 16, 4)).astype(np.float32).astype(np.float64)
    x[0, 0, 0] = 448.0
    assert np.array_equal(e4m3.tile_qdq(x, 4, "float32"), e4m3.e4m3_round(x))


def test_tile_groups_all_key_rows_and_block_v_value_columns():
    rng = np.random.default_rng(3)
    S = rng.standard_normal((1, 8, 8))
    base = e4m3.tile_qdq(S, 4, "float64")
    # scaling the second [K, 4] tile by a power of two scales its QDQ exactly
    # and leaves the first tile alone; a tile spanning the wrong axis fails this
    S2 = S.copy()
    S2[:, :, 4:] *= 1024.0
    Q2 = e4m3.tile_qdq(S2, 4, "float64")
    assert np.array_equal(Q2[:, :, :4], base[:, :, :4])
    assert np.array_equal(Q2[:, :, 4:], base[:, :, 4:] * 1024.0)
    # one large element in a row of the first tile changes the whole first tile's
    # resolution (amax is over all K rows) but nothing in the second tile
    S3 = S.copy()
    S3[0, 5, 1] = 100.0
    Q3 = e4m3.tile_qdq(S3, 4, "float64")
    assert np.array_equal(Q3[:, :, 4:], base[:, :, 4:])
    assert not np.array_equal(Q3[0, 0, :4], base[0, 0, :4])


# ---------------------------------------------------------------- packed storage (codes + tile scales)

def test_encode_value_inverts_the_table_and_matches_torch_bytes():
    import torch
    tab = e4m3.e4m3_table()
    finite = [c for c in range(256) if not np.isnan(tab[c])]
    assert np.array_equal(e4m3.e4m3_encode_value(tab[finite]), np.array(finite, dtype=np.uint8))
    vals = tab[finite]
    ref = torch.tensor(vals, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3.e4m3_encode_value(vals), ref)


@pytest.mark.parametrize("precision", ["float64", "float32"])
def test_tile_decode_of_encode_is_the_qdq(precision):
    rng = np.random.default_rng(31)
    S = rng.standard_normal((3, 5, 128)) * 0.05
    S[1, :, 64:] = 0.0                                     # an all-zero tile
    codes, scales = e4m3.tile_encode(S, 64, precision)
    assert codes.dtype == np.uint8 and scales.shape == (3, 2)
    assert scales[1, 1] == 0 and np.all(codes[1, :, 64:] == 0)
    tol = 0 if precision == "float64" else 1e-7 * np.abs(S).max()
    np.testing.assert_allclose(e4m3.tile_decode(codes, scales, 64), e4m3.tile_qdq(S, 64, precision),
                               rtol=0, atol=tol + 1e-17)
    # each non-zero tile holds the top code +-448 and its scale is amax / 448
    for h in range(3):
        for t in range(2):
            if scales[h, t] > 0:
                assert np.max(np.abs(e4m3.e4m3_table()[codes[h, :, 64 * t:64 * t + 64]])) == 448.0
                np.testing.assert_allclose(scales[h, t], np.abs(S[h, :, 64 * t:64 * t + 64]).max() / 448,
                                           rtol=1e-6 if precision == "float32" else 1e-15)


@pytest.mark.parametrize("layout", ["K_FIRST", "V_FIRST"])
def test_fp8_pack_layout_and_round_trip(layout):
    rng = np.random.default_rng(32)
    K, V = 4, 128
    codes = rng.integers(0, 256, (2, 3, K, V)).astype(np.uint8)
    scales = rng.uniform(0, 1, (2, 3, 2))
    t = e4m3.pack_fp8_tiles(codes, scales, layout)
    assert t.shape == (2, 3, e4m3.fp8_tile_bytes(K, V)) == (2, 3, K * V + 128)   # whole 128-byte lines
    # element (k, v) at byte k V + v (K_FIRST) or v K + k (V_FIRST); then the float32 scales; zero padding
    k, v = 3, 77
    pos = k * V + v if layout == "K_FIRST" else v * K + k
    assert t[1, 2, pos] == codes[1, 2, k, v]
    assert t[1, 2, K * V + 4:K * V + 8].view(np.float32)[0] == np.float32(scales[1, 2, 1])
    assert np.all(t[..., K * V + 8:] == 0)
    c2, s2 = e4m3.unpack_fp8_tiles(t, K, V, layout)
    assert np.array_equal(c2, codes)
    assert np.array_equal(s2, scales.astype(np.float32).astype(np.float64))
