"""FP8 E4M3 state quantise/dequantise with one amax scale per [K, block_v] tile.

Pages followed:
* modelopt ... linear_attention.config, LinearAttentionConfig: ``state.block_v``
  sets the tile width; every [Dk, block_v] tile of a sequence's head state
  has its own scale, recomputed from the tile each time.
* modelopt ... linear_attention.decode, EncodedLinearAttentionTensor: the
  encoded state holds dequantised values beside detached scales and claims
  no compressed storage.
  ``recurrent_decode`` names ``state_format='fp8_e4m3'`` and ``block_v=64``.

The FP8 format itself is not on the pages; it follows the OCP 8-bit
floating point specification (E4M3): sign bit, 4 exponent bits with bias 7,
3 mantissa bits, exponent field 0 holds subnormals m * 2^-9, the single NaN
pattern is S.1111.111, there are no infinities, the largest finite value is
448.

Readings:
* dynamic scale s = amax / 448, so the tile's largest magnitude maps to the
  top of the grid;
* round to nearest, ties to even mantissa, saturating at +-448; subnormals
  kept; a tile whose amax is 0 is left as it is; NaN propagates.
* the pages do not fix the precision in which the code of each element is
  chosen; the plain reading, and the default, is float64 throughout:
  s = amax / 448, code = E4M3(x / s), value = s * code.
  ``precision='float32'`` is the same rule with every operation rounded to
  float32 in the order y = f32(f32(x) * f32(448 / amax)), value =
  f32(code * f32(amax / 448)); it agrees with float64 except for values
  within a few float32 ulps of a midpoint between two codes, and serves to
  compare code decisions taken in that precision.

Pins (tests/test_oracle_e4m3.py): the 256-code table built from the bit
fields is checked against PyTorch's CPU ``float8_e4m3fn`` decode; every
finite code is a fixed point of ``e4m3_round``; exact midpoints go to the
even code; random values agree with PyTorch's CPU cast inside the finite
range; QDQ is idempotent and maps each tile's extreme element to +-amax.
"""
import numpy as np

E4M3_MAX = 448.0
E4M3_BIAS = 7
E4M3_MIN_NORMAL_EXP = -6  # 2^(1 - bias)


def e4m3_decode_code(code):
    """Value of one 8-bit E4M3 code (0..255) from its bit fields; NaN for S.1111.111."""
    code = int(code)
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - E4M3_BIAS)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - E4M3_BIAS)


def e4m3_table():
    """All 256 code values, index = code."""
    return np.array([e4m3_decode_code(c) for c in range(256)], dtype=np.float64)


def e4m3_round(y):
    """Round float64 values to the E4M3 grid: nearest, ties to even, saturate at +-448.

    Within the binade [2^e, 2^(e+1)) the grid spacing is 2^(e-3); below the
    smallest normal 2^-6 the spacing stays 2^-9 (subnormals).  Dividing by a
    power of two is exact, so ``rint`` (ties to even) on y / spacing picks the
    nearest grid point and, on a tie, the one with an even mantissa field.
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    _, ex = np.frexp(a)                    # a = m * 2^ex, m in [0.5, 1)
    e = np.clip(ex - 1, E4M3_MIN_NORMAL_EXP, 8)
    step = np.ldexp(1.0, e - 3)
    r = np.rint(a / step) * step
    r = np.minimum(r, E4M3_MAX)
    r = np.where(np.isnan(a), np.nan, r)
    return np.copysign(r, y)


def _tiles(S, block_v):
    """S [H, K, V] -> a view [H, K, V // block_v, block_v]: axes 1 and 3 span one [K, block_v] tile."""
    S = np.asarray(S, dtype=np.float64)
    H, K, V = S.shape
    if V % block_v != 0:
        raise ValueError("block_v must divide the value head dim")
    return S.reshape(H, K, V // block_v, block_v)


def tile_qdq(S, block_v=64, precision="float64"):
    """Quantise/dequantise S [H, K, V] with one scale per [K, block_v] tile of each head.

    For each tile: amax = max |S|; if amax == 0 the tile is unchanged;
    otherwise each element x becomes s * E4M3(x / s) with s = amax / 448,
    the division and the product evaluated in ``precision`` (see the module
    docstring).  Every tile of every head is handled at once; the arithmetic
    per element is the same as tile by tile.
    """
    x = _tiles(S, block_v)
    H, K, nt, bv = x.shape
    if precision == "float64":
        amax = np.max(np.abs(x), axis=(1, 3), keepdims=True)
        s = np.where(amax == 0.0, 1.0, amax / E4M3_MAX)
        out = np.where(amax == 0.0, x, s * e4m3_round(x / s))
    elif precision == "float32":
        f = np.float32
        x = x.astype(f)
        amax = np.max(np.abs(x), axis=(1, 3), keepdims=True)
        safe = np.where(amax == 0.0, f(1.0), amax).astype(f)
        inv = (f(E4M3_MAX) / safe).astype(f)
        sc = (safe / f(E4M3_MAX)).astype(f)
        code = e4m3_round((x * inv).astype(f).astype(np.float64)).astype(f)
        out = np.where(amax == 0.0, x, (code * sc).astype(f)).astype(np.float64)
    else:
        raise ValueError(f"unknown precision {precision!r}")
    return out.reshape(H, K, nt * bv)


def tile_scales(S, block_v=64):
    """The per-tile scales s = amax / 448 of S [H, K, V] -> [H, V // block_v]."""
    S = np.asarray(S, dtype=np.float64)
    H, K, V = S.shape
    amax = np.abs(S).reshape(H, K, V // block_v, block_v).max(axis=(1, 3))
    return amax / E4M3_MAX


def e4m3_spacing(y):
    """Grid spacing of E4M3 at magnitude |y| (the size of one quantisation step there)."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    _, ex = np.frexp(a)
    e = np.clip(ex - 1, E4M3_MIN_NORMAL_EXP, 8)
    return np.ldexp(1.0, e - 3)


# ---------------------------------------------------------------- packed storage (codes + tile scales)
#
# This repository's format (the pages keep fp8 states fake-decoded next to
# their scales and claim no compressed storage): a state is kept as its
# E4M3 bytes and its per-tile scales s = amax / 448, and stands for
# code_value * s -- exactly what tile_qdq returns.

def e4m3_encode_value(v):
    """Byte (0..255) of E4M3 grid values v (finite, |v| <= 448, on the grid): sign, exponent, mantissa
    fields; -0.0 gives 0x80."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    sign = np.signbit(v).astype(np.int64) << 7
    _, ex = np.frexp(np.where(a > 0, a, 1.0))          # a = f * 2^ex, f in [0.5, 1)
    e = ex - 1                                          # a in [2^e, 2^(e+1))
    normal = e >= E4M3_MIN_NORMAL_EXP
    field_e = np.where(normal, e + E4M3_BIAS, 0)
    mant = np.where(normal, a / np.ldexp(1.0, e) - 1.0, a / 2.0 ** (1 - E4M3_BIAS)) * 8.0
    code = sign | (field_e.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    return np.where(a > 0, code, sign).astype(np.uint8)


def tile_encode(S, block_v=64, precision="float64"):
    """E4M3 bytes [H, K, V] (uint8) and per-tile scales [H, V // block_v] of S [H, K, V];
    tile_decode(tile_encode(S)) == tile_qdq(S) at the same precision.  An all-zero tile has
    scale 0 and codes 0."""
    x = _tiles(S, block_v)
    H, K, nt, bv = x.shape
    if precision == "float64":
        amax = np.max(np.abs(x), axis=(1, 3), keepdims=True)
        s = np.where(amax == 0.0, 1.0, amax / E4M3_MAX)
        y = x / s
        scale = amax / E4M3_MAX
    elif precision == "float32":
        f = np.float32
        x32 = x.astype(f)
        amax = np.max(np.abs(x32), axis=(1, 3), keepdims=True)
        safe = np.where(amax == 0.0, f(1.0), amax).astype(f)
        inv = (f(E4M3_MAX) / safe).astype(f)
        y = (x32 * inv).astype(f).astype(np.float64)
        scale = np.where(amax == 0.0, f(0.0), (safe / f(E4M3_MAX)).astype(f)).astype(np.float64)
    else:
        raise ValueError(f"unknown precision {precision!r}")
    codes = np.where(amax == 0.0, np.uint8(0), e4m3_encode_value(e4m3_round(y)))
    return codes.reshape(H, K, nt * bv).astype(np.uint8), scale.reshape(H, nt)


def tile_decode(codes, scales, block_v=64):
    """The state [H, K, V] that E4M3 bytes and per-tile scales stand for: code value * scale."""
    codes = np.asarray(codes, dtype=np.uint8)
    vals = e4m3_table()[codes]
    return vals * np.repeat(np.asarray(scales, dtype=np.float64), block_v, axis=-1)[:, None, :]


def fp8_tile_bytes(K, V, block_v=64):
    """Bytes of one packed (row, head) tile: K V codes, then V / block_v float32 scales, the tile zero-padded to
    whole 128-byte lines."""
    return 128 * ((K * V + 4 * (V // block_v) + 127) // 128)


def pack_fp8_tiles(codes, scales, state_layout="K_FIRST", block_v=64):
    """codes [..., K, V] (logical order) and scales [..., V // block_v] -> bytes [..., fp8_tile_bytes]:
    the codes in the pool layout's order (K_FIRST [K][V], V_FIRST [V][K]), then the scales."""
    codes = np.asarray(codes, dtype=np.uint8)
    lead, (K, V) = codes.shape[:-2], codes.shape[-2:]
    c = codes if state_layout == "K_FIRST" else np.swapaxes(codes, -1, -2)
    c = np.ascontiguousarray(c).reshape(lead + (K * V,))
    nt = V // block_v
    s = np.zeros(lead + (fp8_tile_bytes(K, V, block_v) - K * V,), dtype=np.uint8)
    s[..., :4 * nt] = np.ascontiguousarray(np.asarray(scales, dtype=np.float32)).view(np.uint8).reshape(lead + (4 * nt,))
    return np.concatenate([c, s], axis=-1)


def unpack_fp8_tiles(tiles, K, V, state_layout="K_FIRST", block_v=64):
    """Inverse of pack_fp8_tiles -> (codes uint8 [..., K, V] in logical order, scales float64)."""
    t = np.ascontiguousarray(np.asarray(tiles, dtype=np.uint8))
    lead = t.shape[:-1]
    if t.shape[-1] != fp8_tile_bytes(K, V, block_v):
        raise ValueError("tile size does not match K, V and block_v")
    c = t[..., :K * V].reshape(lead + ((K, V) if state_layout == "K_FIRST" else (V, K)))
    codes = np.ascontiguousarray(c if state_layout == "K_FIRST" else np.swapaxes(c, -1, -2))
    nt = V // block_v
    scales = t[..., K * V:K * V + 4 * nt].copy().view(np.float32).reshape(lead + (nt,)).astype(np.float64)
    return codes, scales
