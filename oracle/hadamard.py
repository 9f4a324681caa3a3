"""The int8_hadamard32 state codec: value-basis Hadamard rotation + int8 per (key channel, 32 values).

Pages followed:
* modelopt ... linear_attention.config, LinearAttentionConfig: with the
  int8_hadamard32 codec a scale covers a single key row by a 32-value group
  (not a [Dk, block_v] tile), while ``state.block_v`` keeps its role as the
  execution tile width.  LinearAttentionDecodeConfig: ``state_codec`` is
  'tile' or 'int8_hadamard32'.
* modelopt ... linear_attention.decode, LinearAttentionCarry: the carry has a
  ``value_basis`` and ``reconstruct`` returns the original value basis unless
  told otherwise -- the codec works in a rotated value basis and the state is
  handed back in the original one.

Readings (the pages give no formulas):
* the rotation is the 32-point Walsh-Hadamard transform in Sylvester order,
  normalised to be orthonormal (H / sqrt(32), H the +-1 matrix), applied to
  each group of 32 consecutive value columns of every key row:
  y = x H / sqrt(32); it is its own inverse;
* int8 is symmetric: scale s = amax(|y| over the 32 values) / 127, code =
  round-to-nearest-even(y / s) clamped to [-127, 127]; amax = 0 leaves the
  group unchanged;
* the state returned is (s * code) H / sqrt(32) (the original basis).

Written with z = x H the 1/sqrt(32) factors cancel: y / s = 127 z / amax|z|
and (s * code) H / sqrt(32) = (code H) * amax|z| / (127 * 32).  The code
below uses that form, so that values whose rotation is exactly on the code
grid (ties included) are decided exactly.  The pages do not fix the
precision of the decision; the default is float64 (the plain reading).
With ``precision='float32'`` every operation is rounded to float32 -- z by
radix-2 butterflies (a + b, a - b) over strides 1, 2, 4, 8, 16, inv =
f32(127 / amax|z|), code = rint(f32(z * inv)), result = f32(code H) *
f32(f32(amax|z| / 127) / 32) -- which serves to compare code decisions
taken in that precision.

Packed storage (this repository's format; the pages describe the codec as a
quantise/dequantise emulation and claim no compressed storage): a state is
kept as its codes and scales, int8 code[h, k, v] and scale[h, k, g] =
amax|z| / 127 of group g in the +-1 Hadamard basis z = x H, and stands for
(code H) * scale / 32 -- exactly what int8_hadamard32_qdq returns.
``int8_hadamard32_encode`` / ``int8_hadamard32_decode`` convert, and
``pack_tiles`` / ``unpack_tiles`` lay one (row, head) tile out as its K V
code bytes in [V / 32][K][32] order (each group's codes for all key rows
together) followed by its K V / 32 float32 scales in [V / 32][K] order.

Pins (tests/test_oracle_hadamard.py): H / sqrt(32) is orthonormal and
symmetric, the butterfly transform equals the matrix product, the folded
form equals the definition with explicit normalisation, code points
round-trip exactly, values on the half-code grid round to even exactly, the
error is within half a step per rotated coordinate, groups and key rows are
independent, and a single spike is spread over all 32 coordinates and
reconstructed exactly.
"""
import numpy as np

GROUP = 32
INT8_MAX = 127.0


def hadamard_matrix(n=GROUP):
    """Sylvester Hadamard matrix of order n (entries +-1): H_2n = [[H, H], [H, -H]]."""
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def fwht_butterflies(x, dtype=np.float64):
    """Unnormalised Walsh-Hadamard transform along the last axis (length 32) as radix-2 butterflies."""
    y = np.array(x, dtype=dtype, copy=True)
    n = y.shape[-1]
    h = 1
    while h < n:
        y = y.reshape(y.shape[:-1] + (n // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (n,))
        h *= 2
    return y


def int8_hadamard32_qdq(S, precision="float64"):
    """Quantise/dequantise S [H, K, V] with the int8_hadamard32 codec (V a multiple of 32)."""
    S = np.asarray(S, dtype=np.float64)
    Hh, K, V = S.shape
    if V % GROUP != 0:
        raise ValueError("the value head dim must be a multiple of 32")
    x = S.reshape(Hh, K, V // GROUP, GROUP)
    if precision == "float64":
        z = x @ hadamard_matrix()
        amax = np.max(np.abs(z), axis=-1, keepdims=True)
        safe = np.where(amax > 0, amax, 1.0)
        code = np.clip(np.rint(z * INT8_MAX / safe), -INT8_MAX, INT8_MAX)
        xq = (code @ hadamard_matrix()) * (safe / INT8_MAX / GROUP)
        out = np.where(amax > 0, xq, x)
        return out.reshape(Hh, K, V)
    if precision == "float32":
        f = np.float32
        z = fwht_butterflies(x.astype(f), dtype=f)
        amax = np.max(np.abs(z), axis=-1, keepdims=True)
        safe = np.where(amax > 0, amax, f(1.0)).astype(f)
        inv = (f(INT8_MAX) / safe).astype(f)
        c = ((safe / f(INT8_MAX)).astype(f) / f(GROUP)).astype(f)
        code = np.clip(np.rint((z * inv).astype(f)), -INT8_MAX, INT8_MAX).astype(f)
        xq = (fwht_butterflies(code, dtype=f) * c).astype(f)
        out = np.where(amax > 0, xq, x.astype(f))
        return out.reshape(Hh, K, V).astype(np.float64)
    raise ValueError(f"unknown precision {precision!r}")


def int8_hadamard32_encode(S, precision="float64"):
    """Codes (int8) and scales (float64) of S [H, K, V] under the codec; decode(encode(S)) == qdq(S).

    scale = amax|z| / 127 per (head, key row, group of 32) with z = S H (the +-1 matrix); an
    all-zero group has scale 0 and codes 0.  The codes are decided exactly as in
    int8_hadamard32_qdq at the same precision.
    """
    S = np.asarray(S, dtype=np.float64)
    Hh, K, V = S.shape
    if V % GROUP != 0:
        raise ValueError("the value head dim must be a multiple of 32")
    x = S.reshape(Hh, K, V // GROUP, GROUP)
    if precision == "float64":
        z = x @ hadamard_matrix()
        amax = np.max(np.abs(z), axis=-1, keepdims=True)
        safe = np.where(amax > 0, amax, 1.0)
        code = np.clip(np.rint(z * INT8_MAX / safe), -INT8_MAX, INT8_MAX)
        scale = amax / INT8_MAX
    elif precision == "float32":
        f = np.float32
        z = fwht_butterflies(x.astype(f), dtype=f)
        amax = np.max(np.abs(z), axis=-1, keepdims=True)
        safe = np.where(amax > 0, amax, f(1.0)).astype(f)
        inv = (f(INT8_MAX) / safe).astype(f)
        code = np.clip(np.rint((z * inv).astype(f)), -INT8_MAX, INT8_MAX)
        scale = (amax / f(INT8_MAX)).astype(f).astype(np.float64)
    else:
        raise ValueError(f"unknown precision {precision!r}")
    code = np.where(amax > 0, code, 0.0)
    return code.reshape(Hh, K, V).astype(np.int8), scale.reshape(Hh, K, V // GROUP)


def int8_hadamard32_decode(code, scale):
    """The state [H, K, V] that codes [H, K, V] and scales [H, K, V / 32] stand for: (code H) scale / 32."""
    code = np.asarray(code, dtype=np.float64)
    Hh, K, V = code.shape
    z = code.reshape(Hh, K, V // GROUP, GROUP)
    x = (z @ hadamard_matrix()) * (np.asarray(scale, dtype=np.float64)[..., None] / GROUP)
    return x.reshape(Hh, K, V)


def packed_tile_bytes(K, V):
    """Bytes of one packed (row, head) tile: K V codes, then K V / 32 float32 scales."""
    return K * V + 4 * K * (V // GROUP)


def pack_tiles(code, scale):
    """codes [..., K, V] int8 and scales [..., K, V / 32] -> bytes [..., packed_tile_bytes(K, V)] (uint8):
    the codes in [V / 32][K][32] order, then the scales in [V / 32][K] order."""
    code = np.asarray(code, dtype=np.int8)
    lead, (K, V) = code.shape[:-2], code.shape[-2:]
    G = V // GROUP
    cg = np.moveaxis(code.reshape(lead + (K, G, GROUP)), -2, -3)           # [..., G, K, 32]
    c = np.ascontiguousarray(cg).reshape(lead + (K * V,)).view(np.uint8)
    sg = np.moveaxis(np.asarray(scale, dtype=np.float32).reshape(lead + (K, G)), -1, -2)   # [..., G, K]
    s = np.ascontiguousarray(sg).reshape(lead + (K * G,))
    return np.concatenate([c, s.view(np.uint8).reshape(lead + (4 * K * G,))], axis=-1)


def unpack_tiles(tiles, K, V):
    """Inverse of pack_tiles: bytes [..., packed_tile_bytes(K, V)] -> (codes int8 [..., K, V], scales float64)."""
    t = np.ascontiguousarray(np.asarray(tiles, dtype=np.uint8))
    lead = t.shape[:-1]
    if t.shape[-1] != packed_tile_bytes(K, V):
        raise ValueError("tile size does not match K and V")
    G = V // GROUP
    cg = t[..., :K * V].copy().view(np.int8).reshape(lead + (G, K, GROUP))
    code = np.ascontiguousarray(np.moveaxis(cg, -3, -2)).reshape(lead + (K, V))
    sg = t[..., K * V:].copy().view(np.float32).reshape(lead + (G, K))
    scale = np.ascontiguousarray(np.moveaxis(sg, -1, -2)).astype(np.float64)
    return code, scale
