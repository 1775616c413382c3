"""Number formats of the NVFP4 path, restated in plain NumPy (oracle; test use only).

Sources on the pages:

* E2M1: blog "Z-Image NVFP4 efficient inference: 4-bit quantisation on
  Blackwell GPUs", section "NVFP4 technical background / what is NVFP4": one
  sign bit, two exponent bits, one mantissa bit. The value grid
  {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6} is the only grid such a 1+2+1
  layout yields with exponent bias 1 and a subnormal at exponent 0.
* float8_e4m3fn block scales: model card "nunchaku-z-image-turbo-svdq", header
  (E2M1 + per-16-K fp8_e4m3fn scales) and the tensor table of section
  "What's stored on disk" (wscales dtype); the SD.Next / SDNQ guide, section
  "quantisation type library", gives its range as about +-448.
* bf16: the pipeline dtype (model card, section "Usage", torch_dtype).

Readings where the pages are silent (each listed in the design notes):
rounding is round-to-nearest, ties-to-even (even code / even mantissa) for
both E2M1 and e4m3; encoders saturate (E2M1 at 6, e4m3 at 448) instead of
producing NaN; the sign bit of an E2M1 code is the sign bit of the input,
also when the magnitude rounds to zero.

bf16 values are carried as their uint16 bit patterns (NumPy has no bf16).
"""

import numpy as np

# ---------------------------------------------------------------------------
# bf16 <-> float64
# ---------------------------------------------------------------------------


def bf16_to_f64(bits):
    """uint16 bf16 bit patterns -> float64 (exact: bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(v):
    """float64 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Rounds directly from float64 (no intermediate float32 rounding). A finite
    value with |v| in [2**(e-1), 2**e) has bf16 quantum 2**(e-8) (8 significant
    bits), never finer than the subnormal quantum 2**-133. Scaling by that
    power of two is exact, np.rint rounds half to even, and the rounded value
    is exactly representable in float32 and in bf16.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.float64)
    finite = np.isfinite(v) & (v != 0)
    _, e = np.frexp(np.where(finite, v, 1.0))
    q = np.maximum(e.astype(np.int64) - 8, -133)
    scaled = np.ldexp(np.where(finite, v, 0.0), -q)
    out[...] = np.where(finite, np.ldexp(np.rint(scaled), q), v)
    # values beyond the largest finite bf16 overflow to inf (never reached by
    # this path's data, kept for completeness)
    big = np.abs(out) > 3.3895313892515355e38
    out = np.where(big & finite, np.copysign(np.inf, out), out)
    f32 = out.astype(np.float32)
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def f32_to_bf16(v):
    """float32 values -> bf16 bits (RNE), via the exact float64 route."""
    return f64_to_bf16(np.asarray(v, dtype=np.float32).astype(np.float64))


# ---------------------------------------------------------------------------
# E2M1 (FP4)
# ---------------------------------------------------------------------------

# Magnitude code m = c & 7 -> value. Exponent bits e = m >> 1, mantissa bit
# f = m & 1: e == 0 is subnormal (f * 0.5), otherwise 2**(e-1) * (1 + f/2).
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes):
    """4-bit codes (uint8 in 0..15) -> float64. Bit 3 is the sign."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_GRID[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def _nearest_on_grid_even(t, grid):
    """Index of the grid value nearest to t (t >= 0, grid ascending).

    Ties go to the even index; values above the last grid point saturate to
    the last index. Index parity is code parity for both formats used here
    (the code's least significant bit is the mantissa's least significant bit).
    """
    t = np.minimum(np.asarray(t, dtype=np.float64), grid[-1])
    hi = np.searchsorted(grid, t, side="left")          # grid[hi-1] < t <= grid[hi]
    hi = np.clip(hi, 0, len(grid) - 1)
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    dlo = t - grid[lo]
    dhi = grid[hi] - t
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo).astype(np.uint8)


def e2m1_encode_mag(t):
    """Magnitude t >= 0 -> magnitude code 0..7, RNE, saturating at 6."""
    return _nearest_on_grid_even(t, E2M1_GRID)


# ---------------------------------------------------------------------------
# float8_e4m3fn
# ---------------------------------------------------------------------------


def e4m3_decode(b):
    """e4m3fn bytes -> float64. Bias 7, subnormals at e == 0, no infinities,
    NaN only for S.1111.111 (0x7F, 0xFF). Largest finite value 448 (0x7E)."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    f = b & 7
    mag = np.where(e == 0, f * 2.0 ** -9, np.ldexp(1.0 + f / 8.0, e - 7))
    mag = np.where((e == 15) & (f == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


# Finite non-negative e4m3fn values in code order 0x00..0x7E (ascending).
E4M3_POS_GRID = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(s):
    """s >= 0 -> e4m3fn byte in 0x00..0x7E: RNE on the e4m3 grid, saturating
    at 448 (never NaN, sign bit always clear)."""
    return _nearest_on_grid_even(s, E4M3_POS_GRID)


# ---------------------------------------------------------------------------
# Nibble packing: low nibble = even k (model card, tensor table: qweight is an
# int8 FP4 nibble pack with the low nibble holding the even-k element).
# ---------------------------------------------------------------------------


def pack_nibbles(codes):
    """codes [..., K] (uint8 0..15) -> bytes [..., K/2]; byte j = c[2j] | c[2j+1] << 4."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """bytes [..., K/2] -> codes [..., K]; inverse of pack_nibbles."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out
