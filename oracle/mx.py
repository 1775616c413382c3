"""MXFP4 datatype variant of the layer (oracle; test use only).

The pages define the layer with NVFP4: E2M1 values and one e4m3 scale per 16
K elements (model card "nunchaku-z-image-turbo-svdq", header and section
"What's stored on disk"). gfx950's block-scaled matrix instructions take the
OCP microscaling form instead: E2M1 values with one E8M0 (power-of-two) scale
per 32 K elements. This variant re-rounds both operands into that form, giving
up the pages' exact arithmetic for the faster instructions; it is measured as
a separate, out-of-tolerance speed point.

MX quantisation of a 32-block of real values v (OCP MX rule for E2M1, whose
largest exponent is 2): X = floor(log2(max |v|)) - 2, clamped to [-127, 127],
stored as the byte X + 127; codes = E2M1 nearest-even of |v| / 2^X, saturating
at 6, with the sign bit of v. An all-zero block gets X = -127 (byte 0) and
zero magnitudes.

Variant layer (same epilogue, low-rank branch and bias as the NVFP4 layer):
  a = MX(x * smooth) per token row, w = MX(dequant_NVFP4(qweight, wscales)) per
  output row (re-rounded from the exact NVFP4 values),
  y = bf16( (sum_k a w) * wtscale * wcscales[n] + (x @ proj_down) @ proj_up^T + bias ).
"""

import numpy as np

from . import formats as F
from . import svdq as S

MX_BLOCK = 32


def mx_quantize(v):
    """Rows of float64 values v [rows, K] (K % 32 == 0) -> (codes [rows, K] uint8,
    scale bytes [rows, K/32] uint8)."""
    v = np.asarray(v, dtype=np.float64)
    rows, K = v.shape
    assert K % MX_BLOCK == 0
    vb = v.reshape(rows, K // MX_BLOCK, MX_BLOCK)
    amax = np.abs(vb).max(axis=2)
    nz = amax > 0
    _, e = np.frexp(np.where(nz, amax, 1.0))      # amax = m * 2^e, m in [0.5, 1): floor(log2) = e - 1
    X = np.where(nz, e.astype(np.int64) - 1 - 2, -127)
    X = np.clip(X, -127, 127)
    t = np.abs(vb) / np.ldexp(1.0, X)[:, :, None]
    mag = F.e2m1_encode_mag(t)
    sign = np.where(np.signbit(vb), 8, 0).astype(np.uint8)
    codes = (mag | sign).reshape(rows, K)
    return codes, (X + 127).astype(np.uint8)


def mx_dequant(codes, scales):
    """codes [rows, K] + scale bytes [rows, K/32] -> float64 values."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, K = codes.shape
    vals = F.e2m1_decode(codes).reshape(rows, K // MX_BLOCK, MX_BLOCK)
    X = np.asarray(scales, dtype=np.int64) - 127
    return (vals * np.ldexp(1.0, X)[:, :, None]).reshape(rows, K)


def quantize_act_mx(x_bits, smooth_bits):
    """a = MX(x * smooth): codes [M, K], scale bytes [M, K/32]."""
    v = F.bf16_to_f64(x_bits) * F.bf16_to_f64(smooth_bits)[None, :]
    return mx_quantize(v)


def reround_weight_mx(qweight, wscales):
    """w = MX(exact NVFP4 values): codes [N, K], scale bytes [N, K/32]."""
    return mx_quantize(S.dequant(qweight, wscales))


def linear_mxfp4(x_bits, smooth_bits, qweight, wscales, wcscales_bits, wtscale_bits,
                 proj_down_bits, proj_up_bits, bias_bits):
    """The variant layer. Returns (y64, y bf16 bits, act codes, act scales, w codes, w scales)."""
    ac, asc = quantize_act_mx(x_bits, smooth_bits)
    wc, wsc = reround_weight_mx(qweight, wscales)
    main = mx_dequant(ac, asc) @ mx_dequant(wc, wsc).T
    R = 0 if proj_down_bits is None else np.shape(proj_down_bits)[1]
    lr = S.lowrank(x_bits, proj_down_bits, proj_up_bits) if R > 0 else None
    y64 = S.epilogue(main, wcscales_bits, wtscale_bits, lr, bias_bits)
    return y64, F.f64_to_bf16(y64), ac, asc, wc, wsc
