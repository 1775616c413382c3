"""SVDQuant W4A4 NVFP4 linear layer, restated step by step (oracle; test use only).

The layer is defined on the model card "nunchaku-z-image-turbo-svdq",
section "What's stored on disk", by its runtime reconstruction

    y = scaled_mma(quant(x * smooth), qweight, ascales, wscales) * wtscale * wcscales
        + (x @ proj_down) @ proj_up^T + bias

with the on-disk tensors of the same section's table: qweight [N, K/2] int8
(FP4 nibble pack, low nibble = even k), wscales [K/16, N] float8_e4m3fn,
wcscales [N] bf16, wtscale [1] bf16, smooth_factor [K] bf16, proj_down [K, R]
and proj_up [N, R] bf16 (the rank-R SVD residual). The header of the card
fixes the element format: E2M1 values with one fp8_e4m3fn scale per 16
consecutive K elements.

What the pages leave open is read as follows (each reading is listed in the
design notes):

* "x * smooth" multiplies (not divides), per K channel, in fp32; a bf16 x bf16
  product is exact there (and in float64).
* The activation scale of a 16-block is the block's absolute maximum divided
  by 6 (the largest E2M1 magnitude), rounded to e4m3 (RNE, saturating at 448).
  There is no tensor-level activation scale.
* Codes are round-to-nearest-even of |v| / scale on the E2M1 grid, saturating
  at 6; the sign bit is the sign bit of v (so -tiny gives code 8). A block
  whose scale rounds to zero gets magnitude 0 everywhere.
* ascales is laid out [K/16, M] (mirroring wscales) and the activation codes
  [M, K/2] with the low nibble holding the even k (mirroring qweight).
* The residual branch takes the raw, unsmoothed x.
* bias is bf16 [N] and optional; the output is bf16 (RNE) of the float64 sum.

All arithmetic here is float64 / int64 on exact inputs: the main term is the
exact dot product of exactly dequantised operands (every E2M1 x e4m3 product
and every partial sum is representable), only the final bf16 cast rounds.
"""

import numpy as np

from . import formats as F

BLOCK = 16  # NVFP4 block length along K (model card header: per-16-K scales)


# ---------------------------------------------------------------------------
# Activation quantisation: quant(x * smooth) -> (codes packed, ascales)
# ---------------------------------------------------------------------------


def _quantize_blocks(v):
    """Quantise rows of float64 values v [rows, K] per 16-block along K.

    Returns (codes [rows, K] uint8 in 0..15, scale bytes [rows, K/16] uint8).
    Steps per block: amax = max |v|; s = amax / 6; sc = e4m3 RNE (saturating)
    of s; s_d = decode(sc); magnitude code = E2M1 RNE of |v| / s_d (0 when
    s_d == 0); sign bit from v.
    """
    rows, K = v.shape
    assert K % BLOCK == 0
    vb = v.reshape(rows, K // BLOCK, BLOCK)
    amax = np.abs(vb).max(axis=2)
    s = amax / 6.0
    sc = F.e4m3_encode(s)
    s_d = F.e4m3_decode(sc)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.abs(vb) / s_d[:, :, None]
    t = np.where(s_d[:, :, None] > 0, t, 0.0)
    mag = F.e2m1_encode_mag(t)
    sign = np.where(np.signbit(vb), 8, 0).astype(np.uint8)
    codes = (mag | sign).reshape(rows, K)
    return codes, sc


def quantize_act(x_bits, smooth_bits):
    """quant(x * smooth) for bf16 x [M, K] and bf16 smooth [K] (uint16 bit patterns).

    Returns qact [M, K/2] uint8 (low nibble = even k) and ascales [K/16, M]
    uint8 (e4m3fn bytes).
    """
    x = F.bf16_to_f64(x_bits)
    sm = F.bf16_to_f64(smooth_bits)
    v = x * sm[None, :]  # exact: 8-bit x 8-bit significands
    codes, sc = _quantize_blocks(v)
    return F.pack_nibbles(codes), np.ascontiguousarray(sc.T)


def quantize_weight(W, wcscales_bits, wtscale_bits):
    """Produce the on-disk NVFP4 weight tensors from a float weight W [N, K].

    Input preparation, not part of the layer (the pages do not say how the
    checkpoint was made): W'[n, k] = W[n, k] / (wtscale * wcscales[n]) is
    quantised with the activation rule above (no smooth), in float64.
    Returns qweight [N, K/2] uint8 and wscales [K/16, N] uint8.
    """
    W = np.asarray(W, dtype=np.float64)
    alpha = F.bf16_to_f64(wtscale_bits).reshape(()) * F.bf16_to_f64(wcscales_bits)
    codes, sc = _quantize_blocks(W / alpha[:, None])
    return F.pack_nibbles(codes), np.ascontiguousarray(sc.T)


# ---------------------------------------------------------------------------
# Dequantisation and the main scaled GEMM
# ---------------------------------------------------------------------------


def dequant(packed, scales):
    """packed codes [R, K/2] + scales [K/16, R] -> exact float64 values [R, K]."""
    vals = F.e2m1_decode(F.unpack_nibbles(packed))
    s = F.e4m3_decode(scales).T  # [R, K/16]
    return vals * np.repeat(s, BLOCK, axis=1)


def main_term(qact, ascales, qweight, wscales):
    """scaled_mma: sum over k of dequant(A)[m, k] * dequant(W)[n, k], float64.

    Exact: every dequantised value is a 2-bit significand times a 4-bit one,
    and the sums stay far inside float64's 53 bits for the shapes used.
    """
    return dequant(qact, ascales) @ dequant(qweight, wscales).T


def main_term_int64(qact, ascales, qweight, wscales):
    """The same contraction in exact integer arithmetic, scaled by 2**-20.

    With a' = 2 * E2M1 (integers in [-12, 12]) and s' = 2**9 * e4m3 (integers:
    every e4m3fn value is a multiple of 2**-9),
        main = 2**-20 * sum_b s'_a[b, m] * s'_w[b, n] * sum_{k in b} a'[m, k] * w'[n, k].
    Returns the int64 numerator (exact) so callers can compare bit for bit.
    """
    a = (2 * F.e2m1_decode(F.unpack_nibbles(qact))).astype(np.int64)
    w = (2 * F.e2m1_decode(F.unpack_nibbles(qweight))).astype(np.int64)
    sa = (F.e4m3_decode(ascales) * 512).astype(np.int64)  # [K/16, M]
    sw = (F.e4m3_decode(wscales) * 512).astype(np.int64)  # [K/16, N]
    M, K = a.shape
    N = w.shape[0]
    total = np.zeros((M, N), dtype=np.int64)
    for b in range(K // BLOCK):
        ks = slice(b * BLOCK, (b + 1) * BLOCK)
        partial = a[:, ks] @ w[:, ks].T  # |.| <= 16 * 144
        total += sa[b][:, None] * sw[b][None, :] * partial
    return total


# ---------------------------------------------------------------------------
# Residual, epilogue, whole layer
# ---------------------------------------------------------------------------


def lowrank_down(x_bits, proj_down_bits):
    """x @ proj_down in float64 (raw x, no rounding): [M, R]."""
    return F.bf16_to_f64(x_bits) @ F.bf16_to_f64(proj_down_bits)


def lowrank(x_bits, proj_down_bits, proj_up_bits):
    """(x @ proj_down) @ proj_up^T in float64: [M, N]."""
    return lowrank_down(x_bits, proj_down_bits) @ F.bf16_to_f64(proj_up_bits).T


def epilogue(main, wcscales_bits, wtscale_bits, lr, bias_bits):
    """main * wtscale * wcscales[n] + lr + bias[n], float64."""
    wt = F.bf16_to_f64(wtscale_bits).reshape(())
    wc = F.bf16_to_f64(wcscales_bits)
    y = main * wt * wc[None, :]
    if lr is not None:
        y = y + lr
    if bias_bits is not None:
        y = y + F.bf16_to_f64(bias_bits)[None, :]
    return y


def gemm_w4a4(qact, ascales, lora_act, qweight, wscales, wcscales_bits, wtscale_bits,
              proj_up_bits, bias_bits):
    """Layer from pre-quantised activations and a given down-projection result
    lora_act [M, R] (float64 values; None when R == 0). Returns float64 y."""
    main = main_term(qact, ascales, qweight, wscales)
    lr = None
    if lora_act is not None and proj_up_bits is not None and np.size(proj_up_bits) > 0:
        lr = np.asarray(lora_act, dtype=np.float64) @ F.bf16_to_f64(proj_up_bits).T
    return epilogue(main, wcscales_bits, wtscale_bits, lr, bias_bits)


def linear_w4a4(x_bits, smooth_bits, qweight, wscales, wcscales_bits, wtscale_bits,
                proj_down_bits, proj_up_bits, bias_bits):
    """The whole layer. Returns (y64 float64 [M, N], y bf16 bits, qact, ascales)."""
    qact, ascales = quantize_act(x_bits, smooth_bits)
    main = main_term(qact, ascales, qweight, wscales)
    R = 0 if proj_down_bits is None else np.shape(proj_down_bits)[1]
    lr = lowrank(x_bits, proj_down_bits, proj_up_bits) if R > 0 else None
    y64 = epilogue(main, wcscales_bits, wtscale_bits, lr, bias_bits)
    return y64, F.f64_to_bf16(y64), qact, ascales


# ---------------------------------------------------------------------------
# Static (calibrated) activation scale
# ---------------------------------------------------------------------------
#
# The blog page's section on the Comfy-Org Z-Image Turbo NVFP4 checkpoint says it
# uses calibrated static activation scales; the pages give no rule. Reading
# (NVFP4's two-level form): a per-tensor global scale g is fixed offline from
# calibration activations, g = bf16(max |x * smooth| / (6 * 448)) (1 when that
# maximum is 0), and the per-16 e4m3 block scales are still computed per call,
# relative to g:
#     s = e4m3(amax / (6 g)) (nearest even, saturating at 448),
#     codes = E2M1 nearest even of |v| / (dec(s) * g) (saturating at 6, sign kept).
# The layer's main term then carries a factor g: A_eff = E2M1 * dec(s) * g, so
# y = main * g * wtscale * wcscales + lowrank + bias. With g = 1 this is the
# dynamic rule above. g is a bf16 value (8 significant bits).


def _quantize_blocks_static(v, g):
    """Per 16-block of float64 rows v [rows, K] with the global scale g (float64):
    (codes [rows, K] 0..15, scale bytes [rows, K/16])."""
    rows, K = v.shape
    assert K % BLOCK == 0 and g > 0
    vb = v.reshape(rows, K // BLOCK, BLOCK)
    amax = np.abs(vb).max(axis=2)
    sc = F.e4m3_encode(amax / (6.0 * g))
    d = F.e4m3_decode(sc) * g              # exact: a 4-bit times an 8-bit significand
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.abs(vb) / d[:, :, None]
    t = np.where(d[:, :, None] > 0, t, 0.0)
    mag = F.e2m1_encode_mag(t)
    sign = np.where(np.signbit(vb), 8, 0).astype(np.uint8)
    return (mag | sign).reshape(rows, K), sc


def calibrate_gscale(x_bits, smooth_bits):
    """The static global activation scale from calibration activations x [M, K] (bf16
    bits): bf16(max |x * smooth| / (6 * 448)), or bf16(1) when the maximum is 0.
    Returns a uint16 array of shape (1,)."""
    v = F.bf16_to_f64(x_bits) * F.bf16_to_f64(smooth_bits)[None, :]
    amax = float(np.abs(v).max()) if v.size else 0.0
    g = amax / 2688.0 if amax > 0 else 1.0
    return F.f64_to_bf16(np.array([g]))


def quantize_act_static(x_bits, smooth_bits, gscale_bits):
    """quant(x * smooth) relative to the static global scale g (bf16 bits, shape (1,)):
    qact [M, K/2] uint8 (low nibble = even k), ascales [K/16, M] uint8."""
    g = float(F.bf16_to_f64(gscale_bits).reshape(-1)[0])
    v = F.bf16_to_f64(x_bits) * F.bf16_to_f64(smooth_bits)[None, :]
    codes, sc = _quantize_blocks_static(v, g)
    return F.pack_nibbles(codes), np.ascontiguousarray(sc.T)


def linear_w4a4_static(x_bits, smooth_bits, gscale_bits, qweight, wscales, wcscales_bits, wtscale_bits,
                       proj_down_bits, proj_up_bits, bias_bits):
    """The layer with static activation scales. Returns (y64, y bf16 bits, qact, ascales)."""
    g = float(F.bf16_to_f64(gscale_bits).reshape(-1)[0])
    qact, ascales = quantize_act_static(x_bits, smooth_bits, gscale_bits)
    main = main_term(qact, ascales, qweight, wscales) * g
    R = 0 if proj_down_bits is None else np.shape(proj_down_bits)[1]
    lr = lowrank(x_bits, proj_down_bits, proj_up_bits) if R > 0 else None
    y64 = epilogue(main, wcscales_bits, wtscale_bits, lr, bias_bits)
    return y64, F.f64_to_bf16(y64), qact, ascales


# ---------------------------------------------------------------------------
# FFN neighbour: gated combination of the w1 / w3 outputs
# ---------------------------------------------------------------------------
#
# The blog page's layer table and its key insight name the DiT feed-forward
# layers w1, w2, w3 (quantised to NVFP4, unlike attention); the pages do not
# spell out how they combine. Reading: a gated FFN, w2(silu(w1 x) * (w3 x)),
# with w1 and w3 run as one SVDQuant layer of 2F output channels that share x,
# smooth, wtscale, proj_down and R (columns [0, F) = w1, [F, 2F) = w3).


def silu(z):
    """z * sigmoid(z) = z / (1 + exp(-z)), float64."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu(y64, F_out):
    """h = silu(y[:, :F]) * y[:, F:2F] in float64 from the 2F-wide layer output."""
    y64 = np.asarray(y64, dtype=np.float64)
    assert y64.shape[1] == 2 * F_out
    return silu(y64[:, :F_out]) * y64[:, F_out:]


def linear_w4a4_swiglu(x_bits, smooth_bits, qweight, wscales, wcscales_bits, wtscale_bits,
                       proj_down_bits, proj_up_bits, bias_bits):
    """The fused w1/w3 layer (2F output channels) followed by the gate:
    returns (h64 float64 [M, F], h bf16 bits). The layer output itself is not
    rounded to bf16 here (the fused path never materialises it)."""
    y64, _, _, _ = linear_w4a4(x_bits, smooth_bits, qweight, wscales, wcscales_bits, wtscale_bits,
                               proj_down_bits, proj_up_bits, bias_bits)
    F_out = y64.shape[1] // 2
    h64 = swiglu(y64, F_out)
    return h64, F.f64_to_bf16(h64)


# ---------------------------------------------------------------------------
# Layers kept in bf16
# ---------------------------------------------------------------------------
#
# The blog page's variant table keeps some linears of the DiT in bf16 (its
# "Ultra" variant: attention qkv/out everywhere, and every linear of blocks
# 0-4 and 25-29). Such a layer is the original model's linear,
# y = x @ W^T + bias, with bf16 x [M, K], W [N, K] (the layout of the bf16
# checkpoint's weight), bias [N]; the output is rounded to bf16 once.


def linear_bf16(x_bits, w_bits, bias_bits):
    """Plain bf16 linear: returns (y64 float64 [M, N], y bf16 bits).

    Every bf16 x bf16 product is exact in float64; only the sum over K
    (float64) and the final bf16 cast round."""
    x = F.bf16_to_f64(x_bits)
    w = F.bf16_to_f64(w_bits)
    y64 = x @ w.T
    if bias_bits is not None:
        y64 = y64 + F.bf16_to_f64(bias_bits)[None, :]
    return y64, F.f64_to_bf16(y64)


def normwise_rel_err(y, y_ref):
    """||y - y_ref||_F / ||y_ref||_F in float64 (the acceptance metric for y)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.linalg.norm(y_ref)
    return float(np.linalg.norm(y - y_ref) / den) if den > 0 else float(np.linalg.norm(y))
