"""Pins of the MXFP4 variant's oracle (oracle/mx.py): the OCP MX scale rule on
powers of two and by exact-rational brute force, nearest-even codes with
saturation, idempotence on MX-representable blocks, exact dequantisation, and the
variant layer on lossless inputs."""

from fractions import Fraction

import numpy as np

import workloads
from oracle import formats as F
from oracle import mx as X
from oracle import svdq as S

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def brute_block(vals):
    """Exact rational MX quantisation of one 32-block (list of floats)."""
    fr = [Fraction(v) for v in vals]
    amax = max(abs(f) for f in fr)
    if amax == 0:
        return [8 if np.signbit(v) else 0 for v in vals], 0
    e = 0   # floor(log2 amax)
    while Fraction(2) ** (e + 1) <= amax:
        e += 1
    while Fraction(2) ** e > amax:
        e -= 1
    Xe = max(-127, min(127, e - 2))
    s = Fraction(2) ** Xe
    codes = []
    for v, f in zip(vals, fr):
        t = abs(f) / s
        best = None
        for c, g in enumerate(GRID):
            d = abs(t - g)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        c = 7 if t >= 6 else best[1]
        codes.append(c | (8 if np.signbit(v) else 0))
    return codes, Xe + 127


def test_scale_rule_on_powers_of_two():
    for e in range(-20, 21):
        v = np.zeros((1, 32))
        v[0, 5] = 2.0 ** e
        v[0, 9] = -(2.0 ** (e - 3))
        codes, sc = X.mx_quantize(v)
        assert sc[0, 0] == e - 2 + 127
        assert codes[0, 5] == 6                     # 2^e / 2^(e-2) = 4 -> code 6
        assert codes[0, 9] == 8 | 1                 # 0.5 -> code 1, negative


def test_brute_force_random_blocks():
    rng = np.random.default_rng(0)
    for trial in range(40):
        scale = 2.0 ** rng.integers(-30, 30)
        v = rng.standard_normal((1, 32)) * scale
        if trial % 5 == 0:
            v[0, rng.integers(0, 32)] *= 50.0            # outlier inside the block
        v = F.bf16_to_f64(F.f64_to_bf16(v))
        codes, sc = X.mx_quantize(v)
        bc, bs = brute_block(list(v[0]))
        assert sc[0, 0] == bs
        assert list(codes[0]) == bc


def test_exact_ties_and_saturation():
    # block scale 2^0 (amax in [4, 8)): ties at 5 -> code 6 (4, even), 7 -> saturates at 6,
    # 2.5 -> code 4 (2, even), 0.25 -> code 0 (even)
    v = np.zeros((1, 32))
    v[0, :6] = [5.0, 7.0, 2.5, 0.25, 1.25, 7.99]
    codes, sc = X.mx_quantize(v)
    assert sc[0, 0] == 127
    assert list(codes[0, :6]) == [6, 7, 4, 0, 2, 7]


def test_zero_block_and_signed_zero():
    v = np.zeros((1, 32))
    v[0, 3] = -0.0
    codes, sc = X.mx_quantize(v)
    assert sc[0, 0] == 0 and codes[0, 3] == 8 and codes[0, :3].sum() == 0


def test_idempotent_on_representable_blocks():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 16, (4, 64)).astype(np.uint8)
    codes[:, 0] = 7
    codes[:, 32] = 7          # a +6 in every block fixes its scale
    scales = rng.integers(100, 150, (4, 2)).astype(np.uint8)
    v = X.mx_dequant(codes, scales)
    c2, s2 = X.mx_quantize(v)
    assert np.array_equal(s2, scales)
    assert np.array_equal(X.mx_dequant(c2, s2), v)


def test_variant_layer_is_exact_on_lossless_inputs():
    """x * smooth and the NVFP4 weight both MX-representable: the variant's main term
    equals the NVFP4 layer's exactly."""
    rng = np.random.default_rng(2)
    M, K, N = 16, 64, 24
    ca = rng.integers(0, 16, (M, K)).astype(np.uint8)
    ca[:, ::16] = 7           # a 6 in every 16-block: lossless for NVFP4 as well
    sa = rng.integers(120, 130, (M, K // 32)).astype(np.uint8)
    x = X.mx_dequant(ca, sa)
    x_bits = workloads.f32_to_bf16_bits(x)
    assert np.array_equal(F.bf16_to_f64(x_bits), x)
    ones = workloads.f32_to_bf16_bits(np.ones(K))
    # weight: NVFP4 with power-of-two block scales equal within each 32-block
    cw = rng.integers(0, 16, (N, K)).astype(np.uint8)
    cw[:, ::16] = 7
    e = rng.integers(-4, 3, (N, K // 32))
    sc = np.repeat(e, 2, axis=1)
    ws = F.e4m3_encode(np.ldexp(1.0, sc)).T.copy()       # [K/16, N]
    qw = F.pack_nibbles(cw)
    one = workloads.f32_to_bf16_bits(np.ones(1))
    wc = workloads.f32_to_bf16_bits(np.ones(N))
    y_mx = X.linear_mxfp4(x_bits, ones, qw, ws, wc, one, None, None, None)[0]
    y_nv = S.linear_w4a4(x_bits, ones, qw, ws, wc, one, None, None, None)[0]
    assert np.array_equal(y_mx, y_nv)
    assert np.allclose(y_nv, x @ S.dequant(qw, ws).T, rtol=0, atol=0)


def test_quantize_act_mx_applies_smooth():
    """quantize_act_mx(x, smooth) = MX(x * smooth), checked by the rational brute force on
    each 32-block with per-channel power-of-two smooth factors (exact products), so a dropped
    or misplaced smooth changes the scales or the codes."""
    rng = np.random.default_rng(3)
    M, K = 6, 96
    x = F.bf16_to_f64(F.f64_to_bf16(rng.standard_normal((M, K))))
    sm = np.ldexp(1.0, rng.integers(-3, 4, K))
    sm[::7] = 8.0
    x_bits, sm_bits = F.f64_to_bf16(x), F.f64_to_bf16(sm)
    codes, scales = X.quantize_act_mx(x_bits, sm_bits)
    v = x * sm
    for m in range(M):
        for b in range(K // 32):
            bc, bs = brute_block(list(v[m, 32 * b: 32 * b + 32]))
            assert scales[m, b] == bs
            assert list(codes[m, 32 * b: 32 * b + 32]) == bc
    c_plain, _ = X.quantize_act_mx(x_bits, F.f64_to_bf16(np.ones(K)))
    assert not np.array_equal(c_plain, codes)


def test_reround_weight_mx_identity_on_representable_weight():
    """An NVFP4 weight whose 16-block scales are equal powers of two within each 32-block and
    whose blocks hold a 6 is MX-representable: re-rounding keeps every value, and the MX
    scale byte is the block's power of two (2^e * 6 has floor log2 = e + 2, minus 2)."""
    rng = np.random.default_rng(4)
    N, K = 10, 128
    cw = rng.integers(0, 16, (N, K)).astype(np.uint8)
    cw[:, ::32] = 7
    e = rng.integers(-5, 4, (N, K // 32))
    ws = F.e4m3_encode(np.ldexp(1.0, np.repeat(e, 2, axis=1))).T.copy()
    qw = F.pack_nibbles(cw)
    codes, scales = X.reround_weight_mx(qw, ws)
    assert np.array_equal(X.mx_dequant(codes, scales), S.dequant(qw, ws))
    assert np.array_equal(scales.astype(np.int64) - 127, e)
