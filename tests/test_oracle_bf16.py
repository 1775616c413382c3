"""Pins of the oracle's plain bf16 linear (the layers the blog page's variant
table keeps in bf16): exact rational brute force, permutation weights, integer
inputs, and agreement with the NVFP4 layer where both are lossless."""

from fractions import Fraction

import numpy as np

import workloads
from oracle import formats as F
from oracle import svdq as S


def _bf16_round(q):
    """Nearest bf16 value of the rational q (ties to even), as a Fraction;
    normal range only (8 significant bits)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    n = a * 128            # in [128, 256)
    f = n.numerator // n.denominator
    rem = n - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return sign * Fraction(f, 128) * Fraction(2) ** e


def _near_bf16_midpoint(q, tol):
    """True if q lies within tol of a rounding boundary between bf16 values."""
    return _bf16_round(q - tol) != _bf16_round(q + tol)


def test_rational_brute_force():
    d = workloads.make_bf16_linear(6, 48, 9, kind="dit", seed=77)
    y64, yb = S.linear_bf16(d["x"], d["W"], d["bias"])
    x = F.bf16_to_f64(d["x"])
    w = F.bf16_to_f64(d["W"])
    b = F.bf16_to_f64(d["bias"])
    K = 48
    checked = 0
    for m in range(6):
        for n in range(9):
            terms = [Fraction(float(x[m, k])) * Fraction(float(w[n, k])) for k in range(K)]
            exact = sum(terms) + Fraction(float(b[n]))
            bound = (sum(abs(t) for t in terms) + abs(Fraction(float(b[n])))) * Fraction(K + 2, 2 ** 52)
            assert abs(Fraction(float(y64[m, n])) - exact) <= bound
            if not _near_bf16_midpoint(exact, bound):
                assert Fraction(float(F.bf16_to_f64(yb[m, n]))) == _bf16_round(exact)
                checked += 1
    assert checked >= 50


def test_permutation_weight_selects_input_columns():
    """W[n, perm[n]] = 1: y[:, n] is x[:, perm[n]] exactly (catches a transposed W)."""
    rng = np.random.default_rng(5)
    K = 32
    x = workloads.f32_to_bf16_bits(rng.standard_normal((7, K)).astype(np.float32))
    perm = rng.permutation(K)
    W = np.zeros((K, K), np.float32)
    W[np.arange(K), perm] = 1.0
    _, yb = S.linear_bf16(x, workloads.f32_to_bf16_bits(W), None)
    assert np.array_equal(yb, x[:, perm])
    # with a bias: one rounding of x[m, perm[n]] + bias[n]
    bias = workloads.f32_to_bf16_bits(rng.standard_normal(K).astype(np.float32))
    _, yb = S.linear_bf16(x, workloads.f32_to_bf16_bits(W), bias)
    xv, bv = F.bf16_to_f64(x), F.bf16_to_f64(bias)
    for m in range(7):
        for n in range(K):
            q = Fraction(float(xv[m, perm[n]])) + Fraction(float(bv[n]))
            assert Fraction(float(F.bf16_to_f64(yb[m, n]))) == _bf16_round(q)


def test_integer_inputs_are_exact():
    rng = np.random.default_rng(9)
    M, K, N = 5, 64, 6
    xi = rng.integers(-2, 3, size=(M, K))
    wi = rng.integers(-2, 3, size=(N, K))
    _, yb = S.linear_bf16(workloads.f32_to_bf16_bits(xi.astype(np.float32)),
                          workloads.f32_to_bf16_bits(wi.astype(np.float32)), None)
    got = F.bf16_to_f64(yb)
    for m in range(M):
        for n in range(N):
            ref = sum(int(xi[m, k]) * int(wi[n, k]) for k in range(K))   # |ref| <= 256: exact in bf16
            assert got[m, n] == ref


def test_agrees_with_lossless_nvfp4_layer():
    """With R = 0, smooth = 1, wtscale = wcscales = 1 and an NVFP4-representable x,
    the NVFP4 layer is the plain linear on the dequantised weight (E2M1 x e4m3
    products have at most 6 significant bits, so that weight is exact in bf16)."""
    d = workloads.make_linear(32, 64, 24, 0, kind="tiny", seed=31)
    ones_k = workloads.f32_to_bf16_bits(np.ones(64))
    ones_n = workloads.f32_to_bf16_bits(np.ones(24))
    one = workloads.f32_to_bf16_bits(np.ones(1))
    qw, ws = S.quantize_weight(d["W"], ones_n, one)
    w_deq = S.dequant(qw, ws)
    w_bits = workloads.f32_to_bf16_bits(w_deq)
    assert np.array_equal(F.bf16_to_f64(w_bits), w_deq)
    # x: codes on the E2M1 grid times a power of two per block -> lossless quant
    rng = np.random.default_rng(3)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    xv = rng.choice(grid, size=(32, 64)) * rng.choice([-1, 1], size=(32, 64))
    xv[:, ::16] = 6.0
    xv = xv * np.repeat(2.0 ** rng.integers(-3, 3, size=(32, 4)), 16, axis=1)
    x_bits = workloads.f32_to_bf16_bits(xv)
    y64_q, _, _, _ = S.linear_w4a4(x_bits, ones_k, qw, ws, ones_n, one, None, None, d["bias"])
    y64_b, _ = S.linear_bf16(x_bits, w_bits, d["bias"])
    assert np.allclose(y64_q, y64_b, rtol=0, atol=1e-12)
