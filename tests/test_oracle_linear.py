"""Pins of the oracle's scaled GEMM, low-rank residual and whole-layer formula.

The model card "nunchaku-z-image-turbo-svdq" (section "What's stored on disk")
gives y = scaled_mma(quant(x*smooth), qweight, ascales, wscales) * wtscale *
wcscales + (x @ proj_down) @ proj_up^T + bias. Pins: the int64-exact form of
the main term, a pure-Python integer brute force on tiny shapes, and the
formula's closed-form special cases (R = 0: a plain quantised GEMM;
qweight = 0: a pure low-rank product; lossless inputs: an exact GEMM).
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads
from oracle import formats as F
from oracle import svdq as S


def _tiny(seed=None, **over):
    cfg = dict(workloads.TINY)
    if seed is not None:
        cfg["seed"] = seed
    cfg.update(over)
    d = workloads.make_linear(**cfg)
    d["qweight"], d["wscales"] = S.quantize_weight(d["W"], d["wcscales"], d["wtscale"])
    return d


def test_main_term_fp64_equals_int64_exact():
    d = _tiny()
    qact, ascales = S.quantize_act(d["x"], d["smooth"])
    main = S.main_term(qact, ascales, d["qweight"], d["wscales"])
    exact = S.main_term_int64(qact, ascales, d["qweight"], d["wscales"])
    assert np.abs(exact).max() < 2 ** 53
    assert np.array_equal(main, exact.astype(np.float64) * 2.0 ** -20)


def test_main_term_dit_int64_exact():
    d = workloads.make_linear(M=32, K=1024, N=64, R=0, kind="dit", seed=77)
    qw, ws = S.quantize_weight(d["W"], d["wcscales"], d["wtscale"])
    qact, ascales = S.quantize_act(d["x"], d["smooth"])
    main = S.main_term(qact, ascales, qw, ws)
    exact = S.main_term_int64(qact, ascales, qw, ws)
    assert np.array_equal(main, exact.astype(np.float64) * 2.0 ** -20)


def test_main_term_pure_python_brute_force():
    """Sum over k of (E2M1 * e4m3) products with Python Fractions, element by element."""
    d = _tiny()
    qact, ascales = S.quantize_act(d["x"], d["smooth"])
    main = S.main_term(qact, ascales, d["qweight"], d["wscales"])
    grid = [0, Fraction(1, 2), 1, Fraction(3, 2), 2, 3, 4, 6]

    def e2m1(c):
        return -grid[c & 7] if c & 8 else grid[c & 7]

    def e4m3(b):
        e, f = (b >> 3) & 15, b & 7
        return Fraction(f, 512) if e == 0 else (1 + Fraction(f, 8)) * Fraction(2) ** (e - 7)

    K = d["K"]
    for m, n in [(0, 0), (5, 17), (63, 127), (31, 64), (10, 99)]:
        acc = Fraction(0)
        for k in range(K):
            ab = int(qact[m, k // 2])
            wb = int(d["qweight"][n, k // 2])
            a = e2m1(ab & 15 if k % 2 == 0 else ab >> 4) * e4m3(int(ascales[k // 16, m]))
            w = e2m1(wb & 15 if k % 2 == 0 else wb >> 4) * e4m3(int(d["wscales"][k // 16, n]))
            acc += a * w
        assert Fraction(main[m, n]) == acc


def test_r0_is_plain_quantised_gemm():
    d = _tiny(R=0)
    y64, y, qact, ascales = S.linear_w4a4(d["x"], d["smooth"], d["qweight"], d["wscales"],
                                          d["wcscales"], d["wtscale"], d["proj_down"],
                                          d["proj_up"], d["bias"])
    A = S.dequant(qact, ascales)
    W = S.dequant(d["qweight"], d["wscales"])
    alpha = F.bf16_to_f64(d["wtscale"])[0] * F.bf16_to_f64(d["wcscales"])
    ref = torch.from_numpy(A) @ torch.from_numpy(W).T * torch.from_numpy(alpha) + \
        torch.from_numpy(F.bf16_to_f64(d["bias"]))
    assert np.allclose(y64, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_zero_weight_is_pure_lowrank_product():
    d = _tiny()
    qw0 = np.zeros_like(d["qweight"])
    y64, y, _, _ = S.linear_w4a4(d["x"], d["smooth"], qw0, d["wscales"], d["wcscales"],
                                 d["wtscale"], d["proj_down"], d["proj_up"], d["bias"])
    x = torch.from_numpy(F.bf16_to_f64(d["x"]))
    pd = torch.from_numpy(F.bf16_to_f64(d["proj_down"]))
    pu = torch.from_numpy(F.bf16_to_f64(d["proj_up"]))
    b = torch.from_numpy(F.bf16_to_f64(d["bias"]))
    ref = torch.matmul(torch.matmul(x, pd), pu.T) + b
    assert np.allclose(y64, ref.numpy(), rtol=1e-12, atol=1e-14)
    # output rounding: the bf16 result is RNE of the float64 result
    assert np.array_equal(y, F.f64_to_bf16(ref.numpy())) or \
        np.mean(y != F.f64_to_bf16(ref.numpy())) < 1e-3


def test_lossless_inputs_give_exact_gemm():
    """smooth = 1 and x built from NVFP4 values: quantisation is lossless, so the
    main term is x @ W_eff^T exactly."""
    rng = np.random.default_rng(4)
    M, K, N = 16, 128, 32
    codes = rng.integers(0, 16, size=(M, K), dtype=np.uint8)
    codes[:, ::16] = 7
    sc = rng.integers(0x10, 0x60, size=(M, K // 16), dtype=np.uint8)
    xv = F.e2m1_decode(codes) * np.repeat(F.e4m3_decode(sc), 16, axis=1)
    x_bits = F.f64_to_bf16(xv)
    ones = F.f64_to_bf16(np.ones(K))
    d = workloads.make_linear(M=M, K=K, N=N, R=0, kind="tiny", seed=8)
    qw, ws = S.quantize_weight(d["W"], d["wcscales"], d["wtscale"])
    qact, ascales = S.quantize_act(x_bits, ones)
    main = S.main_term(qact, ascales, qw, ws)
    assert np.array_equal(main, xv @ S.dequant(qw, ws).T)


def test_epilogue_scales_only_the_main_term():
    d = _tiny()
    qact, ascales = S.quantize_act(d["x"], d["smooth"])
    main = S.main_term(qact, ascales, d["qweight"], d["wscales"])
    lr = S.lowrank(d["x"], d["proj_down"], d["proj_up"])
    wc2 = F.f64_to_bf16(2 * F.bf16_to_f64(d["wcscales"]))
    y1 = S.epilogue(main, d["wcscales"], d["wtscale"], lr, None)
    y2 = S.epilogue(main, wc2, d["wtscale"], lr, None)
    assert np.allclose(y2 - y1, main * F.bf16_to_f64(d["wcscales"])[None, :], rtol=1e-12, atol=1e-15)


def test_lowrank_uses_raw_x():
    d = _tiny()
    x = F.bf16_to_f64(d["x"])
    ref = (x @ F.bf16_to_f64(d["proj_down"])) @ F.bf16_to_f64(d["proj_up"]).T
    assert np.allclose(S.lowrank(d["x"], d["proj_down"], d["proj_up"]), ref, rtol=1e-13, atol=1e-16)


def test_w4a4_is_close_to_unquantised_product_when_self_consistent():
    """Sanity of the whole formula (not a parity gate): for W = W_q + proj_up proj_down^T
    quantised faithfully, y approximates x @ W^T."""
    rng = np.random.default_rng(12)
    M, K, N, R = 32, 256, 64, 16
    x = rng.standard_normal((M, K))
    x_bits = F.f64_to_bf16(x)
    pd = F.f64_to_bf16(rng.standard_normal((K, R)) * 0.02)
    pu = F.f64_to_bf16(rng.standard_normal((N, R)) * 0.02)
    Wr = rng.standard_normal((N, K)) * 0.02
    ones = F.f64_to_bf16(np.ones(K))
    wc = F.f64_to_bf16(np.abs(Wr).max(axis=1) / (6 * 448))
    wt = F.f64_to_bf16(np.ones(1))
    qw, ws = S.quantize_weight(Wr, wc, wt)
    y64, _, _, _ = S.linear_w4a4(x_bits, ones, qw, ws, wc, wt, pd, pu, None)
    W_full = Wr + F.bf16_to_f64(pu) @ F.bf16_to_f64(pd).T
    ref = F.bf16_to_f64(x_bits) @ W_full.T
    cos = np.sum(y64 * ref) / np.linalg.norm(y64) / np.linalg.norm(ref)
    assert cos > 0.98


def test_normwise_metric():
    a = np.array([[3.0, 4.0]])
    assert S.normwise_rel_err(a, a) == 0.0
    assert S.normwise_rel_err(np.array([[3.0, 0.0]]), a) == pytest.approx(4.0 / 5.0)


def test_lowrank_exact_rational_brute_force():
    """(x @ proj_down) @ proj_up^T on a tiny slice with Python Fractions (exact), against
    the oracle's float64 result within float64 rounding of the sums."""
    d = _tiny()
    rows, cols = [0, 7, 63], [0, 5, 127]
    x = F.bf16_to_f64(d["x"])
    pd = F.bf16_to_f64(d["proj_down"])
    pu = F.bf16_to_f64(d["proj_up"])
    K, R = pd.shape
    lr = S.lowrank(d["x"], d["proj_down"], d["proj_up"])
    down = S.lowrank_down(d["x"], d["proj_down"])
    for m in rows:
        t = [sum(Fraction(float(x[m, k])) * Fraction(float(pd[k, r])) for k in range(K)) for r in range(R)]
        mag = [sum(abs(Fraction(float(x[m, k])) * Fraction(float(pd[k, r]))) for k in range(K)) for r in range(R)]
        for r in range(R):
            assert abs(Fraction(float(down[m, r])) - t[r]) <= mag[r] * Fraction(K + 1, 2 ** 52)
        for n in cols:
            exact = sum(t[r] * Fraction(float(pu[n, r])) for r in range(R))
            bound = sum(mag[r] * abs(Fraction(float(pu[n, r]))) for r in range(R)) * Fraction(K + R + 2, 2 ** 52)
            assert abs(Fraction(float(lr[m, n])) - exact) <= bound


# --- gated FFN combination (w1 / w3 run as one 2F-wide layer) ---

def test_silu_closed_form_values():
    """silu(0) = 0; silu(z) - silu(-z) = z (sigmoid(z) + sigmoid(-z) = 1); silu(ln 3) =
    ln 3 * 3/4; large |z| tends to max(z, 0)."""
    assert S.silu(0.0) == 0.0
    z = np.linspace(-30, 30, 601)
    assert np.allclose(S.silu(z) - S.silu(-z), z, rtol=0, atol=1e-12)
    assert abs(S.silu(np.log(3.0)) - np.log(3.0) * 0.75) < 1e-15
    assert abs(S.silu(50.0) - 50.0) < 1e-15 and abs(S.silu(-50.0)) < 1e-18


def test_swiglu_pairs_column_n_with_n_plus_f():
    """Column n of the gate half pairs with column F + n of the up half, nothing else."""
    rng = np.random.default_rng(11)
    F_out = 7
    y = rng.standard_normal((3, 2 * F_out))
    h = S.swiglu(y, F_out)
    for m in range(3):
        for n in range(F_out):
            g, u = y[m, n], y[m, F_out + n]
            assert h[m, n] == g / (1.0 + np.exp(-g)) * u


def test_linear_swiglu_equals_gate_times_up_of_the_plain_layer():
    d = workloads.make_linear(M=16, K=128, N=2 * 24, R=16, kind="dit", seed=12)
    qw, ws = S.quantize_weight(d["W"], d["wcscales"], d["wtscale"])
    y64, _, _, _ = S.linear_w4a4(d["x"], d["smooth"], qw, ws, d["wcscales"], d["wtscale"],
                                 d["proj_down"], d["proj_up"], d["bias"])
    h64, h = S.linear_w4a4_swiglu(d["x"], d["smooth"], qw, ws, d["wcscales"], d["wtscale"],
                                  d["proj_down"], d["proj_up"], d["bias"])
    gate, up = y64[:, :24], y64[:, 24:]
    assert np.array_equal(h64, gate / (1.0 + np.exp(-gate)) * up)
    assert np.array_equal(h, F.f64_to_bf16(h64))


# ---------------------------------------------------------------------------
# gemm_w4a4: the layer from pre-quantised activations and a given lora_act
# ---------------------------------------------------------------------------
#
# Pins of oracle.svdq.gemm_w4a4 (model card "nunchaku-z-image-turbo-svdq",
# section "What's stored on disk", runtime formula without the quant step):
#  * an exact-rational brute force of the formula, element by element, with the
#    E2M1 grid and the e4m3fn closed form written out here;
#  * bit-for-bit equality with the pinned whole layer when lora_act is the
#    layer's own x @ proj_down (the two evaluate the same float64 products);
#  * qweight = 0 gives lora_act @ proj_up^T + bias (torch float64 matmul).
# Planted mistakes (the low-rank term dropped or scaled by the weight scales,
# the bias dropped, wcscales applied per row) must fail the brute force.

_GRID = [0, Fraction(1, 2), 1, Fraction(3, 2), 2, 3, 4, 6]


def _e2m1_q(c):
    return -_GRID[c & 7] if c & 8 else _GRID[c & 7]


def _e4m3_q(b):
    e, f = (b >> 3) & 15, b & 7
    return Fraction(f, 512) if e == 0 else (1 + Fraction(f, 8)) * Fraction(2) ** (e - 7)


def _bf16_q(bits):
    """Exact value of a bf16 bit pattern (finite) as a Fraction."""
    return Fraction(float(F.bf16_to_f64(np.array([bits], dtype=np.uint16))[0]))


def _gemm_brute(qact, ascales, lora, qweight, wscales, wc_bits, wt_bits, pu_bits, bias_bits, m, n):
    K = 2 * qact.shape[1]
    main = Fraction(0)
    for k in range(K):
        ab, wb = int(qact[m, k // 2]), int(qweight[n, k // 2])
        a = _e2m1_q(ab & 15 if k % 2 == 0 else ab >> 4) * _e4m3_q(int(ascales[k // 16, m]))
        w = _e2m1_q(wb & 15 if k % 2 == 0 else wb >> 4) * _e4m3_q(int(wscales[k // 16, n]))
        main += a * w
    y = main * _bf16_q(int(wt_bits[0])) * _bf16_q(int(wc_bits[n]))
    if lora is not None:
        for r in range(lora.shape[1]):
            y += Fraction(float(lora[m, r])) * _bf16_q(int(pu_bits[n, r]))
    if bias_bits is not None:
        y += _bf16_q(int(bias_bits[n]))
    return y


def _gemm_case(seed=11, **over):
    d = _tiny(seed=seed, **over)
    d["wtscale"] = F.f64_to_bf16(np.array([0.625]))   # any global alpha: the inputs are arbitrary here
    qact, ascales = S.quantize_act(d["x"], d["smooth"])
    lora = S.lowrank_down(d["x"], d["proj_down"]) if d["R"] > 0 else None
    return d, qact, ascales, lora


def _gemm_pin_error(gemm_fn, d, qact, ascales, lora, points):
    """Largest |gemm_fn - brute force| / scale over the sampled points, where scale is
    the sum of the magnitudes of the formula's terms (so float64 rounding is ~1e-16)."""
    y = gemm_fn(qact, ascales, lora, d["qweight"], d["wscales"], d["wcscales"], d["wtscale"],
                d["proj_up"], d["bias"])
    worst = 0.0
    for m, n in points:
        exact = _gemm_brute(qact, ascales, lora, d["qweight"], d["wscales"], d["wcscales"], d["wtscale"],
                            d["proj_up"], d["bias"], m, n)
        mag = abs(float(exact)) + 1e-3
        worst = max(worst, abs(float(Fraction(float(y[m, n])) - exact)) / mag)
    return worst


_POINTS = [(0, 0), (5, 17), (63, 127), (31, 64), (10, 99), (47, 3)]


def test_gemm_w4a4_rational_brute_force():
    case = _gemm_case()
    assert _gemm_pin_error(S.gemm_w4a4, *case, _POINTS) < 1e-13


def test_gemm_w4a4_rational_brute_force_dit_rows():
    """DiT-shaped inputs (outlier channels, normal-range weight scales, R = 32)."""
    d = workloads.make_linear(M=8, K=256, N=24, R=32, kind="dit", seed=1003)
    d["qweight"], d["wscales"] = S.quantize_weight(d["W"], d["wcscales"], d["wtscale"])
    qact, ascales = S.quantize_act(d["x"], d["smooth"])
    lora = S.lowrank_down(d["x"], d["proj_down"])
    pts = [(0, 0), (7, 23), (3, 11), (5, 2)]
    assert _gemm_pin_error(S.gemm_w4a4, d, qact, ascales, lora, pts) < 1e-13


def test_gemm_w4a4_equals_whole_layer_bitwise():
    for d in (_tiny(seed=12),
              workloads.make_linear(M=32, K=512, N=48, R=32, kind="dit", seed=1003)):
        if "qweight" not in d:
            d["qweight"], d["wscales"] = S.quantize_weight(d["W"], d["wcscales"], d["wtscale"])
        y64, _, qact, ascales = S.linear_w4a4(d["x"], d["smooth"], d["qweight"], d["wscales"], d["wcscales"],
                                              d["wtscale"], d["proj_down"], d["proj_up"], d["bias"])
        lora = S.lowrank_down(d["x"], d["proj_down"])
        y = S.gemm_w4a4(qact, ascales, lora, d["qweight"], d["wscales"], d["wcscales"], d["wtscale"],
                        d["proj_up"], d["bias"])
        assert np.array_equal(y, y64)


def test_gemm_w4a4_zero_weight_is_lowrank_plus_bias():
    d, qact, ascales, lora = _gemm_case(seed=13)
    y = S.gemm_w4a4(qact, ascales, lora, np.zeros_like(d["qweight"]), d["wscales"], d["wcscales"],
                    d["wtscale"], d["proj_up"], d["bias"])
    ref = torch.from_numpy(lora) @ torch.from_numpy(F.bf16_to_f64(d["proj_up"])).T + \
        torch.from_numpy(F.bf16_to_f64(d["bias"]))
    assert np.allclose(y, ref.numpy(), rtol=1e-13, atol=1e-15)


def test_gemm_w4a4_r0_and_no_bias():
    d, qact, ascales, _ = _gemm_case(seed=14, R=0)
    d["bias"] = None
    y = S.gemm_w4a4(qact, ascales, None, d["qweight"], d["wscales"], d["wcscales"], d["wtscale"],
                    None, None)
    A = S.dequant(qact, ascales)
    W = S.dequant(d["qweight"], d["wscales"])
    alpha = F.bf16_to_f64(d["wtscale"])[0] * F.bf16_to_f64(d["wcscales"])
    assert np.allclose(y, (A @ W.T) * alpha[None, :], rtol=1e-13, atol=0)
    assert _gemm_pin_error(S.gemm_w4a4, d, qact, ascales, None, _POINTS) < 1e-13


def _mut_drop_lowrank(qact, ascales, lora, *rest):
    return S.gemm_w4a4(qact, ascales, None, *rest)


def _mut_scale_lowrank(qact, ascales, lora, qweight, wscales, wc, wt, pu, bias):
    main = S.main_term(qact, ascales, qweight, wscales)
    lr = np.asarray(lora) @ F.bf16_to_f64(pu).T
    return S.epilogue(main + lr, wc, wt, None, bias)


def _mut_drop_bias(qact, ascales, lora, qweight, wscales, wc, wt, pu, bias):
    return S.gemm_w4a4(qact, ascales, lora, qweight, wscales, wc, wt, pu, None)


def _mut_row_scales(qact, ascales, lora, qweight, wscales, wc, wt, pu, bias):
    # wcscales applied along the wrong axis (rows instead of output channels)
    main = S.main_term(qact, ascales, qweight, wscales)
    M = main.shape[0]
    wcm = F.bf16_to_f64(wc)[:M]
    y = main * F.bf16_to_f64(wt)[0] * wcm[:, None]
    return y + np.asarray(lora) @ F.bf16_to_f64(pu).T + F.bf16_to_f64(bias)[None, :]


def _mut_drop_wtscale(qact, ascales, lora, qweight, wscales, wc, wt, pu, bias):
    return S.gemm_w4a4(qact, ascales, lora, qweight, wscales, wc, F.f64_to_bf16(np.array([1.0])), pu, bias)


@pytest.mark.parametrize("mutant", [_mut_drop_lowrank, _mut_scale_lowrank, _mut_drop_bias, _mut_row_scales,
                                    _mut_drop_wtscale])
def test_gemm_pin_catches_planted_mistakes(mutant):
    case = _gemm_case()
    assert _gemm_pin_error(mutant, *case, _POINTS) > 1e-6
