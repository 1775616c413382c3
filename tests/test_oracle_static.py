"""Pins of the oracle's static-activation-scale variant (blog page "Z-Image NVFP4 ...",
section on the Comfy-Org Z-Image Turbo NVFP4 checkpoint: calibrated static activation
scales; the rule is a reading, stated in oracle/svdq.py).

* An exact-rational brute force of the rule, with the e4m3fn and E2M1 grids enumerated
  here (ties to the even code), on random blocks, outlier rows and a non-power-of-two g.
* g = 1 is the dynamic rule bit for bit; g = 2^k is the dynamic rule on smooth * 2^-k.
* Saturation: a block far above 6 * 448 * g gets scale byte 0x7E and code magnitude 7.
* Calibration: g is the bf16 rounding of max|x * smooth| / 2688, checked with rationals.
* The layer: g = 1 equals the dynamic layer bit for bit; sampled outputs equal a rational
  brute force; planted mistakes (g on the low-rank term, g dropped, block scales taken
  without g) fail it.
"""

from fractions import Fraction

import numpy as np
import pytest

import workloads
from oracle import formats as F
from oracle import svdq as S

_E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
         Fraction(6)]


def _e4m3_grid():
    """(value, byte) for every finite non-negative e4m3fn code, 0x00 .. 0x7E."""
    out = []
    for b in range(0x7F):
        e, f = b >> 3, b & 7
        v = Fraction(f, 512) if e == 0 else (1 + Fraction(f, 8)) * Fraction(2) ** (e - 7)
        out.append((v, b))
    return out


_E4M3 = _e4m3_grid()


def _nearest_even(t, grid):
    """Index of the nearest grid value to t >= 0, ties to the even index; saturates."""
    if t >= grid[-1]:
        return len(grid) - 1
    best = 0
    for i in range(len(grid)):
        di, db = abs(grid[i] - t), abs(grid[best] - t)
        if di < db or (di == db and i % 2 == 0 and best % 2 == 1):
            best = i
    return best


def _brute_block(vals, neg, g):
    """vals: Fractions |v|; neg: sign bits; g: Fraction. -> (codes, scale byte)."""
    amax = max(vals)
    q = amax / (6 * g)
    sb = _E4M3[_nearest_even(q, [v for v, _ in _E4M3])][1]
    d = _E4M3[sb][0] * g
    codes = []
    for a, n in zip(vals, neg):
        m = 0 if d == 0 else _nearest_even(a / d, _E2M1)
        codes.append((8 if n else 0) | m)
    return codes, sb


def _frac(x):
    return Fraction(float(x))


def _check_rows(x_bits, sm_bits, g_bits, rows):
    qact, asc = S.quantize_act_static(x_bits, sm_bits, g_bits)
    codes = F.unpack_nibbles(qact)
    g = _frac(F.bf16_to_f64(g_bits)[0])
    xv = F.bf16_to_f64(x_bits)
    sv = F.bf16_to_f64(sm_bits)
    K = xv.shape[1]
    for m in rows:
        for b in range(K // 16):
            ks = range(16 * b, 16 * b + 16)
            prods = [_frac(xv[m, k]) * _frac(sv[k]) for k in ks]
            neg = [bool(np.signbit(xv[m, k] * sv[k])) for k in ks]
            bc, bs = _brute_block([abs(p) for p in prods], neg, g)
            assert int(asc[b, m]) == bs, (m, b)
            assert [int(c) for c in codes[m, 16 * b:16 * b + 16]] == bc, (m, b)


def test_static_rule_rational_brute_force_tiny():
    d = workloads.make_linear(**workloads.TINY)
    g = F.f64_to_bf16(np.array([0.0123]))      # not a power of two (8 significant bits)
    _check_rows(d["x"], d["smooth"], g, rows=[0, 7, 33, 63])


def test_static_rule_rational_brute_force_outlier_rows():
    d = workloads.make_linear(M=6, K=512, N=16, R=0, kind="dit", seed=1003)
    g = S.calibrate_gscale(d["x"], d["smooth"])
    _check_rows(d["x"], d["smooth"], g, rows=range(6))
    g2 = F.f64_to_bf16(np.array([3.7e-4]))     # small g: many blocks saturate at 448
    _check_rows(d["x"], d["smooth"], g2, rows=[0, 5])


def test_g_one_is_the_dynamic_rule():
    for d in (workloads.make_linear(**workloads.TINY),
              workloads.make_linear(M=32, K=1024, N=8, R=0, kind="dit", seed=1002)):
        one = F.f64_to_bf16(np.array([1.0]))
        qs, ss = S.quantize_act_static(d["x"], d["smooth"], one)
        qd, sd = S.quantize_act(d["x"], d["smooth"])
        assert np.array_equal(qs, qd) and np.array_equal(ss, sd)


@pytest.mark.parametrize("k", [-3, 5])
def test_power_of_two_g_is_dynamic_rule_on_scaled_smooth(k):
    d = workloads.make_linear(M=32, K=512, N=8, R=0, kind="dit", seed=1013)
    g = F.f64_to_bf16(np.array([2.0 ** k]))
    sm2 = F.f64_to_bf16(F.bf16_to_f64(d["smooth"]) * 2.0 ** -k)   # exact: a power-of-two rescale
    qs, ss = S.quantize_act_static(d["x"], d["smooth"], g)
    qd, sd = S.quantize_act(d["x"], sm2)
    assert np.array_equal(qs, qd) and np.array_equal(ss, sd)


def test_saturation_far_above_the_global_scale():
    K = 32
    x = np.zeros((2, K))
    x[0, :16] = np.linspace(-7000.0, 9000.0, 16)
    x[1, 16:] = 1.0
    xb = F.f64_to_bf16(x)
    one = F.f64_to_bf16(np.ones(K))
    g = F.f64_to_bf16(np.array([0.5]))           # 6 * 448 * g = 1344 < 9000
    q, s = S.quantize_act_static(xb, one, g)
    codes = F.unpack_nibbles(q)
    assert s[0, 0] == 0x7E                       # saturated block scale
    assert codes[0, 15] == 7 and codes[0, 0] == 8 | 7
    # row 1, block 1: amax 1 -> 1 / (6 g) = 1/3 -> e4m3 1.375 * 2^-2 (byte 0x2B); 1 / (0.34375 * 0.5) -> 6
    assert s[1, 1] == 0x2B and np.all(codes[1, 16:] == 7)
    assert s[1, 0] == 0x00 and s[0, 1] == 0x00 and np.all(codes[1, :16] == 0)   # all-zero blocks


def test_calibration_is_bf16_of_amax_over_2688():
    d = workloads.make_linear(M=48, K=256, N=8, R=0, kind="dit", seed=1023)
    g = S.calibrate_gscale(d["x"], d["smooth"])
    xv, sv = F.bf16_to_f64(d["x"]), F.bf16_to_f64(d["smooth"])
    amax = max(abs(_frac(xv[m, k]) * _frac(sv[k])) for m in range(48) for k in range(256))
    q = amax / 2688
    # bf16 nearest-even of the rational q, by brute force over the 2 neighbours of its binade
    e = 0
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    while Fraction(2) ** e > q:
        e -= 1
    step = Fraction(2) ** (e - 7)
    lo = (q // step) * step
    hi = lo + step
    pick = lo if (q - lo < hi - q or (q - lo == hi - q and (lo / step) % 2 == 0)) else hi
    assert Fraction(float(F.bf16_to_f64(g)[0])) == pick
    zero = np.zeros((4, 32), dtype=np.uint16)
    assert F.bf16_to_f64(S.calibrate_gscale(zero, d["smooth"][:32]))[0] == 1.0


def _static_layer_case(seed=21):
    d = workloads.make_linear(M=16, K=256, N=24, R=16, kind="dit", seed=seed)
    d["qweight"], d["wscales"] = S.quantize_weight(d["W"], d["wcscales"], d["wtscale"])
    d["wtscale"] = F.f64_to_bf16(np.array([0.75]))
    d["g"] = F.f64_to_bf16(np.array([0.00731]))
    return d


def _layer_brute(d, m, n):
    qact, asc = S.quantize_act_static(d["x"], d["smooth"], d["g"])
    g = _frac(F.bf16_to_f64(d["g"])[0])
    K = d["K"]
    main = Fraction(0)
    grid = [Fraction(0), Fraction(1, 2), 1, Fraction(3, 2), 2, 3, 4, 6]

    def e2m1(c):
        return -grid[c & 7] if c & 8 else grid[c & 7]

    for k in range(K):
        ab, wb = int(qact[m, k // 2]), int(d["qweight"][n, k // 2])
        a = e2m1(ab & 15 if k % 2 == 0 else ab >> 4) * _E4M3[int(asc[k // 16, m])][0] * g
        w = e2m1(wb & 15 if k % 2 == 0 else wb >> 4) * _E4M3[int(d["wscales"][k // 16, n])][0]
        main += a * w
    y = main * _frac(F.bf16_to_f64(d["wtscale"])[0]) * _frac(F.bf16_to_f64(d["wcscales"])[n])
    xv, pd, pu = F.bf16_to_f64(d["x"]), F.bf16_to_f64(d["proj_down"]), F.bf16_to_f64(d["proj_up"])
    for r in range(d["R"]):
        la = sum(_frac(xv[m, k]) * _frac(pd[k, r]) for k in range(K))
        y += la * _frac(pu[n, r])
    return y + _frac(F.bf16_to_f64(d["bias"])[n])


def _static_layer(d, fn=None):
    fn = fn or S.linear_w4a4_static
    return fn(d["x"], d["smooth"], d["g"], d["qweight"], d["wscales"], d["wcscales"], d["wtscale"],
              d["proj_down"], d["proj_up"], d["bias"])[0]


def _pin_error(d, y64, pts):
    worst = 0.0
    for m, n in pts:
        ex = _layer_brute(d, m, n)
        worst = max(worst, abs(float(Fraction(float(y64[m, n])) - ex)) / (abs(float(ex)) + 1e-3))
    return worst


_PTS = [(0, 0), (15, 23), (7, 11), (3, 19)]


def test_static_layer_rational_brute_force():
    d = _static_layer_case()
    assert _pin_error(d, _static_layer(d), _PTS) < 1e-12


def test_static_layer_g_one_is_dynamic_layer():
    d = _static_layer_case(seed=22)
    d["g"] = F.f64_to_bf16(np.array([1.0]))
    ys = _static_layer(d)
    yd = S.linear_w4a4(d["x"], d["smooth"], d["qweight"], d["wscales"], d["wcscales"], d["wtscale"],
                       d["proj_down"], d["proj_up"], d["bias"])[0]
    assert np.array_equal(ys, yd)


def _mut_g_on_lowrank(x, sm, gb, qw, ws, wc, wt, pd, pu, b):
    g = float(F.bf16_to_f64(gb)[0])
    qact, asc = S.quantize_act_static(x, sm, gb)
    y = S.epilogue(S.main_term(qact, asc, qw, ws), wc, wt, None, None)
    return (g * (y + S.lowrank(x, pd, pu)) + F.bf16_to_f64(b)[None, :]), None


def _mut_g_dropped(x, sm, gb, qw, ws, wc, wt, pd, pu, b):
    qact, asc = S.quantize_act_static(x, sm, gb)
    return S.epilogue(S.main_term(qact, asc, qw, ws), wc, wt, S.lowrank(x, pd, pu), b), None


def _mut_dynamic_scales(x, sm, gb, qw, ws, wc, wt, pd, pu, b):
    g = float(F.bf16_to_f64(gb)[0])
    qact, asc = S.quantize_act(x, sm)
    return S.epilogue(S.main_term(qact, asc, qw, ws) * g, wc, wt, S.lowrank(x, pd, pu), b), None


@pytest.mark.parametrize("mutant", [_mut_g_on_lowrank, _mut_g_dropped, _mut_dynamic_scales])
def test_static_pin_catches_planted_mistakes(mutant):
    d = _static_layer_case()
    assert _pin_error(d, _static_layer(d, mutant), _PTS) > 1e-6


def test_calibrated_static_layer_tracks_dynamic_layer():
    """Calibrated on a different seeded batch of the same distribution, the static layer stays
    close to the dynamic one (most blocks keep normal-range scales)."""
    cfg = dict(M=64, K=512, N=64, R=16, kind="dit")
    d = workloads.make_linear(**cfg, seed=31)
    cal = workloads.make_linear(**cfg, seed=32)
    qw, ws = S.quantize_weight(d["W"], d["wcscales"], d["wtscale"])
    g = S.calibrate_gscale(cal["x"], d["smooth"])
    ys = S.linear_w4a4_static(d["x"], d["smooth"], g, qw, ws, d["wcscales"], d["wtscale"], d["proj_down"],
                              d["proj_up"], d["bias"])[0]
    yd = S.linear_w4a4(d["x"], d["smooth"], qw, ws, d["wcscales"], d["wtscale"], d["proj_down"], d["proj_up"],
                       d["bias"])[0]
    assert S.normwise_rel_err(ys, yd) < 0.1
