"""Pins of the oracle's activation quantisation quant(x * smooth).

No checkpoint, kernel or test vector is on the pages, so the rule is pinned
against: an exact-rational pure-Python brute force written from the reading
(per-16 amax / 6 -> e4m3 RNE saturating; codes = E2M1 RNE of |v| / s_d with
the sign of v), invariants that follow from the format, idempotence on
NVFP4-representable blocks, and exact ties.
"""

from fractions import Fraction

import numpy as np
import pytest

import workloads
from oracle import formats as F
from oracle import svdq as S


def _e4m3_value(code):
    e, f = (code >> 3) & 15, code & 7
    if e == 0:
        return Fraction(f, 8) * Fraction(1, 64)
    return (1 + Fraction(f, 8)) * Fraction(2) ** (e - 7)


E4M3_VALUES = [_e4m3_value(c) for c in range(0x7F)]
E2M1_VALUES = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
               Fraction(3), Fraction(4), Fraction(6)]


def _nearest_even(t, values):
    t = min(t, values[-1])
    best = None
    for c, v in enumerate(values):
        d = abs(t - v)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def _bf16_fraction(bits):
    return Fraction(float(F.bf16_to_f64(np.array([bits]))[0]))


def brute_quant_row(x_bits_row, smooth_bits):
    """Exact rational quantisation of one row: returns (codes list, scale codes list)."""
    K = len(x_bits_row)
    v = [_bf16_fraction(x_bits_row[k]) * _bf16_fraction(smooth_bits[k]) for k in range(K)]
    neg = [bool(np.signbit(F.bf16_to_f64(np.array([x_bits_row[k]]))[0])) !=
           bool(np.signbit(F.bf16_to_f64(np.array([smooth_bits[k]]))[0])) for k in range(K)]
    codes, scales = [], []
    for b in range(K // 16):
        blk = v[16 * b: 16 * b + 16]
        amax = max(abs(t) for t in blk)
        sc = _nearest_even(amax / 6, E4M3_VALUES)
        sd = E4M3_VALUES[sc]
        scales.append(sc)
        for i, t in enumerate(blk):
            mag = 0 if sd == 0 else _nearest_even(abs(t) / sd, E2M1_VALUES)
            codes.append(mag | (8 if neg[16 * b + i] else 0))
    return codes, scales


def test_quant_matches_exact_brute_force_on_tiny_config():
    d = workloads.make_linear(**workloads.TINY)
    qact, ascales = S.quantize_act(d["x"], d["smooth"])
    codes = F.unpack_nibbles(qact)
    rows = range(0, d["M"], 3)  # every third row keeps the pure-Python part short
    for m in rows:
        bc, bs = brute_quant_row(d["x"][m], d["smooth"])
        assert list(codes[m]) == bc
        assert list(ascales[:, m]) == bs


def test_quant_brute_force_dit_outlier_rows():
    x, sm = workloads.make_activation(8, 512, kind="dit", seed=99)
    qact, ascales = S.quantize_act(x, sm)
    codes = F.unpack_nibbles(qact)
    for m in range(8):
        bc, bs = brute_quant_row(x[m], sm)
        assert list(codes[m]) == bc
        assert list(ascales[:, m]) == bs


def test_amax_element_gets_code_7_for_normal_scales():
    x, sm = workloads.make_activation(128, 1024, kind="dit", seed=5)
    qact, ascales = S.quantize_act(x, sm)
    codes = F.unpack_nibbles(qact).reshape(128, 64, 16)
    v = np.abs(F.bf16_to_f64(x) * F.bf16_to_f64(sm)[None, :]).reshape(128, 64, 16)
    normal = ascales.T >= 0x08
    amax_idx = v.argmax(axis=2)
    top = np.take_along_axis(codes, amax_idx[:, :, None], axis=2)[:, :, 0] & 7
    assert normal.sum() > 1000
    assert np.all(top[normal] == 7)


def test_codes_are_nearest_grid_points():
    x, sm = workloads.make_activation(32, 256, kind="tiny", seed=11)
    qact, ascales = S.quantize_act(x, sm)
    codes = F.unpack_nibbles(qact)
    v = F.bf16_to_f64(x) * F.bf16_to_f64(sm)[None, :]
    sd = np.repeat(F.e4m3_decode(ascales).T, 16, axis=1)
    t = np.abs(v) / sd
    got = F.E2M1_GRID[codes & 7]
    err = np.abs(np.minimum(t, 6.0) - got)
    # no grid value is strictly closer than the chosen one
    for g in F.E2M1_GRID:
        assert np.all(err <= np.abs(np.minimum(t, 6.0) - g) + 0.0)
    assert np.array_equal((codes & 8) != 0, np.signbit(v))


def test_idempotent_on_nvfp4_representable_blocks():
    rng = np.random.default_rng(21)
    M, K = 16, 128
    codes = rng.integers(0, 16, size=(M, K), dtype=np.uint8)
    codes[:, ::16] = np.where(rng.random((M, K // 16)) < 0.5, 7, 15)  # one +-6 per block
    sc = rng.integers(0x08, 0x70, size=(M, K // 16), dtype=np.uint8)   # normal scales
    vals = F.e2m1_decode(codes) * np.repeat(F.e4m3_decode(sc), 16, axis=1)
    x_bits = F.f64_to_bf16(vals)
    assert np.array_equal(F.bf16_to_f64(x_bits), vals)   # representable in bf16
    one = F.f64_to_bf16(np.ones(K))
    qact, ascales = S.quantize_act(x_bits, one)
    got = F.unpack_nibbles(qact)
    # -0 codes (8) decode like +0; compare values and the exact code where nonzero
    assert np.array_equal(F.e2m1_decode(got), F.e2m1_decode(codes))
    assert np.array_equal(ascales.T, sc)


def test_exact_ties_round_to_even_codes():
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    expect = [0, 2, 2, 4, 4, 6, 6]
    s_d = F.e4m3_decode(np.array([0x30]))[0]            # 0.5: normal scale
    blk = np.zeros(16)
    blk[0] = 6.0 * s_d                                    # sets amax so sc == 0x30
    blk[1:8] = mids * s_d
    blk[8:15] = -mids * s_d
    x_bits = F.f64_to_bf16(blk[None, :])
    assert np.array_equal(F.bf16_to_f64(x_bits)[0], blk)
    qact, ascales = S.quantize_act(x_bits, F.f64_to_bf16(np.ones(16)))
    assert ascales[0, 0] == 0x30
    c = F.unpack_nibbles(qact)[0]
    assert c[0] == 7
    assert list(c[1:8]) == expect
    assert list(c[8:15]) == [e | 8 for e in expect]
    assert c[15] == 0


def test_zero_block_and_negative_zero_and_underflow():
    blk = np.zeros((1, 32))
    blk[0, 16:] = -2.0 ** -20      # tiny: scale rounds to 0, codes keep the sign
    blk[0, 3] = -0.0
    x_bits = F.f64_to_bf16(blk)
    x_bits[0, 3] = 0x8000
    qact, ascales = S.quantize_act(x_bits, F.f64_to_bf16(np.ones(32)))
    c = F.unpack_nibbles(qact)[0]
    assert list(ascales[:, 0]) == [0, 0]
    assert c[3] == 8 and all(c[i] == 0 for i in range(16) if i != 3)
    assert all(c[16:] == 8)


def test_saturating_scale_for_huge_blocks():
    blk = np.full((1, 16), 3000.0)      # amax / 6 = 500 > 448 -> scale 448, codes saturate
    qact, ascales = S.quantize_act(F.f64_to_bf16(blk), F.f64_to_bf16(np.ones(16)))
    assert ascales[0, 0] == 0x7E
    assert np.all(F.unpack_nibbles(qact)[0] == 7)


@pytest.mark.parametrize("seed", [1, 2])
def test_weight_quant_layout_and_scale_range(seed):
    d = workloads.make_linear(M=4, K=256, N=64, R=0, kind="dit", seed=seed)
    qw, ws = S.quantize_weight(d["W"], d["wcscales"], d["wtscale"])
    assert qw.shape == (64, 128) and ws.shape == (16, 64)
    assert ws.min() >= 0x08 and ws.max() <= 0x7E      # dit recipe: normal e4m3 range
    deq = S.dequant(qw, ws) * F.bf16_to_f64(d["wcscales"])[:, None]
    rel = np.linalg.norm(deq - d["W"]) / np.linalg.norm(d["W"])
    assert rel < 0.12          # 4-bit weights: coarse but faithful
