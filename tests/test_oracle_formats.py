"""Pins of the oracle's number formats against the pages, closed forms and torch casts."""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _minifloat_value(code, ebits, mbits, bias):
    """Generic sign/exponent/mantissa decode with subnormals at exponent 0 (exact)."""
    s = (code >> (ebits + mbits)) & 1
    e = (code >> mbits) & ((1 << ebits) - 1)
    f = code & ((1 << mbits) - 1)
    if e == 0:
        mag = Fraction(f, 1 << mbits) * Fraction(2) ** (1 - bias)
    else:
        mag = (1 + Fraction(f, 1 << mbits)) * Fraction(2) ** (e - bias)
    return -mag if s else mag


def test_e2m1_grid_matches_pages_and_bit_structure():
    grid = [(int(c), float(v)) for c, v in _read_table("e2m1_grid.txt")]
    for code in range(16):
        mag = dict(grid)[code & 7]
        expect = -mag if code & 8 else mag
        assert F.e2m1_decode(np.array([code]))[0] == expect
        # 1 sign + 2 exponent + 1 mantissa bits, bias 1, subnormal at exponent 0
        assert float(_minifloat_value(code, 2, 1, 1)) == expect


def test_e2m1_encode_exact_ties_and_saturation():
    for mid, code in _read_table("e2m1_ties.txt"):
        assert int(F.e2m1_encode_mag(np.array([float(mid)]))[0]) == int(code)
    assert int(F.e2m1_encode_mag(np.array([6.0001]))[0]) == 7
    assert int(F.e2m1_encode_mag(np.array([1e30]))[0]) == 7
    assert int(F.e2m1_encode_mag(np.array([0.0]))[0]) == 0


def test_e2m1_encode_brute_force_nearest():
    """Every multiple of 2**-12 in [0, 8] against a direct search over the 8 codes."""
    grid = [Fraction(str(v)) for v in F.E2M1_GRID]
    ts = [Fraction(i, 4096) for i in range(0, 8 * 4096 + 1)]
    got = F.e2m1_encode_mag(np.array([float(t) for t in ts]))
    for t, g in zip(ts[::7], got[::7]):
        tc = min(t, Fraction(6))
        best = None
        for c, v in enumerate(grid):
            d = abs(tc - v)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        assert g == best[1], (t, g, best)


def test_e4m3_decode_all_codes_vs_torch_and_closed_form():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert ours[c] == float(_minifloat_value(c, 4, 3, 7))


def test_e4m3_facts_from_pages():
    facts = {r[0]: r[1:] for r in _read_table("e4m3_facts.txt")}
    assert F.e4m3_decode(np.array([int(facts["max_finite_code"][0], 16)]))[0] == float(facts["max_finite"][0])
    assert F.E4M3_POS_GRID.max() == float(facts["max_finite"][0])
    nan_codes = [int(c, 16) for c in facts["nan_codes"]]
    assert all(np.isnan(F.e4m3_decode(np.array(nan_codes))))
    assert F.E4M3_POS_GRID[1] == float(facts["min_subnormal"][0])
    assert F.e4m3_decode(np.array([0x08]))[0] == float(facts["min_normal"][0])
    assert np.all(np.diff(F.E4M3_POS_GRID) > 0)


def test_e4m3_encode_vs_torch_on_all_bf16_up_to_448():
    bits = np.arange(0, 0x43E1, dtype=np.uint32) << 16      # bf16 patterns 0 .. 448
    vals = bits.view(np.float32)
    vals = vals[vals <= 448.0]
    ours = F.e4m3_encode(vals.astype(np.float64))
    ref = torch.from_numpy(vals.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_midpoints_vs_torch():
    g = F.E4M3_POS_GRID
    mids = ((g[:-1] + g[1:]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(1e4))
    down = np.nextafter(mids, np.float32(0))
    vals = np.concatenate([mids, up, down])
    ours = F.e4m3_encode(vals.astype(np.float64))
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    # ties go to the even mantissa
    assert np.all(ours[: len(mids)] % 2 == 0)


def test_e4m3_encode_saturates_instead_of_nan():
    for v in (448.0, 460.0, 464.0, 470.0, 1e4, 1e30):
        assert int(F.e4m3_encode(np.array([v]))[0]) == 0x7E
    # smallest cases: 2**-10 is the tie between 0 and the first subnormal -> 0 (even)
    assert int(F.e4m3_encode(np.array([2.0 ** -10]))[0]) == 0
    assert int(F.e4m3_encode(np.array([1.5 * 2.0 ** -10]))[0]) == 1


def test_pack_unpack_round_trip_all_bytes():
    b = np.arange(256, dtype=np.uint8).reshape(16, 16)
    codes = F.unpack_nibbles(b)
    assert np.array_equal(codes[:, 0::2], b & 15)        # low nibble = even k
    assert np.array_equal(F.pack_nibbles(codes), b)
    rng = np.random.default_rng(7)
    c = rng.integers(0, 16, size=(5, 64), dtype=np.uint8)
    assert np.array_equal(F.unpack_nibbles(F.pack_nibbles(c)), c)


def test_bf16_round_trip_and_rne():
    rng = np.random.default_rng(3)
    v = rng.standard_normal(10000).astype(np.float32) * 100
    ours = F.f32_to_bf16(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(F.bf16_to_f64(ours), torch.from_numpy(v).to(torch.bfloat16).double().numpy())
    # direct rounding from float64: 1 + 2**-8 + 2**-30 is above the midpoint between
    # 1 and 1 + 2**-7, so it rounds up (a float32 detour would tie and round down).
    assert F.bf16_to_f64(F.f64_to_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -30])))[0] == 1 + 2.0 ** -7
    assert F.bf16_to_f64(F.f64_to_bf16(np.array([1 + 2.0 ** -8])))[0] == 1.0
    assert F.bf16_to_f64(F.f64_to_bf16(np.array([1 + 3 * 2.0 ** -8])))[0] == 1 + 2 * 2.0 ** -7


@pytest.mark.parametrize("v", [2.0 ** -133, 3 * 2.0 ** -134, -1.5 * 2.0 ** -130])
def test_bf16_subnormals(v):
    out = F.bf16_to_f64(F.f64_to_bf16(np.array([v])))[0]
    ref = torch.tensor([v], dtype=torch.float32).to(torch.bfloat16).double().item()
    assert out == ref
