"""GPU parity of the scaled GEMM + low-rank up-projection + epilogue (svdq_gemm_w4a4).

Inputs: the oracle's own quantised activations and weights and a bf16 lora_act,
so the GPU and the oracle see identical operands; the oracle then evaluates the
formula in float64. Gate: normwise relative error <= 5e-3 on the bf16 output.
Diagnostic bound (also asserted): nearly every element is within one bf16 ulp of
the float64 result, since only fp32 accumulation and the final cast round.

Cases: canonical and packed weight layouts (bit-identical outputs), R = 0,
qweight = 0 (pure low-rank product), no bias, ragged M and N, K of one block and
K not a multiple of the 64-wide stage, the 1024^2 FFN shape sampled by rows.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import formats as F
from oracle import svdq as S
from tests.gpu_util import dev_bf16, dev_u8, host_bits, make_layer, ulp_bf16, within_ulps

pytestmark = pytest.mark.gpu

TOL = 5e-3


_CACHE = {}


def _oracle_inputs(cfg, with_bias, zero_weight):
    key = (tuple(sorted(cfg.items())), with_bias, zero_weight)
    if key not in _CACHE:
        d, layer = make_layer(cfg, with_bias=with_bias, zero_weight=zero_weight)
        qact, ascales = S.quantize_act(d["x"], d["smooth"])
        lora_bits = F.f64_to_bf16(S.lowrank_down(d["x"], d["proj_down"])) if d["R"] > 0 else None
        _CACHE.clear()
        _CACHE[key] = (d, layer, qact, ascales, lora_bits)
    return _CACHE[key]


def gemm_case(ops, cfg, packed=False, with_bias=True, zero_weight=False, rows=None):
    d, layer, qact, ascales, lora_bits = _oracle_inputs(cfg, with_bias, zero_weight)
    R = d["R"]
    if packed:
        layer = layer.packed()
    y = ops.gemm_w4a4(dev_u8(qact), dev_u8(ascales), dev_bf16(lora_bits) if R > 0 else None, layer)
    torch.cuda.synchronize()
    y_bits = host_bits(y)
    sel = slice(None) if rows is None else rows
    y64 = S.gemm_w4a4(qact[sel], ascales[:, sel], F.bf16_to_f64(lora_bits)[sel] if R > 0 else None,
                      d["qweight"], d["wscales"], d["wcscales"], d["wtscale"],
                      d["proj_up"] if R > 0 else None, d["bias"])
    got = y_bits[sel]
    err = S.normwise_rel_err(F.bf16_to_f64(got), y64)
    assert err <= TOL, err
    frac = within_ulps(got, y64, 1).mean()
    assert frac >= 0.999, frac
    return y_bits, err


@pytest.mark.parametrize("cfg", [
    dict(M=64, K=256, N=128, R=16, kind="tiny", seed=1001),
    dict(M=200, K=3840, N=384, R=128, kind="dit", seed=21),
    dict(M=1, K=256, N=16, R=16, kind="dit", seed=22),
    dict(M=63, K=16, N=100, R=16, kind="tiny", seed=23),
    dict(M=130, K=336, N=4100, R=32, kind="dit", seed=24),     # K % 64 != 0, ragged N
    dict(M=257, K=1024, N=257, R=0, kind="dit", seed=25),      # R = 0
    dict(M=96, K=10240, N=256, R=128, kind="swiglu", seed=26),
    dict(M=300, K=512, N=700, R=272, kind="dit", seed=27),      # rank in three passes (8 + 8 + 1 steps)
])
@pytest.mark.parametrize("packed", [False, True])
def test_gemm_parity(gpu_lib, cfg, packed):
    gemm_case(gpu_lib, cfg, packed=packed)


@pytest.mark.parametrize("packed", [False, True])
def test_gemm_wide_ragged_n(gpu_lib, packed):
    """N = 70000 (not a multiple of 32 * 5 * 2 = 320) with one row block: the packed
    path picks its 320-wide tiles here (more than 256 tiles of 256 columns), so the
    ragged last column block of that configuration is covered."""
    gemm_case(gpu_lib, dict(M=64, K=256, N=70000, R=16, kind="dit", seed=35), packed=packed)


def test_gemm_layouts_bit_identical(gpu_lib):
    cfg = dict(M=300, K=768, N=520, R=64, kind="dit", seed=31)
    a, _ = gemm_case(gpu_lib, cfg, packed=False)
    b, _ = gemm_case(gpu_lib, cfg, packed=True)
    assert np.array_equal(a, b)


def test_gemm_zero_weight_is_lowrank_plus_bias(gpu_lib):
    gemm_case(gpu_lib, dict(M=128, K=512, N=192, R=128, kind="dit", seed=32), zero_weight=True)


def test_gemm_no_bias(gpu_lib):
    gemm_case(gpu_lib, dict(M=128, K=512, N=192, R=16, kind="dit", seed=33), with_bias=False)


@pytest.mark.parametrize("packed", [False, True])
def test_gemm_full_ffn_shape_sampled_rows(gpu_lib, packed):
    """M=4096, K=3840, N=10240, R=128 (FFN w1 at 1024^2): the whole output on the GPU,
    checked against the oracle on 48 sampled rows (all columns)."""
    cfg = workloads.FFN_W1_1024
    rows = np.sort(np.random.default_rng(5).choice(cfg["M"], size=48, replace=False))
    rows[0], rows[-1] = 0, cfg["M"] - 1
    gemm_case(gpu_lib, cfg, packed=packed, rows=rows)


def test_gemm_deterministic(gpu_lib):
    cfg = dict(M=256, K=1024, N=512, R=128, kind="dit", seed=34)
    a, _ = gemm_case(gpu_lib, cfg)
    b, _ = gemm_case(gpu_lib, cfg)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("cfg", [
    dict(M=64, K=256, N=128, R=16, kind="tiny", seed=1001),
    dict(M=200, K=3840, N=384, R=128, kind="dit", seed=21),
    dict(M=130, K=336, N=4100, R=32, kind="dit", seed=24),
    dict(M=257, K=1024, N=257, R=0, kind="dit", seed=25),
    dict(M=300, K=512, N=700, R=272, kind="dit", seed=27),
    dict(M=33, K=64, N=40, R=16, kind="dit", seed=28),          # one panel: only the peeled iteration
    dict(M=70, K=128, N=96, R=16, kind="dit", seed=36),         # two panels: one loop pass, no refill
    dict(M=290, K=192, N=650, R=32, kind="dit", seed=37),       # three panels; partial column tile
    dict(M=40, K=80, N=64, R=0, kind="tiny", seed=38),          # two panels, the second K-ragged
])
def test_gemm_packed_activations(gpu_lib, cfg):
    """Packed activations (placed by the oracle's statement of the layout) through the
    LDS-free kernel: within tolerance of the oracle and bit-identical to the
    canonical-activation kernel on the same operands."""
    from oracle import repack as P
    d, layer, qact, ascales, lora_bits = _oracle_inputs(cfg, True, False)
    R = d["R"]
    pl = layer.packed()
    lora = dev_bf16(lora_bits) if R > 0 else None
    y_pk = gpu_lib.gemm_w4a4(dev_u8(P.repack(qact, ascales)), None, lora, pl, M=d["M"])
    y_can = gpu_lib.gemm_w4a4(dev_u8(qact), dev_u8(ascales), lora, pl)
    torch.cuda.synchronize()
    a, b = host_bits(y_pk), host_bits(y_can)
    assert np.array_equal(a, b)
    y64 = S.gemm_w4a4(qact, ascales, F.bf16_to_f64(lora_bits) if R > 0 else None, d["qweight"],
                      d["wscales"], d["wcscales"], d["wtscale"], d["proj_up"] if R > 0 else None, d["bias"])
    assert S.normwise_rel_err(F.bf16_to_f64(a), y64) <= TOL


@pytest.mark.parametrize("cfg", [
    dict(M=77, K=336, N=200, R=32, kind="dit", seed=41),        # K % 64 == 16: the last canonical row segment is half past K
    dict(M=300, K=1040, N=650, R=16, kind="dit", seed=42),
    dict(M=33, K=16, N=40, R=0, kind="tiny", seed=43),          # one 16-K block
])
def test_gemm_packed_activations_canonical_weight(gpu_lib, cfg):
    """Packed activations with the weight in its on-disk layout (read by the kernel without
    the load-time repack): bit-identical to the packed weight, and within the oracle's gate."""
    from oracle import repack as P
    d, layer, qact, ascales, lora_bits = _oracle_inputs(cfg, True, False)
    R = d["R"]
    qpk = dev_u8(P.repack(qact, ascales))
    lora = dev_bf16(lora_bits) if R > 0 else None
    y_c = gpu_lib.gemm_w4a4(qpk, None, lora, layer, M=d["M"])
    y_p = gpu_lib.gemm_w4a4(qpk, None, lora, layer.packed(), M=d["M"])
    torch.cuda.synchronize()
    a, b = host_bits(y_c), host_bits(y_p)
    assert np.array_equal(a, b)
    y64 = S.gemm_w4a4(qact, ascales, F.bf16_to_f64(lora_bits) if R > 0 else None, d["qweight"],
                      d["wscales"], d["wcscales"], d["wtscale"], d["proj_up"] if R > 0 else None, d["bias"])
    assert S.normwise_rel_err(F.bf16_to_f64(a), y64) <= TOL


def test_gemm_packed_full_ffn_shape_sampled_rows(gpu_lib):
    from oracle import repack as P
    cfg = workloads.FFN_W1_1024
    d, layer, qact, ascales, lora_bits = _oracle_inputs(cfg, True, False)
    y = gpu_lib.gemm_w4a4(dev_u8(P.repack(qact, ascales)), None, dev_bf16(lora_bits), layer.packed(),
                          M=d["M"])
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(6).choice(cfg["M"], size=40, replace=False))
    y64 = S.gemm_w4a4(qact[rows], ascales[:, rows], F.bf16_to_f64(lora_bits)[rows], d["qweight"],
                      d["wscales"], d["wcscales"], d["wtscale"], d["proj_up"], d["bias"])
    got = host_bits(y)[rows]
    assert S.normwise_rel_err(F.bf16_to_f64(got), y64) <= TOL
    assert within_ulps(got, y64, 1).mean() >= 0.999


@pytest.mark.parametrize("R", [0, 16])
@pytest.mark.parametrize("mode", ["canonical", "packed_weight", "packed_both"])
def test_gemm_output_rounding_bit_exact(gpu_lib, R, mode):
    """Operands chosen so that every fp32 quantity before the final bf16 cast is exact:
    unit block scales, wcscales = wtscale = 1, a residual of small dyadic bf16 values, and
    biases of 256, 1024, -512 or 0, so that y lands on many bf16 rounding ties (256 + an
    odd integer, 1024 + 4 mod 8, ...). The only rounding left is the cast, so the output
    must equal the oracle's round-to-nearest-even of its float64 value bit for bit."""
    rng = np.random.default_rng(4100 + R)
    M, K, N = 70, 64, 100
    qact = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    qweight = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    one = F.e4m3_encode(np.array([1.0]))[0]
    ascales = np.full((K // 16, M), one, dtype=np.uint8)
    wscales = np.full((K // 16, N), one, dtype=np.uint8)
    ones_n = F.f64_to_bf16(np.ones(N))
    bias = F.f64_to_bf16(rng.choice([256.0, 1024.0, -512.0, 0.0], size=N))
    lora = F.f64_to_bf16(rng.choice([0.0, 1.0, -1.0, 0.5, 2.0], size=(M, R))) if R else None
    proj_up = F.f64_to_bf16(rng.choice([0.0, 1.0, -0.5, 2.0], size=(N, R))) if R else None
    from bit_w4a4_quantized_quantize_amd import ops
    layer = ops.SVDQLinearWeights(
        N=N, K=K, weight=dev_u8(qweight), wscales=dev_u8(wscales), wcscales=dev_bf16(ones_n),
        wtscale=dev_bf16(F.f64_to_bf16(np.ones(1))), smooth=dev_bf16(F.f64_to_bf16(np.ones(K))),
        proj_down=dev_bf16(F.f64_to_bf16(np.zeros((K, R)))) if R else None,
        proj_up=dev_bf16(proj_up) if R else None, bias=dev_bf16(bias))
    if mode != "canonical":
        layer = layer.packed()
    if mode == "packed_both":      # the packed-activation kernel of the whole layer
        from oracle import repack as P
        y = gpu_lib.gemm_w4a4(dev_u8(P.repack(qact, ascales)), None, dev_bf16(lora) if R else None, layer, M=M)
    else:
        y = gpu_lib.gemm_w4a4(dev_u8(qact), dev_u8(ascales), dev_bf16(lora) if R else None, layer)
    torch.cuda.synchronize()
    y64 = S.gemm_w4a4(qact, ascales, F.bf16_to_f64(lora) if R else None, qweight, wscales, ones_n,
                      F.f64_to_bf16(np.ones(1)), proj_up, bias)
    ties = np.sum(np.abs(y64 / ulp_bf16(y64) % 1 - 0.5) < 1e-12)
    assert ties > 50, ties          # the case really exercises ties
    assert np.array_equal(host_bits(y), F.f64_to_bf16(y64))
