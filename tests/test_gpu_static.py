"""GPU parity of the static-activation-scale variant (svdq_calibrate_act_gscale,
svdq_quantize_act_static, svdq_linear_w4a4_static) against the oracle's
calibrate_gscale / quantize_act_static / linear_w4a4_static.

Codes, block scales and the calibrated global scale are bit-exact; the layer output is
within the normwise 5e-3 gate and the per-element bound of the arithmetic (the global
scale multiplies alpha exactly). Cases: calibrated scales from another seeded batch,
non-power-of-two and very small scales (saturating blocks), g = 1 (the dynamic rule),
every e4m3 scale with E2M1 ties and e4m3-midpoint block maxima, both activation layouts,
R = 0 and 128, the full FFN w1 shape.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import formats as F
from oracle import repack as P
from oracle import svdq as S
from tests.gpu_util import dev_bf16, host_bits, host_u8, make_layer, ulp_bf16

pytestmark = pytest.mark.gpu


def g_bits(v):
    return F.f64_to_bf16(np.array([v]))


@pytest.mark.parametrize("M,K,kind,seed", [
    (64, 256, "tiny", 1001),
    (4096, 3840, "dit", 1003),
    (96, 10240, "swiglu", 1023),
    (5, 48, "dit", 7),
])
def test_calibration_matches_oracle(gpu_lib, M, K, kind, seed):
    x, sm = workloads.make_activation(M, K, kind=kind, seed=seed)
    g = gpu_lib.calibrate_act_gscale(dev_bf16(x), dev_bf16(sm))
    torch.cuda.synchronize()
    assert host_bits(g)[0] == S.calibrate_gscale(x, sm)[0]


def test_calibration_of_zeros_is_one(gpu_lib):
    x = torch.zeros(40, 64, dtype=torch.bfloat16, device="cuda")
    sm = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    g = gpu_lib.calibrate_act_gscale(x, sm)
    assert float(g.float().item()) == 1.0


def _quant_static(ops, x_bits, sm_bits, gb, packed=False, pd_bits=None):
    M, K = x_bits.shape
    out = ops.quantize_act_static(dev_bf16(x_bits), dev_bf16(sm_bits), dev_bf16(gb),
                                  dev_bf16(pd_bits) if pd_bits is not None else None, packed=packed)
    torch.cuda.synchronize()
    return out


G_CHOICES = ["calibrated", 0.0123, 3.7e-4, 1.0]


def _g_for(choice, M, K, kind, seed, sm):
    if choice == "calibrated":
        xc, _ = workloads.make_activation(M, K, kind=kind, seed=seed + 1000)
        return S.calibrate_gscale(xc, sm)
    return g_bits(choice)


@pytest.mark.parametrize("M,K,kind,seed", [(64, 256, "tiny", 1001), (300, 3840, "dit", 61),
                                           (96, 10240, "swiglu", 62), (2049, 1040, "dit", 69)])
@pytest.mark.parametrize("gc", G_CHOICES)
@pytest.mark.parametrize("R", [0, 128])
def test_static_quant_canonical_bit_exact(gpu_lib, M, K, kind, seed, gc, R):
    d = workloads.make_linear(M, K, 16, R, kind=kind, seed=seed, with_bias=False)
    gb = _g_for(gc, M, K, kind, seed, d["smooth"])
    q, s, lora = _quant_static(gpu_lib, d["x"], d["smooth"], gb, pd_bits=d["proj_down"] if R > 0 else None)
    q_ref, s_ref = S.quantize_act_static(d["x"], d["smooth"], gb)
    assert np.array_equal(host_u8(s), s_ref)
    assert np.array_equal(host_u8(q), q_ref)
    if gc == 1.0:
        qd, sd = S.quantize_act(d["x"], d["smooth"])
        assert np.array_equal(host_u8(q), qd) and np.array_equal(host_u8(s), sd)


@pytest.mark.parametrize("M,K,R,seed", [(77, 336, 32, 63), (600, 3840, 128, 64), (130, 1024, 0, 65),
                                         (4096, 1280, 128, 68)])   # split-free fused kernel
@pytest.mark.parametrize("gc", ["calibrated", 3.7e-4])
def test_static_quant_packed_bit_exact(gpu_lib, M, K, R, seed, gc):
    from tests.test_gpu_quant import _unspecified_rows_mask
    d = workloads.make_linear(M, K, 16, R, kind="dit", seed=seed, with_bias=False)
    gb = _g_for(gc, M, K, "dit", seed, d["smooth"])
    buf, asc, _ = _quant_static(gpu_lib, d["x"], d["smooth"], gb, packed=True,
                                pd_bits=d["proj_down"] if R > 0 else None)
    assert asc is None
    got = host_u8(buf)
    q_ref, s_ref = S.quantize_act_static(d["x"], d["smooth"], gb)
    expect = P.repack(q_ref, s_ref)
    keep = ~_unspecified_rows_mask(M, K)
    bad = np.argwhere((got != expect) & keep)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:4].ravel().tolist()}"


def test_static_every_scale_with_ties(gpu_lib):
    """smooth = g, so v = x * g exactly. For each nonzero e4m3 scale s: a block with
    x = 6 s (scale code exactly s) and the E2M1 midpoints times s (code ties); and a block
    whose maximum is 6 tau for an e4m3 rounding midpoint tau (a scale tie)."""
    g = 0.0234375                       # 3/128: two significant bits
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    grid = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    rows = []
    for code in range(1, 0x7E):
        s = grid[code]
        blk = np.zeros(32)
        blk[0] = 6 * s
        blk[1:8] = mids * s
        blk[8:15] = -mids * s
        tau = 0.5 * (grid[code] + grid[code + 1])
        blk[16] = 6 * tau
        blk[17:24] = mids * tau
        rows.append(blk)
    x = np.array(rows)
    xb = F.f64_to_bf16(x)
    assert np.array_equal(F.bf16_to_f64(xb), x), "test values must be bf16-exact"
    sm = F.f64_to_bf16(np.full(32, g))
    gb = g_bits(g)
    q, s, _ = _quant_static(gpu_lib, xb, sm, gb)
    q_ref, s_ref = S.quantize_act_static(xb, sm, gb)
    assert np.array_equal(host_u8(s), s_ref)
    assert np.array_equal(host_u8(q), q_ref)


def static_linear_case(ops, cfg, gc, packed, rows=None):
    d, layer = make_layer(cfg)
    if packed:
        layer = layer.packed()
    gb = _g_for(gc, cfg["M"], cfg["K"], cfg["kind"], cfg["seed"], d["smooth"])
    y = ops.linear_w4a4_static(dev_bf16(d["x"]), layer, dev_bf16(gb))
    torch.cuda.synchronize()
    sel = slice(None) if rows is None else rows
    R = d["R"]
    y64, _, qa, sa = S.linear_w4a4_static(d["x"][sel], d["smooth"], gb, d["qweight"], d["wscales"],
                                          d["wcscales"], d["wtscale"], d["proj_down"] if R > 0 else None,
                                          d["proj_up"] if R > 0 else None, d["bias"])
    got = F.bf16_to_f64(host_bits(y)[sel])
    err = S.normwise_rel_err(got, y64)
    assert err <= 5e-3, err
    g = F.bf16_to_f64(gb)[0]
    alpha = np.abs(g * F.bf16_to_f64(d["wtscale"])[0] * F.bf16_to_f64(d["wcscales"]))
    main_abs = np.abs(S.dequant(qa, sa)) @ np.abs(S.dequant(d["qweight"], d["wscales"])).T * alpha
    bound = ulp_bf16(y64) + (d["K"] / 16 + 3) * 2.0 ** -24 * main_abs
    if R > 0:
        x = d["x"][sel]
        pu_abs = np.abs(F.bf16_to_f64(d["proj_up"])).T
        lr_abs = np.abs(S.lowrank_down(x, d["proj_down"])) @ pu_abs
        lr_acc = (np.abs(F.bf16_to_f64(x)) @ np.abs(F.bf16_to_f64(d["proj_down"]))) @ pu_abs
        bound = bound + 2.0 ** -8 * lr_abs + (d["K"] + R + 2) * 2.0 ** -24 * lr_acc
    bad = np.argwhere(np.abs(got - y64) > bound)
    assert bad.size == 0, f"{len(bad)} elements beyond the arithmetic bound, first {bad[:3].tolist()}"
    return d, layer, y


@pytest.mark.parametrize("cfg", [workloads.TINY, dict(M=512, K=3840, N=1152, R=128, kind="dit", seed=66),
                                 dict(M=77, K=1024, N=300, R=0, kind="dit", seed=67)])
@pytest.mark.parametrize("gc", ["calibrated", 0.0123])
@pytest.mark.parametrize("packed", [False, True])
def test_static_linear_parity(gpu_lib, cfg, gc, packed):
    static_linear_case(gpu_lib, cfg, gc, packed)


@pytest.mark.parametrize("packed", [False, True])
def test_static_linear_g_one_equals_dynamic_layer(gpu_lib, packed):
    cfg = dict(M=300, K=1024, N=640, R=64, kind="dit", seed=68)
    d, layer = make_layer(cfg)
    if packed:
        layer = layer.packed()
    x = dev_bf16(d["x"])
    ys = gpu_lib.linear_w4a4_static(x, layer, dev_bf16(g_bits(1.0)))
    yd = gpu_lib.linear_w4a4(x, layer)
    torch.cuda.synchronize()
    assert torch.equal(ys.view(torch.int16), yd.view(torch.int16))


def test_static_linear_full_ffn_shape_sampled_rows(gpu_lib):
    cfg = workloads.FFN_W1_1024
    rows = np.sort(np.random.default_rng(19).choice(cfg["M"], size=24, replace=False))
    static_linear_case(gpu_lib, cfg, "calibrated", packed=True, rows=rows)
