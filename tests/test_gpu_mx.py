"""GPU parity of the MXFP4 datatype variant (svdq_quantize_act_mxfp4,
svdq_reround_weight_mxfp4, svdq_gemm_mxfp4, svdq_linear_mxfp4) against
oracle/mx.py: codes and E8M0 scales bit-exact; y within a normwise 5e-3 of the
variant's float64 evaluation and within the elementwise bound of its arithmetic
(one bf16 ulp, plus (K + 2) 2^-24 of |a| |w|^T |alpha| for the fp32 accumulation
of exact E2M1 x E2M1 x 2^k products, plus the low-rank terms of the NVFP4
layer's bound). The variant's distance from the pages' NVFP4 result is
measured too: it is an out-of-tolerance speed point, not the layer."""

import numpy as np
import pytest
import torch

import workloads
from oracle import formats as F
from oracle import mx as X
from oracle import svdq as S
from tests.gpu_util import dev_bf16, host_bits, host_u8, make_layer

pytestmark = pytest.mark.gpu


def unpack_mx_codes(buf, rows, K):
    """MX code buffer (layout of include/svdq.h) -> codes [rows, K]."""
    P = (rows + 31) // 32
    b = np.asarray(buf, dtype=np.uint8)[: (K // 64) * P * 1024].reshape(K // 64, P, 2, 32, 16)
    nib = np.stack([b & 15, b >> 4], axis=-1)              # [s, p, h, c, j, t]
    codes = nib.transpose(1, 3, 0, 2, 4, 5).reshape(P * 32, K)
    return codes[:rows]


def unpack_mx_scales(buf, rows, K):
    P = (rows + 31) // 32
    return np.asarray(buf, dtype=np.uint8)[: (K // 32) * P * 32].reshape(K // 32, P * 32).T[:rows]


@pytest.mark.parametrize("M,K", [(64, 128), (300, 256), (1, 384), (4096, 3840)])
def test_activation_mx_quant_bit_exact(gpu_lib, M, K):
    x, sm = workloads.make_activation(M, K, kind="dit", seed=M + K)
    codes, scales = gpu_lib.quantize_act_mxfp4(dev_bf16(x), dev_bf16(sm))
    torch.cuda.synchronize()
    ca, sa = X.quantize_act_mx(x, sm)
    got_c = unpack_mx_codes(host_u8(codes), M, K)
    got_s = unpack_mx_scales(host_u8(scales), M, K)
    assert np.array_equal(got_s, sa)
    assert np.array_equal(got_c, ca)
    P = (M + 31) // 32
    if P * 32 > M:   # padding rows: zero codes, scale byte 0
        assert not unpack_mx_codes(host_u8(codes), P * 32, K)[M:].any()
        assert not unpack_mx_scales(host_u8(scales), P * 32, K)[M:].any()


@pytest.mark.parametrize("N,K,kind", [(128, 256, "tiny"), (200, 384, "dit"), (10240, 3840, "dit")])
def test_weight_reround_bit_exact(gpu_lib, N, K, kind):
    d, layer = make_layer(dict(M=4, K=K, N=N, R=0, kind=kind, seed=N + K))
    codes, scales = gpu_lib.reround_weight_mxfp4(layer)
    torch.cuda.synchronize()
    cw, sw = X.reround_weight_mx(d["qweight"], d["wscales"])
    assert np.array_equal(unpack_mx_scales(host_u8(scales), N, K), sw)
    assert np.array_equal(unpack_mx_codes(host_u8(codes), N, K), cw)


def check_layer(gpu_lib, cfg, rows=None, with_bias=True):
    d, layer = make_layer(cfg, with_bias=with_bias)
    wc, ws = gpu_lib.reround_weight_mxfp4(layer)
    y = gpu_lib.linear_mxfp4(dev_bf16(d["x"]), layer, wc, ws)
    torch.cuda.synchronize()
    sel = slice(None) if rows is None else rows
    R = d["R"]
    x = d["x"][sel]
    y64, _, ac, asc, cw, sw = X.linear_mxfp4(x, d["smooth"], d["qweight"], d["wscales"], d["wcscales"], d["wtscale"],
                                             d["proj_down"] if R else None, d["proj_up"] if R else None, d["bias"])
    got = F.bf16_to_f64(host_bits(y)[sel])
    err = S.normwise_rel_err(got, y64)
    assert err <= 5e-3, err
    alpha = np.abs(F.bf16_to_f64(d["wtscale"])[0] * F.bf16_to_f64(d["wcscales"]))
    main_abs = np.abs(X.mx_dequant(ac, asc)) @ np.abs(X.mx_dequant(cw, sw)).T * alpha
    from tests.gpu_util import ulp_bf16
    bound = ulp_bf16(y64) + (d["K"] + 2) * 2.0 ** -24 * main_abs
    if R:
        pu_abs = np.abs(F.bf16_to_f64(d["proj_up"])).T
        lr_abs = np.abs(S.lowrank_down(x, d["proj_down"])) @ pu_abs
        lr_acc = (np.abs(F.bf16_to_f64(x)) @ np.abs(F.bf16_to_f64(d["proj_down"]))) @ pu_abs
        bound = bound + 2.0 ** -8 * lr_abs + (d["K"] + R + 2) * 2.0 ** -24 * lr_acc
    bad = np.argwhere(np.abs(got - y64) > bound)
    assert bad.size == 0, f"{len(bad)} elements beyond the bound, first {bad[:3].tolist()}"
    # distance of the variant from the pages' NVFP4 layer on the same inputs
    y_nv, _, _, _ = S.linear_w4a4(x, d["smooth"], d["qweight"], d["wscales"], d["wcscales"], d["wtscale"],
                                  d["proj_down"] if R else None, d["proj_up"] if R else None, d["bias"])
    return S.normwise_rel_err(y64, y_nv)


@pytest.mark.parametrize("cfg,bias", [
    (dict(M=64, K=256, N=128, R=16, kind="tiny", seed=1), True),
    (dict(M=300, K=384, N=200, R=32, kind="dit", seed=2), True),     # ragged M and N
    (dict(M=77, K=128, N=72, R=0, kind="dit", seed=3), False),       # one panel, no residual, no bias
    (dict(M=513, K=1024, N=640, R=128, kind="swiglu", seed=4), True),
    (dict(M=96, K=128, N=330, R=48, kind="dit", seed=5), True),      # odd R steps; residual panels in the prologue
    (dict(M=200, K=512, N=256, R=80, kind="dit", seed=6), True),     # odd R steps over three residual panels
    (dict(M=64, K=128, N=320, R=128, kind="dit", seed=7), False),    # one matrix panel, four residual panels
])
def test_variant_layer_matches_oracle(gpu_lib, cfg, bias):
    dist = check_layer(gpu_lib, cfg, with_bias=bias)
    assert dist < 0.2   # an out-of-tolerance variant: a few percent from the NVFP4 result


def test_variant_layer_full_size_sampled(gpu_lib):
    rows = np.array([0, 255, 256, 2049, 4095])
    dist = check_layer(gpu_lib, dict(workloads.FFN_W1_1024), rows=rows)
    assert dist < 0.2


def test_variant_layer_wide_tile_ragged_sampled(gpu_lib):
    # M = 4000, N = 4200: 208 tiles of 256 x 320 (one round on 256 CUs) against 272 of
    # 256 x 256, so the launcher takes the 320-wide tile; both edges are ragged
    # (4000 = 15 x 256 + 160 rows, 4200 = 13 x 320 + 40 columns)
    rows = np.array([0, 255, 256, 3839, 3840, 3999])
    dist = check_layer(gpu_lib, dict(M=4000, K=256, N=4200, R=32, kind="dit", seed=8), with_bias=True, rows=rows)
    assert dist < 0.2


def _lora_within_bound(got_bits, x_bits, pd_bits, K):
    got = F.bf16_to_f64(got_bits)
    ref = S.lowrank_down(x_bits, pd_bits)
    scale = np.abs(F.bf16_to_f64(x_bits)) @ np.abs(F.bf16_to_f64(pd_bits))
    tol = np.abs(ref) * 2.0 ** -8 + scale * K * 2.0 ** -23 + 1e-30
    assert not np.any(np.abs(got - ref) > tol)


@pytest.mark.parametrize("M,K,R", [
    (64, 128, 16), (300, 256, 32), (1, 384, 128), (130, 1024, 256),   # R above one 128-wide chunk
    (2049, 1280, 128), (4096, 3840, 128),
])
def test_fused_quant_down_mx(gpu_lib, M, K, R):
    """svdq_quantize_act with the MXFP4 layout: codes and scales bit for bit those of the
    standalone MX quantiser (padding rows included) and of the oracle, and lora_act within
    the down-projection's bound, from one pass over x."""
    d = workloads.make_linear(M, K, 16, R, kind="dit", seed=M + K + R, with_bias=False)
    x, sm, pd = dev_bf16(d["x"]), dev_bf16(d["smooth"]), dev_bf16(d["proj_down"])
    codes, scales, lora = gpu_lib.quantize_act(x, sm, pd, mx=True)
    c1, s1 = gpu_lib.quantize_act_mxfp4(x, sm)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(codes), host_u8(c1))
    assert np.array_equal(host_u8(scales), host_u8(s1))
    ca, sa = X.quantize_act_mx(d["x"], d["smooth"])
    assert np.array_equal(unpack_mx_scales(host_u8(scales), M, K), sa)
    assert np.array_equal(unpack_mx_codes(host_u8(codes), M, K), ca)
    _lora_within_bound(host_bits(lora), d["x"], d["proj_down"], K)


def test_gemm_entry_matches_linear(gpu_lib):
    d, layer = make_layer(dict(M=128, K=256, N=96, R=16, kind="dit", seed=9))
    wc, ws = gpu_lib.reround_weight_mxfp4(layer)
    x = dev_bf16(d["x"])
    ac, asc = gpu_lib.quantize_act_mxfp4(x, layer.smooth)
    _, _, lora = gpu_lib.quantize_act(x, layer.smooth, layer.proj_down)
    y1 = gpu_lib.gemm_mxfp4(ac, asc, lora, wc, ws, layer, 128)
    y2 = gpu_lib.linear_mxfp4(x, layer, wc, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_gemm_entry_on_fused_operands_matches_linear(gpu_lib):
    """The layer equals the GEMM entry point on the one-pass quantiser's operands, bit for bit."""
    d, layer = make_layer(dict(M=300, K=1024, N=200, R=128, kind="dit", seed=10))
    wc, ws = gpu_lib.reround_weight_mxfp4(layer)
    x = dev_bf16(d["x"])
    ac, asc, lora = gpu_lib.quantize_act(x, layer.smooth, layer.proj_down, mx=True)
    y1 = gpu_lib.gemm_mxfp4(ac, asc, lora, wc, ws, layer, 300)
    y2 = gpu_lib.linear_mxfp4(x, layer, wc, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
