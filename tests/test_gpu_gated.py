"""GPU parity of the gated FFN step (w1 and w3 as one 2F-channel SVDQuant layer,
h = silu(y[:, :F]) * y[:, F:]) against the oracle's float64 evaluation.

Gate: normwise relative error <= 5e-3 on h. Also asserted per element, the bound
that follows from the arithmetic: one bf16 ulp of h, plus the layer's own fp32
error bound E (as in the linear tests: (K/16+2) 2^-24 |A||W||alpha| for the main
term, 2^-8 |lora||proj_up| for the bf16 lora_act, (K+R+2) 2^-24 (|x||proj_down|)|proj_up|
for its accumulation) propagated through the gate (|d silu| <= 1.1), plus 2^-20 |h|
for the fp32 silu evaluation.

Cases: tiny, ragged F (not a multiple of the 160-column half tile) and M, R = 0,
no bias, rank above one 128-wide chunk, and the 1024^2 FFN shape (F = 10240) on
sampled rows.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import formats as F
from oracle import svdq as S
from tests.gpu_util import dev_bf16, host_bits, make_layer, ulp_bf16

pytestmark = pytest.mark.gpu


def gated_case(ops, cfg, rows=None, with_bias=True):
    d, layer = make_layer(cfg, with_bias=with_bias)
    F_out = d["N"] // 2
    h = ops.linear_w4a4_gated(dev_bf16(d["x"]), layer.packed())
    torch.cuda.synchronize()
    h_bits = host_bits(h)
    sel = slice(None) if rows is None else rows
    R = d["R"]
    x = d["x"][sel]
    y64, _, qa, sa = S.linear_w4a4(x, d["smooth"], d["qweight"], d["wscales"], d["wcscales"], d["wtscale"],
                                   d["proj_down"] if R > 0 else None, d["proj_up"] if R > 0 else None,
                                   d["bias"])
    h64 = S.swiglu(y64, F_out)
    got = F.bf16_to_f64(h_bits[sel])
    err = S.normwise_rel_err(got, h64)
    assert err <= 5e-3, err
    alpha = np.abs(F.bf16_to_f64(d["wtscale"])[0] * F.bf16_to_f64(d["wcscales"]))
    E = (d["K"] / 16 + 2) * 2.0 ** -24 * (np.abs(S.dequant(qa, sa)) @ np.abs(S.dequant(d["qweight"], d["wscales"])).T * alpha)
    if R > 0:
        pu_abs = np.abs(F.bf16_to_f64(d["proj_up"])).T
        E = E + 2.0 ** -8 * (np.abs(S.lowrank_down(x, d["proj_down"])) @ pu_abs)
        E = E + (d["K"] + R + 2) * 2.0 ** -24 * ((np.abs(F.bf16_to_f64(x)) @ np.abs(F.bf16_to_f64(d["proj_down"]))) @ pu_abs)
    E = E + 2.0 ** -23 * np.abs(y64)
    gate, up = y64[:, :F_out], y64[:, F_out:]
    bound = (ulp_bf16(h64) + 1.1 * E[:, :F_out] * (np.abs(up) + E[:, F_out:])
             + np.abs(S.silu(gate)) * E[:, F_out:] + 2.0 ** -20 * np.abs(h64))
    bad = np.argwhere(np.abs(got - h64) > bound)
    assert bad.size == 0, f"{len(bad)} elements beyond the arithmetic bound, first {bad[:3].tolist()}"
    return h_bits, err


@pytest.mark.parametrize("cfg", [
    dict(M=64, K=256, N=2 * 128, R=16, kind="tiny", seed=71),
    dict(M=130, K=512, N=2 * 352, R=32, kind="dit", seed=72),      # F = 11 panels: partial last tile
    dict(M=77, K=336, N=2 * 96, R=0, kind="dit", seed=73),         # R = 0, K % 64 != 0
    dict(M=300, K=1024, N=2 * 640, R=272, kind="swiglu", seed=74), # rank in three passes
])
def test_gated_parity(gpu_lib, cfg):
    gated_case(gpu_lib, cfg)


def test_gated_no_bias(gpu_lib):
    gated_case(gpu_lib, dict(M=96, K=256, N=2 * 160, R=16, kind="dit", seed=75), with_bias=False)


def test_gated_full_ffn_shape_sampled_rows(gpu_lib):
    """w1 and w3 at 1024^2 as one layer: M = 4096, K = 3840, F = 10240, R = 128."""
    cfg = dict(M=4096, K=3840, N=2 * 10240, R=128, kind="dit", seed=1003)
    rows = np.sort(np.random.default_rng(76).choice(cfg["M"], size=24, replace=False))
    rows[0], rows[-1] = 0, cfg["M"] - 1
    gated_case(gpu_lib, cfg, rows=rows)


def test_gated_deterministic(gpu_lib):
    cfg = dict(M=128, K=512, N=2 * 320, R=64, kind="dit", seed=77)
    a, _ = gated_case(gpu_lib, cfg)
    b, _ = gated_case(gpu_lib, cfg)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# The gated step that also quantises h for w2 (svdq_gemm_w4a4_gated_quant)
# ---------------------------------------------------------------------------


def gated_quant_case(ops, cfg, w2_seed=81):
    """Returns (d, layer, h_bits, next_qact bytes, plain gated h bits, smooth2 bits)."""
    from oracle import repack as P
    from tests.test_gpu_quant import _unspecified_rows_mask
    d, layer = make_layer(cfg)
    packed = layer.packed()
    M, F_out = d["M"], d["N"] // 2
    _, sm2 = workloads.make_activation(8, F_out, kind="swiglu", seed=w2_seed)
    qpk, _, lora = ops.quantize_act(dev_bf16(d["x"]), packed.smooth, packed.proj_down, packed=True)
    h, q2 = ops.gemm_w4a4_gated_quant(qpk, lora, packed, M, dev_bf16(sm2))
    h_plain = ops.gemm_w4a4_gated(qpk, lora, packed, M)
    torch.cuda.synchronize()
    h_bits = host_bits(h)
    assert np.array_equal(h_bits, host_bits(h_plain)), "h differs from the plain gated step"
    got = q2.detach().cpu().numpy()
    q_ref, s_ref = S.quantize_act(h_bits, sm2)
    expect = P.repack(q_ref, s_ref)
    keep = ~_unspecified_rows_mask(M, F_out)
    bad = np.argwhere((got[: expect.size] != expect) & keep)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:4].ravel().tolist()}"
    return d, packed, h, q2, sm2


@pytest.mark.parametrize("cfg", [
    dict(M=64, K=256, N=2 * 128, R=16, kind="tiny", seed=78),
    dict(M=77, K=512, N=2 * 192, R=32, kind="dit", seed=79),       # ragged M, a partial column tile
    dict(M=300, K=1024, N=2 * 640, R=0, kind="swiglu", seed=80),   # R = 0
])
def test_gated_quant_codes_bit_exact(gpu_lib, cfg):
    """w2's codes and scales from the gated epilogue == the oracle's quantisation of the h
    the same call wrote (and h itself == the plain gated step's)."""
    gated_quant_case(gpu_lib, cfg)


def test_gated_quant_full_ffn_shape(gpu_lib):
    """F = 10240 at 1024^2: every code and scale of w2's [4096, 10240] input."""
    gated_quant_case(gpu_lib, dict(M=4096, K=3840, N=2 * 10240, R=128, kind="dit", seed=1003))


def test_ffn_block_through_quantising_gate(gpu_lib):
    """The whole FFN block by the fused path: gated step with w2's quantisation, w2's
    down-projection alone, then w2's GEMM on the packed codes; y against the oracle's
    w2 layer on the h the call wrote."""
    ops = gpu_lib
    cfg = dict(M=200, K=512, N=2 * 256, R=32, kind="dit", seed=82)
    d, packed, h, q2, sm2 = gated_quant_case(ops, cfg)
    M, F_out = d["M"], d["N"] // 2
    d2 = workloads.make_linear(M, F_out, 384, 32, kind="swiglu", seed=83)
    qw2, ws2 = S.quantize_weight(d2["W"], d2["wcscales"], d2["wtscale"])
    from bit_w4a4_quantized_quantize_amd.ops import SVDQLinearWeights
    w2 = SVDQLinearWeights(N=384, K=F_out, weight=torch.from_numpy(qw2).cuda(), wscales=torch.from_numpy(ws2).cuda(),
                           wcscales=dev_bf16(d2["wcscales"]), wtscale=dev_bf16(d2["wtscale"]), smooth=dev_bf16(sm2),
                           proj_down=dev_bf16(d2["proj_down"]), proj_up=dev_bf16(d2["proj_up"]),
                           bias=dev_bf16(d2["bias"])).packed()
    lora2 = ops.lowrank_down(h, w2.proj_down)
    y = ops.gemm_w4a4(q2, None, lora2, w2, M=M)
    y_ref_path = ops.linear_w4a4(h, w2)
    torch.cuda.synchronize()
    h_bits = host_bits(h)
    y64, _, _, _ = S.linear_w4a4(h_bits, sm2, qw2, ws2, d2["wcscales"], d2["wtscale"], d2["proj_down"],
                                 d2["proj_up"], d2["bias"])
    err = S.normwise_rel_err(F.bf16_to_f64(host_bits(y)), y64)
    assert err <= 5e-3, err
    # the two paths differ only in how lora_act's fp32 sums are associated
    diff = S.normwise_rel_err(F.bf16_to_f64(host_bits(y)), F.bf16_to_f64(host_bits(y_ref_path)))
    assert diff <= 2e-3, diff


def test_gated_quant_needs_f_multiple_of_64(gpu_lib):
    ops = gpu_lib
    d, layer = make_layer(dict(M=64, K=256, N=2 * 96, R=16, kind="tiny", seed=84))
    packed = layer.packed()
    qpk, _, lora = ops.quantize_act(dev_bf16(d["x"]), packed.smooth, packed.proj_down, packed=True)
    with pytest.raises(ops.SvdqError, match="multiple of 64"):
        ops.gemm_w4a4_gated_quant(qpk, lora, packed, 64, torch.ones(96, dtype=torch.bfloat16, device="cuda"))
