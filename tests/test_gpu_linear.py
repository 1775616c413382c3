"""GPU parity of the whole layer svdq_linear_w4a4 against the oracle's float64 evaluation of
y = scaled_mma(quant(x*smooth), qweight, ascales, wscales)*wtscale*wcscales
    + (x @ proj_down) @ proj_up^T + bias
(model card "nunchaku-z-image-turbo-svdq", section "What's stored on disk").
Gate: normwise relative error <= 5e-3 on the bf16 output. Also asserted, for every
element, the bound that follows from the arithmetic: a bf16 ulp of output
rounding (one ulp, as the fp32 value may cross a binade), plus 2^-8 of
|lora| @ |proj_up|^T (lora_act is rounded to bf16) and (K + R + 2) * 2^-24 of
(|x| @ |proj_down|) @ |proj_up|^T (its fp32 accumulation), plus (K/16 + 2) * 2^-24 of |A| @ |W|^T * |alpha| for the fp32
accumulation of exact per-block products."""

import numpy as np
import pytest
import torch

import workloads
from oracle import formats as F
from oracle import svdq as S
from tests.gpu_util import dev_bf16, host_bits, make_layer, ulp_bf16

pytestmark = pytest.mark.gpu


def linear_case(ops, cfg, packed=False, rows=None, with_bias=True):
    d, layer = make_layer(cfg, with_bias=with_bias)
    if packed:
        layer = layer.packed()
    y = ops.linear_w4a4(dev_bf16(d["x"]), layer)
    torch.cuda.synchronize()
    y_bits = host_bits(y)
    sel = slice(None) if rows is None else rows
    R = d["R"]
    y64, _, _, _ = S.linear_w4a4(d["x"][sel], d["smooth"], d["qweight"], d["wscales"], d["wcscales"],
                                 d["wtscale"], d["proj_down"] if R > 0 else None,
                                 d["proj_up"] if R > 0 else None, d["bias"])
    err = S.normwise_rel_err(F.bf16_to_f64(y_bits[sel]), y64)
    assert err <= 5e-3, err
    got = F.bf16_to_f64(y_bits[sel])
    x = d["x"][sel]
    qa, sa = S.quantize_act(x, d["smooth"])
    alpha = np.abs(F.bf16_to_f64(d["wtscale"])[0] * F.bf16_to_f64(d["wcscales"]))
    main_abs = np.abs(S.dequant(qa, sa)) @ np.abs(S.dequant(d["qweight"], d["wscales"])).T * alpha
    bound = ulp_bf16(y64) + (d["K"] / 16 + 2) * 2.0 ** -24 * main_abs
    if R > 0:
        pu_abs = np.abs(F.bf16_to_f64(d["proj_up"])).T
        lr_abs = np.abs(S.lowrank_down(x, d["proj_down"])) @ pu_abs
        lr_acc = (np.abs(F.bf16_to_f64(x)) @ np.abs(F.bf16_to_f64(d["proj_down"]))) @ pu_abs
        bound = bound + 2.0 ** -8 * lr_abs + (d["K"] + R + 2) * 2.0 ** -24 * lr_acc
    bad = np.argwhere(np.abs(got - y64) > bound)
    assert bad.size == 0, f"{len(bad)} elements beyond the arithmetic bound, first {bad[:3].tolist()}"
    return y_bits, err


@pytest.mark.parametrize("cfg", [
    workloads.TINY,
    dict(M=512, K=3840, N=1152, R=128, kind="dit", seed=41),
    dict(M=77, K=1024, N=300, R=0, kind="dit", seed=42),
    dict(M=129, K=2048, N=640, R=128, kind="swiglu", seed=43),
])
@pytest.mark.parametrize("packed", [False, True])
def test_linear_parity(gpu_lib, cfg, packed):
    linear_case(gpu_lib, cfg, packed=packed)


def test_linear_full_ffn_shape_sampled_rows(gpu_lib):
    cfg = workloads.FFN_W1_1024
    rows = np.sort(np.random.default_rng(9).choice(cfg["M"], size=32, replace=False))
    linear_case(gpu_lib, cfg, packed=True, rows=rows)


@pytest.mark.parametrize("name,cfg", [
    ("qkv_1024", workloads.QKV_1024),
    ("w2_1024", workloads.FFN_W2_1024),
    ("qkv_2048px", workloads.LAYERS_2048["qkv"]),
    ("out_2048px", workloads.LAYERS_2048["out"]),
    ("w2_2048px", workloads.LAYERS_2048["w2"]),
    ("qkv_1024_tp8", workloads.SHARDS_TP8_1024["qkv"]),
    ("w1_1024_tp8", workloads.SHARDS_TP8_1024["w1"]),
    ("w2_1024_tp8", workloads.SHARDS_TP8_1024["w2"]),
])
def test_linear_full_size_sampled_rows(gpu_lib, name, cfg):
    """The other full-size layers (fused QKV N = 11520; w2 with K = 10240 on SwiGLU-like
    inputs; the 2048px token count M = 16896; one GPU's share of the 1024^2 layers under
    8-way tensor parallelism, whose GEMMs take the 128-row tiles and whose w2 share
    (K = 1280) takes the split-free quantiser), whole output computed with packed weights
    as the layer runs, 24 sampled rows checked against the oracle."""
    rows = np.sort(np.random.default_rng(cfg["seed"]).choice(cfg["M"], size=24, replace=False))
    rows[0], rows[-1] = 0, cfg["M"] - 1
    linear_case(gpu_lib, cfg, packed=True, rows=rows)


def test_linear_workspace_reuse_and_smaller_second_call(gpu_lib):
    """The same workspace serves a large call then a smaller one (no stale state)."""
    cfg1 = dict(M=600, K=1024, N=256, R=128, kind="dit", seed=44)
    cfg2 = dict(M=40, K=1024, N=256, R=128, kind="dit", seed=45)
    d1, l1 = make_layer(cfg1)
    ws = torch.empty(gpu_lib.linear_workspace_bytes(600, 256, 1024, 128), dtype=torch.uint8, device="cuda")
    y1 = gpu_lib.linear_w4a4(dev_bf16(d1["x"]), l1, workspace=ws)
    d2, l2 = make_layer(cfg2)
    y2 = gpu_lib.linear_w4a4(dev_bf16(d2["x"]), l2, workspace=ws)
    torch.cuda.synchronize()
    for d, y in ((d1, y1), (d2, y2)):
        y64, _, _, _ = S.linear_w4a4(d["x"], d["smooth"], d["qweight"], d["wscales"], d["wcscales"],
                                     d["wtscale"], d["proj_down"], d["proj_up"], d["bias"])
        assert S.normwise_rel_err(F.bf16_to_f64(host_bits(y)), y64) <= 5e-3
