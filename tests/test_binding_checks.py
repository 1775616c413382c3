"""The Python binding's argument checks, on any host: every tensor handed to the C ABI
(which sees only raw pointers) is checked against the problem sizes first, so a
mis-sized tensor raises ValueError before any launch.

Tensors here live on the CPU. The binding checks dtype and shape before the device,
so a size mistake is reported as such; a correctly sized CPU tensor is then refused
as "must be a GPU tensor". Either way nothing reaches the library's compute calls.
"""

import pytest
import torch

from bit_w4a4_quantized_quantize_amd import ops

M, K, N, R = 64, 256, 96, 16
bf, u8 = torch.bfloat16, torch.uint8


def layer(packed=False, **over):
    L = ops._lib.lib()
    t = dict(
        weight=torch.zeros(L.svdq_repack_weight_bytes(N, K), dtype=u8) if packed else torch.zeros(N, K // 2, dtype=u8),
        wscales=None if packed else torch.zeros(K // 16, N, dtype=u8),
        wcscales=torch.zeros(N, dtype=bf), wtscale=torch.zeros(1, dtype=bf), smooth=torch.zeros(K, dtype=bf),
        proj_down=torch.zeros(K, R, dtype=bf), proj_up=torch.zeros(N, R, dtype=bf), bias=torch.zeros(N, dtype=bf))
    t.update(over)
    return ops.SVDQLinearWeights(N=N, K=K, layout=ops.WEIGHT_PACKED if packed else ops.WEIGHT_CANONICAL, **t)


@pytest.mark.parametrize("field,bad", [
    ("weight", torch.zeros(N, K // 2 + 1, dtype=u8)),
    ("wscales", torch.zeros(K // 16, N - 1, dtype=u8)),
    ("wcscales", torch.zeros(N + 1, dtype=bf)),
    ("wtscale", torch.zeros(2, dtype=bf)),
    ("smooth", torch.zeros(K - 16, dtype=bf)),
    ("proj_down", torch.zeros(K, R + 16, dtype=bf)),
    ("proj_up", torch.zeros(N - 1, R, dtype=bf)),
    ("bias", torch.zeros(N - 1, dtype=bf)),
])
def test_layer_tensor_shapes(field, bad):
    w = layer(**{field: bad})
    x = torch.zeros(M, K, dtype=bf)
    with pytest.raises(ValueError, match="must have shape"):
        ops.linear_w4a4(x, w)


def test_packed_weight_too_small():
    w = layer(packed=True, weight=torch.zeros(100, dtype=u8))
    with pytest.raises(ValueError, match="at least"):
        ops.linear_w4a4(torch.zeros(M, K, dtype=bf), w)


def test_packed_weight_with_wscales_refused():
    w = layer(packed=True, wscales=torch.zeros(K // 16, N, dtype=u8))
    with pytest.raises(ValueError, match="must be None"):
        ops.linear_w4a4(torch.zeros(M, K, dtype=bf), w)


def test_linear_output_and_workspace():
    w = layer()
    x = torch.zeros(M, K, dtype=bf)
    with pytest.raises(ValueError, match="y must have shape"):
        ops.linear_w4a4(x, w, y=torch.zeros(M, N + 1, dtype=bf))
    with pytest.raises(ValueError, match="y must be torch.bfloat16"):
        ops.linear_w4a4(x, w, y=torch.zeros(M, N, dtype=torch.float16))
    with pytest.raises(ValueError, match="x has K"):
        ops.linear_w4a4(torch.zeros(M, K + 16, dtype=bf), w)
    need = ops.linear_workspace_bytes(M, N, K, R)
    with pytest.raises(ValueError, match="workspace has"):
        ops.linear_w4a4(x, w, y=torch.zeros(M, N, dtype=bf), workspace=torch.zeros(need - 1, dtype=u8))
    # everything sized right: only the device is wrong
    with pytest.raises(ValueError, match="GPU tensor"):
        ops.linear_w4a4(x, w, y=torch.zeros(M, N, dtype=bf), workspace=torch.zeros(need, dtype=u8))


def test_quantize_act_outputs():
    x = torch.zeros(M, K, dtype=bf)
    sm = torch.zeros(K, dtype=bf)
    pd = torch.zeros(K, R, dtype=bf)
    with pytest.raises(ValueError, match="smooth must have shape"):
        ops.quantize_act(x, torch.zeros(K + 16, dtype=bf))
    with pytest.raises(ValueError, match="proj_down must have shape"):
        ops.quantize_act(x, sm, torch.zeros(K - 16, R, dtype=bf))
    with pytest.raises(ValueError, match="qact must have shape"):
        ops.quantize_act(x, sm, qact=torch.zeros(M, K // 2 - 1, dtype=u8))
    with pytest.raises(ValueError, match="ascales must have shape"):
        ops.quantize_act(x, sm, ascales=torch.zeros(K // 16, M + 1, dtype=u8))
    with pytest.raises(ValueError, match="lora_act must have shape"):
        ops.quantize_act(x, sm, pd, lora_act=torch.zeros(M, R + 1, dtype=bf))
    nbytes = ops._lib.lib().svdq_packed_act_bytes(M, K)
    with pytest.raises(ValueError, match="at least"):
        ops.quantize_act(x, sm, pd, qact=torch.zeros(nbytes - 16, dtype=u8), packed=True)
    with pytest.raises(ValueError, match="must be None"):
        ops.quantize_act(x, sm, pd, qact=torch.zeros(nbytes, dtype=u8), ascales=torch.zeros(1, dtype=u8),
                         packed=True)
    need = ops.quantize_act_workspace_bytes(M, K, R)
    if need > 0:
        with pytest.raises(ValueError, match="at least"):
            ops.quantize_act(x, sm, pd, workspace=torch.zeros(need - 1, dtype=u8))
    with pytest.raises(ValueError, match="multiple of 16"):
        ops.quantize_act(torch.zeros(M, 40, dtype=bf), torch.zeros(40, dtype=bf))


def test_gemm_operands():
    w = layer()
    qact = torch.zeros(M, K // 2, dtype=u8)
    asc = torch.zeros(K // 16, M, dtype=u8)
    lora = torch.zeros(M, R, dtype=bf)
    with pytest.raises(ValueError, match="ascales must have shape"):
        ops.gemm_w4a4(qact, torch.zeros(K // 16 + 1, M, dtype=u8), lora, w)
    with pytest.raises(ValueError, match="lora_act must have shape"):
        ops.gemm_w4a4(qact, asc, torch.zeros(M + 1, R, dtype=bf), w)
    with pytest.raises(ValueError, match="y must have shape"):
        ops.gemm_w4a4(qact, asc, lora, w, y=torch.zeros(M, N - 8, dtype=bf))
    with pytest.raises(ValueError, match="at least"):
        ops.gemm_w4a4(torch.zeros(10, dtype=u8), None, lora, w, M=M)
    wp = layer(packed=True)
    with pytest.raises(ValueError, match="at least"):
        ops.gemm_w4a4(torch.zeros(10, dtype=u8), None, lora, wp, M=M)


def test_gated_operands():
    w = layer(packed=True)   # N = 96 = 2F with F = 48
    nbytes = ops._lib.lib().svdq_packed_act_bytes(M, K)
    lora = torch.zeros(M, R, dtype=bf)
    with pytest.raises(ValueError, match="h must have shape"):
        ops.gemm_w4a4_gated(torch.zeros(nbytes, dtype=u8), lora, w, M, h=torch.zeros(M, N, dtype=bf))
    with pytest.raises(ValueError, match="at least"):
        ops.gemm_w4a4_gated(torch.zeros(nbytes - 1, dtype=u8), lora, w, M)
    with pytest.raises(ValueError, match="packed weight layout"):
        ops.linear_w4a4_gated(torch.zeros(M, K, dtype=bf), layer())


def test_repack_and_bf16_and_prep():
    with pytest.raises(ValueError, match="wscales must have shape"):
        ops.repack_weight(torch.zeros(N, K // 2, dtype=u8), torch.zeros(K // 16, N + 1, dtype=u8))
    with pytest.raises(ValueError, match="at least"):
        ops.unpack_weight(torch.zeros(16, dtype=u8), N, K)
    x = torch.zeros(M, K, dtype=bf)
    with pytest.raises(ValueError, match="bias must have shape"):
        ops.linear_bf16(x, torch.zeros(N, K, dtype=bf), torch.zeros(N + 1, dtype=bf))
    with pytest.raises(ValueError, match="y must have shape"):
        ops.linear_bf16(x, torch.zeros(N, K, dtype=bf), y=torch.zeros(N, M, dtype=bf))
    with pytest.raises(ValueError, match="smooth must have shape"):
        ops.prepare_weight(torch.zeros(N, K, dtype=bf), torch.zeros(K - 16, dtype=bf))
    with pytest.raises(ValueError, match="proj_up must have shape"):
        ops.prepare_residual(torch.zeros(N, K, dtype=bf), torch.zeros(K, dtype=bf), torch.zeros(K, R, dtype=bf),
                             torch.zeros(N, R + 16, dtype=bf))


def test_mx_operands():
    w = layer()
    L = ops._lib.lib()
    ac = torch.zeros(L.svdq_mx_codes_bytes(M, K), dtype=u8)
    asl = torch.zeros(L.svdq_mx_scales_bytes(M, K), dtype=u8)
    wc = torch.zeros(L.svdq_mx_codes_bytes(N, K), dtype=u8)
    wsl = torch.zeros(L.svdq_mx_scales_bytes(N, K), dtype=u8)
    lora = torch.zeros(M, R, dtype=bf)
    with pytest.raises(ValueError, match="w_codes has"):
        ops.gemm_mxfp4(ac, asl, lora, wc[:-16], wsl, w, M)
    with pytest.raises(ValueError, match="act_scales has"):
        ops.gemm_mxfp4(ac, asl[:-1], lora, wc, wsl, w, M)
    with pytest.raises(ValueError, match="w_scales has"):
        ops.linear_mxfp4(torch.zeros(M, K, dtype=bf), w, wc, wsl[:-1])
