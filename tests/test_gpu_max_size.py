"""GPU parity at the largest operands the library accepts. x of M = 279620 rows by
K = 3840 (M K 2 bytes = 2^31 - 2048, just under the 2 GiB limit of the 32-bit buffer
offsets; M is not a multiple of the 128-row blocks). The rows farthest into the buffers
are where an offset overflow would show, so the sampled rows include the last ones.

x is drawn on the device by torch's seeded generator (an input, not a result of these
kernels); the sampled rows are copied back and the oracle evaluates them:
- codes and scales of the canonical quantisation, bit for bit;
- the whole layer (packed weights, R = 128, bias), normwise error <= 5e-3 and every
  element within the arithmetic bound of the layer (as in test_gpu_linear.py).
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import formats as F
from oracle import svdq as S
from tests.gpu_util import host_bits, host_u8, make_layer, ulp_bf16

pytestmark = pytest.mark.gpu

M_MAX, K, N, R = 279620, 3840, 200, 128


def test_layer_at_the_largest_activation(gpu_lib):
    assert M_MAX * K * 2 < 2 ** 31 <= (M_MAX + 1) * K * 2
    d, layer = make_layer(dict(M=8, K=K, N=N, R=R, kind="dit", seed=77))   # weights, smooth, proj
    layer = layer.packed()
    g = torch.Generator(device="cuda").manual_seed(78)
    x = torch.randn(M_MAX, K, dtype=torch.bfloat16, device="cuda", generator=g)
    rows = np.concatenate([[0, 1, 127, 128], np.sort(np.random.default_rng(79).choice(M_MAX - 8, 24, replace=False)),
                           np.arange(M_MAX - 6, M_MAX)])
    x_rows = host_bits(x[torch.from_numpy(rows).cuda()])

    qact, ascales, _ = gpu_lib.quantize_act(x, layer.smooth)
    torch.cuda.synchronize()
    q_ref, s_ref = S.quantize_act(x_rows, d["smooth"])
    assert np.array_equal(host_u8(qact[torch.from_numpy(rows).cuda()]), q_ref)
    assert np.array_equal(host_u8(ascales[:, torch.from_numpy(rows).cuda()]), s_ref)
    del qact, ascales

    y = gpu_lib.linear_w4a4(x, layer)
    torch.cuda.synchronize()
    got_bits = host_bits(y[torch.from_numpy(rows).cuda()])
    y64, _, _, _ = S.linear_w4a4(x_rows, d["smooth"], d["qweight"], d["wscales"], d["wcscales"], d["wtscale"],
                                 d["proj_down"], d["proj_up"], d["bias"])
    got = F.bf16_to_f64(got_bits)
    assert S.normwise_rel_err(got, y64) <= 5e-3
    alpha = np.abs(F.bf16_to_f64(d["wtscale"])[0] * F.bf16_to_f64(d["wcscales"]))
    main_abs = np.abs(S.dequant(q_ref, s_ref)) @ np.abs(S.dequant(d["qweight"], d["wscales"])).T * alpha
    pu_abs = np.abs(F.bf16_to_f64(d["proj_up"])).T
    lr_abs = np.abs(S.lowrank_down(x_rows, d["proj_down"])) @ pu_abs
    lr_acc = (np.abs(F.bf16_to_f64(x_rows)) @ np.abs(F.bf16_to_f64(d["proj_down"]))) @ pu_abs
    bound = (ulp_bf16(y64) + (K / 16 + 2) * 2.0 ** -24 * main_abs + 2.0 ** -8 * lr_abs
             + (K + R + 2) * 2.0 ** -24 * lr_acc)
    bad = np.argwhere(np.abs(got - y64) > bound)
    assert bad.size == 0, f"{len(bad)} elements beyond the arithmetic bound, first {bad[:3].tolist()}"


def test_one_row_more_is_rejected(gpu_lib):
    """M + 1 rows put x past 2 GiB: the call is refused before any launch."""
    from bit_w4a4_quantized_quantize_amd import _lib
    x = torch.empty((M_MAX + 1) * K, dtype=torch.bfloat16, device="cuda")
    d, layer = make_layer(dict(M=8, K=K, N=N, R=R, kind="dit", seed=77))
    with pytest.raises(_lib.SvdqError):
        gpu_lib.quantize_act(x.view(M_MAX + 1, K), layer.smooth)


def test_gemm_at_the_largest_weight(gpu_lib):
    """The largest N whose packed weight stays under 2 GiB at K = 10240 (N = 372,000 or so):
    random codes and valid block scales drawn on the device, repacked by the library, then
    the scaled GEMM + rank-16 residual + bias from the oracle's quantised activations, in both
    activation layouts. Sampled columns include the last ones (the largest weight offsets)."""
    from bit_w4a4_quantized_quantize_amd import _lib, ops
    from oracle import repack as P
    from tests.gpu_util import dev_bf16, dev_u8
    L = _lib.lib()
    Kw, Rw, Mw = 10240, 16, 64
    lo, hi = 1, 1 << 22
    while lo < hi:                       # largest N with a packed weight under 2 GiB
        mid = (lo + hi + 1) // 2
        lo, hi = (mid, hi) if L.svdq_repack_weight_bytes(mid, Kw) < 2 ** 31 else (lo, mid - 1)
    Nw = lo
    assert L.svdq_repack_weight_bytes(Nw + 1, Kw) >= 2 ** 31
    g = torch.Generator(device="cuda").manual_seed(80)
    qweight = torch.randint(0, 256, (Nw, Kw // 2), dtype=torch.uint8, device="cuda", generator=g)
    wscales = torch.randint(0x28, 0x40, (Kw // 16, Nw), dtype=torch.uint8, device="cuda", generator=g)
    rng = np.random.default_rng(81)
    wcs_bits = F.f64_to_bf16(rng.uniform(0.5, 1.5, Nw) * 2.0 ** -6)
    bias_bits = F.f64_to_bf16(rng.normal(0, 0.01, Nw))
    pu_bits = F.f64_to_bf16(rng.normal(0, 0.02, (Nw, Rw)))
    wt_bits = F.f64_to_bf16(np.ones(1))
    layer = ops.SVDQLinearWeights(N=Nw, K=Kw, weight=qweight, wscales=wscales, wcscales=dev_bf16(wcs_bits),
                                  wtscale=dev_bf16(wt_bits), smooth=dev_bf16(F.f64_to_bf16(np.ones(Kw))),
                                  proj_down=dev_bf16(F.f64_to_bf16(np.zeros((Kw, Rw)))), proj_up=dev_bf16(pu_bits),
                                  bias=dev_bf16(bias_bits))
    cols = np.concatenate([[0, 1, 31, 32], np.sort(rng.choice(Nw - 8, 24, replace=False)), np.arange(Nw - 6, Nw)])
    cidx = torch.from_numpy(cols).cuda()
    qw_cols, ws_cols = host_u8(qweight[cidx]), host_u8(wscales[:, cidx])
    packed = layer.packed()
    del layer, qweight, wscales
    d = workloads.make_linear(Mw, Kw, 8, Rw, kind="dit", seed=82, with_bias=False)
    qact, ascales = S.quantize_act(d["x"], d["smooth"])
    lora_bits = F.f64_to_bf16(rng.normal(0, 0.5, (Mw, Rw)))
    y64 = S.gemm_w4a4(qact, ascales, F.bf16_to_f64(lora_bits), qw_cols, ws_cols, wcs_bits[cols], wt_bits,
                      pu_bits[cols], bias_bits[cols])
    for act in ("canonical", "packed"):
        if act == "canonical":
            y = gpu_lib.gemm_w4a4(dev_u8(qact), dev_u8(ascales), dev_bf16(lora_bits), packed)
        else:
            y = gpu_lib.gemm_w4a4(dev_u8(P.repack(qact, ascales)), None, dev_bf16(lora_bits), packed, M=Mw)
        torch.cuda.synchronize()
        got_bits = host_bits(y[:, cidx])
        got = F.bf16_to_f64(got_bits)
        assert S.normwise_rel_err(got, y64) <= 5e-3, act
        frac = float(np.mean(np.abs(got - y64) <= ulp_bf16(y64) + 1e-30))
        assert frac >= 0.999, (act, frac)
        del y
