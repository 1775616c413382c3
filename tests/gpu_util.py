"""Helpers for the GPU parity tests: numpy <-> device tensors and layer setup.

Expected values always come from oracle/ on the same seeded inputs; nothing
here computes any part of the layer.
"""

import numpy as np
import torch

import workloads
from oracle import formats as F
from oracle import svdq as S


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def host_bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host_u8(t):
    return t.detach().cpu().contiguous().numpy()


def make_layer(cfg, with_bias=True, zero_weight=False):
    """Seeded layer inputs (numpy), the oracle's NVFP4 weight, and device copies."""
    from bit_w4a4_quantized_quantize_amd import ops
    d = workloads.make_linear(cfg["M"], cfg["K"], cfg["N"], cfg["R"], kind=cfg.get("kind", "dit"),
                              seed=cfg.get("seed", 0), with_bias=with_bias)
    qw, ws = S.quantize_weight(d["W"], d["wcscales"], d["wtscale"])
    if zero_weight:
        qw = np.zeros_like(qw)
    d["qweight"], d["wscales"] = qw, ws
    R = d["R"]
    layer = ops.SVDQLinearWeights(
        N=d["N"], K=d["K"], weight=dev_u8(qw), wscales=dev_u8(ws),
        wcscales=dev_bf16(d["wcscales"]), wtscale=dev_bf16(d["wtscale"]),
        smooth=dev_bf16(d["smooth"]),
        proj_down=dev_bf16(d["proj_down"]) if R > 0 else None,
        proj_up=dev_bf16(d["proj_up"]) if R > 0 else None,
        bias=dev_bf16(d["bias"]) if d["bias"] is not None else None)
    return d, layer


def ulp_bf16(v):
    """Spacing of bf16 numbers at |v| (float64), for diagnostics."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    e = np.floor(np.log2(a))
    return 2.0 ** (e - 7)


def within_ulps(y_bits, y64, n=1):
    y = F.bf16_to_f64(y_bits)
    return np.abs(y - y64) <= n * ulp_bf16(y64) + 1e-30
