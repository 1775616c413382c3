"""PyTorch-facing binding of the HIP library: argument marshalling only.

Every function checks dtype/device/contiguity, allocates outputs with torch
(device memory and the current stream are the only things torch provides),
and calls the C ABI with raw pointers. All arithmetic happens in the HIP
kernels; there is no CPU or PyTorch fallback.

Tensors (bf16 unless stated): x [M, K]; smooth [K]; qweight uint8 [N, K/2]
(low nibble = even k); wscales uint8 [K/16, N] (e4m3fn bytes; a
torch.float8_e4m3fn tensor is accepted and viewed as bytes); wcscales [N];
wtscale [1]; proj_down [K, R]; proj_up [N, R]; bias [N] or None.
"""

from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import ACT_CANONICAL, ACT_PACKED, WEIGHT_CANONICAL, WEIGHT_PACKED, SvdqError  # noqa: F401


def _bytes(t):
    if t.dtype == torch.float8_e4m3fn or t.dtype == torch.int8:
        return t.view(torch.uint8)
    return t


def _need(t, name, dtype, ndim=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _p(t):
    return None if t is None else t.data_ptr()


def _stream(device=None):
    return torch.cuda.current_stream(device).cuda_stream


def quantize_act(x, smooth, proj_down=None, qact=None, ascales=None, lora_act=None, packed=False,
                 workspace=None):
    """quant(x * smooth) and, with proj_down, lora_act = x @ proj_down.

    Returns (qact, ascales, lora_act): canonical qact uint8 [M, K/2] and ascales
    uint8 [K/16, M]; or, with packed=True, one packed uint8 buffer (the packed
    weight layout with rows = tokens) and ascales None. lora_act bf16 [M, R] or None.
    workspace: optional uint8 device tensor of at least
    quantize_act_workspace_bytes(M, K, R) bytes (allocated here when None).
    """
    _need(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    _need(smooth, "smooth", torch.bfloat16, 1)
    R = 0
    if proj_down is not None:
        _need(proj_down, "proj_down", torch.bfloat16, 2)
        R = proj_down.shape[1]
    dev = x.device
    L = _lib.lib()
    if packed:
        nbytes = L.svdq_packed_act_bytes(M, K)
        if qact is None:
            qact = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        ascales = None
    else:
        if qact is None:
            qact = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        if ascales is None:
            ascales = torch.empty((K // 16, M), dtype=torch.uint8, device=dev)
    if R > 0 and lora_act is None:
        lora_act = torch.empty((M, R), dtype=torch.bfloat16, device=dev)
    ws_need = quantize_act_workspace_bytes(M, K, R)
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else _need(workspace, "workspace", torch.uint8, 1).numel()
    _lib.check("svdq_quantize_act", L.svdq_quantize_act(
        _p(x), _p(smooth), M, K, _p(proj_down), R, ACT_PACKED if packed else ACT_CANONICAL,
        _p(qact), _p(ascales), _p(lora_act) if R > 0 else None, _p(workspace), ws_bytes, _stream(dev)))
    return qact, ascales, (lora_act if R > 0 else None)


def quantize_act_workspace_bytes(M, K, R):
    """Scratch bytes svdq_quantize_act needs (fp32 partials when K is split)."""
    return int(_lib.lib().svdq_quantize_act_workspace_bytes(M, K, R))


def repack_weight(qweight, wscales):
    """qweight [N, K/2] + wscales [K/16, N] -> packed uint8 buffer (MFMA order)."""
    qweight = _need(_bytes(qweight), "qweight", torch.uint8, 2)
    wscales = _need(_bytes(wscales), "wscales", torch.uint8, 2)
    N, Kh = qweight.shape
    K = 2 * Kh
    L = _lib.lib()
    nbytes = L.svdq_repack_weight_bytes(N, K)
    packed = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=qweight.device)
    _lib.check("svdq_repack_weight", L.svdq_repack_weight(
        _p(qweight), _p(wscales), N, K, _p(packed), nbytes, _stream(qweight.device)))
    return packed


def unpack_weight(packed, N, K):
    """Inverse of repack_weight: -> (qweight uint8 [N, K/2], wscales uint8 [K/16, N])."""
    _need(packed, "packed", torch.uint8, 1)
    qweight = torch.empty((N, K // 2), dtype=torch.uint8, device=packed.device)
    wscales = torch.empty((K // 16, N), dtype=torch.uint8, device=packed.device)
    L = _lib.lib()
    _lib.check("svdq_unpack_weight", L.svdq_unpack_weight(
        _p(packed), packed.numel(), N, K, _p(qweight), _p(wscales), _stream(packed.device)))
    return qweight, wscales


@dataclass
class SVDQLinearWeights:
    """One quantised linear layer's tensors, on the GPU.

    weight is qweight [N, K/2] (layout WEIGHT_CANONICAL, wscales given) or a
    buffer from repack_weight (layout WEIGHT_PACKED, wscales None).
    """
    N: int
    K: int
    weight: torch.Tensor
    wscales: Optional[torch.Tensor]
    wcscales: torch.Tensor
    wtscale: torch.Tensor
    smooth: torch.Tensor
    proj_down: Optional[torch.Tensor]
    proj_up: Optional[torch.Tensor]
    bias: Optional[torch.Tensor] = None
    layout: int = WEIGHT_CANONICAL

    @property
    def R(self):
        return 0 if self.proj_down is None else int(self.proj_down.shape[1])

    def packed(self):
        """A copy of this layer with the weight repacked (load-time step)."""
        if self.layout == WEIGHT_PACKED:
            return self
        buf = repack_weight(self.weight, self.wscales)
        return SVDQLinearWeights(self.N, self.K, buf, None, self.wcscales, self.wtscale, self.smooth,
                                 self.proj_down, self.proj_up, self.bias, WEIGHT_PACKED)


def _check_layer(w: SVDQLinearWeights):
    if w.layout == WEIGHT_CANONICAL:
        _need(_bytes(w.weight), "qweight", torch.uint8, 2)
        _need(_bytes(w.wscales), "wscales", torch.uint8, 2)
    else:
        _need(w.weight, "packed weight", torch.uint8, 1)
    _need(w.wcscales, "wcscales", torch.bfloat16, 1)
    _need(w.wtscale, "wtscale", torch.bfloat16, 1)
    if w.R > 0:
        _need(w.proj_down, "proj_down", torch.bfloat16, 2)
        _need(w.proj_up, "proj_up", torch.bfloat16, 2)
    if w.bias is not None:
        _need(w.bias, "bias", torch.bfloat16, 1)


def gemm_w4a4(qact, ascales, lora_act, w: SVDQLinearWeights, y=None, M=None):
    """The scaled GEMM + low-rank up-projection + epilogue from quantised activations.

    Canonical activations: qact [M, K/2], ascales [K/16, M]. Packed activations
    (from quantize_act(..., packed=True)): qact is the packed buffer, ascales
    None, and M must be given; the layer's weight must be packed too.
    """
    _check_layer(w)
    act_packed = ascales is None
    if act_packed:
        _need(qact, "qact (packed)", torch.uint8, 1)
        if M is None:
            raise ValueError("M is required with packed activations")
    else:
        _need(qact, "qact", torch.uint8, 2)
        _need(ascales, "ascales", torch.uint8, 2)
        M = qact.shape[0]
    if w.R > 0:
        _need(lora_act, "lora_act", torch.bfloat16, 2)
    if y is None:
        y = torch.empty((M, w.N), dtype=torch.bfloat16, device=qact.device)
    L = _lib.lib()
    _lib.check("svdq_gemm_w4a4", L.svdq_gemm_w4a4(
        _p(qact), _p(ascales), ACT_PACKED if act_packed else ACT_CANONICAL,
        _p(lora_act) if w.R > 0 else None,
        _p(_bytes(w.weight)), _p(_bytes(w.wscales)) if w.wscales is not None else None, w.layout,
        _p(w.wcscales), _p(w.wtscale), _p(w.proj_up) if w.R > 0 else None, _p(w.bias),
        M, w.N, w.K, w.R, _p(y), _stream(qact.device)))
    return y


def linear_workspace_bytes(M, N, K, R):
    return _lib.lib().svdq_linear_workspace_bytes(M, N, K, R)


def linear_w4a4(x, w: SVDQLinearWeights, y=None, workspace=None):
    """The whole layer: y [M, N] bf16."""
    _check_layer(w)
    _need(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    if K != w.K:
        raise ValueError(f"x has K={K}, the layer K={w.K}")
    if y is None:
        y = torch.empty((M, w.N), dtype=torch.bfloat16, device=x.device)
    L = _lib.lib()
    nbytes = L.svdq_linear_workspace_bytes(M, w.N, K, w.R)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    _lib.check("svdq_linear_w4a4", L.svdq_linear_w4a4(
        _p(x), _p(w.smooth), _p(_bytes(w.weight)),
        _p(_bytes(w.wscales)) if w.wscales is not None else None, w.layout,
        _p(w.wcscales), _p(w.wtscale), _p(w.proj_down) if w.R > 0 else None,
        _p(w.proj_up) if w.R > 0 else None, _p(w.bias), M, w.N, K, w.R,
        _p(y), _p(workspace), workspace.numel(), _stream(x.device)))
    return y


def _check_gated(w: SVDQLinearWeights):
    _check_layer(w)
    if w.layout != WEIGHT_PACKED:
        raise ValueError("the gated layer needs the packed weight layout (use .packed())")
    if w.N % 2 != 0:
        raise ValueError(f"the gated layer has 2F output channels, got N={w.N}")
    return w.N // 2


def gemm_w4a4_gated(qact, lora_act, w: SVDQLinearWeights, M, h=None):
    """Gated FFN step from packed activations: h [M, F] = silu(y[:, :F]) * y[:, F:]
    of the 2F-channel layer w (w1 and w3 as one layer), bf16."""
    F_out = _check_gated(w)
    _need(qact, "qact (packed)", torch.uint8, 1)
    if w.R > 0:
        _need(lora_act, "lora_act", torch.bfloat16, 2)
    if h is None:
        h = torch.empty((M, F_out), dtype=torch.bfloat16, device=qact.device)
    L = _lib.lib()
    _lib.check("svdq_gemm_w4a4_gated", L.svdq_gemm_w4a4_gated(
        _p(qact), _p(lora_act) if w.R > 0 else None, _p(_bytes(w.weight)), _p(w.wcscales),
        _p(w.wtscale), _p(w.proj_up) if w.R > 0 else None, _p(w.bias), M, F_out, w.K, w.R,
        _p(h), _stream(qact.device)))
    return h


def linear_w4a4_gated(x, w: SVDQLinearWeights, h=None, workspace=None):
    """The whole gated step from x: h [M, F] bf16 (w is the 2F-channel w1/w3 layer)."""
    F_out = _check_gated(w)
    _need(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    if K != w.K:
        raise ValueError(f"x has K={K}, the layer K={w.K}")
    if h is None:
        h = torch.empty((M, F_out), dtype=torch.bfloat16, device=x.device)
    L = _lib.lib()
    nbytes = L.svdq_linear_gated_workspace_bytes(M, F_out, K, w.R)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    _lib.check("svdq_linear_w4a4_gated", L.svdq_linear_w4a4_gated(
        _p(x), _p(w.smooth), _p(_bytes(w.weight)), _p(w.wcscales), _p(w.wtscale),
        _p(w.proj_down) if w.R > 0 else None, _p(w.proj_up) if w.R > 0 else None, _p(w.bias),
        M, F_out, K, w.R, _p(h), _p(workspace), workspace.numel(), _stream(x.device)))
    return h


def linear_bf16(x, weight, bias=None, y=None):
    """A linear kept in bf16: y [M, N] = bf16(x @ weight^T + bias), with x [M, K],
    weight [N, K] and bias [N] (or None), all bf16."""
    _need(x, "x", torch.bfloat16, 2)
    _need(weight, "weight", torch.bfloat16, 2)
    M, K = x.shape
    N = weight.shape[0]
    if weight.shape[1] != K:
        raise ValueError(f"x has K={K}, weight has K={weight.shape[1]}")
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, 1)
        if bias.numel() != N:
            raise ValueError(f"bias has {bias.numel()} entries, N={N}")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    else:
        _need(y, "y", torch.bfloat16, 2)
        if tuple(y.shape) != (M, N):
            raise ValueError(f"y must be [{M}, {N}], got {tuple(y.shape)}")
    L = _lib.lib()
    _lib.check("svdq_linear_bf16", L.svdq_linear_bf16(
        _p(x), _p(weight), _p(bias), M, N, K, _p(y), _stream(x.device)))
    return y


def prepare_workspace_bytes(N, K, R):
    return _lib.lib().svdq_prepare_workspace_bytes(N, K, R)


def _prep_outputs(N, K, R, dev):
    u8 = torch.uint8
    return dict(qweight=torch.empty((N, K // 2), dtype=u8, device=dev),
                wscales=torch.empty((K // 16, N), dtype=u8, device=dev),
                wcscales=torch.empty(N, dtype=torch.bfloat16, device=dev),
                wtscale=torch.empty(1, dtype=torch.bfloat16, device=dev))


def prepare_weight(weight, smooth, omega=None, iters=2, bias=None, workspace=None):
    """SVDQuant preparation of a bf16 weight [N, K] with smooth [K]: the rank-R
    split (R = omega.shape[1]; omega [K, R] float32 Gaussian, or None for R = 0),
    the residual's two-level scales and NVFP4 codes. Returns SVDQLinearWeights
    (canonical layout)."""
    _need(weight, "weight", torch.bfloat16, 2)
    _need(smooth, "smooth", torch.bfloat16, 1)
    N, K = weight.shape
    R = 0
    if omega is not None:
        _need(omega, "omega", torch.float32, 2)
        if omega.shape[0] != K:
            raise ValueError(f"omega must be [K={K}, R], got {tuple(omega.shape)}")
        R = omega.shape[1]
    dev = weight.device
    out = _prep_outputs(N, K, R, dev)
    pd = torch.empty((K, R), dtype=torch.bfloat16, device=dev) if R else None
    pu = torch.empty((N, R), dtype=torch.bfloat16, device=dev) if R else None
    L = _lib.lib()
    nbytes = L.svdq_prepare_workspace_bytes(N, K, R)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _lib.check("svdq_prepare_weight", L.svdq_prepare_weight(
        _p(weight), _p(smooth), _p(omega), N, K, R, iters, _p(out["qweight"]), _p(out["wscales"]),
        _p(out["wcscales"]), _p(out["wtscale"]), _p(pd), _p(pu), _p(workspace), workspace.numel(),
        _stream(dev)))
    return SVDQLinearWeights(N=N, K=K, weight=out["qweight"], wscales=out["wscales"], wcscales=out["wcscales"],
                             wtscale=out["wtscale"], smooth=smooth, proj_down=pd, proj_up=pu, bias=bias)


def prepare_residual(weight, smooth, proj_down=None, proj_up=None, workspace=None):
    """Steps 3-5 of the preparation for given bf16 factors: returns
    (qweight, wscales, wcscales, wtscale)."""
    _need(weight, "weight", torch.bfloat16, 2)
    _need(smooth, "smooth", torch.bfloat16, 1)
    N, K = weight.shape
    R = 0 if proj_down is None else proj_down.shape[1]
    if R:
        _need(proj_down, "proj_down", torch.bfloat16, 2)
        _need(proj_up, "proj_up", torch.bfloat16, 2)
    dev = weight.device
    out = _prep_outputs(N, K, R, dev)
    L = _lib.lib()
    nbytes = L.svdq_prepare_workspace_bytes(N, K, R)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _lib.check("svdq_prepare_residual", L.svdq_prepare_residual(
        _p(weight), _p(smooth), _p(proj_down), _p(proj_up), N, K, R, _p(out["qweight"]), _p(out["wscales"]),
        _p(out["wcscales"]), _p(out["wtscale"]), _p(workspace), workspace.numel(), _stream(dev)))
    return out["qweight"], out["wscales"], out["wcscales"], out["wtscale"]


def mx_buffers(rows, K, dev):
    L = _lib.lib()
    return (torch.empty(L.svdq_mx_codes_bytes(rows, K), dtype=torch.uint8, device=dev),
            torch.empty(L.svdq_mx_scales_bytes(rows, K), dtype=torch.uint8, device=dev))


def reround_weight_mxfp4(w: "SVDQLinearWeights"):
    """MXFP4 variant: the layer's canonical NVFP4 weight re-rounded to MX codes and
    scales (load time). Returns (mx_codes, mx_scales) uint8 buffers."""
    _check_layer(w)
    if w.layout != WEIGHT_CANONICAL:
        raise ValueError("re-rounding reads the canonical weight layout")
    codes, scales = mx_buffers(w.N, w.K, w.weight.device)
    L = _lib.lib()
    _lib.check("svdq_reround_weight_mxfp4", L.svdq_reround_weight_mxfp4(
        _p(_bytes(w.weight)), _p(_bytes(w.wscales)), w.N, w.K, _p(codes), _p(scales), _stream(w.weight.device)))
    return codes, scales


def quantize_act_mxfp4(x, smooth):
    """MX(x * smooth): returns (mx_codes, mx_scales) uint8 buffers."""
    _need(x, "x", torch.bfloat16, 2)
    _need(smooth, "smooth", torch.bfloat16, 1)
    M, K = x.shape
    codes, scales = mx_buffers(M, K, x.device)
    L = _lib.lib()
    _lib.check("svdq_quantize_act_mxfp4", L.svdq_quantize_act_mxfp4(
        _p(x), _p(smooth), M, K, _p(codes), _p(scales), _stream(x.device)))
    return codes, scales


def gemm_mxfp4(act_codes, act_scales, lora_act, w_codes, w_scales, w: "SVDQLinearWeights", M, y=None):
    """The variant's GEMM + low-rank up-projection + epilogue: y [M, N] bf16."""
    if y is None:
        y = torch.empty((M, w.N), dtype=torch.bfloat16, device=act_codes.device)
    L = _lib.lib()
    _lib.check("svdq_gemm_mxfp4", L.svdq_gemm_mxfp4(
        _p(act_codes), _p(act_scales), _p(lora_act) if w.R > 0 else None, _p(w_codes), _p(w_scales),
        _p(w.wcscales), _p(w.wtscale), _p(w.proj_up) if w.R > 0 else None, _p(w.bias), M, w.N, w.K, w.R,
        _p(y), _stream(act_codes.device)))
    return y


def linear_mxfp4(x, w: "SVDQLinearWeights", w_codes, w_scales, y=None, workspace=None):
    """The whole MXFP4 variant layer from x (w supplies smooth, wcscales, wtscale,
    the low-rank factors and bias; w_codes / w_scales from reround_weight_mxfp4)."""
    _need(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    if K != w.K:
        raise ValueError(f"x has K={K}, the layer K={w.K}")
    if y is None:
        y = torch.empty((M, w.N), dtype=torch.bfloat16, device=x.device)
    L = _lib.lib()
    nbytes = L.svdq_linear_mxfp4_workspace_bytes(M, K, w.R)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    _lib.check("svdq_linear_mxfp4", L.svdq_linear_mxfp4(
        _p(x), _p(w.smooth), _p(w_codes), _p(w_scales), _p(w.wcscales), _p(w.wtscale),
        _p(w.proj_down) if w.R > 0 else None, _p(w.proj_up) if w.R > 0 else None, _p(w.bias),
        M, w.N, K, w.R, _p(y), _p(workspace), workspace.numel(), _stream(x.device)))
    return y
