"""GPU: every output byte is written and none outside the output, for each entry point.

Each output (and each workspace) is placed inside a larger buffer with 4 KB guard bands
before and after it, filled with 0xA5. The output region itself is pre-filled twice, with
0x00 and with 0xFF (bf16 +0 and a NaN pattern; for codes, two different bytes), and both
runs must give the bytes of the same call into freshly allocated tensors: a byte that the
kernels skip keeps its fill in one of the two runs. The guard bands must come back
untouched. The shapes are ragged in M, N and K and span several tiles, and every tile shape
of the packed GEMM is forced once.

Packed activation buffers leave the rows beyond M in their last 32-row panel unspecified,
so their cases use M a multiple of 32; the workspaces' contents are unspecified, so only
their guard bands are checked. The reference calls' own outputs are checked against the
oracle by the parity tests of each entry point; here they are only required to be finite.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import formats as F
from oracle import repack as P
from oracle import svdq as S
from tests.gpu_util import dev_bf16, dev_u8, make_layer

pytestmark = pytest.mark.gpu

G = 4096          # guard band bytes on each side
GUARD = 0xA5


class Guarded:
    """A device tensor of `shape` and `dtype` inside a uint8 buffer with guard bands."""

    def __init__(self, shape, dtype, fill):
        self.shape, self.dtype = tuple(shape), dtype
        self.nbytes = int(np.prod(self.shape)) * torch.empty(0, dtype=dtype).element_size()
        self.base = torch.full((self.nbytes + 2 * G,), GUARD, dtype=torch.uint8, device="cuda")
        self.base[G:G + self.nbytes].fill_(fill)
        self.t = self.base[G:G + self.nbytes].view(dtype).view(self.shape)

    def check_guards(self, name):
        b = self.base.cpu().numpy()
        assert np.all(b[:G] == GUARD), f"{name}: written before its start"
        assert np.all(b[G + self.nbytes:] == GUARD), f"{name}: written past its end"

    def body(self):
        return self.base[G:G + self.nbytes].cpu().numpy()


def _bytes_of(t):
    return t.detach().contiguous().view(torch.uint8).cpu().numpy().reshape(-1)


def _finite_bf16(t):
    return bool(torch.isfinite(t.float()).all())


def _run_guarded(name, specs, call, ref):
    """specs: {arg: (shape, dtype, compare)}; call(**tensors) runs the entry point into the
    given tensors; ref: {arg: reference tensor} for the compared outputs."""
    for fill in (0x00, 0xFF):
        bufs = {k: Guarded(shape, dt, fill) for k, (shape, dt, _) in specs.items()}
        call(**{k: g.t for k, g in bufs.items()})
        torch.cuda.synchronize()
        for k, g in bufs.items():
            g.check_guards(f"{name}.{k} (fill {fill:#04x})")
            if specs[k][2]:
                assert np.array_equal(g.body(), _bytes_of(ref[k])), f"{name}.{k}: bytes left unwritten (fill {fill:#04x})"


LAYERS = [
    dict(M=130, K=336, N=700, R=16, kind="dit", seed=91),     # ragged M, N; K % 64 != 0
    dict(M=1, K=256, N=333, R=32, kind="dit", seed=92),       # one row
    dict(M=300, K=640, N=1000, R=0, kind="dit", seed=93),     # R = 0, several tiles
]


@pytest.fixture
def tile_reset(gpu_lib):
    yield gpu_lib
    gpu_lib.set_gemm_tile(0)


@pytest.mark.parametrize("cfg", LAYERS)
@pytest.mark.parametrize("layout", ["packed", "canonical"])
def test_linear_writes_exactly_y(tile_reset, cfg, layout):
    ops = tile_reset
    d, layer = make_layer(cfg)
    if layout == "packed":
        layer = layer.packed()
    M, N, K, R = d["M"], d["N"], d["K"], d["R"]
    x = dev_bf16(d["x"])
    ws_bytes = ops.linear_workspace_bytes(M, N, K, R)
    for tile in (0, 1, 2, 3, 4):
        ops.set_gemm_tile(tile)
        y_ref = ops.linear_w4a4(x, layer)
        torch.cuda.synchronize()
        assert _finite_bf16(y_ref)
        _run_guarded(f"linear_w4a4[{layout}, tile {tile}]",
                     {"y": ((M, N), torch.bfloat16, True), "workspace": ((max(ws_bytes, 1),), torch.uint8, False)},
                     lambda y, workspace: ops.linear_w4a4(x, layer, y=y, workspace=workspace), {"y": y_ref})


@pytest.mark.parametrize("cfg", LAYERS[:2])
def test_gemm_both_canonical_writes_exactly_y(gpu_lib, cfg):
    """Canonical activations with the canonical weight (the per-wave dequantising kernel)."""
    ops = gpu_lib
    d, layer = make_layer(cfg)
    qact, ascales = S.quantize_act(d["x"], d["smooth"])
    qa, sa = dev_u8(qact), dev_u8(ascales)
    lora = ops.lowrank_down(dev_bf16(d["x"]), layer.proj_down) if d["R"] > 0 else None
    y_ref = ops.gemm_w4a4(qa, sa, lora, layer)
    torch.cuda.synchronize()
    assert _finite_bf16(y_ref)
    _run_guarded("gemm_w4a4[canonical, canonical]", {"y": ((d["M"], d["N"]), torch.bfloat16, True)},
                 lambda y: ops.gemm_w4a4(qa, sa, lora, layer, y=y), {"y": y_ref})


@pytest.mark.parametrize("M,K,R", [
    (96, 336, 16),       # K % 64 != 0
    (256, 1280, 128),    # short K: the split-free form
    (64, 3840, 128),     # K split across workgroups, partial sums in the workspace
])
@pytest.mark.parametrize("packed", [False, True])
def test_quantize_writes_exactly_outputs(gpu_lib, M, K, R, packed):
    ops = gpu_lib
    x, sm = workloads.make_activation(M, K, kind="dit", seed=M + K + R)
    pd = np.random.default_rng(K + R).standard_normal((K, R)) * 0.05
    xd, smd, pdd = dev_bf16(x), dev_bf16(sm), dev_bf16(F.f64_to_bf16(pd))
    q_ref, s_ref, l_ref = ops.quantize_act(xd, smd, pdd, packed=packed)
    torch.cuda.synchronize()
    assert _finite_bf16(l_ref)
    L = ops._lib.lib()
    ws_bytes = ops.quantize_act_workspace_bytes(M, K, R)
    specs = {"lora_act": ((M, R), torch.bfloat16, True)}
    ref = {"lora_act": l_ref}
    if packed:
        specs["qact"] = ((L.svdq_packed_act_bytes(M, K),), torch.uint8, True)
        ref["qact"] = q_ref
    else:
        specs["qact"] = ((M, K // 2), torch.uint8, True)
        specs["ascales"] = ((K // 16, M), torch.uint8, True)
        ref["qact"], ref["ascales"] = q_ref, s_ref
    if ws_bytes > 0:
        specs["workspace"] = ((ws_bytes,), torch.uint8, False)

    def call(qact, lora_act, ascales=None, workspace=None):
        ops.quantize_act(xd, smd, pdd, qact=qact, ascales=ascales, lora_act=lora_act, packed=packed,
                         workspace=workspace)

    _run_guarded(f"quantize_act[packed={packed}]", specs, call, ref)


@pytest.mark.parametrize("M,K,R", [(130, 384, 32), (64, 3840, 128)])
def test_quantize_mx_writes_exactly_outputs(gpu_lib, M, K, R):
    """The MXFP4 layout of svdq_quantize_act: codes and scales of the padded rows, lora_act."""
    ops = gpu_lib
    x, sm = workloads.make_activation(M, K, kind="dit", seed=M + K)
    pd = dev_bf16(F.f64_to_bf16(np.random.default_rng(K).standard_normal((K, R)) * 0.05))
    xd, smd = dev_bf16(x), dev_bf16(sm)
    c_ref, s_ref, l_ref = ops.quantize_act(xd, smd, pd, mx=True)
    torch.cuda.synchronize()
    L = ops._lib.lib()
    specs = {"qact": ((L.svdq_mx_codes_bytes(M, K),), torch.uint8, True),
             "ascales": ((L.svdq_mx_scales_bytes(M, K),), torch.uint8, True),
             "lora_act": ((M, R), torch.bfloat16, True)}
    ws_bytes = ops.quantize_act_workspace_bytes(M, K, R)
    if ws_bytes > 0:
        specs["workspace"] = ((ws_bytes,), torch.uint8, False)

    def call(qact, ascales, lora_act, workspace=None):
        ops.quantize_act(xd, smd, pd, qact=qact, ascales=ascales, lora_act=lora_act, workspace=workspace, mx=True)

    _run_guarded("quantize_act[mx]", specs, call, {"qact": c_ref, "ascales": s_ref, "lora_act": l_ref})


def test_lowrank_down_writes_exactly_lora(gpu_lib):
    ops = gpu_lib
    M, K, R = 77, 3840, 128
    x, _ = workloads.make_activation(M, K, kind="dit", seed=94)
    pd = dev_bf16(F.f64_to_bf16(np.random.default_rng(95).standard_normal((K, R)) * 0.05))
    xd = dev_bf16(x)
    l_ref = ops.lowrank_down(xd, pd)
    torch.cuda.synchronize()
    ws_bytes = ops.quantize_act_workspace_bytes(M, K, R)
    specs = {"lora_act": ((M, R), torch.bfloat16, True)}
    if ws_bytes > 0:
        specs["workspace"] = ((ws_bytes,), torch.uint8, False)
    _run_guarded("lowrank_down", specs, lambda lora_act, workspace=None: ops.lowrank_down(
        xd, pd, lora_act=lora_act, workspace=workspace), {"lora_act": l_ref})


@pytest.mark.parametrize("tile", [0, 1, 3])
def test_gated_writes_exactly_h_and_next_codes(tile_reset, tile):
    ops = tile_reset
    cfg = dict(M=96, K=512, N=2 * 384, R=32, kind="swiglu", seed=96)
    d, layer = make_layer(cfg)
    layer = layer.packed()
    M, F_out = d["M"], d["N"] // 2
    qact, ascales = S.quantize_act(d["x"], d["smooth"])
    qpk = dev_u8(P.repack(qact, ascales))
    lora = ops.lowrank_down(dev_bf16(d["x"]), layer.proj_down)
    nsm = dev_bf16(F.f64_to_bf16(np.random.default_rng(97).uniform(0.5, 2.0, size=F_out)))
    ops.set_gemm_tile(tile)
    h_ref = ops.gemm_w4a4_gated(qpk, lora, layer, M)
    h2_ref, q_ref = ops.gemm_w4a4_gated_quant(qpk, lora, layer, M, nsm)
    torch.cuda.synchronize()
    assert _finite_bf16(h_ref)
    _run_guarded("gemm_w4a4_gated", {"h": ((M, F_out), torch.bfloat16, True)},
                 lambda h: ops.gemm_w4a4_gated(qpk, lora, layer, M, h=h), {"h": h_ref})
    nbytes = ops._lib.lib().svdq_packed_act_bytes(M, F_out)
    _run_guarded("gemm_w4a4_gated_quant",
                 {"h": ((M, F_out), torch.bfloat16, True), "next_qact": ((nbytes,), torch.uint8, True)},
                 lambda h, next_qact: ops.gemm_w4a4_gated_quant(qpk, lora, layer, M, nsm, h=h, next_qact=next_qact),
                 {"h": h2_ref, "next_qact": q_ref})
    x = dev_bf16(d["x"])
    hl_ref = ops.linear_w4a4_gated(x, layer)
    torch.cuda.synchronize()
    ws_bytes = ops._lib.lib().svdq_linear_gated_workspace_bytes(M, F_out, d["K"], d["R"])
    _run_guarded("linear_w4a4_gated",
                 {"h": ((M, F_out), torch.bfloat16, True), "workspace": ((max(ws_bytes, 1),), torch.uint8, False)},
                 lambda h, workspace: ops.linear_w4a4_gated(x, layer, h=h, workspace=workspace), {"h": hl_ref})


@pytest.mark.parametrize("M,N,K", [(130, 700, 336), (1, 200, 64), (300, 1000, 640)])
def test_linear_bf16_writes_exactly_y(gpu_lib, M, N, K):
    ops = gpu_lib
    d = workloads.make_bf16_linear(M, K, N, kind="dit", seed=M + N)
    x, w, b = dev_bf16(d["x"]), dev_bf16(d["W"]), dev_bf16(d["bias"])
    y_ref = ops.linear_bf16(x, w, b)
    torch.cuda.synchronize()
    assert _finite_bf16(y_ref)
    _run_guarded("linear_bf16", {"y": ((M, N), torch.bfloat16, True)},
                 lambda y: ops.linear_bf16(x, w, b, y=y), {"y": y_ref})


@pytest.mark.parametrize("cfg", [dict(M=130, K=384, N=700, R=16, kind="dit", seed=98),
                                 dict(M=1, K=256, N=333, R=0, kind="dit", seed=99)])
def test_linear_mxfp4_writes_exactly_y(gpu_lib, cfg):
    ops = gpu_lib
    d, layer = make_layer(cfg)
    wc, wsc = ops.reround_weight_mxfp4(layer)
    x = dev_bf16(d["x"])
    y_ref = ops.linear_mxfp4(x, layer, wc, wsc)
    torch.cuda.synchronize()
    assert _finite_bf16(y_ref)
    ws_bytes = ops._lib.lib().svdq_linear_mxfp4_workspace_bytes(d["M"], d["K"], d["R"])
    _run_guarded("linear_mxfp4",
                 {"y": ((d["M"], d["N"]), torch.bfloat16, True), "workspace": ((max(ws_bytes, 1),), torch.uint8, False)},
                 lambda y, workspace: ops.linear_mxfp4(x, layer, wc, wsc, y=y, workspace=workspace), {"y": y_ref})
