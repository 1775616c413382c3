"""svdq_linear_w4a4_noalloc (the layer with the library's static device scratch as
workspace) against svdq_linear_w4a4 with a caller workspace: bit-identical outputs on
two calls in a row, the second smaller than the first, in both weight layouts; and
against the oracle's float64 layer within the output tolerance (normwise <= 5e-3).
A problem whose workspace exceeds the static array is refused on the host."""

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import svdq as S
from tests.gpu_util import dev_bf16, host_bits, make_layer

pytestmark = pytest.mark.gpu

# the first call needs K-split partial sums in the scratch; the second is smaller
CASES = [dict(M=1000, K=3840, N=640, R=128, kind="dit", seed=71),
         dict(M=96, K=256, N=128, R=16, kind="dit", seed=72)]


@pytest.mark.parametrize("packed", [False, True])
def test_noalloc_matches_workspace_entry_point(gpu_lib, packed):
    ops = gpu_lib
    for cfg in CASES:
        print(f"[noalloc] packed={packed} {cfg}", flush=True)
        need = ops.linear_workspace_bytes(cfg["M"], cfg["N"], cfg["K"], cfg["R"])
        assert 0 < need <= ops.noalloc_scratch_bytes()
        d, layer = make_layer(cfg)
        if packed:
            layer = layer.packed()
        x = dev_bf16(d["x"])
        y_ws = ops.linear_w4a4(x, layer)
        y_na = torch.full_like(y_ws, float("nan"))
        ops.linear_w4a4_noalloc(x, layer, y_na)
        torch.cuda.synchronize()
        assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16))
        y64, _, _, _ = S.linear_w4a4(d["x"], d["smooth"], d["qweight"], d["wscales"], d["wcscales"], d["wtscale"],
                                     d["proj_down"], d["proj_up"], d["bias"])
        err = S.normwise_rel_err(F.bf16_to_f64(host_bits(y_na)), y64)
        assert err <= 5e-3, err


def test_noalloc_repeat_is_deterministic(gpu_lib):
    """The same call twice (the array keeps the first call's contents): identical."""
    ops = gpu_lib
    cfg = CASES[0]
    d, layer = make_layer(cfg)
    x = dev_bf16(d["x"])
    y1 = torch.empty((cfg["M"], cfg["N"]), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty_like(y1)
    ops.linear_w4a4_noalloc(x, layer, y1)
    ops.linear_w4a4_noalloc(x, layer, y2)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_noalloc_refuses_oversized_problem(gpu_lib):
    """Real (zero) tensors of a problem whose workspace exceeds the static array: refused
    with SVDQ_ERR_WORKSPACE before anything is enqueued; y is left untouched."""
    ops = gpu_lib
    M, K, N, R = 16896, 10240, 3840, 128
    assert ops.linear_workspace_bytes(M, N, K, R) > ops.noalloc_scratch_bytes()
    bf, u8 = torch.bfloat16, torch.uint8
    dev = "cuda"
    L = ops._lib.lib()
    layer = ops.SVDQLinearWeights(
        N=N, K=K, weight=torch.zeros(L.svdq_repack_weight_bytes(N, K), dtype=u8, device=dev), wscales=None,
        wcscales=torch.zeros(N, dtype=bf, device=dev), wtscale=torch.zeros(1, dtype=bf, device=dev),
        smooth=torch.zeros(K, dtype=bf, device=dev), proj_down=torch.zeros(K, R, dtype=bf, device=dev),
        proj_up=torch.zeros(N, R, dtype=bf, device=dev), bias=None, layout=ops.WEIGHT_PACKED)
    x = torch.zeros(M, K, dtype=bf, device=dev)
    y = torch.full((M, N), 7.0, dtype=bf, device=dev)
    with pytest.raises(ops.SvdqError, match="static scratch"):
        ops.linear_w4a4_noalloc(x, layer, y)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
