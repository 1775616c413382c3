"""GPU: every tile shape of the packed W4A4 GEMM gives the same output bit for bit, and
that output meets the oracle's gate.

The shapes are forced through svdq_set_gemm_tile (0 automatic, 1 256 x 320, 2 256 x 256,
3 128 x 320, 4 128 x 160 outputs per workgroup). Each output element is the same sequence
of matrix instructions and roundings whatever tile holds it, so any difference is a
tiling bug (a wrong row or column offset, a missed ragged edge, a chunk dealt to the
wrong wave). The gated GEMM has no 128 x 160 shape: forcing 4 there falls back to the
automatic choice, which must still give the same result.

Each case also runs the canonical (on-disk) weight layout, which the kernel reads without a
repack, and canonical activations with the packed weight, and requires the same bits. Cases: ragged M and N over several tiles of every shape,
K not a multiple of the 64-wide panel (so K not a multiple of 32 inside a canonical row), R = 0,
a rank in three residual passes, one GPU's share of the 1024^2 FFN w1
under 8-way tensor parallelism (N = 1280, where the automatic choice is 128 x 160) on
sampled rows, and the gated step with and without w2's quantisation in its epilogue.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import formats as F
from oracle import repack as P
from oracle import svdq as S
from tests.gpu_util import dev_bf16, dev_u8, host_bits, make_layer, within_ulps

pytestmark = pytest.mark.gpu

TILES = (0, 1, 2, 3, 4)


@pytest.fixture
def tile_reset(gpu_lib):
    yield gpu_lib
    gpu_lib.set_gemm_tile(0)


def _gemm_all_tiles(ops, d, layer, qact, ascales, lora_bits):
    """Packed activations with the packed weight under every tile shape; the same with the
    canonical (on-disk) weight read without a repack, and canonical activations with the
    packed weight, must agree bit for bit."""
    R = d["R"]
    qpk = dev_u8(P.repack(qact, ascales))
    lora = dev_bf16(lora_bits) if R > 0 else None
    pl = layer.packed()
    qc, sc = dev_u8(qact), dev_u8(ascales)
    out = {}
    for t in TILES:
        ops.set_gemm_tile(t)
        y = ops.gemm_w4a4(qpk, None, lora, pl, M=d["M"])
        yc = ops.gemm_w4a4(qpk, None, lora, layer, M=d["M"])
        ya = ops.gemm_w4a4(qc, sc, lora, pl)
        torch.cuda.synchronize()
        out[t] = host_bits(y)
        assert np.array_equal(host_bits(yc), out[t]), f"tile {t}: canonical weight differs from packed"
        assert np.array_equal(host_bits(ya), out[t]), f"tile {t}: canonical activations differ from packed"
    ops.set_gemm_tile(0)
    return out


@pytest.mark.parametrize("cfg", [
    dict(M=300, K=640, N=1000, R=32, kind="dit", seed=61),
    dict(M=130, K=336, N=700, R=16, kind="dit", seed=62),       # K % 64 != 0
    dict(M=257, K=512, N=333, R=0, kind="dit", seed=63),        # R = 0
    dict(M=100, K=256, N=480, R=272, kind="dit", seed=64),      # rank in three passes
    dict(M=33, K=64, N=40, R=16, kind="tiny", seed=65),         # one panel, one partial tile
])
def test_tiles_bit_identical(tile_reset, cfg):
    ops = tile_reset
    d, layer = make_layer(cfg)
    qact, ascales = S.quantize_act(d["x"], d["smooth"])
    R = d["R"]
    lora_bits = F.f64_to_bf16(S.lowrank_down(d["x"], d["proj_down"])) if R > 0 else None
    out = _gemm_all_tiles(ops, d, layer, qact, ascales, lora_bits)
    for t in TILES[1:]:
        assert np.array_equal(out[t], out[0]), f"tile {t} differs from the automatic choice"
    y64 = S.gemm_w4a4(qact, ascales, F.bf16_to_f64(lora_bits) if R > 0 else None, d["qweight"], d["wscales"],
                      d["wcscales"], d["wtscale"], d["proj_up"] if R > 0 else None, d["bias"])
    assert S.normwise_rel_err(F.bf16_to_f64(out[0]), y64) <= 5e-3
    assert within_ulps(out[0], y64, 1).mean() >= 0.999


def test_tiles_tp8_shard_sampled_rows(tile_reset):
    """One GPU's share of the 1024^2 FFN w1 at 8-way tensor parallelism (M = 4096,
    K = 3840, N = 1280): every shape bit-identical, the output checked against the
    oracle on 32 sampled rows."""
    ops = tile_reset
    cfg = workloads.SHARDS_TP8_1024["w1"]
    d, layer = make_layer(cfg)
    qact, ascales = S.quantize_act(d["x"], d["smooth"])
    lora_bits = F.f64_to_bf16(S.lowrank_down(d["x"], d["proj_down"]))
    out = _gemm_all_tiles(ops, d, layer, qact, ascales, lora_bits)
    for t in TILES[1:]:
        assert np.array_equal(out[t], out[0]), f"tile {t} differs from the automatic choice"
    rows = np.sort(np.random.default_rng(66).choice(cfg["M"], size=32, replace=False))
    rows[0], rows[-1] = 0, cfg["M"] - 1
    y64 = S.gemm_w4a4(qact[rows], ascales[:, rows], F.bf16_to_f64(lora_bits)[rows], d["qweight"], d["wscales"],
                      d["wcscales"], d["wtscale"], d["proj_up"], d["bias"])
    got = out[0][rows]
    assert S.normwise_rel_err(F.bf16_to_f64(got), y64) <= 5e-3
    assert within_ulps(got, y64, 1).mean() >= 0.999


@pytest.mark.parametrize("cfg", [
    dict(M=130, K=512, N=2 * 384, R=32, kind="dit", seed=67),      # F = 12 panels: partial last tile
    dict(M=300, K=256, N=2 * 1280, R=16, kind="swiglu", seed=68),
])
def test_gated_tiles_bit_identical(tile_reset, cfg):
    """The gated step (h = silu(gate) * up), and the same step writing w2's packed NVFP4
    input: h, and the codes and scales, equal for every forced shape; h within the
    normwise gate of the oracle."""
    ops = tile_reset
    d, layer = make_layer(cfg)
    F_out = d["N"] // 2
    qact, ascales = S.quantize_act(d["x"], d["smooth"])
    lora_bits = F.f64_to_bf16(S.lowrank_down(d["x"], d["proj_down"]))
    qpk = dev_u8(P.repack(qact, ascales))
    lora = dev_bf16(lora_bits)
    pl = layer.packed()
    next_smooth = dev_bf16(F.f64_to_bf16(np.random.default_rng(69).uniform(0.5, 2.0, size=F_out)))
    hs, qs = {}, {}
    for t in TILES:
        ops.set_gemm_tile(t)
        h = ops.gemm_w4a4_gated(qpk, lora, pl, d["M"])
        q2 = torch.zeros(max(1, ops._lib.lib().svdq_packed_act_bytes(d["M"], F_out)), dtype=torch.uint8,
                         device=qpk.device)
        h2, q2 = ops.gemm_w4a4_gated_quant(qpk, lora, pl, d["M"], next_smooth, next_qact=q2)
        torch.cuda.synchronize()
        hs[t] = host_bits(h)
        assert np.array_equal(host_bits(h2), hs[t])
        qs[t] = q2.cpu().numpy()
    ops.set_gemm_tile(0)
    for t in TILES[1:]:
        assert np.array_equal(hs[t], hs[0]), f"tile {t}: h differs"
        assert np.array_equal(qs[t], qs[0]), f"tile {t}: w2's codes differ"
    y64 = S.gemm_w4a4(qact, ascales, F.bf16_to_f64(lora_bits), d["qweight"], d["wscales"], d["wcscales"],
                      d["wtscale"], d["proj_up"], d["bias"])
    h64 = S.swiglu(y64, F_out)
    assert S.normwise_rel_err(F.bf16_to_f64(hs[0]), h64) <= 5e-3
