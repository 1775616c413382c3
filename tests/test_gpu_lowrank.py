"""GPU parity of the down-projection lora_act = bf16(x @ proj_down) against the oracle's
float64 product: each element within bf16 rounding plus fp32 accumulation error.

The down-projection runs inside the fused quantisation kernel: 32 rows per
workgroup, with K split across workgroups (fp32 partials added in a fixed order
by a second kernel) when there are few row blocks, or, for short K, the
split-free form (each workgroup 32 rows and 64 of the columns over all of K).
Covers split and unsplit K, the split-free form (ragged M and K, R = 96), ragged
M, R = 16 .. 256, K = 16 and 10240, and determinism.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import formats as F
from oracle import svdq as S
from tests.gpu_util import dev_bf16, host_bits

pytestmark = pytest.mark.gpu


def check_lora(ops, M, K, R, kind, seed):
    d = workloads.make_linear(M, K, 16, R, kind=kind, seed=seed, with_bias=False)
    x = dev_bf16(d["x"])
    _, _, lora = ops.quantize_act(x, dev_bf16(d["smooth"]), dev_bf16(d["proj_down"]))
    torch.cuda.synchronize()
    got = F.bf16_to_f64(host_bits(lora))
    ref = S.lowrank_down(d["x"], d["proj_down"])
    # bf16 output rounding (2^-9 relative) + fp32 accumulation over K terms
    scale = np.abs(F.bf16_to_f64(d["x"])) @ np.abs(F.bf16_to_f64(d["proj_down"]))
    tol = np.abs(ref) * 2.0 ** -8 + scale * K * 2.0 ** -23 + 1e-30
    bad = np.argwhere(np.abs(got - ref) > tol)
    assert bad.size == 0, f"{len(bad)} elements off, first {bad[:3].tolist()}"
    assert S.normwise_rel_err(got, ref) < 3e-3
    return host_bits(lora)


@pytest.mark.parametrize("M,K,R,kind,seed", [
    (64, 256, 16, "tiny", 1001),
    (4096, 3840, 128, "dit", 1003),     # the 1024^2 activation
    (17000, 256, 32, "dit", 12),        # many rows: two row tiles per wave, ragged last tile
    (100, 10240, 128, "swiglu", 13),    # long K, ragged M
    (33, 16, 16, "tiny", 14),           # a single 16-wide K block
    (48, 384, 256, "dit", 15),          # R above one 128-wide chunk
    (300, 3840, 256, "dit", 16),        # K split over 7 workgroups, two R chunks, ragged M
    (4096, 1280, 128, "swiglu", 17),    # short K: the split-free form (rank split across workgroups)
    (2049, 1040, 96, "dit", 18),        # split-free, ragged M and K, a half-empty column half
    (1000, 1040, 128, "dit", 19),       # split-free, a partial last super-panel
])
def test_lora_down(gpu_lib, M, K, R, kind, seed):
    check_lora(gpu_lib, M, K, R, kind, seed)


@pytest.mark.parametrize("K", [3840, 1280])
def test_lora_down_deterministic(gpu_lib, K):
    """Both fused forms (K split with ordered partial sums at K = 3840, split-free at
    K = 1280) give the same bits on every call."""
    a = check_lora(gpu_lib, 4096, K, 128, "dit", 1003)
    b = check_lora(gpu_lib, 4096, K, 128, "dit", 1003)
    assert np.array_equal(a, b)
