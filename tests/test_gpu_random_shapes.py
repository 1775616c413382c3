"""GPU parity over seeded random shapes, beside the hand-picked cases of the other
files: ragged M and N, any K that is a multiple of 16 (the format's only
constraint), ranks R = 0 .. 256 (multiples of 16, the kernels' constraint),
canonical and packed layouts, with and without bias.

- the whole layer against the oracle's float64 evaluation, with the normwise 5e-3
  gate and the elementwise bound of the arithmetic (see test_gpu_linear.py);
- the activation codes and scales of the fused quantisation + down-projection,
  bit for bit, in both output layouts.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import svdq as S
from oracle import repack as P
from tests.gpu_util import dev_bf16, host_u8
from tests.test_gpu_linear import linear_case

pytestmark = pytest.mark.gpu

KINDS = ("dit", "swiglu", "tiny")


def random_cfg(rng, max_m=600, max_n=700, max_k16=200):
    return dict(M=int(rng.integers(1, max_m + 1)), N=int(rng.integers(1, max_n + 1)),
                K=16 * int(rng.integers(1, max_k16 + 1)), R=16 * int(rng.integers(0, 17)),
                kind=KINDS[int(rng.integers(0, len(KINDS)))], seed=int(rng.integers(0, 2 ** 31)))


@pytest.mark.parametrize("case", range(12))
def test_linear_random_shapes(gpu_lib, case):
    rng = np.random.default_rng(7100 + case)
    cfg = random_cfg(rng)
    packed = bool(case % 2)
    with_bias = case % 3 != 0
    print(f"case {case}: {cfg} packed={packed} bias={with_bias}", flush=True)
    linear_case(gpu_lib, cfg, packed=packed, with_bias=with_bias)


@pytest.mark.parametrize("case", range(10))
def test_quant_random_shapes_bit_exact(gpu_lib, case):
    rng = np.random.default_rng(7200 + case)
    cfg = random_cfg(rng, max_m=2000, max_n=16, max_k16=700)
    M, K, R = cfg["M"], cfg["K"], cfg["R"]
    print(f"case {case}: M={M} K={K} R={R} kind={cfg['kind']}", flush=True)
    d = workloads.make_linear(M, K, 16, R, kind=cfg["kind"], seed=cfg["seed"], with_bias=False)
    q_ref, s_ref = S.quantize_act(d["x"], d["smooth"])
    pd = dev_bf16(d["proj_down"]) if R > 0 else None
    # canonical
    q, s, _ = gpu_lib.quantize_act(dev_bf16(d["x"]), dev_bf16(d["smooth"]), pd)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(s), s_ref)
    assert np.array_equal(host_u8(q), q_ref)
    # packed: the oracle's unpack of the whole buffer gives the canonical codes back
    buf, _, _ = gpu_lib.quantize_act(dev_bf16(d["x"]), dev_bf16(d["smooth"]), pd, packed=True)
    torch.cuda.synchronize()
    q2, s2 = P.unpack(host_u8(buf), M, K)
    assert np.array_equal(q2, q_ref) and np.array_equal(s2, s_ref)
