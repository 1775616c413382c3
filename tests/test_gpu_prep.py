"""GPU parity of the load-time SVDQuant weight preparation (svdq_prepare_weight,
svdq_prepare_residual) against oracle/prep.py.

* Residual, two-level scales and NVFP4 codes, given the bf16 factors: bit-exact
  (qweight, wscales, wcscales, wtscale), since both sides evaluate the same
  float64 definition in the same order.
* The randomized rank-R split (fp32 products, fp64 Gram and Cholesky on the
  device; float64 in the oracle, same omega): proj_up / proj_down within a
  normwise 3e-3 of the oracle's float64 factors (bf16 storage alone gives about
  1e-3), at least 95% of elements equal to the oracle's bf16 rounding, and the
  projection error within 0.1% of the oracle's.
* The prepared layer in svdq_linear_w4a4 against the bf16 product x @ W^T.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import formats as F
from oracle import prep as P
from oracle import svdq as S
from tests.gpu_util import dev_bf16, host_bits, host_u8

pytestmark = pytest.mark.gpu


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def check_residual(ops, W, sm, pu, pd, rows=None):
    """GPU residual stage on the given factors vs the oracle, bit for bit (rows: a
    sample of rows checked, the oracle being row-local)."""
    R = 0 if pu is None else pu.shape[1]
    qw, ws, wc, wt = ops.prepare_residual(dev_bf16(W), dev_bf16(sm), dev_bf16(pd) if R else None,
                                          dev_bf16(pu) if R else None)
    torch.cuda.synchronize()
    sel = slice(None) if rows is None else rows
    E = P.residual(W[sel], sm, pu[sel] if R else None, pd if R else None)
    q_o, s_o, wc_o, wt_o, _ = P.quantize_residual(E)
    assert np.array_equal(host_u8(qw)[sel], q_o)
    assert np.array_equal(host_u8(ws)[:, sel], s_o)
    assert np.array_equal(host_bits(wc)[sel], wc_o)
    assert np.array_equal(host_bits(wt), wt_o)


@pytest.mark.parametrize("N,K,R", [(96, 128, 16), (300, 336, 32), (77, 64, 0), (513, 1024, 128)])
def test_residual_stage_bit_exact(gpu_lib, N, K, R):
    W, sm, _ = workloads.make_prep_weight(N, K, seed=N + K)
    rng = np.random.default_rng(R + 1)
    pu = workloads.f32_to_bf16_bits(rng.standard_normal((N, R)) * 0.05) if R else None
    pd = workloads.f32_to_bf16_bits(rng.standard_normal((K, R)) * 0.05) if R else None
    check_residual(gpu_lib, W, sm, pu, pd)


@pytest.mark.parametrize("N,K,R,iters,strong", [(512, 384, 32, 2, 8), (640, 768, 64, 1, 0), (257, 160, 16, 0, 4),
                                                  (400, 256, 96, 1, 6)])   # R above 64, not a power of two
def test_randomized_split_matches_oracle(gpu_lib, N, K, R, iters, strong):
    W, sm, _ = workloads.make_prep_weight(N, K, seed=3 * N + K, strong=strong)
    omega = workloads.make_omega(K, R, seed=R + iters)
    lay = gpu_lib.prepare_weight(dev_bf16(W), dev_bf16(sm), dev_f32(omega), iters=iters)
    torch.cuda.synchronize()
    pu_g, pd_g = host_bits(lay.proj_up), host_bits(lay.proj_down)
    pu_o, pd_o = P.lowrank_randomized(W, sm, omega, iters)
    for g, o in ((pu_g, pu_o), (pd_g, pd_o)):
        assert S.normwise_rel_err(F.bf16_to_f64(g), o) <= 3e-3
        assert np.mean(g == F.f64_to_bf16(o)) >= 0.95
    Ws = P.smoothed(W, sm)
    smv = F.bf16_to_f64(sm)[:, None]
    e_g = np.linalg.norm(Ws - F.bf16_to_f64(pu_g) @ (F.bf16_to_f64(pd_g) / smv).T)
    e_o = np.linalg.norm(Ws - pu_o @ (pd_o / smv).T)
    assert e_g <= 1.001 * e_o + 1e-6
    # the rest of the preparation, on the device's own factors, is the oracle's exactly
    E = P.residual(W, sm, pu_g, pd_g)
    q_o, s_o, wc_o, wt_o, _ = P.quantize_residual(E)
    assert np.array_equal(host_u8(lay.weight), q_o)
    assert np.array_equal(host_u8(lay.wscales), s_o)
    assert np.array_equal(host_bits(lay.wcscales), wc_o)


def test_full_size_dit_weight_sampled(gpu_lib):
    """The FFN w1 shape (N=10240, K=3840, R=128): factors orthonormal (proj_up) up to
    bf16 rounding, the residual stage bit-exact on sampled rows."""
    N, K, R = 10240, 3840, 128
    W, sm, _ = workloads.make_prep_weight(N, K, seed=77)
    omega = workloads.make_omega(K, R, seed=78)
    lay = gpu_lib.prepare_weight(dev_bf16(W), dev_bf16(sm), dev_f32(omega), iters=2)
    torch.cuda.synchronize()
    pu = F.bf16_to_f64(host_bits(lay.proj_up))
    G = pu.T @ pu
    assert np.abs(G - np.eye(R)).max() < 2e-2
    rows = np.array([0, 1, 4095, 5000, 10238, 10239])
    pu_b, pd_b = host_bits(lay.proj_up), host_bits(lay.proj_down)
    E = P.residual(W[rows], sm, pu_b[rows], pd_b)
    q_o, s_o, wc_o, _, _ = P.quantize_residual(E)
    assert np.array_equal(host_u8(lay.weight)[rows], q_o)
    assert np.array_equal(host_u8(lay.wscales)[:, rows], s_o)
    assert np.array_equal(host_bits(lay.wcscales)[rows], wc_o)


def test_prepared_layer_tracks_the_bf16_linear(gpu_lib):
    N, K, R = 1024, 768, 64
    W, sm, x = workloads.make_prep_weight(N, K, seed=91)
    omega = workloads.make_omega(K, R, seed=92)
    ref = F.bf16_to_f64(x) @ F.bf16_to_f64(W).T
    errs = {}
    for r in (0, R):
        lay = gpu_lib.prepare_weight(dev_bf16(W), dev_bf16(sm), dev_f32(omega[:, :r]) if r else None, iters=2)
        y = gpu_lib.linear_w4a4(dev_bf16(x), lay.packed())
        torch.cuda.synchronize()
        errs[r] = S.normwise_rel_err(F.bf16_to_f64(host_bits(y)), ref)
    assert errs[R] < 0.1, errs
    assert errs[R] < errs[0], errs
