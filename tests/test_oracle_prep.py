"""Pins of the oracle's SVDQuant weight preparation (oracle/prep.py): the
Cholesky QR against orthonormality and the triangular factor, the rank-R split
against the Eckart-Young optimum computed from eigenvalues (a different
routine), exact recovery of exactly-low-rank weights, the residual against an
exact rational brute force, the two-level scale rule and its range, the R = 0
reduction to plain weight quantisation, and the layer's fidelity to x @ W^T."""

from fractions import Fraction

import numpy as np
import pytest

import workloads
from oracle import formats as F
from oracle import prep as P
from oracle import svdq as S


def bf(a):
    return workloads.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def weights(N, K, seed, decay=False):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((N, K)) * 0.02
    if decay:   # a spectrum with a few strong directions, as in trained weights
        A = rng.standard_normal((N, 8)) * np.geomspace(1.0, 0.05, 8)[None, :]
        W = W + A @ rng.standard_normal((8, K)) * 0.05
    smooth = rng.uniform(0.25, 2.0, K)
    return bf(W), bf(smooth)


def test_chol_qr_orthonormal_and_triangular():
    rng = np.random.default_rng(1)
    Y = rng.standard_normal((200, 16)) @ np.diag(np.geomspace(1, 1e-3, 16))
    Q = P.orth(Y)
    assert np.allclose(Q.T @ Q, np.eye(16), atol=1e-12)
    Rm = Q.T @ Y                      # Y = Q R with R upper triangular, positive diagonal
    assert np.allclose(np.tril(Rm, -1), 0, atol=1e-10)
    assert (np.diag(Rm) > 0).all()
    assert np.allclose(Q @ Rm, Y, atol=1e-12)


def test_chol_qr_drops_a_dependent_column():
    rng = np.random.default_rng(2)
    Y = rng.standard_normal((50, 4))
    Y[:, 2] = Y[:, 0] * 3.0
    Q = P.chol_qr(Y)
    assert np.all(np.isfinite(Q))
    nz = np.linalg.norm(Q, axis=0) > 0.5
    assert nz.sum() == 3 and not nz[2] or nz.sum() == 4


def test_svd_split_is_the_eckart_young_optimum():
    W, sm = weights(96, 64, 3, decay=True)
    R = 8
    pu, pd = P.lowrank_svd(W, sm, R)
    Ws = P.smoothed(W, sm)
    L = pu @ (pd / F.bf16_to_f64(sm)[:, None]).T
    err2 = np.linalg.norm(Ws - L) ** 2
    ev = np.sort(np.linalg.eigvalsh(Ws.T @ Ws))[::-1]
    assert np.isclose(err2, ev[R:].sum(), rtol=1e-9)


def test_randomized_split_recovers_exactly_low_rank_weights():
    rng = np.random.default_rng(4)
    N, K, R = 80, 48, 6
    # small integers: the rank-6 product (|entries| <= 24) is exact in bf16
    W = bf((rng.integers(-2, 3, (N, R)) @ rng.integers(-2, 3, (R, K))) * 0.0625)
    sm = bf(np.ones(K))
    omega = rng.standard_normal((K, R))
    pu, pd = P.lowrank_randomized(W, sm, omega, 0)
    Ws = P.smoothed(W, sm)
    assert np.linalg.norm(Ws - pu @ pd.T) <= 1e-9 * np.linalg.norm(Ws)
    assert np.allclose(pu.T @ pu, np.eye(R), atol=1e-12)


@pytest.mark.parametrize("gap,slack", [(True, 1.001), (False, 1.10)])
def test_randomized_split_is_near_optimal(gap, slack):
    """With a spectral gap after R, two power rounds reach the optimum; on a flat
    spectrum (no gap) the projection error stays within 10% of it."""
    rng = np.random.default_rng(5)
    N, K, R = 128, 96, 8
    W = rng.standard_normal((N, K)) * 0.02
    if gap:
        W = W + (rng.standard_normal((N, R)) * np.geomspace(1.0, 0.5, R)[None, :]) @ rng.standard_normal((R, K)) * 0.2
    W = bf(W)
    sm = bf(rng.uniform(0.5, 2.0, K))
    omega = np.random.default_rng(6).standard_normal((K, R))
    Ws = P.smoothed(W, sm)
    smv = F.bf16_to_f64(sm)
    pu_o, pd_o = P.lowrank_svd(W, sm, R)
    opt = np.linalg.norm(Ws - pu_o @ (pd_o / smv[:, None]).T)
    pu, pd = P.lowrank_randomized(W, sm, omega, 2)
    got = np.linalg.norm(Ws - pu @ (pd / smv[:, None]).T)
    assert opt * (1 - 1e-12) <= got <= slack * opt, (got, opt)


def test_residual_exact_rational_brute_force():
    W, sm = weights(6, 32, 7)
    rng = np.random.default_rng(8)
    pu = bf(rng.standard_normal((6, 4)) * 0.1)
    pd = bf(rng.standard_normal((32, 4)) * 0.1)
    E = P.residual(W, sm, pu, pd)
    Wf, smf, puf, pdf = (F.bf16_to_f64(a) for a in (W, sm, pu, pd))
    for n in range(6):
        for k in range(32):
            terms = [Fraction(float(puf[n, r])) * Fraction(float(pdf[k, r])) for r in range(4)]
            num = Fraction(float(Wf[n, k])) - sum(terms)
            exact = num / Fraction(float(smf[k]))
            mag = (abs(Fraction(float(Wf[n, k]))) + sum(abs(t) for t in terms)) / abs(Fraction(float(smf[k])))
            assert abs(Fraction(float(E[n, k])) - exact) <= mag * Fraction(6, 2 ** 53)


def test_two_level_scales_and_range():
    W, sm = weights(40, 64, 9)
    E = P.residual(W, sm, None, None)
    qw, ws, wc, wt, Wp = P.quantize_residual(E)
    assert F.bf16_to_f64(wt)[0] == 1.0
    wcv = F.bf16_to_f64(wc)
    amax = np.abs(E).max(axis=1)
    # wcscales is the bf16 rounding of amax / 2688 (within half a bf16 ulp, at most 2^-8 relative)
    assert np.all(np.abs(wcv - amax / 2688.0) <= 2.0 ** -8 * amax / 2688.0 * 1.0001)
    # every W' sits inside +-6 * 448 (up to the bf16 rounding of wcscales) and its
    # block scales are normal e4m3 numbers for the row maximum
    Wpv = F.bf16_to_f64(Wp)
    assert np.abs(Wpv).max() <= 6 * 448 * (1 + 2.0 ** -7)
    dq = S.dequant(qw, ws)
    # NVFP4 relative block error: at most a quarter of the block's amax per element
    blocks = Wpv.reshape(40, 4, 16)
    err = np.abs(dq.reshape(40, 4, 16) - blocks)
    assert np.all(err <= np.abs(blocks).max(axis=2, keepdims=True) / 4 + 1e-12)


def test_rank_zero_is_plain_weight_quantisation():
    W, sm = weights(32, 48, 10)
    out = P.prepare_weight(W, sm, None, 0)
    E = F.bf16_to_f64(W) / F.bf16_to_f64(sm)[None, :]
    wc = F.f64_to_bf16(np.abs(E).max(axis=1) / 2688.0)
    Wp = F.f64_to_bf16(E / F.bf16_to_f64(wc)[:, None])
    qa, sa = S.quantize_act(Wp, F.f64_to_bf16(np.ones(48)))
    assert np.array_equal(out["qweight"], qa) and np.array_equal(out["wscales"], sa)
    assert np.array_equal(out["wcscales"], wc)


@pytest.mark.parametrize("R", [0, 16])
def test_prepared_layer_approximates_the_bf16_linear(R):
    """The prepared layer run through the oracle's W4A4 formula stays close to x @ W^T,
    and the low-rank branch makes it closer on weights with strong directions."""
    M, K, N = 64, 128, 96
    W, _ = weights(N, K, 11, decay=True)
    d = workloads.make_linear(M, K, N, 0, kind="dit", seed=12)
    x, sm = d["x"], d["smooth"]
    omega = np.random.default_rng(13).standard_normal((K, R)) if R else None
    out = P.prepare_weight(W, sm, omega, 2)
    y64, _, _, _ = S.linear_w4a4(x, sm, out["qweight"], out["wscales"], out["wcscales"], out["wtscale"],
                                 out["proj_down"] if R else None, out["proj_up"] if R else None, None)
    ref = F.bf16_to_f64(x) @ F.bf16_to_f64(W).T
    err = S.normwise_rel_err(y64, ref)
    assert err < 0.12, err
    if R:
        out0 = P.prepare_weight(W, sm, None, 0)
        y0, _, _, _ = S.linear_w4a4(x, sm, out0["qweight"], out0["wscales"], out0["wcscales"],
                                    out0["wtscale"], None, None, None)
        assert err < S.normwise_rel_err(y0, ref)
