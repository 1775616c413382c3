"""SVDQuant weight preparation, restated step by step (oracle; test use only).

The model card "nunchaku-z-image-turbo-svdq" (section "What's stored on disk")
lists the tensors a prepared layer carries (qweight, wscales, wcscales,
wtscale, smooth_factor, proj_down, proj_up; R = 128) and the runtime formula,
and cites SVDQuant; it does not give the preparation steps. They are read from
what the formula needs, in float64:

1. Smoothed weight Ws[n, k] = W[n, k] / smooth[k]: the runtime multiplies x by
   smooth, so (x * smooth) @ Ws^T = x @ W^T.
2. A rank-R part L of Ws. The runtime adds (x @ proj_down) @ proj_up^T, which
   equals (x * smooth) @ (proj_up (proj_down / smooth)^T)^T, so
   L = proj_up (proj_down / smooth[k])^T. Two ways to pick it:
   * ``lowrank_svd``: the best rank-R approximation (truncated SVD, the
     reference optimum), split as proj_up = U sqrt(S), proj_down = smooth * V sqrt(S);
   * ``lowrank_randomized``: the randomized range finder the device runs:
     Y = Ws Omega with a caller-supplied Gaussian Omega [K, R], q rounds of
     Y = Ws orth(Ws^T orth(Y)), Q = orth(Y); proj_up = Q and
     proj_down = smooth * (Ws^T Q), so L = Q Q^T Ws, the best approximation
     within span(Q). orth is Cholesky QR applied twice.
3. The residual with the bf16-rounded factors,
   E[n, k] = (W[n, k] - sum_r proj_up[n, r] proj_down[k, r]) / smooth[k],
   summed in float64 in the order r = 0, 1, ..., R-1 (each product of two
   bf16 values is exact), then one division.
4. Two-level scales: wtscale = 1, wcscales[n] = bf16(max_k |E[n, k]| / (6 * 448))
   (this puts each 16-block's scale in e4m3's range), rounded directly from
   float64 to bf16 (nearest even).
5. W'[n, k] = bf16(E[n, k] / wcscales[n]) (a zero wcscales gives W' = 0 for its
   row), quantised per 16-block with the activation rule and smooth = 1, giving
   qweight [N, K/2] and wscales [K/16, N].
"""

import numpy as np

from . import formats as F
from . import svdq as S

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def smoothed(W_bits, smooth_bits):
    """Ws = W / smooth[k] in float64 [N, K]."""
    return F.bf16_to_f64(W_bits) / F.bf16_to_f64(smooth_bits)[None, :]


def chol_qr(Y):
    """One Cholesky QR step: G = Y^T Y = L L^T, returns Y L^-T (float64).

    A pivot that is not positive (after rounding) makes that column zero, and
    the column takes no further part."""
    Y = np.asarray(Y, dtype=np.float64)
    P = Y.shape[1]
    G = Y.T @ Y
    L = np.zeros((P, P))
    live = np.zeros(P, dtype=bool)
    for j in range(P):
        d = G[j, j] - np.dot(L[j, :j], L[j, :j])
        if d <= 0.0:
            continue
        L[j, j] = np.sqrt(d)
        live[j] = True
        if j + 1 < P:
            L[j + 1:, j] = (G[j + 1:, j] - L[j + 1:, :j] @ L[j, :j]) / L[j, j]
    # T = L^-T restricted to live columns (dead columns of L are zero)
    T = np.zeros((P, P))
    idx = np.flatnonzero(live)
    if idx.size:
        Ll = L[np.ix_(idx, idx)]
        T[np.ix_(idx, idx)] = np.linalg.inv(Ll).T
    return Y @ T


def orth(Y):
    """Cholesky QR twice."""
    return chol_qr(chol_qr(Y))


def lowrank_randomized(W_bits, smooth_bits, omega, iters):
    """Randomized range finder: returns (proj_up64 [N, R], proj_down64 [K, R])."""
    Ws = smoothed(W_bits, smooth_bits)
    Y = Ws @ np.asarray(omega, dtype=np.float64)
    for _ in range(iters):
        Z = orth(Ws.T @ orth(Y))
        Y = Ws @ Z
    Q = orth(Y)
    Bt = Ws.T @ Q
    sm = F.bf16_to_f64(smooth_bits)
    return Q, sm[:, None] * Bt


def lowrank_svd(W_bits, smooth_bits, R):
    """Best rank-R split of Ws (truncated SVD): (proj_up64, proj_down64)."""
    Ws = smoothed(W_bits, smooth_bits)
    U, s, Vt = np.linalg.svd(Ws, full_matrices=False)
    r = np.sqrt(s[:R])
    sm = F.bf16_to_f64(smooth_bits)
    return U[:, :R] * r[None, :], sm[:, None] * (Vt[:R].T * r[None, :])


def residual(W_bits, smooth_bits, pu_bits, pd_bits):
    """E = (W - proj_up proj_down^T) / smooth, float64, r summed in order."""
    acc = F.bf16_to_f64(W_bits).copy()
    if pu_bits is not None and np.shape(pu_bits)[1] > 0:
        pu = F.bf16_to_f64(pu_bits)
        pd = F.bf16_to_f64(pd_bits)
        for r in range(pu.shape[1]):
            acc -= pu[:, r:r + 1] * pd[:, r][None, :]
    return acc / F.bf16_to_f64(smooth_bits)[None, :]


def quantize_residual(E):
    """Steps 4-5: returns (qweight, wscales, wcscales bits, wtscale bits, W' bits)."""
    E = np.asarray(E, dtype=np.float64)
    wc_bits = F.f64_to_bf16(np.abs(E).max(axis=1) / (E2M1_MAX * E4M3_MAX))
    wc = F.bf16_to_f64(wc_bits)
    with np.errstate(divide="ignore", invalid="ignore"):
        Wp = np.where(wc[:, None] > 0, E / wc[:, None], 0.0)
    Wp_bits = F.f64_to_bf16(Wp)
    ones = F.f64_to_bf16(np.ones(E.shape[1]))
    qweight, wscales = S.quantize_act(Wp_bits, ones)
    return qweight, wscales, wc_bits, F.f64_to_bf16(np.ones(1)), Wp_bits


def prepare_weight(W_bits, smooth_bits, omega, iters):
    """The whole preparation with the randomized split. Returns a dict of the
    layer's tensors (bf16 bit patterns / bytes) and the float64 factors."""
    if omega is None or np.shape(omega)[1] == 0:
        pu64 = np.zeros((np.shape(W_bits)[0], 0))
        pd64 = np.zeros((np.shape(W_bits)[1], 0))
    else:
        pu64, pd64 = lowrank_randomized(W_bits, smooth_bits, omega, iters)
    pu_bits, pd_bits = F.f64_to_bf16(pu64), F.f64_to_bf16(pd64)
    E = residual(W_bits, smooth_bits, pu_bits, pd_bits)
    qweight, wscales, wc_bits, wt_bits, _ = quantize_residual(E)
    return dict(qweight=qweight, wscales=wscales, wcscales=wc_bits, wtscale=wt_bits,
                proj_up=pu_bits, proj_down=pd_bits, proj_up64=pu64, proj_down64=pd64)
