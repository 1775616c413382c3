// SVDQuant weight preparation on the device: from a bf16 weight W [N, K] and
// smooth [K], the tensors the model card "nunchaku-z-image-turbo-svdq" (section
// "What's stored on disk") stores for a layer: proj_up [N, R], proj_down [K, R],
// wcscales [N], wtscale [1], qweight [N, K/2], wscales [K/16, N].
//
// The card gives the tensors and the runtime formula, not the preparation. It is
// read from what the formula needs:
//  1. Ws = W / smooth[k] (the runtime multiplies x by smooth);
//  2. rank-R split of Ws by the randomized range finder: Y = Ws Omega (Omega
//     [K, R] Gaussian, supplied by the caller), `iters` rounds of
//     Y = Ws orth(Ws^T orth(Y)), Q = orth(Y); proj_up = Q,
//     proj_down = smooth * (Ws^T Q), so that (x @ proj_down) @ proj_up^T equals
//     (x * smooth) @ (Q Q^T Ws)^T; orth = Cholesky QR twice (fp64 Gram and
//     Cholesky, fp32 products);
//  3. residual E = (W - proj_up proj_down^T) / smooth with the bf16 factors,
//     in fp64, r summed in order (bf16 products are exact in fp64), one division;
//  4. wtscale = 1, wcscales[n] = bf16(max_k |E[n, k]| / (6 * 448)) (fp64 -> bf16
//     nearest even, directly);
//  5. W' = bf16(E / wcscales[n]) (0 for a zero wcscales), quantised by the
//     library's activation quantiser with smooth = 1.
// Steps 3-5 are exact: given the factors, the result equals the float64
// definition bit for bit.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace svdq {

namespace {

constexpr int kRMax = 128;   // fp64 Gram / Cholesky of R x R sit in LDS

// ---------------------------------------------------------------------------
// Tall-skinny products with Ws = W / smooth (fp32), 64 x R per workgroup
// ---------------------------------------------------------------------------

// Y[n, r] = sum_k Ws[n, k] B[k, r]; 256 threads, 32 rows per workgroup (enough
// workgroups to fill the chip at N = 10240), thread (rg, cg) owns rows
// 2rg, 2rg+1 and columns 8cg..8cg+7.
__global__ __launch_bounds__(256) void tsmm_nn_kernel(const uint16_t* __restrict__ W,
                                                      const uint16_t* __restrict__ smooth,
                                                      const float* __restrict__ B, float* __restrict__ Y,
                                                      int N, int K, int R) {
  __shared__ float As[32][32 + 4];    // [k][row]
  __shared__ float Bs[32][kRMax];     // [k][r]
  const int t = threadIdx.x;
  const int n0 = blockIdx.x * 32;
  const int rg = t & 15, cg = t >> 4;
  float acc[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
  for (int k0 = 0; k0 < K; k0 += 32) {
    {   // A: row t / 8, 4 k from (t % 8) * 4 (K % 16 == 0: all 4 in or all past K)
      const int row = t >> 3, kk = (t & 7) * 4;
      const int n = n0 + row, k = k0 + kk;
      float v[4];
      if (n < N && k < K) {
        const u32x2 w = *reinterpret_cast<const u32x2*>(W + (size_t)n * K + k);
        const u32x2 sv = *reinterpret_cast<const u32x2*>(smooth + k);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t wb = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          const uint32_t sb = (sv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          v[e] = bf16lo_to_f32(wb) / bf16lo_to_f32(sb);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) As[kk + e][row] = v[e];
    }
    for (int idx = t; idx < 32 * R; idx += 256) {
      const int kk = idx / R, r = idx % R;
      Bs[kk][r] = (k0 + kk < K) ? B[(size_t)(k0 + kk) * R + r] : 0.0f;
    }
    __syncthreads();
    if (8 * cg < R) {
#pragma unroll 8
      for (int kk = 0; kk < 32; ++kk) {
        float a[2], b[8];
#pragma unroll
        for (int i = 0; i < 2; ++i) a[i] = As[kk][2 * rg + i];
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = Bs[kk][8 * cg + j];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      }
    }
    __syncthreads();
  }
  if (8 * cg < R) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int n = n0 + 2 * rg + i;
      if (n < N)
#pragma unroll
        for (int j = 0; j < 8; ++j) Y[(size_t)n * R + 8 * cg + j] = acc[i][j];
    }
  }
}

// Zp[s, k, r] = sum over n in split s of Ws[n, k] Q[n, r]; 64 k per workgroup
// (blockIdx.x), split s = blockIdx.y over rows [s * rows_per, (s+1) * rows_per).
__global__ __launch_bounds__(256) void tsmm_tn_kernel(const uint16_t* __restrict__ W,
                                                      const uint16_t* __restrict__ smooth,
                                                      const float* __restrict__ Q, float* __restrict__ Zp,
                                                      int N, int K, int R, int rows_per) {
  __shared__ float As[32][64 + 4];    // [n][k]
  __shared__ float Qs[32][kRMax];     // [n][r]
  const int t = threadIdx.x;
  const int k0 = blockIdx.x * 64;
  const int s = blockIdx.y;
  const int nb = s * rows_per, ne = min(N, nb + rows_per);
  const int kg = t & 15, cg = t >> 4;
  float acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
  for (int n0 = nb; n0 < ne; n0 += 32) {
    {   // A: row t / 8, 8 k from (t % 8) * 8
      const int row = t >> 3, kk = (t & 7) * 8;
      const int n = n0 + row, k = k0 + kk;
      float v[8];
      if (n < ne && k < K) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(W + (size_t)n * K + k);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t wb = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          const uint16_t sb = smooth[k + e];
          v[e] = bf16lo_to_f32(wb) / bf16lo_to_f32(sb);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) As[row][kk + e] = v[e];
    }
    for (int idx = t; idx < 32 * R; idx += 256) {
      const int nn = idx / R, r = idx % R;
      Qs[nn][r] = (n0 + nn < ne) ? Q[(size_t)(n0 + nn) * R + r] : 0.0f;
    }
    __syncthreads();
    if (8 * cg < R) {
#pragma unroll 4
      for (int nn = 0; nn < 32; ++nn) {
        float a[4], b[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = As[nn][4 * kg + i];
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = Qs[nn][8 * cg + j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      }
    }
    __syncthreads();
  }
  if (8 * cg < R) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = k0 + 4 * kg + i;
      if (k < K)
#pragma unroll
        for (int j = 0; j < 8; ++j) Zp[((size_t)s * K + k) * R + 8 * cg + j] = acc[i][j];
    }
  }
}

// Z[k, r] = sum_s Zp[s, k, r], splits added in order.
__global__ void sum_splits_kernel(const float* __restrict__ Zp, float* __restrict__ Z, int64_t count, int S) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  float v = 0.0f;
  for (int s = 0; s < S; ++s) v += Zp[(size_t)s * count + i];
  Z[i] = v;
}

// ---------------------------------------------------------------------------
// Cholesky QR: G = Y^T Y (fp64), G = L L^T, T = L^-T, Q = Y T
// ---------------------------------------------------------------------------

constexpr int kGramRows = 128;

// Gp[c] = Y[rows of chunk c]^T Y[rows of chunk c], fp64, thread (bi, bj) owns the
// 8 x 8 block (8bi.., 8bj..).
__global__ __launch_bounds__(256) void gram_kernel(const float* __restrict__ Y, double* __restrict__ Gp,
                                                   int rows, int R) {
  __shared__ float Ys[kGramRows][kRMax];
  const int t = threadIdx.x;
  const int r0 = blockIdx.x * kGramRows;
  const int nr = min(kGramRows, rows - r0);
  for (int idx = t; idx < kGramRows * R; idx += 256) {
    const int rr = idx / R, c = idx % R;
    Ys[rr][c] = rr < nr ? Y[(size_t)(r0 + rr) * R + c] : 0.0f;
  }
  __syncthreads();
  const int nb = R / 8;
  const int bi = t / 16, bj = t % 16;
  if (bi >= nb || bj >= nb) return;
  double acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0;
  for (int rr = 0; rr < nr; ++rr) {
    double a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = (double)Ys[rr][8 * bi + i];
#pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = (double)Ys[rr][8 * bj + j];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
  }
  double* g = Gp + (size_t)blockIdx.x * R * R;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) g[(8 * bi + i) * R + 8 * bj + j] = acc[i][j];
}

// G = sum of the chunk Grams, chunks added in order (one thread per entry).
__global__ void gram_sum_kernel(const double* __restrict__ Gp, double* __restrict__ G, int chunks, int RR) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= RR) return;
  double v = 0.0;
  for (int c = 0; c < chunks; ++c) v += Gp[(size_t)c * RR + i];
  G[i] = v;
}

// One workgroup: right-looking Cholesky of G in LDS (a pivot that is not
// positive makes its column zero), then X = L^-1 right-looking (row j of X is
// divided by L[j][j], then X[i][:] -= L[i][j] X[j][:] for i > j). One barrier
// per step: step j updates with the still unscaled column (row) j times
// 1/pivot, and column (row) j itself is scaled during step j+1, which does not
// touch it otherwise. X is lower triangular like L: its off-diagonal entry
// (i, c) is kept at the mirrored slot (c, i) of the same R x R array, its
// diagonal aside. Output T = L^-T = X^T (fp32, upper triangular). 1024 threads
// as 32 x 32 (ty, tx). Dynamic LDS: R*(R+1) + 2R doubles.
__global__ __launch_bounds__(1024) void chol_inv_kernel(const double* __restrict__ G, int R, float* __restrict__ T) {
  extern __shared__ double lds_d[];
  const int S_ = R + 1;   // padded row stride: column walks hit distinct banks
  double* L = lds_d;
  double* xd = lds_d + R * S_;  // diagonal of X
  double* ld = xd + R;          // diagonal of L
  const int t = threadIdx.x;
  const int tx = t & 31, ty = t >> 5;
  for (int idx = t; idx < R * R; idx += 1024) L[(idx / R) * S_ + idx % R] = G[idx];
  __syncthreads();
  double inv_prev = 0.0;   // 1 / pivot of the previous step
  for (int j = 0; j <= R; ++j) {
    if (j > 0)   // scale column j-1 below the diagonal
      for (int i = j + t; i < R; i += 1024) L[i * S_ + j - 1] *= inv_prev;
    if (j == R) break;
    const double d = L[j * S_ + j];
    const bool live = d > 0.0;
    const double l = live ? sqrt(d) : 0.0;
    const double inv_d = live ? 1.0 / d : 0.0;
    if (t == 0) ld[j] = l;
    // trailing block (j+1 .. R-1)^2, lower part, with the unscaled column j
    for (int i = j + 1 + ty; i < R; i += 32) {
      const double lij = L[i * S_ + j] * inv_d;
      for (int k = j + 1 + tx; k <= i; k += 32) L[i * S_ + k] -= lij * L[k * S_ + j];
    }
    inv_prev = live ? 1.0 / l : 0.0;
    __syncthreads();
  }
  __syncthreads();
  // X = I: clear the upper triangle (X's off-diagonal slots), diagonal 1
  for (int a = ty; a < R; a += 32)
    for (int b = a + 1 + tx; b < R; b += 32) L[a * S_ + b] = 0.0;
  for (int i = t; i < R; i += 1024) xd[i] = 1.0;
  __syncthreads();
  for (int j = 0; j <= R; ++j) {
    if (j > 0) {   // scale row j-1 of X: (j-1, c) at slot (c, j-1), c < j-1; diagonal xd[j-1]
      const double lp = ld[j - 1];
      for (int c = t; c < j; c += 1024) {
        if (c < j - 1) L[c * S_ + j - 1] = lp > 0.0 ? L[c * S_ + j - 1] / lp : 0.0;
        else xd[j - 1] = lp > 0.0 ? xd[j - 1] / lp : 0.0;
      }
    }
    if (j == R) break;
    const double lj = ld[j];
    const double inv_l = lj > 0.0 ? 1.0 / lj : 0.0;
    for (int i = j + 1 + ty; i < R; i += 32) {
      const double lij = L[i * S_ + j] * inv_l;
      for (int c = tx; c <= j; c += 32) {
        const double xjc = c < j ? L[c * S_ + j] : xd[j];   // row j of X, not yet scaled
        L[c * S_ + i] -= lij * xjc;   // X(i, c) at slot (c, i); c <= j < i
      }
    }
    __syncthreads();
  }
  __syncthreads();
  for (int idx = t; idx < R * R; idx += 1024) {
    const int a = idx / R, b = idx % R;
    T[idx] = b > a ? (float)L[a * S_ + b] : (b == a ? (float)xd[a] : 0.0f);
  }
}

// Dynamic LDS: R*R + 64*(R+4) floats.
__global__ __launch_bounds__(256) void right_mul_kernel(const float* __restrict__ A, const float* __restrict__ T,
                                                        float* __restrict__ O, int rows, int R) {
  extern __shared__ float lds_f[];
  float* Ts = lds_f;
  float* As = lds_f + R * R;   // [64][R + 4]
  const int ld = R + 4;
  const int t = threadIdx.x;
  const int n0 = blockIdx.x * 64;
  for (int idx = t; idx < R * R; idx += 256) Ts[idx] = T[idx];
  for (int idx = t; idx < 64 * R; idx += 256) {
    const int rr = idx / R, c = idx % R;
    As[rr * ld + c] = (n0 + rr < rows) ? A[(size_t)(n0 + rr) * R + c] : 0.0f;
  }
  __syncthreads();
  const int rg = t & 15, cg = t >> 4;
  if (8 * cg >= R) return;
  float acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
  for (int k = 0; k < R; ++k) {
    float b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = Ts[k * R + 8 * cg + j];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = As[(4 * rg + i) * ld + k];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a, b[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = n0 + 4 * rg + i;
    if (n < rows)
#pragma unroll
      for (int j = 0; j < 8; ++j) O[(size_t)n * R + 8 * cg + j] = acc[i][j];
  }
}

// proj_up = bf16(Q); proj_down[k, r] = bf16(smooth[k] * Z[k, r]).
__global__ void factors_kernel(const float* __restrict__ Q, const float* __restrict__ Z,
                               const uint16_t* __restrict__ smooth, uint16_t* __restrict__ pu,
                               uint16_t* __restrict__ pd, int N, int K, int R) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nu = (int64_t)N * R, nd = (int64_t)K * R;
  if (i < nu) pu[i] = (uint16_t)f32_to_bf16_rne(Q[i]);
  if (i < nd) pd[i] = (uint16_t)f32_to_bf16_rne(bf16lo_to_f32(smooth[i / R]) * Z[i]);
}

// ---------------------------------------------------------------------------
// Residual, two-level scales, W' (exact)
// ---------------------------------------------------------------------------

// float64 -> bf16 bits, nearest even, directly: |v| in [2^(e-1), 2^e) has
// quantum 2^(e-8), never below the bf16 subnormal quantum 2^-133; scaling by
// it is exact and rint rounds half to even.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double v) {
  if (v == 0.0 || !isfinite(v)) return (uint16_t)(__float_as_uint((float)v) >> 16);
  int e;
  frexp(v, &e);
  const int q = max(e - 8, -133);
  const double out = ldexp(rint(ldexp(v, -q)), q);
  return (uint16_t)(__float_as_uint((float)out) >> 16);
}

constexpr int kResRows = 8;   // rows per workgroup of the residual kernels

// E for kResRows rows at column k: acc = W; acc -= pu[n, r] * pd[k, r] for
// r = 0..R-1 (exact products, one rounding each); E = acc / smooth[k].
template <int NR>
__device__ __forceinline__ void residual_col(const uint16_t* __restrict__ W, const uint16_t* __restrict__ pd,
                                             const double* pus, double sm, int n0, int nrows, int K, int R,
                                             int k, double (&E)[NR]) {
#pragma unroll
  for (int i = 0; i < NR; ++i) E[i] = i < nrows ? (double)bf16lo_to_f32(W[(size_t)(n0 + i) * K + k]) : 0.0;
  const uint16_t* p = pd + (size_t)k * R;
  for (int r = 0; r < R; ++r) {
    const double d = (double)bf16lo_to_f32(p[r]);
#pragma unroll
    for (int i = 0; i < NR; ++i) E[i] = fma(-pus[i * kRMax + r], d, E[i]);
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) E[i] = E[i] / sm;
}

// Two passes over each row block: max |E| per row -> wcscales; then
// W' = bf16(E / wcscales).
__global__ __launch_bounds__(256) void residual_kernel(const uint16_t* __restrict__ W,
                                                       const uint16_t* __restrict__ smooth,
                                                       const uint16_t* __restrict__ pu,
                                                       const uint16_t* __restrict__ pd, int N, int K, int R,
                                                       uint16_t* __restrict__ wc_out, uint16_t* __restrict__ Wp) {
  __shared__ double pus[kResRows * kRMax];
  __shared__ double red[kResRows][256];
  __shared__ double wcs[kResRows];
  const int t = threadIdx.x;
  const int n0 = blockIdx.x * kResRows;
  const int nrows = min(kResRows, N - n0);
  for (int idx = t; idx < kResRows * kRMax; idx += 256) {
    const int i = idx / kRMax, r = idx % kRMax;
    pus[idx] = (i < nrows && r < R) ? (double)bf16lo_to_f32(pu[(size_t)(n0 + i) * R + r]) : 0.0;
  }
  __syncthreads();
  double amax[kResRows];
#pragma unroll
  for (int i = 0; i < kResRows; ++i) amax[i] = 0.0;
  for (int k = t; k < K; k += 256) {
    double E[kResRows];
    residual_col<kResRows>(W, pd, pus, (double)bf16lo_to_f32(smooth[k]), n0, nrows, K, R, k, E);
#pragma unroll
    for (int i = 0; i < kResRows; ++i) amax[i] = fmax(amax[i], fabs(E[i]));
  }
#pragma unroll
  for (int i = 0; i < kResRows; ++i) red[i][t] = amax[i];
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w)
#pragma unroll
      for (int i = 0; i < kResRows; ++i) red[i][t] = fmax(red[i][t], red[i][t + w]);
    __syncthreads();
  }
  if (t < nrows) {
    const uint16_t b = f64_to_bf16_rne(red[t][0] / 2688.0);
    wc_out[n0 + t] = b;
    wcs[t] = (double)bf16lo_to_f32(b);
  }
  __syncthreads();
  for (int k = t; k < K; k += 256) {
    double E[kResRows];
    residual_col<kResRows>(W, pd, pus, (double)bf16lo_to_f32(smooth[k]), n0, nrows, K, R, k, E);
#pragma unroll
    for (int i = 0; i < kResRows; ++i)
      if (i < nrows) Wp[(size_t)(n0 + i) * K + k] = wcs[i] > 0.0 ? f64_to_bf16_rne(E[i] / wcs[i]) : (uint16_t)0;
  }
}

__global__ void fill_u16_kernel(uint16_t* __restrict__ p, uint16_t v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

size_t al(size_t v) { return (v + 255) & ~size_t(255); }

struct PrepWs {
  size_t wp, ones, y, q, z, z2, zp, gp, g, tm, total;
  int splits, rows_per;
};

PrepWs prep_ws(int64_t N, int64_t K, int64_t R) {
  PrepWs w{};
  size_t o = 0;
  w.wp = o; o = al(o + (size_t)N * K * 2);
  w.ones = o; o = al(o + (size_t)K * 2);
  if (R > 0) {
    const int64_t kb = (K + 63) / 64;
    int S = (int)((256 + kb - 1) / kb);
    S = S < 1 ? 1 : (S > 16 ? 16 : S);
    int64_t rp = (N + S - 1) / S;
    rp = (rp + 31) / 32 * 32;
    S = (int)((N + rp - 1) / rp);
    w.splits = S;
    w.rows_per = (int)rp;
    const int64_t big = N > K ? N : K;
    w.y = o; o = al(o + (size_t)N * R * 4);
    w.q = o; o = al(o + (size_t)N * R * 4);
    w.z = o; o = al(o + (size_t)K * R * 4);
    w.z2 = o; o = al(o + (size_t)K * R * 4);
    w.zp = o; o = al(o + (size_t)S * K * R * 4);
    w.gp = o; o = al(o + (size_t)((big + kGramRows - 1) / kGramRows) * R * R * 8);
    w.g = o; o = al(o + (size_t)R * R * 8);
    w.tm = o; o = al(o + (size_t)R * R * 4);
  }
  w.total = o;
  return w;
}

}  // namespace

size_t prep_workspace_bytes(int64_t N, int64_t K, int64_t R) { return prep_ws(N, K, R).total; }

// a <- orth(a) (Cholesky QR twice), b is scratch of the same shape
static hipError_t orth(float* a, float* b, int rows, int R, const PrepWs& w, uint8_t* ws, hipStream_t s) {
  double* gp = reinterpret_cast<double*>(ws + w.gp);
  double* g = reinterpret_cast<double*>(ws + w.g);
  float* tm = reinterpret_cast<float*>(ws + w.tm);
  const int chunks = (rows + kGramRows - 1) / kGramRows;
  const int lds_chol = (R * (R + 1) + 2 * R) * 8;
  const int lds_mul = (R * R + 64 * (R + 4)) * 4;
  static std::atomic<uint64_t> chol_set{0}, mul_set{0};
  hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(&chol_inv_kernel), (kRMax * (kRMax + 1) + 2 * kRMax) * 8,
                                    chol_set);
  if (e != hipSuccess) return e;
  e = set_lds_limit_once(reinterpret_cast<const void*>(&right_mul_kernel), (kRMax * kRMax + 64 * (kRMax + 4)) * 4,
                         mul_set);
  if (e != hipSuccess) return e;
  for (int pass = 0; pass < 2; ++pass) {
    float* in = pass == 0 ? a : b;
    float* out = pass == 0 ? b : a;
    hipLaunchKernelGGL(gram_kernel, dim3(chunks), dim3(256), 0, s, in, gp, rows, R);
    hipLaunchKernelGGL(gram_sum_kernel, dim3((R * R + 255) / 256), dim3(256), 0, s, gp, g, chunks, R * R);
    hipLaunchKernelGGL(chol_inv_kernel, dim3(1), dim3(1024), lds_chol, s, g, R, tm);
    hipLaunchKernelGGL(right_mul_kernel, dim3((rows + 63) / 64), dim3(256), lds_mul, s, in, tm, out, rows, R);
  }
  return hipGetLastError();
}

hipError_t launch_prepare_lowrank(const uint16_t* W, const uint16_t* smooth, const float* omega, int64_t N,
                                  int64_t K, int64_t R, int iters, uint16_t* proj_down, uint16_t* proj_up,
                                  uint8_t* ws, hipStream_t s) {
  const PrepWs w = prep_ws(N, K, R);
  float* y = reinterpret_cast<float*>(ws + w.y);
  float* q = reinterpret_cast<float*>(ws + w.q);
  float* z = reinterpret_cast<float*>(ws + w.z);
  float* z2 = reinterpret_cast<float*>(ws + w.z2);
  float* zp = reinterpret_cast<float*>(ws + w.zp);
  const int n = (int)N, k = (int)K, r = (int)R;
  const dim3 g_nn((n + 31) / 32), g_tn((k + 63) / 64, w.splits);
  const int64_t kr = (int64_t)K * R;
  auto tn = [&](const float* qq, float* out) {
    hipLaunchKernelGGL(tsmm_tn_kernel, g_tn, dim3(256), 0, s, W, smooth, qq, zp, n, k, r, w.rows_per);
    hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((kr + 255) / 256)), dim3(256), 0, s, zp, out, kr,
                       w.splits);
  };
  hipError_t e;
  hipLaunchKernelGGL(tsmm_nn_kernel, g_nn, dim3(256), 0, s, W, smooth, omega, y, n, k, r);
  for (int it = 0; it < iters; ++it) {
    if ((e = orth(y, q, n, r, w, ws, s)) != hipSuccess) return e;
    tn(y, z);
    if ((e = orth(z, z2, k, r, w, ws, s)) != hipSuccess) return e;
    hipLaunchKernelGGL(tsmm_nn_kernel, g_nn, dim3(256), 0, s, W, smooth, z, y, n, k, r);
  }
  if ((e = orth(y, q, n, r, w, ws, s)) != hipSuccess) return e;
  tn(y, z);
  const int64_t cnt = (N > K ? N : K) * R;
  hipLaunchKernelGGL(factors_kernel, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, s, y, z, smooth, proj_up,
                     proj_down, n, k, r);
  return hipGetLastError();
}

hipError_t launch_prepare_residual(const uint16_t* W, const uint16_t* smooth, const uint16_t* proj_down,
                                   const uint16_t* proj_up, int64_t N, int64_t K, int64_t R, uint8_t* qweight,
                                   uint8_t* wscales, uint16_t* wcscales, uint16_t* wtscale, uint8_t* ws,
                                   hipStream_t s) {
  const PrepWs w = prep_ws(N, K, R);
  uint16_t* wp = reinterpret_cast<uint16_t*>(ws + w.wp);
  uint16_t* ones = reinterpret_cast<uint16_t*>(ws + w.ones);
  hipLaunchKernelGGL(residual_kernel, dim3((unsigned)((N + kResRows - 1) / kResRows)), dim3(256), 0, s, W, smooth,
                     proj_up, proj_down, (int)N, (int)K, (int)R, wcscales, wp);
  hipLaunchKernelGGL(fill_u16_kernel, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, s, ones, (uint16_t)0x3F80, K);
  hipLaunchKernelGGL(fill_u16_kernel, dim3(1), dim3(64), 0, s, wtscale, (uint16_t)0x3F80, (int64_t)1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_quant_act(wp, ones, qweight, wscales, N, K, s);
}

}  // namespace svdq
