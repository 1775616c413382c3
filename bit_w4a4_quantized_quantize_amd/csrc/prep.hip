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
// Tall-skinny products with Ws = W / smooth (fp32) on the fp32 matrix instruction
// v_mfma_f32_32x32x2_f32: lane l supplies A[l % 32][l / 32] and B[l / 32][l % 32] of
// a 32 x 2 by 2 x 32 product; accumulator element i of lane l is row
// 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32. A workgroup of 4 waves owns a
// 64 x 128 output tile: wave (wm, wn) rows 32 wm .. + 31 and columns 64 wn .. + 63
// (two 32 x 32 blocks; columns past R multiply zeros and are not stored, which keeps
// the loop free of branches so the accumulators stay in place). The reduction walks 32-wide
// chunks through two LDS stages, the next chunk's global loads in registers while
// the current one multiplies.
// ---------------------------------------------------------------------------

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 8 consecutive bf16 of W and the matching 8 of smooth (past the bounds W = 0 and
// smooth = 1; the division waits until the chunk's matrix instructions are issued)
struct Ws8 {
  u32x4 w, s;
};
__device__ __forceinline__ Ws8 ws8_load(const uint16_t* __restrict__ W, const uint16_t* __restrict__ smooth,
                                        int64_t n, int k, bool in, int K) {
  Ws8 r;
  r.w = in ? *reinterpret_cast<const u32x4*>(W + n * K + k) : u32x4{0u, 0u, 0u, 0u};
  r.s = in ? *reinterpret_cast<const u32x4*>(smooth + k) : u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  return r;
}
__device__ __forceinline__ float ws8_value(const Ws8& r, int e) {
  const uint32_t wb = (r.w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
  const uint32_t sb = (r.s[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
  return bf16lo_to_f32(wb) / bf16lo_to_f32(sb);
}

// Y[n, r] = sum_k Ws[n, k] B[k, r] (B [K, R] fp32): 64 rows per workgroup; the
// reduction may be split (blockIdx.y = split s over k in [s kper, (s+1) kper), kper a
// multiple of 32, partial sums to Y + s N R, added in split order by sum_splits_kernel).
// K % 16 == 0, so a thread's 8 k are all inside the range or all past it.
__global__ __launch_bounds__(256) void tsmm_nn_kernel(const uint16_t* __restrict__ W,
                                                      const uint16_t* __restrict__ smooth,
                                                      const float* __restrict__ B, float* __restrict__ Y,
                                                      int N, int K, int R, int kper) {
  __shared__ __attribute__((aligned(16))) float As[2][32][64 + 4];   // [stage][k][row]
  __shared__ __attribute__((aligned(16))) float Bs[2][32][kRMax];    // [stage][k][r]
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int wm = wave & 1, wn = wave >> 1;
  const int n0 = blockIdx.x * 64;
  const int kb = (int)blockIdx.y * kper, ke = min(K, kb + kper);
  Y += (size_t)blockIdx.y * N * R;
  // loads: A row t / 4, k (t % 4) * 8 .. + 7 of the chunk; B pieces t + 256 u (u < 4): k = piece / 32,
  // r = 4 (piece % 32)
  const int ar = t >> 2, ak = (t & 3) * 8;
  Ws8 av;
  f32x4_t bv[4];
  auto load = [&](int k0) {
    av = ws8_load(W, smooth, n0 + ar, k0 + ak, n0 + ar < N && k0 + ak < ke, K);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pc = t + 256 * u, kk = pc >> 5, r = 4 * (pc & 31);
      bv[u] = (k0 + kk < ke && r < R) ? *reinterpret_cast<const f32x4_t*>(B + (size_t)(k0 + kk) * R + r)
                                      : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  auto store = [&](int st) {
#pragma unroll
    for (int e = 0; e < 8; ++e) As[st][ak + e][ar] = ws8_value(av, e);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pc = t + 256 * u;
      *reinterpret_cast<f32x4_t*>(&Bs[st][pc >> 5][4 * (pc & 31)]) = bv[u];
    }
  };
  f32x16_t acc[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.0f;
  const int nk = (ke - kb + 31) / 32;
  if (nk > 0) {
    load(kb);
    store(0);
  }
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const int st = kc & 1;
    if (kc + 1 < nk) load(kb + 32 * (kc + 1));
    float fa[16], fb0[16], fb1[16];   // the chunk's operands, read before its matrix instructions
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) {
      fa[s2] = As[st][2 * s2 + h][32 * wm + l32];
      fb0[s2] = Bs[st][2 * s2 + h][64 * wn + l32];
      fb1[s2] = Bs[st][2 * s2 + h][64 * wn + 32 + l32];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) {
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[s2], fb0[s2], acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[s2], fb1[s2], acc[1], 0, 0, 0);
    }
    if (kc + 1 < nk) store(st ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int col = 64 * wn + 32 * c + l32;
    if (col >= R) continue;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int n = n0 + 32 * wm + 8 * (i >> 2) + 4 * h + (i & 3);
      if (n < N) Y[(size_t)n * R + col] = acc[c][i];
    }
  }
}

// Zp[s, k, r] = sum over n in split s of Ws[n, k] Q[n, r]; 64 k per workgroup
// (blockIdx.x), split s = blockIdx.y over rows [s * rows_per, (s+1) * rows_per).
__global__ __launch_bounds__(256) void tsmm_tn_kernel(const uint16_t* __restrict__ W,
                                                      const uint16_t* __restrict__ smooth,
                                                      const float* __restrict__ Q, float* __restrict__ Zp,
                                                      int N, int K, int R, int rows_per) {
  __shared__ __attribute__((aligned(16))) float As[2][32][64 + 4];   // [stage][n][k]
  __shared__ __attribute__((aligned(16))) float Qs[2][32][kRMax];    // [stage][n][r]
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int wm = wave & 1, wn = wave >> 1;
  const int k0 = blockIdx.x * 64;
  const int sp = blockIdx.y;
  const int nb = sp * rows_per, ne = min(N, nb + rows_per);
  // loads: A row t / 8 of the chunk, k (t % 8) * 8 .. + 7; Q pieces as B above
  const int ar = t >> 3, ak = (t & 7) * 8;
  Ws8 av;
  f32x4_t qv[4];
  auto load = [&](int n0) {
    av = ws8_load(W, smooth, n0 + ar, k0 + ak, n0 + ar < ne && k0 + ak < K, K);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pc = t + 256 * u, nn = pc >> 5, r = 4 * (pc & 31);
      qv[u] = (n0 + nn < ne && r < R) ? *reinterpret_cast<const f32x4_t*>(Q + (size_t)(n0 + nn) * R + r)
                                      : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  auto store = [&](int st) {
    *reinterpret_cast<f32x4_t*>(&As[st][ar][ak]) =
        f32x4_t{ws8_value(av, 0), ws8_value(av, 1), ws8_value(av, 2), ws8_value(av, 3)};
    *reinterpret_cast<f32x4_t*>(&As[st][ar][ak + 4]) =
        f32x4_t{ws8_value(av, 4), ws8_value(av, 5), ws8_value(av, 6), ws8_value(av, 7)};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pc = t + 256 * u;
      *reinterpret_cast<f32x4_t*>(&Qs[st][pc >> 5][4 * (pc & 31)]) = qv[u];
    }
  };
  f32x16_t acc[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.0f;
  const int nc = (ne - nb + 31) / 32;
  if (nc > 0) {
    load(nb);
    store(0);
  }
  __syncthreads();
  for (int ic = 0; ic < nc; ++ic) {
    const int st = ic & 1;
    if (ic + 1 < nc) load(nb + 32 * (ic + 1));
    float fa[16], fb0[16], fb1[16];   // the chunk's operands, read before its matrix instructions
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) {
      fa[s2] = As[st][2 * s2 + h][32 * wm + l32];
      fb0[s2] = Qs[st][2 * s2 + h][64 * wn + l32];
      fb1[s2] = Qs[st][2 * s2 + h][64 * wn + 32 + l32];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) {
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[s2], fb0[s2], acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[s2], fb1[s2], acc[1], 0, 0, 0);
    }
    if (ic + 1 < nc) store(st ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int col = 64 * wn + 32 * c + l32;
    if (col >= R) continue;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int k = k0 + 32 * wm + 8 * (i >> 2) + 4 * h + (i & 3);
      if (k < K) Zp[((size_t)sp * K + k) * R + col] = acc[c][i];
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

// Gp[c] = Y[rows of chunk c]^T Y[rows of chunk c], fp64; each chunk is split over
// four workgroups by quadrant of G (R % 8 == 0), so that the chip has work for
// 4 x (rows / 128) workgroups.
__global__ __launch_bounds__(256) void gram_kernel(const float* __restrict__ Y, double* __restrict__ Gp,
                                                   int rows, int R) {
  // workgroup (chunk, quadrant): quadrant q of G, rows (q / 2) R/2 .., columns (q % 2) R/2 ..;
  // thread (bi, bj) of 16 x 16 owns its 4 x 4 elements (4 bi.., 4 bj.. within the quadrant)
  __shared__ float Ys[kGramRows][kRMax];
  const int t = threadIdx.x;
  const int r0 = blockIdx.x * kGramRows;
  const int nr = min(kGramRows, rows - r0);
  const int half = R / 2;
  const int q = blockIdx.y, gi0 = (q >> 1) * half, gj0 = (q & 1) * half;
  for (int idx = t; idx < kGramRows * R; idx += 256) {
    const int rr = idx / R, c = idx % R;
    Ys[rr][c] = rr < nr ? Y[(size_t)(r0 + rr) * R + c] : 0.0f;
  }
  __syncthreads();
  const int bi = t >> 4, bj = t & 15;
  if (4 * bi >= half || 4 * bj >= half) return;
  const int i0 = gi0 + 4 * bi, j0 = gj0 + 4 * bj;
  double acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
  for (int rr = 0; rr < nr; ++rr) {   // the chunk's rows in order, as a whole-G loop would take them
    double a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = (double)Ys[rr][i0 + i];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = (double)Ys[rr][j0 + j];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
  }
  double* g = Gp + (size_t)blockIdx.x * R * R;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) g[(i0 + i) * R + j0 + j] = acc[i][j];
}

// G = sum of the chunk Grams, chunks added in order (one thread per entry).
__global__ void gram_sum_kernel(const double* __restrict__ Gp, double* __restrict__ G, int chunks, int RR) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= RR) return;
  double v = 0.0;
  for (int c = 0; c < chunks; ++c) v += Gp[(size_t)c * RR + i];
  G[i] = v;
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Cholesky QR's factorisation, in two kernels. G = L L^T right-looking in one
// workgroup (a pivot that is not positive makes its column zero), one barrier per
// step: step j updates with the still unscaled column j times 1/pivot, and column j
// itself is scaled during step j+1, which does not touch it otherwise. Then
// X = L^-1, one column per wave: column c of X is the forward substitution of e_c,
// right-looking (row j of X is divided by L[j][j], then X[i][c] -= L[i][j] X[j][c]
// for i > j), so each element sees the same operations in the same order as in a
// right-looking inversion of the whole matrix. Output T = L^-T = X^T (fp32, upper
// triangular).

// 1024 threads as 32 x 32 (ty, tx). Lout [R, R] (lower triangle and diagonal; the
// upper triangle is not written), ld_out [R] = the diagonal. Dynamic LDS:
// R*(R+1) + R doubles.
__global__ __launch_bounds__(1024) void chol_kernel(const double* G, int R, double* Lout,   // Lout may be G
                                                   double* __restrict__ ld_out) {
  extern __shared__ double lds_d[];
  const int S_ = R + 1;   // padded row stride: column walks hit distinct banks
  double* L = lds_d;
  double* ld = lds_d + R * S_;  // diagonal of L
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
  // L (scaled, diagonal = roots of the pivots) and its diagonal out
  for (int idx = t; idx < R * R; idx += 1024) {
    const int i = idx / R, j = idx % R;
    if (j < i) Lout[idx] = L[i * S_ + j];
    else if (j == i) Lout[idx] = ld[i];
  }
  for (int i = t; i < R; i += 1024) ld_out[i] = ld[i];
}

// T[c, :] = column c of X = L^-1, divided row by row by L[i][i]; wave w of workgroup
// b takes c = 4 b + w. Lane l holds rows l and l + 64 of the column; the pivot row's
// value comes from its lane. Dynamic LDS: R*(R+1) + R doubles (L, 1 / L[j][j]).
__global__ __launch_bounds__(256) void inv_kernel(const double* __restrict__ Lg, const double* __restrict__ ldg,
                                                  int R, float* __restrict__ T) {
  extern __shared__ double lds_d[];
  const int S_ = R + 1;
  double* L = lds_d;
  double* il = lds_d + R * S_;
  const int t = threadIdx.x;
  for (int idx = t; idx < R * R; idx += 256) {
    const int i = idx / R, j = idx % R;
    if (j < i) L[i * S_ + j] = Lg[idx];
  }
  for (int j = t; j < R; j += 256) {
    const double lj = ldg[j];
    il[j] = lj > 0.0 ? 1.0 / lj : 0.0;
  }
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const int c = 4 * (int)blockIdx.x + wave;
  if (c >= R) return;
  const int r0 = lane, r1 = lane + 64;
  double x0 = r0 == c ? 1.0 : 0.0, x1 = r1 == c ? 1.0 : 0.0;   // X(r, c), rows not yet divided
  for (int j = c; j < R - 1; ++j) {
    const double xj = readlane_f64(j < 64 ? x0 : x1, j & 63);
    const double inv_l = il[j];
    const double l0 = L[min(r0, R - 1) * S_ + j] * inv_l, l1 = L[min(r1, R - 1) * S_ + j] * inv_l;
    const double u0 = x0 - l0 * xj, u1 = x1 - l1 * xj;
    x0 = r0 > j && r0 < R ? u0 : x0;
    x1 = r1 > j && r1 < R ? u1 : x1;
  }
  if (r0 < R) {
    const double l = ldg[r0];
    T[c * R + r0] = r0 >= c ? (float)(l > 0.0 ? x0 / l : 0.0) : 0.0f;
  }
  if (r1 < R) {
    const double l = ldg[r1];
    T[c * R + r1] = r1 >= c ? (float)(l > 0.0 ? x1 / l : 0.0) : 0.0f;
  }
}

// O[n, r] = sum_k A[n, k] T[k, r] (A [rows, R], T [R, R], fp32) on the fp32 matrix
// instruction, with the tiles and two-stage chunks of tsmm_nn_kernel.
__global__ __launch_bounds__(256) void right_mul_kernel(const float* __restrict__ A, const float* __restrict__ T,
                                                        float* __restrict__ O, int rows, int R) {
  __shared__ __attribute__((aligned(16))) float As[2][32][64 + 4];   // [stage][k][row]
  __shared__ __attribute__((aligned(16))) float Bs[2][32][kRMax];    // [stage][k][r]
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63, h = lane >> 5, l32 = lane & 31;
  const int wm = wave & 1, wn = wave >> 1;
  const int n0 = blockIdx.x * 64;
  const int ar = t >> 2, ak = (t & 3) * 8;   // A row t / 4, k (t % 4) * 8 .. + 7 of the chunk
  f32x4_t av[2], bv[4];
  auto load = [&](int k0) {
    const bool in = n0 + ar < rows && k0 + ak < R;   // R % 16 == 0: all 8 in or all out
    const float* src = A + (size_t)(in ? n0 + ar : 0) * R + (in ? k0 + ak : 0);
    av[0] = in ? *reinterpret_cast<const f32x4_t*>(src) : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    av[1] = in ? *reinterpret_cast<const f32x4_t*>(src + 4) : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pc = t + 256 * u, kk = pc >> 5, r = 4 * (pc & 31);
      bv[u] = (k0 + kk < R && r < R) ? *reinterpret_cast<const f32x4_t*>(T + (size_t)(k0 + kk) * R + r)
                                     : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  auto store = [&](int st) {
#pragma unroll
    for (int e = 0; e < 8; ++e) As[st][ak + e][ar] = av[e >> 2][e & 3];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pc = t + 256 * u;
      *reinterpret_cast<f32x4_t*>(&Bs[st][pc >> 5][4 * (pc & 31)]) = bv[u];
    }
  };
  f32x16_t acc[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.0f;
  const int nk = (R + 31) / 32;
  load(0);
  store(0);
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const int st = kc & 1;
    if (kc + 1 < nk) load(32 * (kc + 1));
    float fa[16], fb0[16], fb1[16];
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) {
      fa[s2] = As[st][2 * s2 + h][32 * wm + l32];
      fb0[s2] = Bs[st][2 * s2 + h][64 * wn + l32];
      fb1[s2] = Bs[st][2 * s2 + h][64 * wn + 32 + l32];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) {
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[s2], fb0[s2], acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[s2], fb1[s2], acc[1], 0, 0, 0);
    }
    if (kc + 1 < nk) store(st ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int col = 64 * wn + 32 * c + l32;
    if (col >= R) continue;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int n = n0 + 32 * wm + 8 * (i >> 2) + 4 * h + (i & 3);
      if (n < rows) O[(size_t)n * R + col] = acc[c][i];
    }
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
  // this column's proj_down row, 8 values per 16-byte load (R % 16 == 0)
  const u32x4* p = reinterpret_cast<const u32x4*>(pd + (size_t)k * R);
  for (int r8 = 0; r8 < R / 8; ++r8) {
    const u32x4 v = p[r8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = 8 * r8 + e;
      const double d = (double)bf16lo_to_f32((v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
#pragma unroll
      for (int i = 0; i < NR; ++i) E[i] = fma(-pus[i * kRMax + r], d, E[i]);
    }
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
  size_t wp, ones, y, q, z, z2, zp, gp, g, ldv, tm, total;
  int splits, rows_per;   // Ws^T Q: row splits
  int nn_splits, nn_kper;   // Ws B: reduction splits
};

PrepWs prep_ws(int64_t N, int64_t K, int64_t R) {
  PrepWs w{};
  size_t o = 0;
  w.wp = o; o = al(o + (size_t)N * K * 2);
  w.ones = o; o = al(o + (size_t)K * 2);
  if (R > 0) {
    const int64_t kb = (K + 63) / 64;
    int S = (int)(512 / kb);   // about two workgroups per CU
    S = S < 1 ? 1 : (S > 16 ? 16 : S);
    int64_t rp = (N + S - 1) / S;
    rp = (rp + 31) / 32 * 32;
    S = (int)((N + rp - 1) / rp);
    w.splits = S;
    w.rows_per = (int)rp;
    // Ws B: 64-row workgroups, the reduction split so that about two workgroups run per CU
    const int64_t nb = (N + 63) / 64;
    const int64_t nk32 = (K + 31) / 32;
    int64_t Sn = 512 / nb;
    Sn = Sn < 1 ? 1 : (Sn > 16 ? 16 : Sn);
    Sn = Sn > nk32 ? nk32 : Sn;
    const int64_t kper = (nk32 + Sn - 1) / Sn * 32;
    w.nn_kper = (int)kper;
    w.nn_splits = (int)((K + kper - 1) / kper);
    const int64_t big = N > K ? N : K;
    w.y = o; o = al(o + (size_t)N * R * 4);
    w.q = o; o = al(o + (size_t)N * R * 4);
    w.z = o; o = al(o + (size_t)K * R * 4);
    w.z2 = o; o = al(o + (size_t)K * R * 4);
    const size_t zp_tn = (size_t)S * K * R * 4, zp_nn = w.nn_splits > 1 ? (size_t)w.nn_splits * N * R * 4 : 0;
    w.zp = o; o = al(o + (zp_tn > zp_nn ? zp_tn : zp_nn));
    w.gp = o; o = al(o + (size_t)((big + kGramRows - 1) / kGramRows) * R * R * 8);
    w.g = o; o = al(o + (size_t)R * R * 8);
    w.ldv = o; o = al(o + (size_t)R * 8);
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
  double* ldv = reinterpret_cast<double*>(ws + w.ldv);
  float* tm = reinterpret_cast<float*>(ws + w.tm);
  const int chunks = (rows + kGramRows - 1) / kGramRows;
  const int lds_chol = (R * (R + 1) + R) * 8;   // chol_kernel and inv_kernel alike
  static std::atomic<uint64_t> chol_set{0}, inv_set{0};
  hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(&chol_kernel), (kRMax * (kRMax + 1) + kRMax) * 8,
                                    chol_set);
  if (e != hipSuccess) return e;
  e = set_lds_limit_once(reinterpret_cast<const void*>(&inv_kernel), (kRMax * (kRMax + 1) + kRMax) * 8, inv_set);
  if (e != hipSuccess) return e;
  for (int pass = 0; pass < 2; ++pass) {
    float* in = pass == 0 ? a : b;
    float* out = pass == 0 ? b : a;
    hipLaunchKernelGGL(gram_kernel, dim3(chunks, 4), dim3(256), 0, s, in, gp, rows, R);
    hipLaunchKernelGGL(gram_sum_kernel, dim3((R * R + 255) / 256), dim3(256), 0, s, gp, g, chunks, R * R);
    hipLaunchKernelGGL(chol_kernel, dim3(1), dim3(1024), lds_chol, s, g, R, g, ldv);   // L over G
    hipLaunchKernelGGL(inv_kernel, dim3((R + 3) / 4), dim3(256), lds_chol, s, g, ldv, R, tm);
    hipLaunchKernelGGL(right_mul_kernel, dim3((rows + 63) / 64), dim3(256), 0, s, in, tm, out, rows, R);
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
  const dim3 g_nn((n + 63) / 64, w.nn_splits), g_tn((k + 63) / 64, w.splits);
  const int64_t nr = (int64_t)N * R;
  // y = Ws b, through the split partial sums when the reduction is split
  auto nn = [&](const float* b) {
    float* dst = w.nn_splits > 1 ? zp : y;
    hipLaunchKernelGGL(tsmm_nn_kernel, g_nn, dim3(256), 0, s, W, smooth, b, dst, n, k, r, w.nn_kper);
    if (w.nn_splits > 1)
      hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((nr + 255) / 256)), dim3(256), 0, s, zp, y, nr,
                         w.nn_splits);
  };
  const int64_t kr = (int64_t)K * R;
  auto tn = [&](const float* qq, float* out) {
    hipLaunchKernelGGL(tsmm_tn_kernel, g_tn, dim3(256), 0, s, W, smooth, qq, zp, n, k, r, w.rows_per);
    hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((kr + 255) / 256)), dim3(256), 0, s, zp, out, kr,
                       w.splits);
  };
  hipError_t e;
  nn(omega);
  for (int it = 0; it < iters; ++it) {
    if ((e = orth(y, q, n, r, w, ws, s)) != hipSuccess) return e;
    tn(y, z);
    if ((e = orth(z, z2, k, r, w, ws, s)) != hipSuccess) return e;
    nn(z);
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
