// Activation quantisation quant(x * smooth) for the SVDQuant W4A4 layer
// (model card "nunchaku-z-image-turbo-svdq", section "What's stored on disk":
// the activation operand of scaled_mma, with per-16-K e4m3 block scales).
//
// Per row m and 16-block b: v = x * smooth (fp32, exact for bf16 x bf16),
// s = max|v| / 6 -> e4m3 (nearest even, saturating at 448) = ascales[b, m],
// codes = E2M1 nearest even of v / s_d (saturating, sign kept), packed two per
// byte with the even k in the low nibble.
//
// Exactness of the code decision without a division (see common.h): v has at
// most 16 significant bits and s_d at most 4, so v / s_d is either exactly an
// E2M1 rounding midpoint or at least 2^-16 (relative) away from every
// midpoint. q = v * (1/s_d), with the reciprocal within about 1 unit in the
// last place, is within 3 units of v / s_d; rounding q to 21 significant bits
// puts an exact midpoint back exactly on it and leaves every other quotient on
// its side of every midpoint; the hardware E2M1 conversion then rounds ties to
// even. The scale itself is e4m3(max|v| * RN(1/6)), equal to the exact rule.
//
// With a static global activation scale g (calibrated offline; blog page "Z-Image
// NVFP4 ...", the Comfy-Org checkpoint's calibrated static activation scales) the
// block scale is e4m3(max|v| / (6 g)) and the codes E2M1(v / (s_d g)), decided
// exactly by the same rounding scheme (common.h, BlockScale).
//
// HBM-bound: one workgroup covers 32 rows x 256 columns; each lane loads 8
// consecutive bf16 (16 bytes) per row, a wave reads two 512-byte row
// segments, and the pair of lanes holding one 16-block exchanges its maximum
// with a lane swap. Codes leave as one dword per lane (contiguous per row);
// scales are staged in LDS and leave as 32-byte runs of the [K/16, M] layout.
#include "common.h"
#include "kernels.h"

namespace svdq {

namespace {

constexpr int kRows = 32;     // rows per workgroup
constexpr int kChunk = 256;   // K elements per workgroup (16 blocks)
constexpr int kThreads = 256;


// STATIC: block scales relative to the global activation scale *gscale (see common.h).
template <bool STATIC>
__global__ __launch_bounds__(kThreads) void quant_act_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ smooth,
    uint8_t* __restrict__ qact, uint8_t* __restrict__ ascales, int M, int K, const uint16_t* __restrict__ gscale) {
  __shared__ uint8_t s_scale[kChunk / 16][kRows];
  BlockScale<STATIC> bs;
  bs.init(gscale);

  const int tid = threadIdx.x;
  const int kk = tid & 31;        // 8-element group within the chunk
  const int rsub = tid >> 5;      // 0..7
  const int m_base = blockIdx.x * kRows;
  const int k0 = blockIdx.y * kChunk + kk * 8;
  const bool k_in = k0 < K;       // both halves of a block agree (K % 16 == 0)

  float sm[8];
  if (k_in) {
    const u32x4 s = *reinterpret_cast<const u32x4*>(smooth + k0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sm[2 * j] = bf16lo_to_f32(s[j]);
      sm[2 * j + 1] = bf16hi_to_f32(s[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) sm[j] = 0.0f;
  }

#pragma unroll
  for (int i = 0; i < kRows / 8; ++i) {
    const int mr = rsub + 8 * i;
    const int m = m_base + mr;
    const bool ok = k_in && m < M;
    float v[8];
    float amax = 0.0f;
    if (ok) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(x + (size_t)m * K + k0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = bf16lo_to_f32(w[j]) * sm[2 * j];
        v[2 * j + 1] = bf16hi_to_f32(w[j]) * sm[2 * j + 1];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0.0f;
    }
    // the other half of this 16-block sits in the neighbouring lane (a DPP lane swap)
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(amax), 0xB1, 0xF, 0xF, false)));

    const uint32_t sc = bs.code(amax);
    const float sd = bs.divisor(sc);
    const float inv = sd > 0.0f ? scale_reciprocal(sd) : 0.0f;

    uint32_t packed = 0u;
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, snap21(v[0] * inv), snap21(v[1] * inv), 1.0f, 0);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, snap21(v[2] * inv), snap21(v[3] * inv), 1.0f, 1);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, snap21(v[4] * inv), snap21(v[5] * inv), 1.0f, 2);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, snap21(v[6] * inv), snap21(v[7] * inv), 1.0f, 3);

    if (ok) {
      *reinterpret_cast<uint32_t*>(qact + (size_t)m * (K / 2) + k0 / 2) = packed;
      if ((kk & 1) == 0) s_scale[kk >> 1][mr] = (uint8_t)sc;
    }
  }
  __syncthreads();

  // scales: [K/16, M] layout, 32 consecutive bytes per block row
  const int kb0 = blockIdx.y * (kChunk / 16);
#pragma unroll
  for (int u = 0; u < (kChunk / 16) * kRows / kThreads; ++u) {
    const int idx = tid + u * kThreads;
    const int kbl = idx / kRows;
    const int mr = idx % kRows;
    const int m = m_base + mr;
    const int kb = kb0 + kbl;
    if (m < M && kb * 16 < K) ascales[(size_t)kb * M + m] = s_scale[kbl][mr];
  }
}

// Calibration of the static global activation scale, pass 1: the maximum of
// |x * smooth| over this workgroup's 32 rows x 256 columns (the quantiser's tiling).
__global__ __launch_bounds__(kThreads) void calib_amax_kernel(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ smooth, int M, int K,
                                                              float* __restrict__ partial) {
  __shared__ float s_max[kThreads / 64];
  const int tid = threadIdx.x;
  const int kk = tid & 31;
  const int rsub = tid >> 5;
  const int k0 = blockIdx.y * kChunk + kk * 8;
  float amax = 0.0f;
  if (k0 < K) {
    const u32x4 sv = *reinterpret_cast<const u32x4*>(smooth + k0);
#pragma unroll
    for (int i = 0; i < kRows / 8; ++i) {
      const int m = blockIdx.x * kRows + rsub + 8 * i;
      if (m < M) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(x + (size_t)m * K + k0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          amax = fmaxf(amax, fabsf(bf16lo_to_f32(w[j]) * bf16lo_to_f32(sv[j])));
          amax = fmaxf(amax, fabsf(bf16hi_to_f32(w[j]) * bf16hi_to_f32(sv[j])));
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((tid & 63) == 0) s_max[tid >> 6] = amax;
  __syncthreads();
  if (tid == 0) {
    float r = s_max[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) r = fmaxf(r, s_max[w]);
    partial[(size_t)blockIdx.y * gridDim.x + blockIdx.x] = r;
  }
}

// Pass 2 (one workgroup): gscale = bf16(max / (6 * 448)), or 1 for a zero maximum.
// The quotient is taken in fp64 (correctly rounded) and then rounded to fp32 and to
// bf16: a bf16 rounding midpoint (9 significant bits) times 2688 against the
// maximum (16 bits) is either equal or at least 2^-16 apart, so neither earlier
// rounding changes the bf16 result.
__global__ __launch_bounds__(256) void calib_finish_kernel(const float* __restrict__ partial, int n,
                                                           uint16_t* __restrict__ gscale) {
  __shared__ float s_max[4];
  float amax = 0.0f;
  for (int i = threadIdx.x; i < n; i += 256) amax = fmaxf(amax, partial[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = amax;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float m = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    const float g = m > 0.0f ? (float)((double)m / 2688.0) : 1.0f;
    gscale[0] = (uint16_t)f32_to_bf16_rne(g);
  }
}

}  // namespace

size_t calibrate_workspace_bytes(int64_t M, int64_t K) {
  return (size_t)((M + kRows - 1) / kRows) * (size_t)((K + kChunk - 1) / kChunk) * sizeof(float);
}

hipError_t launch_calibrate(const uint16_t* x, const uint16_t* smooth, int64_t M, int64_t K, uint16_t* gscale,
                            float* workspace, hipStream_t stream) {
  dim3 grid((unsigned)((M + kRows - 1) / kRows), (unsigned)((K + kChunk - 1) / kChunk));
  hipLaunchKernelGGL(calib_amax_kernel, grid, dim3(kThreads), 0, stream, x, smooth, (int)M, (int)K, workspace);
  hipLaunchKernelGGL(calib_finish_kernel, dim3(1), dim3(256), 0, stream, workspace, (int)(grid.x * grid.y), gscale);
  return hipGetLastError();
}

hipError_t launch_quant_act(const uint16_t* x, const uint16_t* smooth, uint8_t* qact,
                            uint8_t* ascales, int64_t M, int64_t K, hipStream_t stream, const uint16_t* gscale) {
  dim3 grid((unsigned)((M + kRows - 1) / kRows), (unsigned)((K + kChunk - 1) / kChunk));
  if (gscale != nullptr)
    hipLaunchKernelGGL(quant_act_kernel<true>, grid, dim3(kThreads), 0, stream, x, smooth, qact, ascales, (int)M,
                       (int)K, gscale);
  else
    hipLaunchKernelGGL(quant_act_kernel<false>, grid, dim3(kThreads), 0, stream, x, smooth, qact, ascales, (int)M,
                       (int)K, gscale);
  return hipGetLastError();
}

}  // namespace svdq
