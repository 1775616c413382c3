// Load-time repack of the canonical NVFP4 weight (qweight [N, K/2],
// wscales [K/16, N]) into the MFMA-order layout read by the GEMM, and the
// exact inverse (model card "nunchaku-z-image-turbo-svdq": section "Why
// row-major" describes a one-shot load-time pack into a kernel's tile order
// forming a bit-exact pair with its unpack; section "Conversion source"
// reports the round trip bit-exact).
//
// Layout (n-panels of 32 channels, k-panels of 64; NP = ceil(N/32),
// KP = ceil(K/64)): code chunk (p, q) = 1024 bytes at 1024*(p*NP + q), whose
// dword (h*32 + c)*4 + t is the 4 canonical bytes of channel 32q + c at
// k = 64p + 16t + 8h; scale chunk (p, q) = 128 bytes at 1024*KP*NP + 128*(p*NP + q),
// byte c*4 + t = wscales[4p + t, 32q + c]. Out-of-range positions are zero.
// Lane l of a wave reading chunk (p, q) with one 16-byte load at l*16 gets the
// four 32x32x16 fragments (channel l%32, k-half l/32) of the k-panel.
//
// Both directions are pure byte moves: one thread per dword of codes and one
// per scale byte.
#include "common.h"
#include "kernels.h"

namespace svdq {

namespace {

__global__ void repack_codes_kernel(const uint8_t* __restrict__ qweight, uint8_t* __restrict__ packed,
                                    int N, int K, int NP, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t chunk = i >> 8;
  const int d = (int)(i & 255);
  const int p = (int)(chunk / NP), q = (int)(chunk % NP);
  const int h = d >> 7, c = (d >> 2) & 31, t = d & 3;
  const int n = 32 * q + c;
  const int k = 64 * p + 16 * t + 8 * h;
  uint32_t v = 0u;
  if (n < N && k < K) v = *reinterpret_cast<const uint32_t*>(qweight + (size_t)n * (K / 2) + k / 2);
  *reinterpret_cast<uint32_t*>(packed + i * 4) = v;
}

__global__ void repack_scales_kernel(const uint8_t* __restrict__ wscales, uint8_t* __restrict__ packed_scales,
                                     int N, int K, int NP, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t chunk = i >> 7;
  const int b = (int)(i & 127);
  const int p = (int)(chunk / NP), q = (int)(chunk % NP);
  const int c = b >> 2, t = b & 3;
  const int n = 32 * q + c;
  const int blk = 4 * p + t;
  packed_scales[i] = (n < N && 16 * blk < K) ? wscales[(size_t)blk * N + n] : (uint8_t)0;
}

__global__ void unpack_codes_kernel(const uint8_t* __restrict__ packed, uint8_t* __restrict__ qweight,
                                    int N, int K, int NP, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t chunk = i >> 8;
  const int d = (int)(i & 255);
  const int p = (int)(chunk / NP), q = (int)(chunk % NP);
  const int h = d >> 7, c = (d >> 2) & 31, t = d & 3;
  const int n = 32 * q + c;
  const int k = 64 * p + 16 * t + 8 * h;
  if (n < N && k < K)
    *reinterpret_cast<uint32_t*>(qweight + (size_t)n * (K / 2) + k / 2) =
        *reinterpret_cast<const uint32_t*>(packed + i * 4);
}

__global__ void unpack_scales_kernel(const uint8_t* __restrict__ packed_scales, uint8_t* __restrict__ wscales,
                                     int N, int K, int NP, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t chunk = i >> 7;
  const int b = (int)(i & 127);
  const int p = (int)(chunk / NP), q = (int)(chunk % NP);
  const int c = b >> 2, t = b & 3;
  const int n = 32 * q + c;
  const int blk = 4 * p + t;
  if (n < N && 16 * blk < K) wscales[(size_t)blk * N + n] = packed_scales[i];
}

}  // namespace

size_t packed_weight_bytes(int64_t N, int64_t K) {
  const int64_t NP = (N + 31) / 32, KP = (K + 63) / 64;
  return (size_t)(NP * KP) * (1024 + 128);
}

hipError_t launch_repack(const uint8_t* qweight, const uint8_t* wscales, uint8_t* packed,
                         int64_t N, int64_t K, hipStream_t stream) {
  const int NP = (int)((N + 31) / 32), KP = (int)((K + 63) / 64);
  const int64_t chunks = (int64_t)NP * KP;
  const int64_t nd = chunks * 256, ns = chunks * 128;
  hipLaunchKernelGGL(repack_codes_kernel, dim3((unsigned)((nd + 255) / 256)), dim3(256), 0, stream,
                     qweight, packed, (int)N, (int)K, NP, nd);
  hipLaunchKernelGGL(repack_scales_kernel, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, stream,
                     wscales, packed + chunks * 1024, (int)N, (int)K, NP, ns);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* packed, uint8_t* qweight, uint8_t* wscales,
                         int64_t N, int64_t K, hipStream_t stream) {
  const int NP = (int)((N + 31) / 32), KP = (int)((K + 63) / 64);
  const int64_t chunks = (int64_t)NP * KP;
  const int64_t nd = chunks * 256, ns = chunks * 128;
  hipLaunchKernelGGL(unpack_codes_kernel, dim3((unsigned)((nd + 255) / 256)), dim3(256), 0, stream,
                     packed, qweight, (int)N, (int)K, NP, nd);
  hipLaunchKernelGGL(unpack_scales_kernel, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, stream,
                     packed + chunks * 1024, wscales, (int)N, (int)K, NP, ns);
  return hipGetLastError();
}

}  // namespace svdq
