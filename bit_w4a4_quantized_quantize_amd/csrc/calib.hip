// Measurement helpers, not part of the layer: the sustained rate of the matrix
// instruction the NVFP4 GEMM runs (v_mfma_f32_32x32x16_f16), and of the
// block-scaled one the MXFP4 variant runs, on operands the caller chooses, with the shader clock sampled in the kernel, and a plain
// streaming device copy. They calibrate the roofline figures the benchmark
// reports next to the published peaks: the chip power-limits its clock under
// sustained matrix work, and by how much depends on how many operand bits
// toggle, so the operand table decides what "sustained" means.
#include "common.h"
#include "kernels.h"

namespace svdq {

namespace {

constexpr int kCalibWaves = 8;     // two waves per SIMD, as in the GEMM
constexpr int kCalibFrags = 8;     // operand fragments per lane
constexpr int kCalibTables = 64;   // distinct per-wave operand sets in the table

// Each wave holds the GEMM's accumulator footprint (2 x 5 tiles of 32 x 32,
// 160 registers) and eight f16 operand fragments. One iteration issues 20
// independent-accumulator matrix instructions whose operand pairs all differ
// from the previous instruction's, so the operand bits keep toggling. Wave 0,
// lane 0 of every workgroup records the core-clock and the constant-rate
// counters at its start and end.
__global__ __launch_bounds__(64 * kCalibWaves) void calib_mfma_kernel(const f16x8* __restrict__ table,
                                                                      int64_t iters, float* __restrict__ out,
                                                                      uint64_t* __restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int set = (int)((blockIdx.x * kCalibWaves + wave) % kCalibTables);
  f16x8 f[kCalibFrags];
#pragma unroll
  for (int i = 0; i < kCalibFrags; ++i) f[i] = table[(set * kCalibFrags + i) * 64 + lane];
  f32x16 acc[10];
#pragma unroll
  for (int t = 0; t < 10; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;

  const bool timer = threadIdx.x == 0;
  uint64_t c0 = 0, w0 = 0;
  if (timer) {
    c0 = (uint64_t)clock64();
    w0 = (uint64_t)wall_clock64();
  }
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 5; ++j)
        acc[5 * i + j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f[i], f[2 + j], acc[5 * i + j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 5; ++j)
        acc[5 * i + j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f[7 - i], f[j], acc[5 * i + j], 0, 0, 0);
  }
  if (timer) {
    const uint64_t c1 = (uint64_t)clock64();
    const uint64_t w1 = (uint64_t)wall_clock64();
    uint64_t* c = clocks + 4 * blockIdx.x;
    c[0] = c0;
    c[1] = c1;
    c[2] = w0;
    c[3] = w1;
  }
  float s = 0.0f;
#pragma unroll
  for (int t = 0; t < 10; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[t][r];
  out[(size_t)blockIdx.x * 64 * kCalibWaves + threadIdx.x] = s;
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// The same measurement for the block-scaled matrix instruction of the MXFP4 variant,
// v_mfma_scale_f32_32x32x64_f8f6f4, with FMT the operand format of both sides (4 = fp4
// E2M1: the first 16 bytes of each operand are used; 0 = fp8 e4m3: all 32 bytes) and
// unit E8M0 scales. Operands are built from the table's bytes: fragment i alone (fp4),
// or fragments i and i+1 (fp8).
template <int FMT>
__global__ __launch_bounds__(64 * kCalibWaves) void calib_mfma_scaled_kernel(const u32x4* __restrict__ table,
                                                                             int64_t iters, float* __restrict__ out,
                                                                             uint64_t* __restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int set = (int)((blockIdx.x * kCalibWaves + wave) % kCalibTables);
  u32x4 raw[kCalibFrags];
#pragma unroll
  for (int i = 0; i < kCalibFrags; ++i) raw[i] = table[(set * kCalibFrags + i) * 64 + lane];
  i32x8 f[kCalibFrags];
#pragma unroll
  for (int i = 0; i < kCalibFrags; ++i) {
    const u32x4 a = raw[i];
    const u32x4 b = FMT == 4 ? zero4() : raw[(i + 1) % kCalibFrags];
    f[i] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
  }
  f32x16 acc[10];
#pragma unroll
  for (int t = 0; t < 10; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;

  const bool timer = threadIdx.x == 0;
  uint64_t c0 = 0, w0 = 0;
  if (timer) {
    c0 = (uint64_t)clock64();
    w0 = (uint64_t)wall_clock64();
  }
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 5; ++j)
        acc[5 * i + j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f[i], f[2 + j], acc[5 * i + j], FMT, FMT, 0,
                                                                         127, 0, 127);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 5; ++j)
        acc[5 * i + j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f[7 - i], f[j], acc[5 * i + j], FMT, FMT, 0,
                                                                         127, 0, 127);
  }
  if (timer) {
    const uint64_t c1 = (uint64_t)clock64();
    const uint64_t w1 = (uint64_t)wall_clock64();
    uint64_t* c = clocks + 4 * blockIdx.x;
    c[0] = c0;
    c[1] = c1;
    c[2] = w0;
    c[3] = w1;
  }
  float s = 0.0f;
#pragma unroll
  for (int t = 0; t < 10; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[t][r];
  out[(size_t)blockIdx.x * 64 * kCalibWaves + threadIdx.x] = s;
}

// LDS bandwidth: 8 waves per workgroup over a 64 KB region, each lane moving 16 bytes per
// instruction at consecutive 16-byte slots (conflict-free). MODE 0: ds_read_b128 only; 1:
// ds_write_b128 only; 2: three reads to one write (the GEMM main loop's mix is about 3:1).
// Each iteration issues 8 instructions per wave; the sums keep the reads live.
template <int MODE>
__global__ __launch_bounds__(64 * kCalibWaves) void calib_lds_kernel(int64_t iters, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) u32x4 buf[4096];   // 64 KB
  const int tid = threadIdx.x;
  for (int i = tid; i < 4096; i += 64 * kCalibWaves) buf[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  u32x4 acc = zero4();
  const u32x4 w = {(uint32_t)tid, 7u, 9u, 11u};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int slot = (tid + 512 * k + (int)(it & 7) * 64) & 4095;
      if (MODE == 0 || (MODE == 2 && (k & 3) != 3)) {
        const u32x4 v = buf[slot];
        acc[0] += v[0]; acc[1] ^= v[1]; acc[2] += v[2]; acc[3] ^= v[3];
      } else {
        buf[slot] = w + acc;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the iteration's accesses are done
  }
  __syncthreads();
  const u32x4 last = buf[(tid * 7) & 4095];   // the writes are observed
  out[(size_t)blockIdx.x * 64 * kCalibWaves + tid] =
      (float)(acc[0] + acc[1] + acc[2] + acc[3] + last[0] + last[1] + last[2] + last[3]);
}

// Grid-stride copy of 16-byte units, four in flight per thread.
__global__ __launch_bounds__(256) void calib_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

size_t calib_table_bytes() { return (size_t)kCalibTables * kCalibFrags * 64 * sizeof(f16x8); }
int calib_waves_per_workgroup() { return kCalibWaves; }
int64_t calib_flop_per_wave_iteration() { return 20 * 2 * 32 * 32 * 16; }
int64_t calib_scaled_flop_per_wave_iteration() { return 20 * 2 * 32 * 32 * 64; }

hipError_t launch_calib_mfma_scaled(const void* table, int64_t iters, int64_t workgroups, int fmt, float* out,
                                    uint64_t* clocks, hipStream_t stream) {
  const u32x4* t = static_cast<const u32x4*>(table);
  if (fmt == 4)
    hipLaunchKernelGGL(calib_mfma_scaled_kernel<4>, dim3((unsigned)workgroups), dim3(64 * kCalibWaves), 0, stream, t,
                       iters, out, clocks);
  else if (fmt == 0)
    hipLaunchKernelGGL(calib_mfma_scaled_kernel<0>, dim3((unsigned)workgroups), dim3(64 * kCalibWaves), 0, stream, t,
                       iters, out, clocks);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_calib_mfma(const void* table, int64_t iters, int64_t workgroups, float* out, uint64_t* clocks,
                             hipStream_t stream) {
  hipLaunchKernelGGL(calib_mfma_kernel, dim3((unsigned)workgroups), dim3(64 * kCalibWaves), 0, stream,
                     static_cast<const f16x8*>(table), iters, out, clocks);
  return hipGetLastError();
}

int64_t calib_lds_bytes_per_iteration(int64_t workgroups) { return workgroups * 64 * kCalibWaves * 8 * 16; }

hipError_t launch_calib_lds(int64_t iters, int64_t workgroups, int mode, float* out, hipStream_t stream) {
  if (mode == 0)
    hipLaunchKernelGGL(calib_lds_kernel<0>, dim3((unsigned)workgroups), dim3(64 * kCalibWaves), 0, stream, iters, out);
  else if (mode == 1)
    hipLaunchKernelGGL(calib_lds_kernel<1>, dim3((unsigned)workgroups), dim3(64 * kCalibWaves), 0, stream, iters, out);
  else if (mode == 2)
    hipLaunchKernelGGL(calib_lds_kernel<2>, dim3((unsigned)workgroups), dim3(64 * kCalibWaves), 0, stream, iters, out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_calib_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  const int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return hipSuccess;
  const int64_t want = (n + 1023) / 1024;
  const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(calib_copy_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), n);
  return hipGetLastError();
}

}  // namespace svdq
