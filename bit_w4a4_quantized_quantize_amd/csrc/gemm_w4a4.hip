// Scaled W4A4 GEMM with the low-rank up-projection and the epilogue fused:
//
//   y = bf16( scaled_mma(qact, qweight, ascales, wscales) * wtscale * wcscales[n]
//             + lora_act @ proj_up^T + bias[n] )
//
// (model card "nunchaku-z-image-turbo-svdq", section "What's stored on disk",
// runtime reconstruction formula, after the activation quantisation step).
//
// Datatype choice. gfx950's block-scaled FP4/FP8 matrix instructions take
// power-of-two (E8M0) scales per 32 K elements, while NVFP4 carries an e4m3
// scale (4 significant bits) per 16. An E2M1 value times an e4m3 scale has up
// to 6 significant bits and lies in [2^-10, 2688], so it is exact in f16. Both
// operands are therefore dequantised exactly to f16 in registers (one
// fp4->f16 conversion and one packed f16 multiply per pair of values) and
// multiplied with v_mfma_f32_32x32x16_f16 into fp32 accumulators. Each 16-K
// instruction covers exactly one NVFP4 block, so every per-block product is
// exact and only the fp32 accumulation over blocks rounds.
//
// Tiling. 256 threads = 4 waves in a 2 x 2 arrangement; a wave owns
// (32*TM) x (32*TN) outputs as TM x TN 32x32 tiles. The K loop advances 64
// (four blocks) per stage. Activation codes and scales are staged through LDS
// (a lane then reads its four 16-K fragments of one row with one 16-byte LDS
// read and its four scales with one 4-byte read); with the canonical weight
// layout the weight tile goes the same way. With the packed layout every
// wave reads its weight fragments straight from global memory: a 1 KB chunk of
// the packed buffer is exactly one 32-channel x 64-K fragment set, one 16-byte
// load per lane, in the order the instruction consumes it.
//
// Epilogue. The accumulators are scaled by wtscale * wcscales[n] (one value
// per lane and column tile), then R/16 more matrix instructions add
// lora_act @ proj_up^T in bf16 (both operands R-contiguous, loaded as 16-byte
// fragments), then bias, then round to bf16.
#include "common.h"
#include "kernels.h"

namespace svdq {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;

// LDS offset of the 16-byte half h of row `row` (codes for k-half h of the four
// 16-blocks of the stage); the halves swap on every fourth row to spread banks.
__device__ __forceinline__ int code_off(int row, int h) {
  return row * 32 + ((h ^ ((row >> 2) & 1)) << 4);
}

template <int ROWS>
struct StageRegs {
  u32x2 codes[ROWS * 4 / kThreads];
  uint32_t scales[ROWS * 4 / kThreads];
};

// Global -> registers for one operand stage (canonical layout): rows [r0, r0+ROWS),
// k-panel kt. codes: [rows_total, K/2]; scales: [K/16, rows_total].
template <int ROWS>
__device__ __forceinline__ void load_stage(StageRegs<ROWS>& st, const uint8_t* __restrict__ codes,
                                           const uint8_t* __restrict__ scales, int r0,
                                           int rows_total, int K, int kt, int tid) {
#pragma unroll
  for (int u = 0; u < ROWS * 4 / kThreads; ++u) {
    const int it = tid + u * kThreads;
    const int row = it >> 2, t = it & 3;
    const int k = kt * kBK + 16 * t;
    u32x2 v = {0u, 0u};
    if (r0 + row < rows_total && k < K)
      v = *reinterpret_cast<const u32x2*>(codes + (size_t)(r0 + row) * (K / 2) + k / 2);
    st.codes[u] = v;
  }
#pragma unroll
  for (int u = 0; u < ROWS * 4 / kThreads; ++u) {
    const int it = tid + u * kThreads;
    const int row = it % ROWS, t = it / ROWS;
    const int blk = kt * 4 + t;
    uint32_t v = 0u;
    if (r0 + row < rows_total && blk * 16 < K) v = scales[(size_t)blk * rows_total + r0 + row];
    st.scales[u] = v;
  }
}

template <int ROWS>
__device__ __forceinline__ void store_stage(const StageRegs<ROWS>& st, uint8_t* lds_codes,
                                            uint8_t* lds_scales, int tid) {
#pragma unroll
  for (int u = 0; u < ROWS * 4 / kThreads; ++u) {
    const int it = tid + u * kThreads;
    const int row = it >> 2, t = it & 3;
    *reinterpret_cast<uint32_t*>(lds_codes + code_off(row, 0) + 4 * t) = st.codes[u][0];
    *reinterpret_cast<uint32_t*>(lds_codes + code_off(row, 1) + 4 * t) = st.codes[u][1];
  }
#pragma unroll
  for (int u = 0; u < ROWS * 4 / kThreads; ++u) {
    const int it = tid + u * kThreads;
    const int row = it % ROWS, t = it / ROWS;
    lds_scales[row * 4 + t] = (uint8_t)st.scales[u];
  }
}

__device__ __forceinline__ _Float16 scale_f16(uint32_t four, int t) {
  return (_Float16)e4m3_to_f32(four, t);
}

template <int TM, int TN, bool PACKED>
__global__ __launch_bounds__(kThreads) void gemm_w4a4_kernel(GemmArgs a) {
  constexpr int BM = 64 * TM;
  constexpr int BN = 64 * TN;
  __shared__ __attribute__((aligned(16))) uint8_t lds_a_codes[BM * 32];
  __shared__ __attribute__((aligned(16))) uint8_t lds_a_scales[BM * 4];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b_codes[PACKED ? 16 : BN * 32];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b_scales[PACKED ? 16 : BN * 4];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wave_m = wave & 1;
  const int wave_n = wave >> 1;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const int M = (int)a.M, N = (int)a.N, K = (int)a.K;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int KT = (K + kBK - 1) / kBK;
  const int NP = (N + 31) / 32;
  const size_t packed_code_bytes = (size_t)KT * NP * 1024;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // packed weight fragments of this wave: column tile j is n-panel pq[j]
  int pq[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) pq[j] = (n0 + wave_n * 32 * TN + 32 * j) / 32;

  StageRegs<BM> sa;
  StageRegs<BN> sb;
  u32x4 pb_codes[TN];
  uint32_t pb_scales[TN];

  auto load_packed = [&](int kt) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      pb_codes[j] = zero4();
      pb_scales[j] = 0u;
      if (pq[j] < NP) {
        const size_t chunk = (size_t)kt * NP + pq[j];
        pb_codes[j] = *reinterpret_cast<const u32x4*>(a.weight + chunk * 1024 + lane * 16);
        pb_scales[j] = *reinterpret_cast<const uint32_t*>(a.weight + packed_code_bytes + chunk * 128 + l32 * 4);
      }
    }
  };

  load_stage<BM>(sa, a.qact, a.ascales, m0, M, K, 0, tid);
  if constexpr (PACKED) load_packed(0);
  else load_stage<BN>(sb, a.weight, a.wscales, n0, N, K, 0, tid);

  for (int kt = 0; kt < KT; ++kt) {
    __syncthreads();
    store_stage<BM>(sa, lds_a_codes, lds_a_scales, tid);
    if constexpr (!PACKED) store_stage<BN>(sb, lds_b_codes, lds_b_scales, tid);
    u32x4 cb[TN];
    uint32_t sbv[TN];
    if constexpr (PACKED) {
#pragma unroll
      for (int j = 0; j < TN; ++j) { cb[j] = pb_codes[j]; sbv[j] = pb_scales[j]; }
    }
    __syncthreads();
    if (kt + 1 < KT) {
      load_stage<BM>(sa, a.qact, a.ascales, m0, M, K, kt + 1, tid);
      if constexpr (PACKED) load_packed(kt + 1);
      else load_stage<BN>(sb, a.weight, a.wscales, n0, N, K, kt + 1, tid);
    }

    u32x4 ca[TM];
    uint32_t sav[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = wave_m * 32 * TM + 32 * i + l32;
      ca[i] = *reinterpret_cast<const u32x4*>(lds_a_codes + code_off(row, h));
      sav[i] = *reinterpret_cast<const uint32_t*>(lds_a_scales + row * 4);
    }
    if constexpr (!PACKED) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = wave_n * 32 * TN + 32 * j + l32;
        cb[j] = *reinterpret_cast<const u32x4*>(lds_b_codes + code_off(row, h));
        sbv[j] = *reinterpret_cast<const uint32_t*>(lds_b_scales + row * 4);
      }
    }

#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f16x8 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i] = dequant8_f16(ca[i][t], scale_f16(sav[i], t));
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = dequant8_f16(cb[j][t], scale_f16(sbv[j], t));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue: * wtscale * wcscales[n], + lora_act @ proj_up^T, + bias ----
  // a static global activation scale (bf16, like wtscale) multiplies in exactly
  const float wt = bf16lo_to_f32(a.wtscale[0]) * (a.act_gscale != nullptr ? bf16lo_to_f32(a.act_gscale[0]) : 1.0f);
  int ncol[TN];
  float alpha[TN], bias_v[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    ncol[j] = n0 + wave_n * 32 * TN + 32 * j + l32;
    const bool in = ncol[j] < N;
    alpha[j] = in ? wt * bf16lo_to_f32(a.wcscales[ncol[j]]) : 0.0f;
    bias_v[j] = (in && a.bias != nullptr) ? bf16lo_to_f32(a.bias[ncol[j]]) : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] *= alpha[j];

  const int R = (int)a.R;
  for (int r0 = 0; r0 < R; r0 += 16) {
    bf16x8 la[TM], pu[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + wave_m * 32 * TM + 32 * i + l32;
      u32x4 v = zero4();
      if (m < M) v = *reinterpret_cast<const u32x4*>(a.lora_act + (size_t)m * R + r0 + 8 * h);
      la[i] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      u32x4 v = zero4();
      if (ncol[j] < N) v = *reinterpret_cast<const u32x4*>(a.proj_up + (size_t)ncol[j] * R + r0 + 8 * h);
      pu[j] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(la[i], pu[j], acc[i][j], 0, 0, 0);
  }

#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if (ncol[j] >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wave_m * 32 * TM + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m < M) a.y[(size_t)m * N + ncol[j]] = (uint16_t)f32_to_bf16_rne(acc[i][j][r] + bias_v[j]);
      }
    }
  }
}

template <int TM, int TN>
hipError_t launch_tile(const GemmArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)((a.N + 64 * TN - 1) / (64 * TN)), (unsigned)((a.M + 64 * TM - 1) / (64 * TM)));
  if (a.packed)
    hipLaunchKernelGGL((gemm_w4a4_kernel<TM, TN, true>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_w4a4_kernel<TM, TN, false>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_w4a4(const GemmArgs& a, hipStream_t stream) {
  return launch_tile<2, 2>(a, stream);
}

}  // namespace svdq
