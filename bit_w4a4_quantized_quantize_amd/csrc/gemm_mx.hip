// MXFP4 datatype variant of the layer: both operands in the OCP microscaling
// form that gfx950's block-scaled matrix instruction takes (E2M1 values, one
// E8M0 power-of-two scale per 32 consecutive K), re-rounded from the pages'
// NVFP4 (E2M1 with one e4m3 scale per 16 K; model card
// "nunchaku-z-image-turbo-svdq", header and section "What's stored on disk").
// This gives up the exactness of the NVFP4 path for v_mfma_scale_f32_32x32x64
// with FP4 operands (on random data it sustains ~3.9x the f16 instruction's
// rate). The epilogue, low-rank branch and bias are the NVFP4 layer's.
//
// MX quantisation of a 32-block (OCP MX rule for E2M1, mx_format.h): X =
// floor(log2 amax) - 2 clamped to [-127, 127], byte X + 127; codes = E2M1
// nearest-even of v * 2^-X (exact scaling), saturating at 6, sign of v kept;
// all-zero block: X = -127.
//
// MX operand layout (rows = tokens or output channels, padded to 32-row panels):
//   codes: per 64-K step s and row panel p a 1 KB chunk at 1024 * (s * P + p);
//          lane l = 32 h + c of the matrix instruction holds bytes 16 l .. 16 l + 15:
//          row 32 p + c, k = 64 s + 32 h + 0..31, low nibble first. Rows past the
//          tensor are zero.
//   scales: [K/32, padded rows] bytes (padded to the 32-row panels, so a panel's
//          32 scales of a block are 4-byte aligned; padding rows hold 0).
#include "common.h"
#include "kernels.h"
#include "mx_format.h"

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

namespace svdq {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// 32 values -> 16 bytes of E2M1 codes (value 2i in the low nibble of byte i)
__device__ __forceinline__ u32x4 mx_codes(const float (&v)[32], int X) {
  u32x4 out;
#pragma unroll
  for (int w = 0; w < 4; ++w) out[w] = mx_codes8(v + 8 * w, X);
  return out;
}

// one thread per (row, 32-block), rows of the padded panels fastest
__global__ void quant_act_mx_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ smooth,
                                    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int M, int K) {
  const int RP = (M + 31) / 32;
  const int rows = RP * 32;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rows * (K / 32)) return;
  const int m = (int)(idx % rows), b = (int)(idx / rows);
  uint8_t* dst = codes + 1024 * ((size_t)(b / 2) * RP + m / 32) + 16 * ((b % 2) * 32 + m % 32);
  if (m >= M) {
    *reinterpret_cast<u32x4*>(dst) = zero4();
    scales[(size_t)b * rows + m] = 0;
    return;
  }
  float v[32];
  const uint16_t* xr = x + (size_t)m * K + 32 * b;
  const uint16_t* sr = smooth + 32 * b;
  float amax = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 xv = *reinterpret_cast<const u32x4*>(xr + 8 * q);
    const u32x4 sv = *reinterpret_cast<const u32x4*>(sr + 8 * q);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t xb = (xv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      const uint32_t sb = (sv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      v[8 * q + e] = bf16lo_to_f32(xb) * bf16lo_to_f32(sb);   // exact in fp32
      amax = fmaxf(amax, fabsf(v[8 * q + e]));
    }
  }
  const int X = mx_exponent(amax);
  *reinterpret_cast<u32x4*>(dst) = mx_codes(v, X);
  scales[(size_t)b * rows + m] = (uint8_t)(X + 127);
}

// NVFP4 weight (canonical qweight [N, K/2], wscales [K/16, N]) -> MX: each value
// decoded exactly (E2M1 x e4m3 has at most 6 significant bits), then MX-quantised.
__global__ void reround_mx_kernel(const uint8_t* __restrict__ qweight, const uint8_t* __restrict__ wscales,
                                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int N, int K) {
  const int NP = (N + 31) / 32;
  const int rows = NP * 32;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rows * (K / 32)) return;
  const int n = (int)(idx % rows), b = (int)(idx / rows);
  uint8_t* dst = codes + 1024 * ((size_t)(b / 2) * NP + n / 32) + 16 * ((b % 2) * 32 + n % 32);
  if (n >= N) {
    *reinterpret_cast<u32x4*>(dst) = zero4();
    scales[(size_t)b * rows + n] = 0;
    return;
  }
  const u32x4 q = *reinterpret_cast<const u32x4*>(qweight + (size_t)n * (K / 2) + 16 * b);
  const float s0 = e4m3_to_f32(wscales[(size_t)(2 * b) * N + n], 0);
  const float s1 = e4m3_to_f32(wscales[(size_t)(2 * b + 1) * N + n], 0);
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t c = (q[i >> 3] >> (4 * (i & 7))) & 0xFu;
    const uint32_t mc = c & 7u;   // E2M1 magnitude: 0.5 m below 2, else 2^(m/2 - 1) * (1 + (m & 1) / 2)
    const float g = mc < 2u ? 0.5f * (float)mc : (float)(1u << ((mc >> 1) - 1u)) * ((mc & 1u) ? 1.5f : 1.0f);
    const float mag = g * (i < 16 ? s0 : s1);
    v[i] = (c & 8u) ? -mag : mag;
    amax = fmaxf(amax, mag);
  }
  const int X = mx_exponent(amax);
  *reinterpret_cast<u32x4*>(dst) = mx_codes(v, X);
  scales[(size_t)b * rows + n] = (uint8_t)(X + 127);
}

// ---------------------------------------------------------------------------
// GEMM: 8 waves (4 x 2), tile 256 x (32 TN 2), 128-K panels (two matrix-
// instruction K steps) in S LDS stages, all copied buffer-to-LDS: per chunk and
// panel two 1 KB code blocks and its 128 scale bytes (4 blocks x 32 rows, one
// 4-byte piece per lane of half a wave). The rank-R residual follows as further
// panels of the same stage ring (two 16-wide R steps each, lora_act and proj_up
// rows in the code blocks' places), so its copies are issued while the last
// matrix panels multiply. Every panel, matrix or residual, costs each wave the
// same number of copies, so one vmcnt count per panel holds throughout. The
// tile's alpha = wtscale * wcscales and bias are staged in LDS at the start.
// Output staging as in gemm_lds.hip.
// ---------------------------------------------------------------------------

constexpr int kGroupM = 4;

template <int N_>
__device__ __forceinline__ void wait_vm() {
  static_assert(N_ >= 0 && N_ < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N_ & 15) | ((N_ >> 4) << 14) | 0x0F70);
}

__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Buffer-to-LDS copies of 16 and 4 bytes per lane. Device functions rather than
// calls inside the kernel's lambdas: the host compilation pass of a lambda rejects
// the 16-byte form (a gfx950 feature) without a diagnostic and then emits no
// launch stub for the kernel.
__device__ __forceinline__ void buf_to_lds16(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(lds), 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void buf_to_lds4(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(lds), 4, voff, soff, 0, 0);
}

template <int WM, int WN, int TM, int TN, int S>
struct MxCfg {
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BM = 32 * TM * WM;
  static constexpr int BN = 32 * TN * WN;
  static constexpr int kChunksA = BM / 32;
  static constexpr int kChunksB = BN / 32;
  static constexpr int kChunks = kChunksA + kChunksB;
  static constexpr int kFull = kChunks / kWaves;
  static constexpr int kRest = kChunks - kFull * kWaves;
  static constexpr int kPerWave = kFull + (kRest ? 1 : 0);
  static constexpr int kCodeBytes = kChunks * 2048;                 // two 1 KB K steps per chunk
  static constexpr int kStageBytes = kCodeBytes + kChunks * 128;     // + 4 scale blocks x 32 rows
  static constexpr int kAlphaOff = S * kStageBytes;                  // f32 alpha [BN], then f32 bias [BN]
  static constexpr int kLdsBytes = kAlphaOff + 8 * BN;
  static constexpr int kOutBytes = kWaves * 32 * (32 * TN) * 2;
  static_assert(kOutBytes <= kAlphaOff, "output staging fits below the column factors");
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
  static_assert(S >= 2 && S <= 4, "panel waits cover up to S - 2 = 2 later panels");
  static_assert((S - 2) * kPerWave * 3 < 64, "vmcnt range");
};

template <int WM, int WN, int TM, int TN, int S>
__global__ __launch_bounds__(64 * WM * WN) void gemm_mx_kernel(MxGemmArgs a) {
  using C = MxCfg<WM, WN, TM, TN, S>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int wave_m = wave % WM;
  const int wave_n = wave / WM;

  const int M = (int)a.M, N = (int)a.N, K = (int)a.K, R = (int)a.R;
  const int KP = K / 128;
  const int r_steps = R / 16;
  const int RP = (r_steps + 1) / 2;   // residual panels
  const int TP = KP + RP;
  const int MP = (M + 31) / 32;
  const int NP = (N + 31) / 32;
  const int NBX = (N + C::BN - 1) / C::BN;
  const int NBY = (M + C::BM - 1) / C::BM;
  const int T = NBX * NBY;
  const int per_xcd = (int)(gridDim.x / 8);
  const int tile = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (tile >= T) return;
  const int per_group = kGroupM * NBX;
  const int first_row = (tile / per_group) * kGroupM;
  const int group_rows = min(NBY - first_row, kGroupM);
  const int by = first_row + (tile % per_group) % group_rows;
  const int bx = (tile % per_group) / group_rows;
  const int mp0 = by * (C::BM / 32);
  const int np0 = bx * (C::BN / 32);

  // this wave's chunks c = wave + kWaves * s (A chunks first) as row-panel indices;
  // panels past the tensor read the last panel (their results are never stored)
  int pan[C::kPerWave];
#pragma unroll
  for (int s = 0; s < C::kPerWave; ++s) {
    const int c = min(wave + C::kWaves * s, C::kChunks - 1);
    pan[s] = c < C::kChunksA ? min(mp0 + c, MP - 1) : min(np0 + c - C::kChunksA, NP - 1);
  }
  const uint32_t a_code_bytes = (uint32_t)MP * 32 * (uint32_t)(K / 2);
  const uint32_t w_code_bytes = (uint32_t)NP * 32 * (uint32_t)(K / 2);
  const bool extra = C::kRest && wave < C::kRest;

  // column factors, loaded before the panels so that the first panel wait covers them
  float* lds_alpha = reinterpret_cast<float*>(smem + C::kAlphaOff);
  float* lds_bias = lds_alpha + C::BN;
  uint32_t wc_raw = 0, b_raw = 0;
  if (tid < C::BN) {
    const int col = np0 * 32 + tid;
    if (col < N) {
      wc_raw = a.wcscales[col];
      if (a.bias != nullptr) b_raw = a.bias[col];
    }
  }

  auto stage_at = [&](int kp) { return smem + (kp % S) * C::kStageBytes; };
  auto copy_chunk = [&](int s, int kp) {
    const int c = wave + C::kWaves * s;
    const bool is_a = c < C::kChunksA;
    uint8_t* st = stage_at(kp);
    if (kp < KP) {
      const int rows = is_a ? MP : NP;
      const auto rc = make_rsrc(is_a ? a.act_codes : a.w_codes, is_a ? a_code_bytes : w_code_bytes);
      const auto rsc = make_rsrc(is_a ? a.act_scales : a.w_scales, (uint32_t)(K / 32) * rows * 32);
#pragma unroll
      for (int u = 0; u < 2; ++u)
        buf_to_lds16(rc, st + (c * 2 + u) * 1024, lane * 16, ((2 * kp + u) * rows + pan[s]) * 1024);
      if (lane < 32)   // blocks 4 kp .. 4 kp + 3 of the chunk's 32 rows
        buf_to_lds4(rsc, st + C::kCodeBytes + c * 128, ((lane >> 3) & 3) * rows * 32 + 4 * (lane & 7),
                    4 * kp * rows * 32 + pan[s] * 32);
    } else {
      // residual panel q: R steps 2q and 2q + 1 of 32 lora_act (A) or proj_up (B) rows,
      // lane (h, l32) holding 8 values of row l32 as the bf16 instruction's operand
      const int q = kp - KP;
      const int g = is_a ? c : c - C::kChunksA;
      const int row = is_a ? min(mp0 * 32 + 32 * g + l32, M - 1) : min(np0 * 32 + 32 * g + l32, N - 1);
      const auto rr = make_rsrc(is_a ? a.lora_act : a.proj_up, (uint32_t)(is_a ? M : N) * (uint32_t)R * 2);
      const int vo = row * R * 2 + 16 * h;
#pragma unroll
      for (int u = 0; u < 2; ++u)   // an odd last step is copied twice; the second copy is not multiplied
        buf_to_lds16(rr, st + (c * 2 + u) * 1024, vo, 32 * min(2 * q + u, r_steps - 1));
      if (lane < 32)   // keeps the per-panel copy count; these bytes are not read
        buf_to_lds4(rr, st + C::kCodeBytes + c * 128, vo, 64 * q);
    }
  };
  auto load_panel = [&](int kp) {
#pragma unroll
    for (int s = 0; s < C::kFull; ++s) copy_chunk(s, kp);
    if (extra) copy_chunk(C::kFull, kp);
  };
  // panel kp landed: copies of panels issued after it may stay in flight
  auto wait_panel = [&](int kp) {
    const int later = min(kp + S - 2, TP - 1) - kp;
    if (later >= 2) {
      if (extra) wait_vm<(S >= 4 ? 2 : 0) * C::kPerWave * 3>(); else wait_vm<(S >= 4 ? 2 : 0) * C::kFull * 3>();
    } else if (later == 1) {
      if (extra) wait_vm<C::kPerWave * 3>(); else wait_vm<C::kFull * 3>();
    } else {
      wait_vm<0>();
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

#pragma unroll
  for (int p = 0; p < S - 1; ++p)
    if (p < TP) load_panel(p);
  if (tid < C::BN) {
    lds_alpha[tid] = bf16lo_to_f32(a.wtscale[0]) * bf16lo_to_f32(wc_raw);
    lds_bias[tid] = bf16lo_to_f32(b_raw);
  }

  for (int kp = 0; kp < KP; ++kp) {
    wait_panel(kp);
    barrier_no_fence();
    if (kp + S - 1 < TP) load_panel(kp + S - 1);
    const uint8_t* cur = stage_at(kp);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      i32x8 fa[TM], fb[TN];
      int sa[TM], sb[TN];   // E8M0 of this lane's row (column) and block 4 kp + 2 u + h
#pragma unroll
      for (int i = 0; i < TM; ++i) sa[i] = cur[C::kCodeBytes + (wave_m * TM + i) * 128 + (2 * u + h) * 32 + l32];
#pragma unroll
      for (int j = 0; j < TN; ++j)
        sb[j] = cur[C::kCodeBytes + (C::kChunksA + wave_n * TN + j) * 128 + (2 * u + h) * 32 + l32];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(cur + ((wave_m * TM + i) * 2 + u) * 1024 + lane * 16);
        fa[i] = i32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(cur + ((C::kChunksA + wave_n * TN + j) * 2 + u) * 1024 + lane * 16);
        fb[j] = i32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 4, 4, 0, sa[i], 0,
                                                                       sb[j]);
    }
  }

  // ---- epilogue: * wtscale * wcscales[n], + lora_act @ proj_up^T, + bias, bf16 ----
  {
    float al[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) al[j] = lds_alpha[(wave_n * TN + j) * 32 + l32];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] *= al[j];
  }
  for (int q = 0; q < RP; ++q) {
    const int kp = KP + q;
    wait_panel(kp);
    barrier_no_fence();
    if (kp + S - 1 < TP) load_panel(kp + S - 1);
    const uint8_t* cur = stage_at(kp);
    const int nu = 2 * q + 1 < r_steps ? 2 : 1;
    for (int u = 0; u < nu; ++u) {
      bf16x8 la[TM], pu[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        la[i] = *reinterpret_cast<const bf16x8*>(cur + ((wave_m * TM + i) * 2 + u) * 1024 + lane * 16);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        pu[j] = *reinterpret_cast<const bf16x8*>(cur + ((C::kChunksA + wave_n * TN + j) * 2 + u) * 1024 + lane * 16);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(la[i], pu[j], acc[i][j], 0, 0, 0);
    }
  }

  const int m_w = (mp0 + wave_m * TM) * 32;
  const int n_w = (np0 + wave_n * TN) * 32;
  float bias_v[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) bias_v[j] = lds_bias[(wave_n * TN + j) * 32 + l32];
  __syncthreads();   // every wave is done with the stages
  constexpr int kCols = 32 * TN;
  constexpr int kPieces = kCols / 8;
  uint16_t* stage_out = reinterpret_cast<uint16_t*>(smem + wave * (32 * kCols * 2));
  const bool vec_ok = (N % 8) == 0;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * h + (r & 3);
        stage_out[row * kCols + 32 * j + l32] = (uint16_t)f32_to_bf16_rne(acc[i][j][r] + bias_v[j]);
      }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < (32 * kPieces + 63) / 64; ++u) {
      const int idx = lane + 64 * u;
      if (idx < 32 * kPieces) {
        const int row = idx / kPieces, piece = idx % kPieces;
        const int m = m_w + 32 * i + row;
        const int n = n_w + 8 * piece;
        if (m < M && n < N) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(stage_out + row * kCols + 8 * piece);
          uint16_t* dst = a.y + (size_t)m * N + n;
          if (vec_ok && n + 8 <= N) {
            *reinterpret_cast<u32x4*>(dst) = v;
          } else {
            for (int e = 0; e < 8 && n + e < N; ++e) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
          }
        }
      }
    }
    __syncthreads();
  }
}

template <int WM, int WN, int TM, int TN, int S>
hipError_t launch_mx_cfg(const MxGemmArgs& a, hipStream_t stream) {
  using C = MxCfg<WM, WN, TM, TN, S>;
  const int64_t tiles = ((a.N + C::BN - 1) / C::BN) * ((a.M + C::BM - 1) / C::BM);
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(&gemm_mx_kernel<WM, WN, TM, TN, S>),
                                    C::kLdsBytes, lds_set);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((tiles + 7) / 8 * 8));
  hipLaunchKernelGGL((gemm_mx_kernel<WM, WN, TM, TN, S>), grid, dim3(C::kThreads), C::kLdsBytes, stream, a);
  return hipGetLastError();
}

constexpr int kMxStages = 4;

}  // namespace

size_t mx_codes_bytes(int64_t rows, int64_t K) { return (size_t)((rows + 31) / 32) * 32 * (size_t)(K / 2); }

hipError_t launch_quant_act_mx(const uint16_t* x, const uint16_t* smooth, uint8_t* codes, uint8_t* scales,
                               int64_t M, int64_t K, hipStream_t stream) {
  const int64_t threads = ((M + 31) / 32) * 32 * (K / 32);
  hipLaunchKernelGGL(quant_act_mx_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, x, smooth,
                     codes, scales, (int)M, (int)K);
  return hipGetLastError();
}

hipError_t launch_reround_mx(const uint8_t* qweight, const uint8_t* wscales, uint8_t* codes, uint8_t* scales,
                             int64_t N, int64_t K, hipStream_t stream) {
  const int64_t threads = ((N + 31) / 32) * 32 * (K / 32);
  hipLaunchKernelGGL(reround_mx_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, qweight,
                     wscales, codes, scales, (int)N, (int)K);
  return hipGetLastError();
}

// tile width 256 or 320 by the same round-count estimate as the other GEMMs
hipError_t launch_gemm_mx(const MxGemmArgs& a, hipStream_t stream) {
  const int64_t row_blocks = (a.M + 255) / 256;
  const int64_t tiles320 = row_blocks * ((a.N + 319) / 320);
  const int64_t tiles256 = row_blocks * ((a.N + 255) / 256);
  const double cost320 = (double)((tiles320 + 255) / 256);
  const double cost256 = 0.82 * (double)((tiles256 + 255) / 256);
  if (cost256 < cost320) return launch_mx_cfg<4, 2, 2, 4, kMxStages>(a, stream);
  return launch_mx_cfg<4, 2, 2, 5, kMxStages>(a, stream);
}

}  // namespace svdq
