// Scaled W4A4 GEMM + low-rank up-projection + epilogue for packed operands,
// with each NVFP4 element dequantised once per workgroup (model card
// "nunchaku-z-image-turbo-svdq", section "What's stored on disk", runtime
// formula; packed layouts: see repack.hip and quant_lora.hip).
//
// Why: the matrix cores need f16 operands (see common.h for the exact
// dequantisation), and dequantising in every wave that uses a fragment costs
// ~8 VALU instructions per 32x32x16 instruction at 64x64 per wave. Here a
// workgroup of WM x WN waves (2 per SIMD) owns a (32*TM*WM) x (32*TN*WN) tile;
// per 64-K panel each packed 1 KB chunk (32 rows x 64 K of codes, plus its
// scale chunk) is loaded by one wave, dequantised once, and written to LDS as
// four 1 KB f16 fragment blocks (lane l at l*16, the v_mfma_f32_32x32x16_f16
// operand layout, so both the writes and the 16-byte fragment reads are
// bank-conflict free). Every wave then reads its TM + TN fragments per 16-K
// step from LDS.
//
// Pipeline (one barrier per panel, two LDS stages): while the waves multiply
// panel p out of stage p%2, each also dequantises its share of panel p+1 (one
// 16-K slice per step, interleaved with its matrix instructions) into stage
// (p+1)%2, and after that issues the global loads of its panel p+2 chunks into
// registers, a whole panel ahead of their use.
//
// Tile order: workgroup w is dispatched to XCD w % 8 and each XCD has its own
// L2, so the 8 XCDs get contiguous ranges of tiles; inside a range, tiles walk
// down kGroupM row blocks before moving right, so the workgroups resident on
// one XCD share activation rows and weight columns. The grid is padded to a
// multiple of 8; the padding workgroups exit at once. Epilogue: accumulators *
// wtscale * wcscales[n], then R/16 bf16 matrix instructions add
// lora_act @ proj_up^T, then bias, then bf16 (RNE), staged through LDS so the
// output leaves as coalesced 16-byte row pieces.
#include "common.h"
#include "kernels.h"

namespace svdq {

namespace {

constexpr int kGroupM = 4;

template <int WM, int WN, int TM, int TN>
struct LdsCfg {
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BM = 32 * TM * WM;
  static constexpr int BN = 32 * TN * WN;
  static constexpr int kChunksA = BM / 32;
  static constexpr int kChunksB = BN / 32;
  static constexpr int kChunks = kChunksA + kChunksB;
  static constexpr int kPerWave = (kChunks + kWaves - 1) / kWaves;   // chunks a wave dequantises
  static constexpr int kStageBytes = kChunks * 4096;                  // f16 fragments of one panel
};

template <int WM, int WN, int TM, int TN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_lds_kernel(GemmArgs a) {
  using C = LdsCfg<WM, WN, TM, TN>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int wave_m = wave % WM;
  const int wave_n = wave / WM;

  const int M = (int)a.M, N = (int)a.N, K = (int)a.K;
  const int KP = (K + 63) / 64;
  const int MP = (M + 31) / 32;
  const int NP = (N + 31) / 32;
  const size_t a_code_bytes = (size_t)KP * MP * 1024;
  const size_t b_code_bytes = (size_t)KP * NP * 1024;

  // XCD-aware grouped tile order (see the header comment)
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

  // this wave's dequantisation chunks: c = wave + kWaves * s (A chunks first)
  u32x4 cc[C::kPerWave];
  uint32_t cs[C::kPerWave];
  auto load_chunks = [&](int kp) {
#pragma unroll
    for (int s = 0; s < C::kPerWave; ++s) {
      const int c = wave + C::kWaves * s;
      cc[s] = zero4();
      cs[s] = 0u;
      if (c < C::kChunksA) {
        if (mp0 + c < MP) {
          const size_t chunk = (size_t)kp * MP + mp0 + c;
          cc[s] = *reinterpret_cast<const u32x4*>(a.qact + chunk * 1024 + lane * 16);
          cs[s] = *reinterpret_cast<const uint32_t*>(a.qact + a_code_bytes + chunk * 128 + l32 * 4);
        }
      } else if (c < C::kChunks) {
        if (np0 + c - C::kChunksA < NP) {
          const size_t chunk = (size_t)kp * NP + np0 + (c - C::kChunksA);
          cc[s] = *reinterpret_cast<const u32x4*>(a.weight + chunk * 1024 + lane * 16);
          cs[s] = *reinterpret_cast<const uint32_t*>(a.weight + b_code_bytes + chunk * 128 + l32 * 4);
        }
      }
    }
  };
  // dequantise 16-K slice t of this wave's chunks into an LDS stage
  auto dequant_slice = [&](uint8_t* stage, int t) {
#pragma unroll
    for (int s = 0; s < C::kPerWave; ++s) {
      const int c = wave + C::kWaves * s;
      if (c < C::kChunks) {
        const f16x2 sp = t >= 2 ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cs[s], 1.0f, true)
                                : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cs[s], 1.0f, false);
        const f16x8 f = dequant8_f16(cc[s][t], sp[t & 1]);
        *reinterpret_cast<f16x8*>(stage + c * 4096 + t * 1024 + lane * 16) = f;
      }
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  uint8_t* stage0 = smem;
  uint8_t* stage1 = smem + C::kStageBytes;

  // prologue: panel 0 into stage 0, panel 1 into registers
  load_chunks(0);
#pragma unroll
  for (int t = 0; t < 4; ++t) dequant_slice(stage0, t);
  if (KP > 1) load_chunks(1);
  __syncthreads();

  for (int kp = 0; kp < KP; ++kp) {
    uint8_t* cur = (kp & 1) ? stage1 : stage0;
    uint8_t* nxt = (kp & 1) ? stage0 : stage1;
    const bool more = kp + 1 < KP;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f16x8 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[i] = *reinterpret_cast<const f16x8*>(cur + (wave_m * TM + i) * 4096 + t * 1024 + lane * 16);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fb[j] = *reinterpret_cast<const f16x8*>(cur + (C::kChunksA + wave_n * TN + j) * 4096 + t * 1024 + lane * 16);
      if (more) dequant_slice(nxt, t);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kp + 2 < KP) load_chunks(kp + 2);
    __syncthreads();
  }

  // ---- epilogue ----
  const int m_w = (mp0 + wave_m * TM) * 32;
  const int n_w = (np0 + wave_n * TN) * 32;
  const float wt = bf16lo_to_f32(a.wtscale[0]);
  int ncol[TN];
  float alpha[TN], bias_v[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    ncol[j] = n_w + 32 * j + l32;
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

  // low-rank up-projection: R/16 bf16 matrix instructions per tile; the
  // operands of step s+2 load while step s multiplies
  const int R = (int)a.R;
  const int r_steps = R / 16;
  auto load_res = [&](bf16x8* la, bf16x8* pu, int rs) {
    const int r0 = 16 * rs;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m_w + 32 * i + l32;
      u32x4 v = zero4();
      if (rs < r_steps && m < M) v = *reinterpret_cast<const u32x4*>(a.lora_act + (size_t)m * R + r0 + 8 * h);
      la[i] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      u32x4 v = zero4();
      if (rs < r_steps && ncol[j] < N) v = *reinterpret_cast<const u32x4*>(a.proj_up + (size_t)ncol[j] * R + r0 + 8 * h);
      pu[j] = __builtin_bit_cast(bf16x8, v);
    }
  };
  if (r_steps > 0) {
    bf16x8 la0[TM], pu0[TN], la1[TM], pu1[TN];
    load_res(la0, pu0, 0);
    load_res(la1, pu1, 1);
    for (int rs = 0; rs < r_steps; rs += 2) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(la0[i], pu0[j], acc[i][j], 0, 0, 0);
      load_res(la0, pu0, rs + 2);
      if (rs + 1 < r_steps) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(la1[i], pu1[j], acc[i][j], 0, 0, 0);
      }
      load_res(la1, pu1, rs + 3);
    }
  }

  // bf16 output through LDS (free after the main loop): each wave writes one
  // 32-row slice of its tile row-major, then stores whole 16-byte row pieces
  constexpr int kCols = 32 * TN;                 // columns of a wave tile
  constexpr int kPieces = kCols / 8;             // 16-byte pieces per row
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

template <int WM, int WN, int TM, int TN>
hipError_t launch_lds_cfg(const GemmArgs& a, hipStream_t stream) {
  using C = LdsCfg<WM, WN, TM, TN>;
  const int64_t tiles = ((a.N + C::BN - 1) / C::BN) * ((a.M + C::BM - 1) / C::BM);
  const unsigned lds = 2 * C::kStageBytes;
  // more than 64 KB of dynamic LDS must be allowed explicitly (set on every
  // launch: cheap, and correct for whichever device is current)
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_lds_kernel<WM, WN, TM, TN>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((tiles + 7) / 8 * 8));
  hipLaunchKernelGGL((gemm_lds_kernel<WM, WN, TM, TN>), grid, dim3(C::kThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_lds(const GemmArgs& a, hipStream_t stream) {
  return launch_lds_cfg<4, 2, 2, 5>(a, stream);
}

}  // namespace svdq
