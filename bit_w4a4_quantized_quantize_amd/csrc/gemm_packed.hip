// Scaled W4A4 GEMM + low-rank up-projection + epilogue for packed operands
// (model card "nunchaku-z-image-turbo-svdq", section "What's stored on disk",
// runtime formula; the packed layouts are this library's load-time /
// quantisation-time fragment order, see repack.hip and quant_lora.hip).
//
// Both operands arrive as 1 KB chunks that are exactly one 32-row x 64-K set
// of v_mfma_f32_32x32x16_f16 fragments (one 16-byte load per lane at lane*16),
// each followed by its 128-byte scale chunk (one dword per lane: the four e4m3
// scales of its row for the four 16-blocks). So a wave needs no LDS and no
// barrier: it loads its TM activation chunks and TN weight chunks for the next
// 64-K panel while it dequantises (exactly, to f16: see common.h) and
// multiplies the current one. A wave owns (32*TM) x (32*TN) outputs; the waves
// of a workgroup are stacked along M and share the weight chunks through the
// cache. The shipped configuration is 64 x 64 per wave, 2 waves per workgroup
// (about 144 registers per lane, 3 waves per SIMD): measured on MI355X at
// M=4096, K=3840, N=10240 it beats 128 x 128 per wave (one wave per SIMD,
// exposed load latency) and 128 x 64.
//
// Epilogue: accumulators * wtscale * wcscales[n], then R/16 bf16 matrix
// instructions add lora_act @ proj_up^T, then bias, then bf16 (RNE) stores.
#include "common.h"
#include "kernels.h"

namespace svdq {

namespace {

constexpr int kGroupM = 4;

template <int TM, int TN>
struct PanelRegs {
  u32x4 a[TM];
  uint32_t as[TM];
  u32x4 b[TN];
  uint32_t bs[TN];
};

template <int TM, int TN, int WAVES_M>
__global__ __launch_bounds__(64 * WAVES_M) void gemm_packed_kernel(GemmArgs a) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const int M = (int)a.M, N = (int)a.N, K = (int)a.K;
  const int KP = (K + 63) / 64;
  const int MP = (M + 31) / 32;
  const int NP = (N + 31) / 32;
  const size_t a_code_bytes = (size_t)KP * MP * 1024;
  const size_t b_code_bytes = (size_t)KP * NP * 1024;

  // Tile order. Workgroup w is dispatched to XCD w % 8 and each XCD has its own
  // L2, so the 8 XCDs get contiguous ranges of tiles; inside a range, tiles
  // walk down kGroupM row blocks before moving right, so the workgroups
  // resident on one XCD share activation rows and weight columns. The grid is
  // padded to a multiple of 8; the padding workgroups exit at once.
  const int NBX = (N + 32 * TN - 1) / (32 * TN);
  const int NBY = (M + 32 * TM * WAVES_M - 1) / (32 * TM * WAVES_M);
  const int T = NBX * NBY;
  const int per_xcd = (int)(gridDim.x / 8);
  const int t = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (t >= T) return;
  const int per_group = kGroupM * NBX;
  const int first_row = (t / per_group) * kGroupM;
  const int group_rows = min(NBY - first_row, kGroupM);
  const int by = first_row + (t % per_group) % group_rows;
  const int bx = (t % per_group) / group_rows;
  const int m_w = by * (32 * TM * WAVES_M) + wave * 32 * TM;
  const int n0 = bx * (32 * TN);
  const int mp0 = m_w / 32, np0 = n0 / 32;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto load = [&](PanelRegs<TM, TN>& p, int kp) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      p.a[i] = zero4();
      p.as[i] = 0u;
      if (mp0 + i < MP) {
        const size_t chunk = (size_t)kp * MP + mp0 + i;
        p.a[i] = *reinterpret_cast<const u32x4*>(a.qact + chunk * 1024 + lane * 16);
        p.as[i] = *reinterpret_cast<const uint32_t*>(a.qact + a_code_bytes + chunk * 128 + l32 * 4);
      }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      p.b[j] = zero4();
      p.bs[j] = 0u;
      if (np0 + j < NP) {
        const size_t chunk = (size_t)kp * NP + np0 + j;
        p.b[j] = *reinterpret_cast<const u32x4*>(a.weight + chunk * 1024 + lane * 16);
        p.bs[j] = *reinterpret_cast<const uint32_t*>(a.weight + b_code_bytes + chunk * 128 + l32 * 4);
      }
    }
  };

  auto compute = [&](const PanelRegs<TM, TN>& p) {
    // scales as f16 pairs (s_t0, s_t1), (s_t2, s_t3) per fragment row
    f16x2 sa01[TM], sa23[TM], sb01[TN], sb23[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      sa01[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(p.as[i], 1.0f, false);
      sa23[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(p.as[i], 1.0f, true);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      sb01[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(p.bs[j], 1.0f, false);
      sb23[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(p.bs[j], 1.0f, true);
    }
    // per 16-K step: the TM activation fragments, then each weight fragment
    // right before the TM matrix instructions that consume it (few live
    // fragments; its dequantisation overlaps the previous instructions)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f16x8 fa[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const f16x2 sc = t < 2 ? sa01[i] : sa23[i];
        fa[i] = dequant8_f16(p.a[i][t], sc[t & 1]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const f16x2 sc = t < 2 ? sb01[j] : sb23[j];
        const f16x8 fb = dequant8_f16(p.b[j][t], sc[t & 1]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb, acc[i][j], 0, 0, 0);
      }
    }
  };

  // the next panel loads while this one computes
  PanelRegs<TM, TN> cur, nxt;
  load(cur, 0);
  for (int kp = 0; kp < KP; ++kp) {
    if (kp + 1 < KP) load(nxt, kp + 1);
    compute(cur);
    cur = nxt;
  }

  // ---- epilogue ----
  const float wt = bf16lo_to_f32(a.wtscale[0]);
  int ncol[TN];
  float alpha[TN], bias_v[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    ncol[j] = n0 + 32 * j + l32;
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
  for (int rb = 0; rb < R; rb += 128) {
#pragma unroll
    for (int rs = 0; rs < 8; ++rs) {
      const int r0 = rb + 16 * rs;
      if (r0 < R) {
        bf16x8 la[TM], pu[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int m = m_w + 32 * i + l32;
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
    }
  }

#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if (ncol[j] >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m_w + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m < M) a.y[(size_t)m * N + ncol[j]] = (uint16_t)f32_to_bf16_rne(acc[i][j][r] + bias_v[j]);
      }
    }
  }
}

template <int TM, int TN, int WAVES_M>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t stream) {
  const int64_t tiles = ((a.N + 32 * TN - 1) / (32 * TN)) *
                        ((a.M + 32 * TM * WAVES_M - 1) / (32 * TM * WAVES_M));
  dim3 grid((unsigned)((tiles + 7) / 8 * 8));
  hipLaunchKernelGGL((gemm_packed_kernel<TM, TN, WAVES_M>), grid, dim3(64 * WAVES_M), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_packed(const GemmArgs& a, hipStream_t stream) {
  return launch_cfg<2, 2, 2>(a, stream);
}

}  // namespace svdq
