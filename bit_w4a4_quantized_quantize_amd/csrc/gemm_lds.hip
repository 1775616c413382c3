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
// (p+1)%2, then issues the global loads of its panel p+2 chunks into
// registers. Chunk loads go through buffer resources, so a panel past the end
// of M or N reads as zeros without a branch; the last panel is peeled.
//
// Tile order: workgroup w is dispatched to XCD w % 8 and each XCD has its own
// L2, so the 8 XCDs get contiguous ranges of tiles; inside a range, tiles walk
// down kGroupM row blocks before moving right, so the workgroups resident on
// one XCD share activation rows and weight columns. The grid is padded to a
// multiple of 8; the padding workgroups exit at once.
//
// Epilogue: wcscales and bias load while the last panel multiplies;
// accumulators * wtscale * wcscales[n] (times the static global activation
// scale when the activations were quantised relative to one); then lora_act @ proj_up^T as
// ceil(R/64) further panels of the same two-stage pipeline (bf16 matrix
// instructions; each residual panel is copied into its stage by direct
// global-to-LDS loads while the panel before it multiplies); then bias, then
// bf16 (RNE), staged through LDS so the output leaves as coalesced 16-byte
// row pieces.
#include "common.h"
#include "kernels.h"

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

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
  static constexpr int kFull = kChunks / kWaves;                 // chunks every wave dequantises
  static constexpr int kRest = kChunks - kFull * kWaves;         // waves 0..kRest-1 take one more
  static constexpr int kPerWave = kFull + (kRest ? 1 : 0);
  static constexpr int kStageBytes = kChunks * 4096;
  // LDS of the output epilogue: the gated exchange region (one f32x16 per lane per
  // column tile and wave row), then 32 staged bf16 rows of every writing wave
  static constexpr int epilogue_bytes(bool gated) {
    return (gated ? WM * TN * 64 * 64 : 0) + (gated ? WM : kWaves) * 32 * (32 * TN) * 2;
  }
  static constexpr int lds_bytes(bool gated) {
    return 2 * kStageBytes > epilogue_bytes(gated) ? 2 * kStageBytes : epilogue_bytes(gated);
  }
};

// GATED: the weight holds 2F output channels (a.N = 2F, a.gated_f = F); the
// workgroup's two wave columns compute matching column ranges of the two
// halves (wave_n = 0: channels c, wave_n = 1: channels F + c), and the output
// is h[:, c] = silu(y[:, c]) * y[:, F + c], [M, F] bf16.
//
// Q2 (gated only): the writer waves also quantise h for the next layer, w2,
// whose input h is: per row and 16-block of h's columns, v = h * next_smooth
// with the activation rule of the quantiser kernels, codes and e4m3 scales
// into next_qact in the packed activation layout (rows = tokens, K = F). A
// 16-block is two 8-column pieces held by an even lane and the next one in the
// store loop below, so the block maximum takes one lane swap; an output tile
// holds whole blocks (its width is a multiple of 32 columns).
// CA / CW: the activations / the weight in the canonical layout (codes [rows, K/2], low
// nibble first; e4m3 scales [K/16, rows]) rather than the packed buffer, for callers that
// skip the load-time repack or hold canonical activations (not both at once: that
// combination takes the older canonical kernel). A lane then loads 16 bytes of one row
// (row l % 32, k from 32 (l / 32) in the panel) and one v_permlane32_swap per pair of dwords
// regroups them into the packed layout's per-lane order (lane (h, c): the four 8-code runs at
// k = 16 t + 8 h); the four block scales come from byte loads. From there on the kernel is
// the same, so both layouts give identical results.
template <int WM, int WN, int TM, int TN, bool GATED, bool Q2 = false, bool CA = false, bool CW = false>
__global__ __launch_bounds__(64 * WM * WN) void gemm_lds_kernel(GemmArgs a) {
  using C = LdsCfg<WM, WN, TM, TN>;
  static_assert(!GATED || WN == 2, "the gated epilogue pairs the two wave columns");
  static_assert(!Q2 || (GATED && (32 * (32 * TN / 8)) % 64 == 0), "Q2: whole 16-blocks in lane pairs");
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
  const uint32_t a_code_bytes = (uint32_t)KP * MP * 1024;
  const uint32_t b_code_bytes = (uint32_t)KP * NP * 1024;

  const int FO = GATED ? (int)a.gated_f : N;          // output columns
  const int FP = (FO + 31) / 32;                       // output panels (per half when gated)
  const int NBX = GATED ? (FP + TN - 1) / TN : (N + C::BN - 1) / C::BN;
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
  // weight panel of B chunk j (0 .. kChunksB-1), and whether it exists
  auto b_panel = [&](int j) -> int {
    return GATED ? (j / TN) * FP + bx * TN + j % TN : np0 + j;
  };
  auto b_panel_in = [&](int j) -> bool {
    return GATED ? bx * TN + j % TN < FP : np0 + j < NP;
  };

  // bytes of each operand buffer (codes, and the canonical scales); the buffer resources are
  // built after choosing the operand, since a select between two resources is lowered
  // through a private-memory array
  const uint32_t qa_bytes = CA ? (uint32_t)M * (uint32_t)(K / 2) : a_code_bytes + (uint32_t)KP * MP * 128;
  const uint32_t qb_bytes = CW ? (uint32_t)N * (uint32_t)(K / 2) : b_code_bytes + (uint32_t)KP * NP * 128;

  // chunk c = wave + kWaves * s; A chunks first. Out-of-range panels read as zero.
  u32x4 cc[C::kPerWave];
  uint32_t cs[C::kPerWave];
  auto load_one = [&](int s, int kp) {
    const int c = wave + C::kWaves * s;
    const bool is_a = c < C::kChunksA;
    const bool in = is_a ? mp0 + c < MP : b_panel_in(c - C::kChunksA);
    const int row = is_a ? mp0 + c : b_panel(c - C::kChunksA);
    if ((CA && is_a) || (CW && !is_a)) {   // uniform per wave: every lane takes part in the swaps
      const int rows_total = is_a ? M : N;
      const int r = 32 * row + l32;
      const int kb = 64 * kp + 32 * h;       // k of this lane's first code
      const bool rin = in && r < rows_total;
      const __amdgpu_buffer_rsrc_t rc = make_rsrc(is_a ? a.qact : a.weight, is_a ? qa_bytes : qb_bytes);
      const __amdgpu_buffer_rsrc_t rsc = make_rsrc(is_a ? a.ascales : a.wscales, (uint32_t)(K / 16) * rows_total);
      u32x4 v = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, rin && kb < K ? (uint32_t)r * (K / 2) + kb / 2 : 0x80000000u,
                                                       0, 0));
      if (kb + 16 >= K) {   // codes from K on belong to the next row (K is a multiple of 16)
        v[2] = 0u;
        v[3] = 0u;
      }
      // lower lane (h = 0) holds dwords 0..3 of the row's 32-byte panel segment, the upper
      // one dwords 4..7; afterwards lane (h, c) holds dwords h, h + 2, h + 4, h + 6
      const auto s01 = __builtin_amdgcn_permlane32_swap(v[0], v[1], false, false);
      const auto s23 = __builtin_amdgcn_permlane32_swap(v[2], v[3], false, false);
      cc[s] = u32x4{s01[0], s23[0], s01[1], s23[1]};
      uint32_t sc = 0u;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int blk = 4 * kp + t;
        const uint32_t off = rin && blk < K / 16 ? (uint32_t)blk * rows_total + r : 0x80000000u;
        sc |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rsc, off, 0, 0) << (8 * t);
      }
      cs[s] = sc;
      return;
    }
    const int rows = is_a ? MP : NP;
    const uint32_t code_bytes = is_a ? a_code_bytes : b_code_bytes;
    const uint32_t chunk = (uint32_t)kp * rows + row;
    const uint32_t off_c = in ? chunk * 1024 + lane * 16 : 0x80000000u;
    const uint32_t off_s = in ? code_bytes + chunk * 128 + l32 * 4 : 0x80000000u;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(is_a ? a.qact : a.weight, is_a ? qa_bytes : qb_bytes);
    cc[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off_c, 0, 0));
    cs[s] = __builtin_amdgcn_raw_buffer_load_b32(r, off_s, 0, 0);
  };
  auto load_chunks = [&](int kp) {
#pragma unroll
    for (int s = 0; s < C::kFull; ++s) load_one(s, kp);
    if (C::kRest && wave < C::kRest) load_one(C::kFull, kp);
  };
  auto dq_one = [&](uint8_t* stage, int s, int t) {
    const int c = wave + C::kWaves * s;
    const f16x2 sp = t >= 2 ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cs[s], 1.0f, true)
                            : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cs[s], 1.0f, false);
    *reinterpret_cast<f16x8*>(stage + c * 4096 + t * 1024 + lane * 16) = dequant8_f16(cc[s][t], sp[t & 1]);
  };
  auto dequant_slice = [&](uint8_t* stage, int t) {
#pragma unroll
    for (int s = 0; s < C::kFull; ++s) dq_one(stage, s, t);
    if (C::kRest && wave < C::kRest) dq_one(stage, C::kFull, t);
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

  load_chunks(0);
#pragma unroll
  for (int t = 0; t < 4; ++t) dequant_slice(stage0, t);
  if (KP > 1) load_chunks(1);
  __syncthreads();

  auto mma_step = [&](const uint8_t* cur, int t) {
    f16x8 fa[TM], fb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
      fa[i] = *reinterpret_cast<const f16x8*>(cur + (wave_m * TM + i) * 4096 + t * 1024 + lane * 16);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      fb[j] = *reinterpret_cast<const f16x8*>(cur + (C::kChunksA + wave_n * TN + j) * 4096 + t * 1024 + lane * 16);
    return [&, fa, fb]() mutable {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    };
  };

  // panels 0 .. KP-2: multiply panel kp, dequantise panel kp+1, load panel kp+2. Panel
  // kp+1 is complete after step 2 (slices 2 and 3 are dequantised there), so the barrier
  // sits before step 3, whose fragments are already read and whose matrix instructions
  // overlap it (1-2% faster than a barrier after the last step).
  for (int kp = 0; kp + 1 < KP; ++kp) {
    const uint8_t* cur = (kp & 1) ? stage1 : stage0;
    uint8_t* nxt = (kp & 1) ? stage0 : stage1;
    {
      auto mm = mma_step(cur, 0);
      dequant_slice(nxt, 0);
      mm();
    }
    {
      auto mm = mma_step(cur, 1);
      dequant_slice(nxt, 1);
      mm();
    }
    {
      auto mm = mma_step(cur, 2);
      dequant_slice(nxt, 2);
      dequant_slice(nxt, 3);
      mm();
    }
    {
      auto mm = mma_step(cur, 3);
      if (kp + 2 < KP) load_chunks(kp + 2);
      __syncthreads();
      mm();
    }
  }
  // epilogue operands load while the last panel multiplies
  const int m_w = (mp0 + wave_m * TM) * 32;
  // this wave's first output column (in the output of width FO)
  const int n_w = GATED ? bx * TN * 32 : (np0 + wave_n * TN) * 32;
  int ncol[TN];      // weight channel of column j of this lane
  bool ncol_in[TN];
  uint32_t wc_raw[TN], bias_raw[TN];
  {
    const __amdgpu_buffer_rsrc_t rwc = make_rsrc(a.wcscales, (uint32_t)N * 2);
    const __amdgpu_buffer_rsrc_t rbi = make_rsrc(a.bias, a.bias != nullptr ? (uint32_t)N * 2 : 0u);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n_w + 32 * j + l32;
      ncol_in[j] = col < FO;
      ncol[j] = (GATED ? wave_n * FO : 0) + col;
      const uint32_t off = ncol_in[j] ? (uint32_t)ncol[j] * 2 : 0x80000000u;
      wc_raw[j] = __builtin_amdgcn_raw_buffer_load_b16(rwc, off, 0, 0);
      bias_raw[j] = __builtin_amdgcn_raw_buffer_load_b16(rbi, off, 0, 0);
    }
  }
  const uint32_t wt_raw = a.wtscale[0];
  const uint32_t gs_raw = a.act_gscale != nullptr ? (uint32_t)a.act_gscale[0] : 0x3F80u;   // bf16 1.0

  // The residual lora_act @ proj_up^T runs as ceil(R/64) more panels of the
  // same pipeline: residual panel p (R steps 4p .. 4p+3) is copied by direct
  // global-to-LDS loads into the stage the previous panel does not use, in
  // the matrix-instruction operand order (chunk c, 16-R step t at
  // c*4096 + t*1024, lane l at l*16), while that previous panel multiplies.
  // Rows beyond M or N are clamped to the last row (their results are never
  // stored).
  const int R = (int)a.R;
  const int r_steps = R / 16;
  const int RP = (r_steps + 3) / 4;
  const int m_wg = mp0 * 32;
  auto res_dma = [&](uint8_t* stage, int p) {
    const int S = min(4, r_steps - 4 * p);
    for (int b = wave; b < C::kChunks * 4; b += C::kWaves) {
      const int c = b >> 2, t = b & 3;
      if (t >= S) continue;
      const int col = 16 * (4 * p + t) + 8 * h;
      const uint16_t* src;
      if (c < C::kChunksA) {
        const int m = min(m_wg + 32 * c + l32, M - 1);
        src = a.lora_act + (size_t)m * R + col;
      } else {
        const int n = min(b_panel(c - C::kChunksA) * 32 + l32, N - 1);
        src = a.proj_up + (size_t)n * R + col;
      }
      __builtin_amdgcn_global_load_lds(src, LDS_PTR(stage + c * 4096 + t * 1024), 16, 0, 0);
    }
  };
  {
    const uint8_t* cur = ((KP - 1) & 1) ? stage1 : stage0;
    if (RP > 0) res_dma(((KP - 1) & 1) ? stage0 : stage1, 0);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      auto mm = mma_step(cur, t);
      mm();
    }
  }

  // ---- epilogue ----
  // a static global activation scale (bf16, like wtscale) multiplies in exactly
  const float wt = bf16lo_to_f32(wt_raw) * bf16lo_to_f32(gs_raw);
  float alpha[TN], bias_v[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    alpha[j] = wt * bf16lo_to_f32(wc_raw[j]);
    bias_v[j] = bf16lo_to_f32(bias_raw[j]);
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] *= alpha[j];

  for (int p = 0; p < RP; ++p) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this panel's copies have landed
    __syncthreads();                      // ... for every wave; the other stage is free
    const uint8_t* cur = ((KP + p) & 1) ? stage1 : stage0;
    if (p + 1 < RP) res_dma(((KP + p) & 1) ? stage0 : stage1, p + 1);
    const int S = min(4, r_steps - 4 * p);
    for (int t = 0; t < S; ++t) {
      bf16x8 la[TM], pu[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        la[i] = *reinterpret_cast<const bf16x8*>(cur + (wave_m * TM + i) * 4096 + t * 1024 + lane * 16);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        pu[j] = *reinterpret_cast<const bf16x8*>(cur + (C::kChunksA + wave_n * TN + j) * 4096 + t * 1024 + lane * 16);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(la[i], pu[j], acc[i][j], 0, 0, 0);
    }
  }

  // bf16 output through LDS: each writing wave stages one 32-row slice of its
  // tile row-major, then stores whole 16-byte row pieces. Gated: the wave_n = 1
  // waves first hand their fp32 values to their wave_n = 0 partners through
  // LDS (exchange region, then the staging region after it).
  __syncthreads();
  constexpr int kCols = 32 * TN;
  constexpr int kPieces = kCols / 8;
  constexpr int kXBytes = GATED ? WM * TN * 64 * 64 : 0;   // f32x16 per lane per column tile
  const bool writer = !GATED || wave_n == 0;
  static_assert(kXBytes + (GATED ? WM : C::kWaves) * 32 * kCols * 2 == C::epilogue_bytes(GATED),
                "the launch sizes LDS for this epilogue");
  uint16_t* stage_out = reinterpret_cast<uint16_t*>(smem + kXBytes + (GATED ? wave_m : wave) * (32 * kCols * 2));
  f32x16* xchg = reinterpret_cast<f32x16*>(smem) + wave_m * TN * 64;
  const bool vec_ok = (FO % 8) == 0;
  // Q2: w2's packed activation buffer ([M, F], K = F a multiple of 64) and smooth
  const uint32_t q2_code_bytes = Q2 ? (uint32_t)(FO / 64) * MP * 1024 : 0u;
  const __amdgpu_buffer_rsrc_t rq2 = make_rsrc(a.next_qact, Q2 ? q2_code_bytes + (uint32_t)(FO / 64) * MP * 128 : 0u);
  const __amdgpu_buffer_rsrc_t rs2 = make_rsrc(a.next_smooth, Q2 ? (uint32_t)FO * 2 : 0u);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    if (GATED) {
      if (wave_n == 1) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          f32x16 v = acc[i][j];
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] += bias_v[j];
          xchg[j * 64 + lane] = v;
        }
      }
      __syncthreads();
    }
    if (writer) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        f32x16 up;
        if (GATED) up = xchg[j * 64 + lane];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 8 * (r >> 2) + 4 * h + (r & 3);
          float v = acc[i][j][r] + bias_v[j];
          if (GATED) v = v / (1.0f + __expf(-v)) * up[r];
          stage_out[row * kCols + 32 * j + l32] = (uint16_t)f32_to_bf16_rne(v);
        }
      }
    }
    __syncthreads();
    if (writer) {
#pragma unroll
      for (int u = 0; u < (32 * kPieces + 63) / 64; ++u) {
        const int idx = lane + 64 * u;
        if (idx < 32 * kPieces) {
          const int row = idx / kPieces, piece = idx % kPieces;
          const int m = m_w + 32 * i + row;
          const int n = n_w + 8 * piece;
          const u32x4 v = *reinterpret_cast<const u32x4*>(stage_out + row * kCols + 8 * piece);
          if (m < M && n < FO) {
            uint16_t* dst = a.y + (size_t)m * FO + n;
            if (vec_ok && n + 8 <= FO) {
              *reinterpret_cast<u32x4*>(dst) = v;
            } else {
              for (int e = 0; e < 8 && n + e < FO; ++e) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
            }
          }
          if (Q2) {
            // this lane's 8 columns are half of the 16-block n & ~15; every lane of the
            // wave is here (whole pieces per iteration), so the lane swap is complete
            const bool n_in = n < FO;
            const u32x4 smv = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs2, n_in ? (uint32_t)n * 2 : 0x80000000u, 0, 0));
            float q[8];
            float amax = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              q[2 * e] = bf16lo_to_f32(v[e]) * bf16lo_to_f32(smv[e]);
              q[2 * e + 1] = bf16hi_to_f32(v[e]) * bf16hi_to_f32(smv[e]);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(q[e]));
            amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(amax), 0xB1, 0xF, 0xF, false)));
            const uint32_t sc = block_scale_code(amax);
            const float sd = e4m3_to_f32(sc, 0);
            const float inv = sd > 0.0f ? scale_reciprocal(sd) : 0.0f;
            uint32_t pk = 0u;
            pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, snap21(q[0] * inv), snap21(q[1] * inv), 1.0f, 0);
            pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, snap21(q[2] * inv), snap21(q[3] * inv), 1.0f, 1);
            pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, snap21(q[4] * inv), snap21(q[5] * inv), 1.0f, 2);
            pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, snap21(q[6] * inv), snap21(q[7] * inv), 1.0f, 3);
            // packed activation layout of [M, F]: chunk (n / 64, m / 32), dword (hh * 32 + c) * 4 + t
            const int mq = m >> 5, c = m & 31, pp = n >> 6, t = (n >> 4) & 3, hh = (n >> 3) & 1;
            const bool ok = n_in && mq < MP;
            const uint32_t chunk = (uint32_t)pp * MP + mq;
            __builtin_amdgcn_raw_buffer_store_b32(pk, rq2, ok ? chunk * 1024 + ((hh * 32 + c) * 4 + t) * 4 : 0x80000000u,
                                                  0, 0);
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sc, rq2,
                                                 ok && hh == 0 ? q2_code_bytes + chunk * 128 + c * 4 + t : 0x80000000u,
                                                 0, 0);
          }
        }
      }
    }
    __syncthreads();
  }
}

template <int WM, int WN, int TM, int TN, bool GATED, bool Q2 = false, bool CA = false, bool CW = false>
hipError_t launch_lds_cfg(const GemmArgs& a, hipStream_t stream) {
  using C = LdsCfg<WM, WN, TM, TN>;
  const int64_t col_tiles = GATED ? ((a.gated_f + 31) / 32 + TN - 1) / TN : (a.N + C::BN - 1) / C::BN;
  const int64_t tiles = col_tiles * ((a.M + C::BM - 1) / C::BM);
  const unsigned lds = C::lds_bytes(GATED);
  static_assert(C::lds_bytes(GATED) <= 160 * 1024, "LDS per workgroup");
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(&gemm_lds_kernel<WM, WN, TM, TN, GATED, Q2, CA, CW>),
                                    (int)lds, lds_set);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((tiles + 7) / 8 * 8));
  hipLaunchKernelGGL((gemm_lds_kernel<WM, WN, TM, TN, GATED, Q2, CA, CW>), grid, dim3(C::kThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

static std::atomic<int> g_gemm_tile{0};

template <bool CA, bool CW>
hipError_t launch_tile(const GemmArgs& a, hipStream_t stream, int pick) {
  static_assert(!(CA && CW), "canonical activations and weights together take the older kernel");
  switch (pick) {
    case 1: return launch_lds_cfg<4, 2, 2, 4, false, false, CA, CW>(a, stream);
    case 2: return launch_lds_cfg<4, 2, 1, 5, false, false, CA, CW>(a, stream);
    case 3: return launch_lds_cfg<4, 1, 1, 5, false, false, CA, CW>(a, stream);
    default: return launch_lds_cfg<4, 2, 2, 5, false, false, CA, CW>(a, stream);
  }
}

// Tile shape. The candidates, with the time of one round of workgroups relative to
// the 256 x 320 shape's, measured at full occupancy (K = 3840):
//   1: 256 x 320, 8 waves of 64 x 160, one workgroup per CU       1.0
//   2: 256 x 256, 8 waves of 64 x 128, one per CU                 0.82
//   3: 128 x 320, 8 waves of 32 x 160, one per CU                 0.62
//   4: 128 x 160, 4 waves of 32 x 160, two per CU                 0.66, or 0.49
//      when no CU has a second one (not gated: that epilogue pairs two wave columns)
// The estimate is rounds x that factor, the smallest wins (ties to the lower
// number). The large tiles keep full-size layers on few dequantisations per
// flop (N = 10240 at M = 4096: 512 tiles of shape 1, two rounds); the small ones
// keep the CUs busy when the output is small, as for one GPU's share of a layer
// split 8 ways by columns (N = 1280: 64 tiles of shape 1, 256 of shape 4).
hipError_t launch_gemm_lds(const GemmArgs& a, hipStream_t stream) {
  const bool gated = a.gated_f > 0;
  const int64_t FP = gated ? (a.gated_f + 31) / 32 : 0;
  auto cols = [&](int TN, int WN) -> int64_t {
    return gated ? (FP + TN - 1) / TN : (a.N + 32 * TN * WN - 1) / (32 * TN * WN);
  };
  const int64_t r256 = (a.M + 255) / 256, r128 = (a.M + 127) / 128;
  const int64_t tiles[4] = {r256 * cols(5, 2), r256 * cols(4, 2), r128 * cols(5, 2), r128 * cols(5, 1)};
  auto rounds = [](int64_t t, int64_t slots) { return (double)((t + slots - 1) / slots); };
  const double cost[4] = {rounds(tiles[0], 256), 0.82 * rounds(tiles[1], 256), 0.62 * rounds(tiles[2], 256),
                          gated ? 1e30 : (tiles[3] <= 256 ? 0.49 : 0.66 * rounds(tiles[3], 512))};
  int pick = 0;
  for (int i = 1; i < 4; ++i)
    if (cost[i] < cost[pick]) pick = i;
  const int forced = g_gemm_tile.load(std::memory_order_relaxed);
  if (forced >= 1 && forced <= 4 && !(gated && forced == 4)) pick = forced - 1;
  if (gated) {
    const bool q2 = a.next_qact != nullptr;
    if (pick == 1)
      return q2 ? launch_lds_cfg<4, 2, 2, 4, true, true>(a, stream) : launch_lds_cfg<4, 2, 2, 4, true>(a, stream);
    if (pick == 2)
      return q2 ? launch_lds_cfg<4, 2, 1, 5, true, true>(a, stream) : launch_lds_cfg<4, 2, 1, 5, true>(a, stream);
    return q2 ? launch_lds_cfg<4, 2, 2, 5, true, true>(a, stream) : launch_lds_cfg<4, 2, 2, 5, true>(a, stream);
  }
  if (a.act_canonical) {
    if (!a.packed) return hipErrorInvalidValue;   // both canonical: not this kernel
    return launch_tile<true, false>(a, stream, pick);
  }
  return a.packed ? launch_tile<false, false>(a, stream, pick) : launch_tile<false, true>(a, stream, pick);
}

int set_gemm_tile(int tile) { return g_gemm_tile.exchange(tile); }

}  // namespace svdq
