// Fused activation quantisation and low-rank down-projection: one pass over x
// produces quant(x * smooth) (codes + e4m3 block scales) and
// lora_act = bf16(x @ proj_down) (model card "nunchaku-z-image-turbo-svdq",
// section "What's stored on disk": the activation operand of scaled_mma and
// the (x @ proj_down) factor of the SVD residual; raw x feeds the residual).
//
// Three kernels. With a down-projection, quant_lora_ws_kernel (below) splits each
// workgroup's waves into quantisers and matrix waves, with K split across
// workgroups; for short K, quant_lora_rs_kernel (further below) splits the rank
// across workgroups instead and needs no partial sums. quant_lora_kernel serves
// the quantisation alone (R = 0, packed output), the down-projection alone, and
// the lora_act columns past the first 128.
//
// Work split. A workgroup of 8 waves owns 128 * RT rows: wave w owns rows
// 16 * RT * w .. +16 * RT - 1 (RT row tiles of 16; RT = 1 is launched). K is
// cut into 32-wide steps; a workgroup walks the steps of its K split
// (blockIdx.y) in order, every wave on its own rows. Each lane holds 8 consecutive k of one row (a
// 16-byte load), which is at once the A fragment of v_mfma_f32_16x16x32_bf16
// and half of an NVFP4 block (the other half sits in lane ^ 16).
//
// proj_down is shared through LDS: per step the 512 threads load the 32 x 128
// slice of proj_down once (one 16-byte row piece each, coalesced) and scatter
// it with 2-byte LDS writes straight into B-fragment order (the [K, R] layout
// is R-contiguous, the fragments are K-contiguous), into one of two stages;
// after one barrier every wave reads its 8 fragments from there. Fragment i
// holds the column set {8c + i : c = 0..15} (c = lane % 16), so the output
// lane layout gives each lane 8 consecutive r of one row. Operands are loaded
// two steps ahead (three register sets rotated by name: the loop is unrolled
// by three, so a load's destination is never copied while in flight).
//
// Each wave accumulates its own rows over the whole split, so no cross-wave
// reduction is needed. With one K split it stores bf16 lora_act directly;
// with several, each split stores fp32 partial sums and a second kernel adds
// them in split order (deterministic).
//
// The code decision follows the same exact scheme as the standalone
// quantisation kernel (see quant_act.hip): q = v * RN(1/s_d), rounded to 21
// significant bits, then the hardware E2M1 round-to-nearest-even.
//
// Output layouts: canonical (qact [M, K/2], ascales [K/16, M]) or the packed
// MFMA-fragment layout used by the GEMM (the same chunk order as the packed
// weights, with rows = tokens): code chunk (p, q) of 1024 bytes at
// 1024*(p*MP + q), dword (h*32 + c)*4 + t = row 32q + c, k = 64p + 16t + 8h;
// scale chunk at 1024*KP*MP + 128*(p*MP + q), byte c*4 + t.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "mx_format.h"

namespace svdq {

namespace {

constexpr int kRChunk = 128;   // lora_act columns per launch
constexpr int kWaves = 8;

template <int RT>
struct XRegs {
  u32x4 x[RT];   // 8 consecutive k of this lane's row in each row tile
  u32x4 sm;      // smooth at the same 8 k
  u32x4 pd;      // proj_down piece this thread scatters into the fragment stage
};

struct QLArgs {
  const uint16_t* x;
  const uint16_t* smooth;
  const uint16_t* proj_down;
  uint8_t* qact;       // canonical [M, K/2] or the packed buffer
  uint8_t* ascales;    // canonical [K/16, M] (unused when packed)
  uint16_t* lora_act;  // [M, R]
  float* partial;      // [splits, M, R] fp32 partial sums when K is split (else NULL)
  int M, K, R;
  int r_base;          // first of the (up to kRChunk) lora_act columns this launch computes
  int split_steps;     // 32-wide K steps per split (blockIdx.y selects the split)
  const uint16_t* gscale;  // static global activation scale bf16 [1] (STATIC kernels only)
};

// QUANT: write the codes and scales; LORA: compute lora_act columns
// r_base .. r_base + kRChunk - 1. A rank above kRChunk takes further launches
// with QUANT = false.
template <int RT, bool PACKED, bool QUANT, bool LORA, bool STATIC = false>
__global__ __launch_bounds__(64 * kWaves) void quant_lora_kernel(QLArgs a) {
  constexpr int ROWS = 16 * RT * kWaves;
  BlockScale<STATIC> bs;
  if (QUANT) bs.init(a.gscale);
  // B fragments of one step: [stage][fragment i][lane] x 16 bytes
  __shared__ __attribute__((aligned(16))) uint8_t s_frag[LORA ? 2 * 8 * 1024 : 16];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int c = lane & 15;   // row within a 16-row tile; fragment column group
  const int g = lane >> 4;   // k group of 8 within a 32-wide step
  const int m_w = blockIdx.x * ROWS + wave * 16 * RT;
  const int ks = blockIdx.y;
  const int M = a.M, K = a.K, R = a.R;
  const int MP = (M + 31) / 32;
  const int KP = (K + 63) / 64;
  // packed output covers whole 64-wide panels: positions beyond K get zero codes
  // and zero scales (the GEMM multiplies them by the weight's zero padding); its
  // rows beyond M inside the last 32-row panel are written as zeros too
  const int steps = PACKED ? 2 * KP : (K + 31) / 32;
  const int s_begin = ks * a.split_steps;
  const int s_end = min(steps, s_begin + a.split_steps);
  const uint32_t code_bytes = (uint32_t)MP * KP * 1024;

  const uint32_t x_bytes = (uint32_t)M * K * 2;
  const uint32_t pd_bytes = (uint32_t)K * R * 2;
  const uint32_t q_bytes = PACKED ? code_bytes + (uint32_t)MP * KP * 128 : (uint32_t)M * (K / 2);
  const uint32_t s_bytes = PACKED ? 0u : (uint32_t)(K / 16) * M;
  const auto rx = make_rsrc(a.x, x_bytes);
  const auto rsm = make_rsrc(a.smooth, (uint32_t)K * 2);
  const auto rpd = make_rsrc(a.proj_down, pd_bytes);
  const auto rq = make_rsrc(a.qact, q_bytes);
  const auto rsc = make_rsrc(a.ascales, s_bytes);

  // this thread's proj_down piece of a step: row k = 32 st + pr, columns
  // r_base + 8 pc .. + 7; it belongs to fragment lane (pr / 8) * 16 + pc,
  // element pr % 8, of fragments i = 0..7
  const int pr = tid >> 4, pc = tid & 15;
  const int p_col = a.r_base + 8 * pc;
  const uint32_t p_dst = (uint32_t)(((pr >> 3) * 16 + pc) * 16 + (pr & 7) * 2);

  f32x4 acc[RT][8];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[t][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // operands of one step; positions outside the tensors read as zero
  auto load = [&](XRegs<RT>& r, int st) {
    const int kg = st * 32 + 8 * g;
    const bool k_in = st < s_end && kg < K;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int m = m_w + 16 * t + c;
      r.x[t] = __builtin_amdgcn_raw_buffer_load_b128(rx, k_in ? ((uint32_t)m * K + kg) * 2 : x_bytes, 0, 0);
    }
    if (QUANT) r.sm = __builtin_amdgcn_raw_buffer_load_b128(rsm, k_in ? kg * 2 : K * 2, 0, 0);
    if (LORA) {
      const int k = st * 32 + pr;
      const bool in = st < s_end && k < K && p_col < R;
      r.pd = __builtin_amdgcn_raw_buffer_load_b128(rpd, in ? ((uint32_t)k * R + p_col) * 2 : pd_bytes, 0, 0);
    }
  };
  auto scatter_pd = [&](const XRegs<RT>& r, int stage) {
    uint8_t* dst = s_frag + stage * 8192 + p_dst;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<uint16_t*>(dst + i * 1024) = (uint16_t)(r.pd[i >> 1] >> (16 * (i & 1)));
  };

  // one 32-wide step: quantise this step's x, multiply it with the fragments in
  // `stage`, and scatter the next step's proj_down piece into the other stage
  auto process = [&](const XRegs<RT>& cur, const XRegs<RT>& next, int st, int stage) {
    const int kg = st * 32 + 8 * g;
    const bool k_in = kg < K;
    if (LORA) {
      __syncthreads();                                   // `stage` written, the other free
      if (st + 1 < s_end) scatter_pd(next, stage ^ 1);
    }
    if (QUANT) {
      float sm[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sm[2 * j] = bf16lo_to_f32(cur.sm[j]);
        sm[2 * j + 1] = bf16hi_to_f32(cur.sm[j]);
      }
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int m = m_w + 16 * t + c;
        float v[8];
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[2 * j] = bf16lo_to_f32(cur.x[t][j]) * sm[2 * j];
          v[2 * j + 1] = bf16hi_to_f32(cur.x[t][j]) * sm[2 * j + 1];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
        amax = fmaxf(amax, __shfl_xor(amax, 16));   // other half of the block
        const uint32_t sc = bs.code(amax);
        const float sd = bs.divisor(sc);
        const float inv = sd > 0.0f ? scale_reciprocal(sd) : 0.0f;
        uint32_t packed = 0u;
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, snap21(v[0] * inv), snap21(v[1] * inv), 1.0f, 0);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, snap21(v[2] * inv), snap21(v[3] * inv), 1.0f, 1);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, snap21(v[4] * inv), snap21(v[5] * inv), 1.0f, 2);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, snap21(v[6] * inv), snap21(v[7] * inv), 1.0f, 3);
        if (PACKED) {
          const int pp = kg >> 6, tt = (kg >> 4) & 3, hh = (kg >> 3) & 1;
          // rows of the last 32-row panel beyond M are written (as zeros); a
          // workgroup's rows past that panel are not stored at all
          const int q = m >> 5, cc = m & 31;
          const bool in_panel = q < MP;
          const uint32_t chunk = (uint32_t)pp * MP + q;
          __builtin_amdgcn_raw_buffer_store_b32(packed, rq, in_panel ? chunk * 1024 + ((hh * 32 + cc) * 4 + tt) * 4 : q_bytes, 0, 0);
          if (hh == 0)
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sc, rq, in_panel ? code_bytes + chunk * 128 + cc * 4 + tt : q_bytes, 0, 0);
        } else {
          const bool ok = k_in && m < M;
          __builtin_amdgcn_raw_buffer_store_b32(packed, rq, ok ? (uint32_t)m * (K / 2) + kg / 2 : q_bytes, 0, 0);
          if ((g & 1) == 0)
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sc, rsc, ok ? (uint32_t)(kg >> 4) * M + m : s_bytes, 0, 0);
        }
      }
    }
    if (LORA) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(s_frag + stage * 8192 + i * 1024 + lane * 16);
#pragma unroll
        for (int t = 0; t < RT; ++t)
          acc[t][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.x[t]), b,
                                                              acc[t][i], 0, 0, 0);
      }
    }
  };

  XRegs<RT> r0, r1, r2;
  load(r0, s_begin);
  load(r1, s_begin + 1);
  if (LORA) scatter_pd(r0, 0);
  int stage = 0;
  for (int st = s_begin; st < s_end; st += 3) {
    load(r2, st + 2);
    process(r0, r1, st, stage);
    stage ^= 1;
    if (st + 1 >= s_end) break;
    load(r0, st + 3);
    process(r1, r2, st + 1, stage);
    stage ^= 1;
    if (st + 2 >= s_end) break;
    load(r1, st + 4);
    process(r2, r0, st + 2, stage);
    stage ^= 1;
  }

  if (LORA) {
    // lane holds rows 16t + 4g + q of its wave and columns rcol .. rcol+7
    const int rcol = a.r_base + 8 * c;
    const bool r_in = rcol < R;
    const uint32_t l_bytes = (uint32_t)M * R * 2;
    const uint32_t p_bytes = a.partial != nullptr ? (uint32_t)gridDim.y * M * R * 4 : 0u;
    const auto rl = make_rsrc(a.lora_act, l_bytes);
    const auto rp = make_rsrc(a.partial, p_bytes);
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m_w + 16 * t + 4 * g + q;
        const bool ok = r_in && m < M;
        if (a.partial == nullptr) {
          u32x4 o;
#pragma unroll
          for (int w = 0; w < 4; ++w) o[w] = pack_bf16x2(acc[t][2 * w][q], acc[t][2 * w + 1][q]);
          __builtin_amdgcn_raw_buffer_store_b128(o, rl, ok ? ((uint32_t)m * R + rcol) * 2 : l_bytes, 0, 0);
        } else {
          u32x4 o0, o1;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            o0[w] = __float_as_uint(acc[t][w][q]);
            o1[w] = __float_as_uint(acc[t][4 + w][q]);
          }
          const uint32_t off = (((uint32_t)ks * M + m) * R + rcol) * 4;
          __builtin_amdgcn_raw_buffer_store_b128(o0, rp, ok ? off : p_bytes, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b128(o1, rp, ok ? off + 16 : p_bytes, 0, 0);
        }
      }
  }
}

// Wave-specialised form of the same operation (quantisation and the first 128
// lora_act columns together), used for R > 0. A workgroup owns 128 rows and walks
// the 64-wide K panels of its split. Waves 0-3 quantise: quantiser wave q reads
// rows 32 q .. 32 q + 31 of each panel with whole 128-byte row pieces (lane l:
// row 8 i + l / 8 of load i, k piece l % 8, so one NVFP4 block sits in a lane
// pair), quantises them, and copies them into LDS for the down-projection. Waves
// 4-7 (wave 4 + q shares a SIMD with quantiser wave q and takes the same rows)
// load proj_down, and multiply lora^T = proj_down^T x^T with
// v_mfma_f32_32x32x16_bf16: the x operand is read from LDS in the instruction's
// layout, proj_down is stored in its own row-major layout (16-byte piece p of
// row k at piece p ^ 4 (k % 4)) and read by the transposing ds_read_tr16_b64.
// Both operands are double-buffered per panel, one barrier per panel; the
// quantisers prefetch x two panels ahead, so their VALU work overlaps the
// down-projection's matrix instructions on the same SIMD. The accumulators leave
// through LDS so that every store writes whole rows of lora_act or of the fp32
// partial sums.
constexpr int kWsRows = 128;
constexpr int kWsX = 16384;                  // x of one panel: 4 waves x 32 rows x 128 bytes
constexpr int kWsStage = kWsX + 64 * 256;    // + proj_down of one panel (64 k x 128 r bf16)

typedef short v4s __attribute__((ext_vector_type(4)));
#define WS_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// MXO: the quantisers write the MXFP4 variant's operand instead (gemm_mx.hip's
// layout and the rule of mx_format.h: a 32-block is the four lanes of a DPP quad,
// whose maximum two quad swaps gather); qact and ascales are then the MX code and
// scale buffers, K % 128 == 0, and PACKED and STATIC are false.
template <bool PACKED, bool STATIC = false, bool MXO = false>
__global__ __launch_bounds__(512) void quant_lora_ws_kernel(QLArgs a) {
  static_assert(!MXO || (!PACKED && !STATIC), "the MX output has its own layout and dynamic scales");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kWsStage];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const bool quantiser = wave < 4;
  const int qw = wave & 3;
  const int M = a.M, K = a.K, R = a.R;
  if ((int)blockIdx.x * kWsRows >= M) return;
  const int KP = (K + 63) / 64;
  const int MP = (M + 31) / 32;
  const int m0 = blockIdx.x * kWsRows + 32 * qw;     // first row of this wave
  const int ks = blockIdx.y;
  const int p_begin = ks * a.split_steps;              // split_steps counts 64-wide panels here
  const int n = min(KP, p_begin + a.split_steps) - p_begin;
  const uint32_t code_bytes = (uint32_t)MP * KP * 1024;
  const uint32_t x_bytes = (uint32_t)M * K * 2;
  const uint32_t pd_bytes = (uint32_t)K * R * 2;
  const uint32_t q_bytes = MXO ? (uint32_t)MP * 32 * (uint32_t)(K / 2)
                               : PACKED ? code_bytes + (uint32_t)MP * KP * 128 : (uint32_t)M * (K / 2);
  const uint32_t s_bytes = MXO ? (uint32_t)(K / 32) * MP * 32 : PACKED ? 0u : (uint32_t)(K / 16) * M;
  const auto rx = make_rsrc(a.x, x_bytes);
  const auto rsm = make_rsrc(a.smooth, (uint32_t)K * 2);
  const auto rpd = make_rsrc(a.proj_down, pd_bytes);
  const auto rq = make_rsrc(a.qact, q_bytes);
  const auto rsc = make_rsrc(a.ascales, s_bytes);

  // ---- quantiser waves: lane's rows r_i = 8 i + lane / 8 (i = 0..3), k piece pc
  const int pc = lane & 7;
  const int rl = lane >> 3;
  auto x_off = [&](int j, int i) -> uint32_t {      // panel j of the split (j may be >= n)
    const int m = m0 + 8 * i + rl;
    const int k = 64 * (p_begin + j) + 8 * pc;
    return j < n && m < M && k < K ? ((uint32_t)m * K + k) * 2 : x_bytes;
  };
  // x in LDS for the down-projection: row r, piece p at r * 128 + (p ^ ((r / 2) % 8)) * 16
  auto x_slot = [](int r, int p) { return r * 128 + ((p ^ ((r >> 1) & 7)) << 4); };

  // ---- down-projection waves
  f32x16 acc[4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[f][r] = 0.0f;
  // proj_down piece e = 256 u + 64 q + lane (u = 0..3) of a panel: row k = e / 16,
  // stored slot e % 16 = lane % 16, source piece (lane % 16) ^ 4 (k % 4)
  const int pd_r = a.r_base + 8 * ((lane & 15) ^ (4 * ((lane >> 4) & 3)));
  const uint32_t pd_lane = ((uint32_t)(lane >> 4) * R + pd_r) * 2;
  auto pd_off = [&](int j, int u) -> uint32_t {
    const int k0 = 64 * (p_begin + j) + 16 * u + 4 * qw;   // rows k0 .. k0 + 3 (lane / 16)
    return j < n && k0 < K && pd_r < R ? (uint32_t)k0 * R * 2 + pd_lane : pd_bytes;
  };
  // transposing reads: source lane (16 grp + 4 jj + qq) points at row 8 (grp / 2) + 4 h + jj,
  // columns 32 f + 16 (grp % 2) + 4 qq of the 16-k step
  const int grp = lane >> 4, jj = (lane >> 2) & 3, qq = lane & 3;
  const int tr_base = (8 * (grp >> 1) + jj) * 256 + (qq & 1) * 8 + (2 * (grp & 1) + (qq >> 1)) * 16;

  u32x4 X0[5], X1[5], X2[5];      // quantisers: x of three panels (4 rows) and their smooth
  u32x4 P0[4], P1[4], P2[4];      // down-projection: proj_down of three panels
  auto load_x = [&](u32x4 (&X)[5], int j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) X[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, x_off(j, i), 0, 0);
    const int k = 64 * (p_begin + j) + 8 * pc;
    X[4] = __builtin_amdgcn_raw_buffer_load_b128(rsm, j < n && k < K ? k * 2 : K * 2, 0, 0);
  };
  auto put_x = [&](const u32x4 (&X)[5], int b) {
    uint8_t* base = smem + b * kWsStage + qw * 4096;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(base + x_slot(8 * i + rl, pc)) = X[i];
  };
  auto load_pd = [&](u32x4 (&P)[4], int j) {
#pragma unroll
    for (int u = 0; u < 4; ++u) P[u] = __builtin_amdgcn_raw_buffer_load_b128(rpd, pd_off(j, u), 0, 0);
  };
  auto put_pd = [&](const u32x4 (&P)[4], int b) {
    uint8_t* base = smem + b * kWsStage + kWsX;
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<u32x4*>(base + (256 * u + 64 * qw + lane) * 16) = P[u];
  };

  BlockScale<STATIC> bs;
  if (quantiser) bs.init(a.gscale);
  // quantise panel j from X (all four rows of the lane), store codes and scales
  auto quantise = [&](const u32x4 (&X)[5], int j) {
    const int p = p_begin + j;
    const int k = 64 * p + 8 * pc;
    const u32x4 sv = X[4];
    float sm[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sm[2 * e] = bf16lo_to_f32(sv[e]);
      sm[2 * e + 1] = bf16hi_to_f32(sv[e]);
    }
    const int t = pc >> 1, h = pc & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * i + rl;
      const int m = m0 + r;
      float v[8];
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = bf16lo_to_f32(X[i][e]) * sm[2 * e];
        v[2 * e + 1] = bf16hi_to_f32(X[i][e]) * sm[2 * e + 1];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
      // the other half of the block sits in lane ^ 1 (a DPP lane swap, no LDS round trip)
      amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(amax), 0xB1, 0xF, 0xF, false)));
      if constexpr (MXO) {
        // the rest of the 32-block sits in lane ^ 2 and lane ^ 3
        amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(amax), 0x4E, 0xF, 0xF, false)));
        const int X = mx_exponent(amax);
        const uint32_t pk = mx_codes8(v, X);
        // chunk (panel p, row panel q): lane 32 hb + r of the matrix instruction holds
        // 32-block hb of the panel, 4 bytes per pc % 4; rows of the last 32-row panel
        // beyond M are written (zero codes, scale byte 0)
        const int q = m0 >> 5, hb = pc >> 2, jq = pc & 3;
        const bool ok = j < n && q < MP;
        const uint32_t chunk = (uint32_t)p * MP + q;
        __builtin_amdgcn_raw_buffer_store_b32(pk, rq, ok ? chunk * 1024 + (32 * hb + r) * 16 + 4 * jq : q_bytes, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(X + 127), rsc,
                                             ok && jq == 0 ? (uint32_t)(2 * p + hb) * (MP * 32) + (uint32_t)(m0 + r)
                                                           : s_bytes,
                                             0, 0);
        continue;
      }
      const uint32_t sc = bs.code(amax);
      const float sd = bs.divisor(sc);
      const float inv = sd > 0.0f ? scale_reciprocal(sd) : 0.0f;
      uint32_t pk = 0u;
      pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, snap21(v[0] * inv), snap21(v[1] * inv), 1.0f, 0);
      pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, snap21(v[2] * inv), snap21(v[3] * inv), 1.0f, 1);
      pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, snap21(v[4] * inv), snap21(v[5] * inv), 1.0f, 2);
      pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, snap21(v[6] * inv), snap21(v[7] * inv), 1.0f, 3);
      if (PACKED) {
        // rows of the last 32-row panel beyond M are written (as zeros); a
        // wave's rows past that panel are not stored at all
        const int q = m0 >> 5;
        const bool ok = j < n && q < MP;
        const uint32_t chunk = (uint32_t)p * MP + q;
        __builtin_amdgcn_raw_buffer_store_b32(pk, rq, ok ? chunk * 1024 + ((h * 32 + r) * 4 + t) * 4 : q_bytes, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sc, rq, ok && h == 0 ? code_bytes + chunk * 128 + r * 4 + t : q_bytes,
                                             0, 0);
      } else {
        const bool ok = j < n && m < M && k < K;
        __builtin_amdgcn_raw_buffer_store_b32(pk, rq, ok ? (uint32_t)m * (K / 2) + k / 2 : q_bytes, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sc, rsc, ok && h == 0 ? (uint32_t)(k >> 4) * M + m : s_bytes, 0, 0);
      }
    }
  };

  // down-projection of panel j out of buffer b
  auto multiply = [&](int b) {
    const uint8_t* xs = smem + b * kWsStage + qw * 4096;
    const uint8_t* ps = smem + b * kWsStage + kWsX;
    const int mr = lane & 31, hh = lane >> 5;
    bf16x8 xb[4];
    v4s lo[4][4], hi[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      xb[tt] = *reinterpret_cast<const bf16x8*>(xs + x_slot(mr, 2 * tt + hh));
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int off = tt * 4096 + tr_base + 64 * (f ^ jj);
        lo[tt][f] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(WS_LDS(v4s, ps + off));
        hi[tt][f] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(WS_LDS(v4s, ps + off + 1024));
      }
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const bf16x8 pf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo[tt][f], hi[tt][f], 0, 1, 2, 3, 4, 5, 6, 7));
        acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf, xb[tt], acc[f], 0, 0, 0);
      }
  };

  // panel j (buffer j % 2): the quantisers prefetch x two panels ahead, quantise
  // panel j and copy panel j + 1 into the other buffer; the down-projection waves
  // prefetch proj_down two panels ahead, multiply panel j (all of its LDS reads
  // issued before its matrix instructions) and copy panel j + 1's proj_down into
  // the other buffer. Three register sets per role, rotated by name; prefetches
  // past the split read zeros. The role is uniform per wave, so each role runs its
  // own loop with one barrier per panel (the same count, n + 1, in both), and only
  // that role's registers are live.
  if (quantiser) {
    auto qstep = [&](const u32x4 (&cur)[5], const u32x4 (&nxt)[5], u32x4 (&ahead)[5], int j) {
      load_x(ahead, j + 2);
      __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of this panel's work
      put_x(nxt, (j + 1) & 1);
      quantise(cur, j);
      __syncthreads();
    };
    load_x(X0, 0);
    load_x(X1, 1);
    put_x(X0, 0);
    __syncthreads();
    for (int j = 0; j < n; j += 3) {
      qstep(X0, X1, X2, j);
      if (j + 1 < n) qstep(X1, X2, X0, j + 1);
      if (j + 2 < n) qstep(X2, X0, X1, j + 2);
    }
    return;
  }
  auto lstep = [&](const u32x4 (&pnxt)[4], u32x4 (&pahead)[4], int j) {
    load_pd(pahead, j + 2);
    __builtin_amdgcn_sched_barrier(0);
    if (j < n) multiply(j & 1);
    put_pd(pnxt, (j + 1) & 1);
    __syncthreads();
  };
  load_pd(P0, 0);
  load_pd(P1, 1);
  put_pd(P0, 0);
  __syncthreads();
  for (int j = 0; j < n; j += 3) {
    lstep(P1, P2, j);
    if (j + 1 < n) lstep(P2, P0, j + 1);
    if (j + 2 < n) lstep(P0, P1, j + 2);
  }

  {
    // The accumulators go out through this wave's 16 KB of LDS (free after the last
    // barrier), so that every store instruction writes whole rows. Lane holds row
    // m0 + lane % 32 and columns r_base + 32 f + 8 G + 4 (lane / 32) + e; the staging area
    // holds 32 rows of 128 fp32 columns, 16-byte slot s of row m at slot s ^ m (bank
    // conflict free both ways).
    float* st = reinterpret_cast<float*>(smem + qw * 16384);
    const int ml = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int G = 0; G < 4; ++G) {
        const int s = 8 * f + 2 * G + hh;
        *reinterpret_cast<f32x4*>(st + ml * 128 + ((s ^ ml) << 2)) =
            f32x4{acc[f][4 * G], acc[f][4 * G + 1], acc[f][4 * G + 2], acc[f][4 * G + 3]};
      }
    if (a.partial != nullptr) {
      // fp32 partials: one instruction writes rows 2 i, 2 i + 1 (lane: 4 columns)
      const uint32_t p_bytes = (uint32_t)gridDim.y * M * R * 4;
      const auto rp = make_rsrc(a.partial, p_bytes);
      const int c = lane & 31;
      f32x4 v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rl = 2 * i + hh;
        v[i] = *reinterpret_cast<const f32x4*>(st + rl * 128 + ((c ^ rl) << 2));
      }
      const int r = a.r_base + 4 * c;
      const uint32_t base = (((uint32_t)ks * M + m0 + hh) * R + r) * 4;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool ok = m0 + 2 * i + hh < M && r < R;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v[i]), rp,
                                               ok ? base + (uint32_t)(2 * i * R * 4) : p_bytes, 0, 0);
      }
    } else {
      // bf16 lora_act: one instruction writes rows 4 i .. 4 i + 3 (lane: 8 columns)
      const uint32_t l_bytes = (uint32_t)M * R * 2;
      const auto rl2 = make_rsrc(a.lora_act, l_bytes);
      const int c8 = lane & 15;
      u32x4 o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int rl = 4 * i + (lane >> 4);
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(st + rl * 128 + (((2 * c8) ^ rl) << 2));
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(st + rl * 128 + (((2 * c8 + 1) ^ rl) << 2));
        o[i] = u32x4{pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]), pack_bf16x2(v1[0], v1[1]),
                     pack_bf16x2(v1[2], v1[3])};
      }
      const int r = a.r_base + 8 * c8;
      const uint32_t base = ((uint32_t)(m0 + (lane >> 4)) * R + r) * 2;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool ok = m0 + 4 * i + (lane >> 4) < M && r < R;
        __builtin_amdgcn_raw_buffer_store_b128(o[i], rl2, ok ? base + (uint32_t)(4 * i * R * 2) : l_bytes, 0, 0);
      }
    }
  }
}

// lora_act = bf16(sum over the K splits of the fp32 partials), the splits
// added in index order (deterministic). One thread per 8 consecutive columns.
__global__ __launch_bounds__(256) void lora_reduce_kernel(const float* __restrict__ partial,
                                                          uint16_t* __restrict__ lora, int M, int R,
                                                          int splits) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // group of 8 columns
  const int64_t groups = (int64_t)M * (R / 8);
  if (i >= groups) return;
  const size_t plane = (size_t)M * R;
  f32x4 s0 = *reinterpret_cast<const f32x4*>(partial + i * 8);
  f32x4 s1 = *reinterpret_cast<const f32x4*>(partial + i * 8 + 4);
  for (int k = 1; k < splits; ++k) {
    s0 += *reinterpret_cast<const f32x4*>(partial + k * plane + i * 8);
    s1 += *reinterpret_cast<const f32x4*>(partial + k * plane + i * 8 + 4);
  }
  u32x4 o;
  o[0] = pack_bf16x2(s0[0], s0[1]);
  o[1] = pack_bf16x2(s0[2], s0[3]);
  o[2] = pack_bf16x2(s1[0], s1[1]);
  o[3] = pack_bf16x2(s1[2], s1[3]);
  *reinterpret_cast<u32x4*>(lora + i * 8) = o;
}

// One row tile per wave (128 rows per workgroup): measured on MI355X, two tiles
// per wave only paid off at M = 16896, K = 10240 (150 vs 164 us) and lost
// elsewhere (a workgroup of 8 waves x ~90 VGPRs leaves room for two per CU).
constexpr int kRowTiles = 1;
constexpr int kRows = 16 * kRowTiles * kWaves;

// K splits. A split multiplies the workgroups but adds fp32 partial sums to
// write and add back. Modelled time: rounds * steps_per_split * 0.65 us +
// splits * M * R * 1.26e-6 us, where a round is one workgroup per CU (256)
// with the down-projection and two per CU without it. Fitted to a sweep of
// 1 .. 16 splits at M = 4096 and 16896, K = 3840 and 10240, R = 128, which it
// reproduces within about 5%; the cheapest split count wins. Without R there
// are no partial sums.
int k_splits(int64_t M, int64_t K, int64_t R, bool packed_out) {
  const int64_t row_blocks = (M + kRows - 1) / kRows;
  const int64_t steps = packed_out ? 2 * ((K + 63) / 64) : (K + 31) / 32;
  const int64_t per_round = R > 0 ? 256 : 512;
  int best = 1;
  double best_cost = 0.0;
  for (int ks = 1; ks <= 16; ++ks) {
    if (ks > 1 && steps / ks < 4) break;
    if (R > 0 && ks > 1 && ks * M * R * 4 >= (int64_t(1) << 31)) break;   // 32-bit partial offsets
    const int64_t rounds = (row_blocks * ks + per_round - 1) / per_round;
    const int64_t per_split = (steps + ks - 1) / ks;
    const double cost = (double)rounds * (double)per_split * 0.65 +
                        (R > 0 && ks > 1 ? (double)ks * (double)M * (double)R * 1.26e-6 : 0.0);
    if (ks == 1 || cost < best_cost) {
      best = ks;
      best_cost = cost;
    }
  }
  return best;
}

// Split-free form (R in (64, 128]): no partial sums and no reduction launch. A
// workgroup owns 32 rows and 64 of the lora_act columns over the whole of K; the
// two workgroups of a row block are dispatched to the same XCD (blocks 16 g + j and
// 16 g + 8 + j, j < 8) and quantise alternate 64-K panels between them. Waves 4-7
// copy x, proj_down and smooth global -> LDS with buffer loads that write LDS
// directly (the swizzle applied on the source side), in 256-K super-panels, three
// stages, two ahead, and run the down-projection on v_mfma_f32_16x16x32_bf16: wave
// 4 + m takes the 64-K sub-panel m of every super-panel, and the four partial sums
// are added in wave order at the end. Waves 0-3 read their x from LDS and quantise.
// Only the matrix waves issue loads, so the quantisers' stores never share a vmcnt
// wait with a load. Every workgroup streams its half of proj_down over all of K, so
// the L2 traffic grows with K; the launcher uses this form where it is the faster.
constexpr int kRsCols = 64;
constexpr int kRsX = 16 * 1024;     // x: 16 blocks (sub-panel i, row group q) of 8 rows x 64 K
constexpr int kRsPd = 32 * 1024;    // proj_down: 32 blocks of 8 k x 64 columns
constexpr int kRsSm = 1024;         // smooth: 256 k (512 bytes used)
constexpr int kRsStage = kRsX + kRsPd + kRsSm;
constexpr int kRsStages = 3;
constexpr int kRsLds = kRsStages * kRsStage;

template <int N>
__device__ __forceinline__ void rs_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ void rs_wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// a barrier without the memory fence of __syncthreads (which would wait for the
// copies of later super-panels); the empty asm keeps LDS accesses on their side
__device__ __forceinline__ void rs_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
#define RS_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// x row r (0..31 of the block), 16-byte piece pc (0..7 of a 64-K sub-panel) at slot
// pc ^ rs_xswz(r) of its 128-byte LDS row; proj_down row k (0..255 of a super-panel),
// piece pp (8 columns) at slot pp ^ rs_pswz(k). Both make the fragment reads
// conflict-free (16-byte reads of 16 rows; transposing 8-byte reads of 8 rows).
__host__ __device__ constexpr int rs_xswz(int r) { return (r >> 1) & 7; }
__host__ __device__ constexpr int rs_pswz(int k) { return 4 * ((k >> 3) & 1) + 2 * ((k >> 1) & 1); }

template <bool PACKED, bool STATIC>
__global__ __launch_bounds__(512) void quant_lora_rs_kernel(QLArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int M = a.M, K = a.K, R = a.R;
  const int w = (int)blockIdx.x;
  const int h = (w >> 3) & 1;                  // column half
  const int b = 8 * (w >> 4) + (w & 7);        // row block
  const int MP = (M + 31) / 32;
  if (b >= MP) return;
  const int m0 = 32 * b;
  const int r0 = kRsCols * h;
  const int KP = (K + 63) / 64;
  const int nsp = (K + 255) / 256;
  const uint32_t x_bytes = (uint32_t)M * K * 2;
  const uint32_t pd_bytes = (uint32_t)K * R * 2;
  const uint32_t code_bytes = (uint32_t)MP * KP * 1024;
  const uint32_t q_bytes = PACKED ? code_bytes + (uint32_t)MP * KP * 128 : (uint32_t)M * (K / 2);
  const uint32_t s_bytes = PACKED ? 0u : (uint32_t)(K / 16) * M;
  auto stage_at = [&](int sp) { return smem + (sp % kRsStages) * kRsStage; };

  if (wave >= 4) {
    const int mw = wave - 4;
    const auto rx = make_rsrc(a.x, x_bytes);
    const auto rpd = make_rsrc(a.proj_down, pd_bytes);
    const auto rsm = make_rsrc(a.smooth, (uint32_t)K * 2);
    // copies: x blocks 4 mw + u (u < 4), proj_down blocks 8 mw + u (u < 8), and wave 4
    // the smooth block; lane l fills slot l of a block (row l / 8, slot l % 8)
    const int rr = lane >> 3, sl = lane & 7;
    uint32_t xo[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int bi = 4 * mw + u, i = bi >> 2, q = bi & 3;
      const int r = 8 * q + rr;
      const int m = m0 + r;
      xo[u] = m < M ? ((uint32_t)m * K + 64 * i + 8 * (sl ^ rs_xswz(r))) * 2 : x_bytes;
    }
    auto issue = [&](int sp) {
      uint8_t* st = stage_at(sp);
      const int kb = 256 * sp;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int bi = 4 * mw + u, i = bi >> 2, q = bi & 3;
        const int pc = sl ^ rs_xswz(8 * q + rr);
        const bool in = xo[u] < x_bytes && kb + 64 * i + 8 * pc < K;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, RS_LDS(void, st + bi * 1024), 16, in ? xo[u] + kb * 2 : x_bytes,
                                                 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int beta = 8 * mw + u;
        const int k = 8 * beta + rr;
        const int pp = sl ^ rs_pswz(k);
        const int kg = kb + k, col = r0 + 8 * pp;
        const uint32_t off = kg < K && col < R ? ((uint32_t)kg * R + col) * 2 : pd_bytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rpd, RS_LDS(void, st + kRsX + beta * 1024), 16, off, 0, 0, 0);
      }
      if (mw == 0) {
        const int k = kb + 8 * lane;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsm, RS_LDS(void, st + kRsX + kRsPd), 16,
                                                 lane < 32 && k < K ? k * 2 : K * 2, 0, 0, 0);
      }
    };

    f32x4 acc[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[t][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // fragments of k-step 2 mw (k-step 2 mw + 1: x pieces 4 further, i.e. slot ^ 4, and
    // proj_down rows 32 further, 4096 bytes): x rows 16 t + l16 (8 k per lane); transposed
    // proj_down reads of column tile c (lane (G, jj, qq): row 8 G + jj, columns 16 c + 4 qq,
    // the rows 4 further 512 bytes on)
    const int G = lane >> 4, jj = (lane >> 2) & 3, qq = lane & 3, l16 = lane & 15;
    uint32_t xa[2], pa[4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r = 16 * t + l16;
      xa[t] = (mw * 4 + (r >> 3)) * 1024 + (r & 7) * 128 + ((G ^ rs_xswz(r)) << 4);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int k = 64 * mw + 8 * G + jj;
      const int pp = 2 * c + (qq >> 1);
      pa[c] = kRsX + (k >> 3) * 1024 + (k & 7) * 128 + ((pp ^ rs_pswz(k)) << 4) + (qq & 1) * 8;
    }
    const uint32_t smem_base = (uint32_t)(uintptr_t)RS_LDS(uint8_t, smem);
    auto multiply = [&](int stg) {
      const uint32_t so = smem_base + stg * kRsStage;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 xf[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
          xf[t] = *reinterpret_cast<const bf16x8*>(smem + stg * kRsStage + (xa[t] ^ (s << 6)));
        typedef int v2i __attribute__((ext_vector_type(2)));
        v2i lo0, hi0, lo1, hi1, lo2, hi2, lo3, hi3;
        const uint32_t b0 = so + pa[0] + s * 4096, b1 = so + pa[1] + s * 4096;
        const uint32_t b2 = so + pa[2] + s * 4096, b3 = so + pa[3] + s * 4096;
        // The eight transposing reads of this k-step, complete when the block ends. As
        // inline assembly: the builtin carries no alias information, so the compiler
        // would wait for every direct-to-LDS copy in flight before it.
        asm volatile(
            "ds_read_b64_tr_b16 %0, %8\n\t"
            "ds_read_b64_tr_b16 %1, %8 offset:512\n\t"
            "ds_read_b64_tr_b16 %2, %9\n\t"
            "ds_read_b64_tr_b16 %3, %9 offset:512\n\t"
            "ds_read_b64_tr_b16 %4, %10\n\t"
            "ds_read_b64_tr_b16 %5, %10 offset:512\n\t"
            "ds_read_b64_tr_b16 %6, %11\n\t"
            "ds_read_b64_tr_b16 %7, %11 offset:512\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=v"(lo0), "=v"(hi0), "=v"(lo1), "=v"(hi1), "=v"(lo2), "=v"(hi2), "=v"(lo3), "=v"(hi3)
            : "v"(b0), "v"(b1), "v"(b2), "v"(b3)
            : "memory");
        bf16x8 pf[4];
        pf[0] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo0, hi0, 0, 1, 2, 3));
        pf[1] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo1, hi1, 0, 1, 2, 3));
        pf[2] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo2, hi2, 0, 1, 2, 3));
        pf[3] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo3, hi3, 0, 1, 2, 3));
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            acc[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[c], xf[t], acc[t][c], 0, 0, 0);
      }
    };

    issue(0);
    if (nsp > 1) issue(1);
    for (int sp = 0; sp < nsp; ++sp) {
      // this wave's copies of super-panel sp have landed (those of sp + 1 may not)
      if (sp + 1 < nsp) {
        if (mw == 0) rs_wait_vm<13>();
        else rs_wait_vm<12>();
      } else {
        rs_wait_vm<0>();
      }
      rs_wait_lgkm0();
      rs_barrier();   // sp visible to every wave; sp - 1's stage is free
      if (sp + 2 < nsp) issue(sp + 2);
      multiply(sp % kRsStages);
    }
    rs_wait_lgkm0();
    rs_barrier();
    // this wave's partial sums through LDS: row r, 16-byte column slot c4 at c4 ^ (r % 16)
    float* e = reinterpret_cast<float*>(smem + mw * 8192);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int r = 16 * t + l16;
        const int c4 = 4 * c + G;
        *reinterpret_cast<f32x4*>(e + r * 64 + ((c4 ^ (r & 15)) << 2)) = acc[t][c];
      }
  } else {
    const int qw = wave;
    const int r = 8 * qw + (lane >> 3);
    const int pc = lane & 7;
    const int m = m0 + r;
    const auto rq = make_rsrc(a.qact, q_bytes);
    const auto rsc = make_rsrc(a.ascales, s_bytes);
    BlockScale<STATIC> bs;
    bs.init(a.gscale);
    auto quantise = [&](const uint8_t* st, int sp, int i) {
      const int p = 4 * sp + i;
      const int k = 64 * p + 8 * pc;
      const u32x4 xv =
          *reinterpret_cast<const u32x4*>(st + (4 * i + qw) * 1024 + (lane >> 3) * 128 + ((pc ^ rs_xswz(r)) << 4));
      const u32x4 sv = *reinterpret_cast<const u32x4*>(st + kRsX + kRsPd + (64 * i + 8 * pc) * 2);
      float v[8];
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = bf16lo_to_f32(xv[e]) * bf16lo_to_f32(sv[e]);
        v[2 * e + 1] = bf16hi_to_f32(xv[e]) * bf16hi_to_f32(sv[e]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
      // the other half of the block sits in lane ^ 1
      amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(amax), 0xB1, 0xF, 0xF, false)));
      const uint32_t sc = bs.code(amax);
      const float sd = bs.divisor(sc);
      const float inv = sd > 0.0f ? scale_reciprocal(sd) : 0.0f;
      uint32_t pk = 0u;
      pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, snap21(v[0] * inv), snap21(v[1] * inv), 1.0f, 0);
      pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, snap21(v[2] * inv), snap21(v[3] * inv), 1.0f, 1);
      pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, snap21(v[4] * inv), snap21(v[5] * inv), 1.0f, 2);
      pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, snap21(v[6] * inv), snap21(v[7] * inv), 1.0f, 3);
      const int t4 = pc >> 1, hh = pc & 1;
      if (PACKED) {
        // rows of the last 32-row panel beyond M are written (as zeros)
        const uint32_t chunk = (uint32_t)p * MP + b;
        __builtin_amdgcn_raw_buffer_store_b32(pk, rq, chunk * 1024 + ((hh * 32 + r) * 4 + t4) * 4, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sc, rq, hh == 0 ? code_bytes + chunk * 128 + r * 4 + t4 : q_bytes,
                                             0, 0);
      } else {
        const bool ok = m < M && k < K;
        __builtin_amdgcn_raw_buffer_store_b32(pk, rq, ok ? (uint32_t)m * (K / 2) + k / 2 : q_bytes, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sc, rsc, ok && hh == 0 ? (uint32_t)(k >> 4) * M + m : s_bytes, 0,
                                             0);
      }
    };
    for (int sp = 0; sp < nsp; ++sp) {
      rs_wait_lgkm0();
      rs_barrier();
      const uint8_t* st = stage_at(sp);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * sp + i < KP && (i & 1) == h) quantise(st, sp, i);
    }
    rs_wait_lgkm0();
    rs_barrier();
  }
  rs_wait_lgkm0();
  rs_barrier();
  // lora_act: thread row tid / 16, columns 4 (tid % 16) .. + 3, the four k classes added in order
  {
    const int rrow = tid >> 4, c4 = tid & 15;
    const float* e = reinterpret_cast<const float*>(smem);
    const int off = rrow * 64 + ((c4 ^ (rrow & 15)) << 2);
    f32x4 sum = *reinterpret_cast<const f32x4*>(e + off);
    sum += *reinterpret_cast<const f32x4*>(e + 2048 + off);
    sum += *reinterpret_cast<const f32x4*>(e + 4096 + off);
    sum += *reinterpret_cast<const f32x4*>(e + 6144 + off);
    const int m = m0 + rrow, col = r0 + 4 * c4;
    if (m < M && col < R) {
      const u32x2 o = u32x2{pack_bf16x2(sum[0], sum[1]), pack_bf16x2(sum[2], sum[3])};
      *reinterpret_cast<u32x2*>(a.lora_act + (size_t)m * R + col) = o;
    }
  }
}

// Which fused form: estimated microseconds, fitted to both kernels over M = 512 ..
// 16896, K = 1280 .. 10240 at R = 128 on MI355X. The split-free form costs about
// 1.5 + 0.0047 K per round of 256 workgroups (two per 32 rows), bound by its
// proj_down traffic from L2; the split form its fitted split model plus ~5 for the
// partial sums' reduction launch. The split-free form is taken only when it is
// estimated at least 1 faster (at M = 4096, K = 3840 the two are within a
// microsecond either way and the split form stays).
bool use_split_free(int64_t M, int64_t K, int64_t R, bool packed_out) {
  if (R <= kRsCols || R > 2 * kRsCols) return false;
  const int64_t wgs = 2 * ((M + 31) / 32);
  const double rs = 1.5 + (double)((wgs + 255) / 256) * 0.0047 * (double)K;
  const int ks = k_splits(M, K, R, packed_out);
  const int64_t row_blocks = (M + kRows - 1) / kRows;
  const int64_t steps = packed_out ? 2 * ((K + 63) / 64) : (K + 31) / 32;
  const int64_t rounds = (row_blocks * ks + 255) / 256;
  const double split = (double)rounds * (double)((steps + ks - 1) / ks) * 0.65 +
                       (ks > 1 ? (double)ks * (double)M * (double)R * 1.26e-6 : 0.0) + 5.0;
  return rs + 1.0 < split;
}

}  // namespace

size_t quant_lora_workspace_bytes(int64_t M, int64_t K, int64_t R) {
  if (R <= 0) return 0;
  // the larger of the two layouts' split counts, so one size serves both
  const int ks = std::max(k_splits(M, K, R, true), k_splits(M, K, R, false));
  return ks > 1 ? (size_t)ks * (size_t)M * (size_t)R * 4 : 0;
}

hipError_t launch_quant_lora(const uint16_t* x, const uint16_t* smooth, const uint16_t* proj_down,
                             uint8_t* qact, uint8_t* ascales, uint16_t* lora_act, float* partial,
                             int64_t M, int64_t K, int64_t R, bool packed_out, hipStream_t stream,
                             const uint16_t* gscale) {
  QLArgs a{x, smooth, proj_down, qact, ascales, lora_act, nullptr, (int)M, (int)K, (int)R, 0, 0, gscale};
  const bool st = gscale != nullptr;
  if (use_split_free(M, K, R, packed_out)) {
    const void* fn = packed_out ? (st ? reinterpret_cast<const void*>(&quant_lora_rs_kernel<true, true>)
                                      : reinterpret_cast<const void*>(&quant_lora_rs_kernel<true, false>))
                                : (st ? reinterpret_cast<const void*>(&quant_lora_rs_kernel<false, true>)
                                      : reinterpret_cast<const void*>(&quant_lora_rs_kernel<false, false>));
    static std::atomic<uint64_t> lds_set[4];
    hipError_t e = set_lds_limit_once(fn, kRsLds, lds_set[(packed_out ? 2 : 0) + (st ? 1 : 0)]);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)(((M + 31) / 32 + 7) / 8 * 16));
    if (packed_out) {
      if (st) hipLaunchKernelGGL((quant_lora_rs_kernel<true, true>), grid, dim3(512), kRsLds, stream, a);
      else hipLaunchKernelGGL((quant_lora_rs_kernel<true, false>), grid, dim3(512), kRsLds, stream, a);
    } else {
      if (st) hipLaunchKernelGGL((quant_lora_rs_kernel<false, true>), grid, dim3(512), kRsLds, stream, a);
      else hipLaunchKernelGGL((quant_lora_rs_kernel<false, false>), grid, dim3(512), kRsLds, stream, a);
    }
    return hipGetLastError();
  }
  const int ks = k_splits(M, K, R, packed_out);
  const int steps = packed_out ? (int)(2 * ((K + 63) / 64)) : (int)((K + 31) / 32);
  a.split_steps = (steps + ks - 1) / ks;
  a.partial = (R > 0 && ks > 1) ? partial : nullptr;
  dim3 grid((unsigned)((M + kRows - 1) / kRows), (unsigned)ks);
  auto launch = [&](bool quant, bool lora) {
    if (quant && lora) {
      // the wave-specialised kernel walks 64-wide panels; same splits and partial planes
      QLArgs w = a;
      const int64_t KP = (K + 63) / 64;
      w.split_steps = (int)((KP + ks - 1) / ks);
      const dim3 wgrid((unsigned)((M + kWsRows - 1) / kWsRows), (unsigned)ks);
      if (packed_out) {
        if (st) hipLaunchKernelGGL((quant_lora_ws_kernel<true, true>), wgrid, dim3(512), 0, stream, w);
        else hipLaunchKernelGGL((quant_lora_ws_kernel<true>), wgrid, dim3(512), 0, stream, w);
      } else {
        if (st) hipLaunchKernelGGL((quant_lora_ws_kernel<false, true>), wgrid, dim3(512), 0, stream, w);
        else hipLaunchKernelGGL((quant_lora_ws_kernel<false>), wgrid, dim3(512), 0, stream, w);
      }
      return;
    }
    if (quant && st) {
      // quantisation alone with a static scale (R = 0; the canonical layout without a
      // down-projection goes to quant_act_kernel instead)
      if (packed_out)
        hipLaunchKernelGGL((quant_lora_kernel<kRowTiles, true, true, false, true>), grid, dim3(64 * kWaves), 0,
                           stream, a);
      else
        hipLaunchKernelGGL((quant_lora_kernel<kRowTiles, false, true, false, true>), grid, dim3(64 * kWaves), 0,
                           stream, a);
      return;
    }
#define SVDQ_QL(RT, P, Q, L) hipLaunchKernelGGL((quant_lora_kernel<RT, P, Q, L>), grid, dim3(64 * kWaves), 0, stream, a)
#define SVDQ_QL_RT(RT)                                                                 \
    if (packed_out) {                                                                  \
      if (quant) SVDQ_QL(RT, true, true, false);                                       \
      else SVDQ_QL(RT, true, false, true);                                             \
    } else {                                                                           \
      if (quant) SVDQ_QL(RT, false, true, false);                                      \
      else SVDQ_QL(RT, false, false, true);                                            \
    }
    SVDQ_QL_RT(kRowTiles)
#undef SVDQ_QL_RT
#undef SVDQ_QL
  };
  launch(true, R > 0);
  for (int64_t r0 = kRChunk; r0 < R; r0 += kRChunk) {
    a.r_base = (int)r0;
    launch(false, true);
  }
  if (R > 0 && ks > 1) {
    const int64_t groups = M * (R / 8);
    hipLaunchKernelGGL(lora_reduce_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const float*>(partial), lora_act, (int)M, (int)R, ks);
  }
  return hipGetLastError();
}

hipError_t launch_quant_lora_mx(const uint16_t* x, const uint16_t* smooth, const uint16_t* proj_down, uint8_t* codes,
                                uint8_t* scales, uint16_t* lora_act, float* partial, int64_t M, int64_t K, int64_t R,
                                hipStream_t stream) {
  if (R <= 0) return launch_quant_act_mx(x, smooth, codes, scales, M, K, stream);
  QLArgs a{x, smooth, proj_down, codes, scales, lora_act, nullptr, (int)M, (int)K, (int)R, 0, 0, nullptr};
  // the canonical layout's split count, so that lora_act has the bits of the
  // canonical quantisation's down-projection by the same kernel
  const int ks = k_splits(M, K, R, false);
  a.partial = ks > 1 ? partial : nullptr;
  QLArgs w = a;
  w.split_steps = (int)((K / 64 + ks - 1) / ks);
  hipLaunchKernelGGL((quant_lora_ws_kernel<false, false, true>),
                     dim3((unsigned)((M + kWsRows - 1) / kWsRows), (unsigned)ks), dim3(512), 0, stream, w);
  a.split_steps = (int)((K / 32 + ks - 1) / ks);
  const dim3 grid((unsigned)((M + kRows - 1) / kRows), (unsigned)ks);
  for (int64_t r0 = kRChunk; r0 < R; r0 += kRChunk) {   // lora_act columns past the first 128
    a.r_base = (int)r0;
    hipLaunchKernelGGL((quant_lora_kernel<kRowTiles, false, false, true>), grid, dim3(64 * kWaves), 0, stream, a);
  }
  if (ks > 1) {
    const int64_t groups = M * (R / 8);
    hipLaunchKernelGGL(lora_reduce_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const float*>(partial), lora_act, (int)M, (int)R, ks);
  }
  return hipGetLastError();
}

hipError_t launch_lowrank_down(const uint16_t* x, const uint16_t* proj_down, uint16_t* lora_act, float* partial,
                               int64_t M, int64_t K, int64_t R, hipStream_t stream) {
  if (R <= 0) return hipSuccess;
  QLArgs a{x, nullptr, proj_down, nullptr, nullptr, lora_act, nullptr, (int)M, (int)K, (int)R, 0, 0, nullptr};
  const int ks = k_splits(M, K, R, false);
  const int steps = (int)((K + 31) / 32);
  a.split_steps = (steps + ks - 1) / ks;
  a.partial = ks > 1 ? partial : nullptr;
  dim3 grid((unsigned)((M + kRows - 1) / kRows), (unsigned)ks);
  for (int64_t r0 = 0; r0 < R; r0 += kRChunk) {
    a.r_base = (int)r0;
    hipLaunchKernelGGL((quant_lora_kernel<kRowTiles, false, false, true>), grid, dim3(64 * kWaves), 0, stream, a);
  }
  if (ks > 1) {
    const int64_t groups = M * (R / 8);
    hipLaunchKernelGGL(lora_reduce_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const float*>(partial), lora_act, (int)M, (int)R, ks);
  }
  return hipGetLastError();
}

}  // namespace svdq
