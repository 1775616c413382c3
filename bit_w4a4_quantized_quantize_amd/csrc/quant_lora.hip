// Fused activation quantisation and low-rank down-projection: one pass over x
// produces quant(x * smooth) (codes + e4m3 block scales) and
// lora_act = bf16(x @ proj_down) (model card "nunchaku-z-image-turbo-svdq",
// section "What's stored on disk": the activation operand of scaled_mma and
// the (x @ proj_down) factor of the SVD residual; raw x feeds the residual).
//
// A workgroup owns 16*RT rows and the whole K range, so the down-projection
// needs no cross-workgroup reduction: its waves take interleaved 32-wide K
// steps (loading the operands two steps ahead while working on the current one,
// three register sets rotated by name)
// and their partial sums are added in a fixed order through LDS at the end
// (deterministic). Each lane holds 8 consecutive k of one row (a 16-byte
// load), which is at once the A fragment of v_mfma_f32_16x16x32_bf16 and half
// of an NVFP4 block; the other half sits in lane ^ 16.
//
// proj_down [K, R] is R-contiguous; each lane loads an 8 (k) x 8 (r) block
// with 16-byte loads and transposes it with byte permutes into 8 B fragments
// whose column sets are {8c + i}; the output lane layout then gives each lane
// 8 consecutive r of one row (a 16-byte bf16 store).
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
#include "common.h"
#include "kernels.h"

namespace svdq {

namespace {

constexpr int kRChunk = 128;

__device__ __forceinline__ uint32_t perm_lo(uint32_t lo_src, uint32_t hi_src) {
  return __builtin_amdgcn_perm(hi_src, lo_src, 0x05040100u);
}
__device__ __forceinline__ uint32_t perm_hi(uint32_t lo_src, uint32_t hi_src) {
  return __builtin_amdgcn_perm(hi_src, lo_src, 0x07060302u);
}

template <int RT>
struct StepRegs {
  u32x4 x[RT];   // 8 consecutive k of this lane's row(s)
  u32x4 sm;      // smooth at the same 8 k
  u32x4 p[8];    // proj_down rows kg .. kg+7, columns rcol .. rcol+7
};

struct QLArgs {
  const uint16_t* x;
  const uint16_t* smooth;
  const uint16_t* proj_down;
  uint8_t* qact;       // canonical [M, K/2] or the packed buffer
  uint8_t* ascales;    // canonical [K/16, M] (unused when packed)
  uint16_t* lora_act;  // [M, R]
  int M, K, R;
  int r_base;          // first of the (up to kRChunk) lora_act columns this launch computes
};

// QUANT: write the codes and scales; LORA: compute lora_act columns
// r_base .. r_base + kRChunk - 1. A rank above kRChunk takes further launches
// with QUANT = false.
template <int RT, int kWaves, bool PACKED, bool QUANT, bool LORA>
__global__ __launch_bounds__(64 * kWaves) void quant_lora_kernel(QLArgs a) {
  constexpr int ROWS = 16 * RT;
  __shared__ f32x4 s_red[kWaves / 2][RT][8][64];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 15;   // row within a 16-row tile; column group of proj_down
  const int g = lane >> 4;   // k group of 8 within a 32-wide step
  const int m0 = blockIdx.x * ROWS;
  const int M = a.M, K = a.K, R = a.R;
  const int MP = (M + 31) / 32;
  const int KP = (K + 63) / 64;
  // packed output covers whole 64-wide panels: positions beyond K get zero codes
  // and zero scales (the GEMM multiplies them by the weight's zero padding); its
  // rows beyond M inside the last 32-row panel are written as zeros too
  const int steps = PACKED ? 2 * KP : (K + 31) / 32;
  const uint32_t code_bytes = (uint32_t)MP * KP * 1024;

  const uint32_t x_bytes = (uint32_t)M * K * 2;
  const uint32_t pd_bytes = (uint32_t)K * R * 2;
  const uint32_t q_bytes = PACKED ? code_bytes + (uint32_t)MP * KP * 128 : (uint32_t)M * (K / 2);
  const uint32_t s_bytes = PACKED ? 0u : (uint32_t)(K / 16) * M;
  const uint32_t l_bytes = (uint32_t)M * R * 2;
  const auto rx = make_rsrc(a.x, x_bytes);
  const auto rsm = make_rsrc(a.smooth, (uint32_t)K * 2);
  const auto rpd = make_rsrc(a.proj_down, pd_bytes);
  const auto rq = make_rsrc(a.qact, q_bytes);
  const auto rsc = make_rsrc(a.ascales, s_bytes);
  const auto rl = make_rsrc(a.lora_act, l_bytes);

  {
    const int rcol = a.r_base + 8 * c;
    const bool r_in = rcol < R;

    f32x4 acc[RT][8];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[t][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // operands of one 32-wide step; positions outside the tensors read as zero
    auto load = [&](StepRegs<RT>& r, int st) {
      const int kg = st * 32 + 8 * g;
      const bool k_in = st < steps && kg < K;
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int m = m0 + 16 * t + c;
        const uint32_t off = k_in ? ((uint32_t)m * K + kg) * 2 : x_bytes;
        r.x[t] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
      }
      if (QUANT) r.sm = __builtin_amdgcn_raw_buffer_load_b128(rsm, k_in ? kg * 2 : K * 2, 0, 0);
      if (LORA) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t off = (r_in && k_in) ? ((uint32_t)(kg + j) * R + rcol) * 2 : pd_bytes;
          r.p[j] = __builtin_amdgcn_raw_buffer_load_b128(rpd, off, 0, 0);
        }
      }
    };

    // one 32-wide step on the operands in `cur`
    auto process = [&](const StepRegs<RT>& cur, int st) {
      const int kg = st * 32 + 8 * g;
      const bool k_in = kg < K;

      if (QUANT) {
        float sm[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sm[2 * j] = bf16lo_to_f32(cur.sm[j]);
          sm[2 * j + 1] = bf16hi_to_f32(cur.sm[j]);
        }
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const int m = m0 + 16 * t + c;
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
          const uint32_t sc = block_scale_code(amax);
          const float sd = e4m3_to_f32(sc, 0);
          const float inv = sd > 0.0f ? scale_reciprocal(sd) : 0.0f;
          uint32_t packed = 0u;
          packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, snap21(v[0] * inv), snap21(v[1] * inv), 1.0f, 0);
          packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, snap21(v[2] * inv), snap21(v[3] * inv), 1.0f, 1);
          packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, snap21(v[4] * inv), snap21(v[5] * inv), 1.0f, 2);
          packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, snap21(v[6] * inv), snap21(v[7] * inv), 1.0f, 3);
          if (PACKED) {
            const int pp = kg >> 6, tt = (kg >> 4) & 3, hh = (kg >> 3) & 1;
            const int q = m >> 5, cc = m & 31;
            const uint32_t chunk = (uint32_t)pp * MP + q;
            __builtin_amdgcn_raw_buffer_store_b32(packed, rq, chunk * 1024 + ((hh * 32 + cc) * 4 + tt) * 4, 0, 0);
            if (hh == 0)
              __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sc, rq, code_bytes + chunk * 128 + cc * 4 + tt, 0, 0);
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
          u32x4 f;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            f[q] = (i & 1) ? perm_hi(cur.p[2 * q][i >> 1], cur.p[2 * q + 1][i >> 1])
                           : perm_lo(cur.p[2 * q][i >> 1], cur.p[2 * q + 1][i >> 1]);
          const bf16x8 b = __builtin_bit_cast(bf16x8, f);
#pragma unroll
          for (int t = 0; t < RT; ++t)
            acc[t][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.x[t]), b,
                                                                acc[t][i], 0, 0, 0);
        }
      }
    };

    // two steps of lookahead: three register sets used in rotation by name
    // (the loop is unrolled by three), so a load's destination is never
    // copied while it is in flight
    StepRegs<RT> r0, r1, r2;
    load(r0, wave);
    load(r1, wave + kWaves);
    for (int st = wave; st < steps; st += 3 * kWaves) {
      load(r2, st + 2 * kWaves);
      process(r0, st);
      if (st + kWaves >= steps) break;
      load(r0, st + 3 * kWaves);
      process(r1, st + kWaves);
      if (st + 2 * kWaves >= steps) break;
      load(r1, st + 4 * kWaves);
      process(r2, st + 2 * kWaves);
    }

    if (LORA) {
      // fixed-order tree over the waves (8: 4..7 -> 0..3, 2,3 -> 0,1, 1 -> 0)
#pragma unroll
      for (int half = kWaves / 2; half >= 1; half >>= 1) {
        __syncthreads();
        if (wave >= half && wave < 2 * half) {
#pragma unroll
          for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int i = 0; i < 8; ++i) s_red[wave - half][t][i][lane] = acc[t][i];
        }
        __syncthreads();
        if (wave < half) {
#pragma unroll
          for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[t][i] += s_red[wave][t][i][lane];
        }
      }
      if (wave == 0) {
        // lane holds rows 16t + 4g + q and columns rcol .. rcol+7
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int m = m0 + 16 * t + 4 * g + q;
            u32x4 o;
#pragma unroll
            for (int w = 0; w < 4; ++w) o[w] = pack_bf16x2(acc[t][2 * w][q], acc[t][2 * w + 1][q]);
            __builtin_amdgcn_raw_buffer_store_b128(o, rl, r_in ? ((uint32_t)m * R + rcol) * 2 : l_bytes, 0, 0);
          }
      }
    }
  }
}

}  // namespace

int quant_lora_row_tiles(int64_t M) { return (M + 31) / 32 >= 256 ? 2 : 1; }

hipError_t launch_quant_lora(const uint16_t* x, const uint16_t* smooth, const uint16_t* proj_down,
                             uint8_t* qact, uint8_t* ascales, uint16_t* lora_act, int64_t M,
                             int64_t K, int64_t R, bool packed_out, hipStream_t stream) {
  QLArgs a{x, smooth, proj_down, qact, ascales, lora_act, (int)M, (int)K, (int)R, 0};
  const int rt = quant_lora_row_tiles(M);
  dim3 grid((unsigned)((M + 16 * rt - 1) / (16 * rt)));
  // 16 rows: 8 waves per workgroup (2 per SIMD); 32 rows: 4 waves, so each wave
  // may hold two row tiles of operands and accumulators in registers
  auto launch = [&](bool quant, bool lora) {
#define SVDQ_QL(RT, W, P, Q, L) hipLaunchKernelGGL((quant_lora_kernel<RT, W, P, Q, L>), grid, dim3(64 * W), 0, stream, a)
#define SVDQ_QL_RT(RT, W)                                                              \
    if (packed_out) {                                                                  \
      if (quant && lora) SVDQ_QL(RT, W, true, true, true);                             \
      else if (quant) SVDQ_QL(RT, W, true, true, false);                               \
      else SVDQ_QL(RT, W, true, false, true);                                          \
    } else {                                                                           \
      if (quant && lora) SVDQ_QL(RT, W, false, true, true);                            \
      else if (quant) SVDQ_QL(RT, W, false, true, false);                              \
      else SVDQ_QL(RT, W, false, false, true);                                         \
    }
    if (rt == 2) { SVDQ_QL_RT(2, 4) } else { SVDQ_QL_RT(1, 8) }
#undef SVDQ_QL_RT
#undef SVDQ_QL
  };
  launch(true, R > 0);
  for (int64_t r0 = kRChunk; r0 < R; r0 += kRChunk) {
    a.r_base = (int)r0;
    launch(false, true);
  }
  return hipGetLastError();
}

}  // namespace svdq
