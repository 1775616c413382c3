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
  float* partial;      // [splits, M, R] fp32 partial sums when K is split (else NULL)
  int split_steps;     // 32-wide K steps per split (blockIdx.y selects the split)
};

// QUANT: write the codes and scales; LORA: compute lora_act columns
// r_base .. r_base + kRChunk - 1. A rank above kRChunk takes further launches
// with QUANT = false.
template <int RT, int kWaves, int DEPTH, bool PACKED, bool QUANT, bool LORA>
__global__ __launch_bounds__(64 * kWaves) void quant_lora_kernel(QLArgs a) {
  constexpr int ROWS = 16 * RT;
  __shared__ f32x4 s_red[kWaves / 2][RT][8][64];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 15;   // row within a 16-row tile; column group of proj_down
  const int g = lane >> 4;   // k group of 8 within a 32-wide step
  const int m0 = blockIdx.x * ROWS;
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
      const bool k_in = st < s_end && kg < K;
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

    // DEPTH steps of lookahead: DEPTH + 1 register sets used in rotation by
    // name (the loop is unrolled by DEPTH + 1), so a load's destination is
    // never copied while it is in flight
    if constexpr (DEPTH == 2) {
      StepRegs<RT> r0, r1, r2;
      load(r0, s_begin + wave);
      load(r1, s_begin + wave + kWaves);
      for (int st = s_begin + wave; st < s_end; st += 3 * kWaves) {
        load(r2, st + 2 * kWaves);
        process(r0, st);
        if (st + kWaves >= s_end) break;
        load(r0, st + 3 * kWaves);
        process(r1, st + kWaves);
        if (st + 2 * kWaves >= s_end) break;
        load(r1, st + 4 * kWaves);
        process(r2, st + 2 * kWaves);
      }
    } else {
      StepRegs<RT> r0, r1;
      load(r0, s_begin + wave);
      for (int st = s_begin + wave; st < s_end; st += 2 * kWaves) {
        load(r1, st + kWaves);
        process(r0, st);
        if (st + kWaves >= s_end) break;
        load(r0, st + 2 * kWaves);
        process(r1, st + kWaves);
      }
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
        const uint32_t p_bytes = a.partial != nullptr ? (uint32_t)gridDim.y * M * R * 4 : 0u;
        const auto rp = make_rsrc(a.partial, p_bytes);
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int m = m0 + 16 * t + 4 * g + q;
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
              const uint32_t off = ok ? (((uint32_t)ks * M + m) * R + rcol) * 4 : p_bytes;
              __builtin_amdgcn_raw_buffer_store_b128(o0, rp, off, 0, 0);
              __builtin_amdgcn_raw_buffer_store_b128(o1, rp, ok ? off + 16 : p_bytes, 0, 0);
            }
          }
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

}  // namespace

// The down-projection path: a workgroup of 8 waves owns 32 rows (2 row tiles
// per wave, accumulators for all 128 columns of an R chunk, one step of
// lookahead), so each proj_down element read through a CU's L1 serves 32 rows
// and each in-register transpose of it serves two row tiles. When that leaves
// fewer than 256 workgroups, K is split across workgroups (blockIdx.y) and the
// fp32 partials are reduced by a second kernel. (Measured on MI355X against 16
// rows per workgroup and against 64 rows with 4 waves, which runs out of
// registers: 20.1 us vs 22.2 and 27.5 at M=4096, K=3840, R=128.)
constexpr int kLoraRT = 2;
constexpr int kLoraWaves = 8;
constexpr int kLoraDepth = 1;

int quant_lora_splits(int64_t M, int64_t K, int64_t R) {
  if (R <= 0) return 1;
  const int64_t row_blocks = (M + 16 * kLoraRT - 1) / (16 * kLoraRT);
  const int64_t steps = 2 * ((K + 63) / 64);
  int64_t ks = (256 + row_blocks - 1) / row_blocks;
  ks = ks < 1 ? 1 : ks;
  ks = ks > 16 ? 16 : ks;
  while (ks > 1 && steps / ks < 2 * kLoraWaves) --ks;               // at least 2 steps per wave
  while (ks > 1 && ks * M * R * 4 >= (int64_t(1) << 31)) --ks;      // 32-bit partial offsets
  return (int)ks;
}

size_t quant_lora_workspace_bytes(int64_t M, int64_t K, int64_t R) {
  const int ks = quant_lora_splits(M, K, R);
  return ks > 1 ? (size_t)ks * (size_t)M * (size_t)R * 4 : 0;
}

hipError_t launch_quant_lora(const uint16_t* x, const uint16_t* smooth, const uint16_t* proj_down,
                             uint8_t* qact, uint8_t* ascales, uint16_t* lora_act, float* partial,
                             int64_t M, int64_t K, int64_t R, bool packed_out, hipStream_t stream) {
  QLArgs a{x, smooth, proj_down, qact, ascales, lora_act, (int)M, (int)K, (int)R, 0, nullptr, 0};
  const int steps_all = packed_out ? (int)(2 * ((K + 63) / 64)) : (int)((K + 31) / 32);
  if (R == 0) {
    // quantisation only: 16 rows and the whole K per workgroup of 8 waves
    a.split_steps = steps_all;
    dim3 grid((unsigned)((M + 15) / 16));
    if (packed_out) hipLaunchKernelGGL((quant_lora_kernel<1, 8, 2, true, true, false>), grid, dim3(512), 0, stream, a);
    else hipLaunchKernelGGL((quant_lora_kernel<1, 8, 2, false, true, false>), grid, dim3(512), 0, stream, a);
    return hipGetLastError();
  }
  const int ks = quant_lora_splits(M, K, R);
  a.split_steps = (steps_all + ks - 1) / ks;
  a.partial = ks > 1 ? partial : nullptr;
  dim3 grid((unsigned)((M + 16 * kLoraRT - 1) / (16 * kLoraRT)), (unsigned)ks);
  auto launch = [&](bool quant) {
#define SVDQ_QL(P, Q) hipLaunchKernelGGL((quant_lora_kernel<kLoraRT, kLoraWaves, kLoraDepth, P, Q, true>), grid, \
                                         dim3(64 * kLoraWaves), 0, stream, a)
    if (packed_out) {
      if (quant) SVDQ_QL(true, true); else SVDQ_QL(true, false);
    } else {
      if (quant) SVDQ_QL(false, true); else SVDQ_QL(false, false);
    }
#undef SVDQ_QL
  };
  launch(true);
  for (int64_t r0 = kRChunk; r0 < R; r0 += kRChunk) {
    a.r_base = (int)r0;
    launch(false);
  }
  if (ks > 1) {
    const int64_t groups = M * (R / 8);
    hipLaunchKernelGGL(lora_reduce_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const float*>(partial), lora_act, (int)M, (int)R, ks);
  }
  return hipGetLastError();
}

}  // namespace svdq
