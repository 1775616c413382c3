// Down-projection of the low-rank branch, lora_act = x @ proj_down
// (model card "nunchaku-z-image-turbo-svdq", section "What's stored on disk":
// the (x @ proj_down) factor of the SVD residual; proj_down is [K, R] bf16).
// The raw x is used (not x * smooth); the result is stored as bf16 after
// fp32 accumulation.
//
// Matrix cores: v_mfma_f32_16x16x32_bf16. A workgroup owns 32 rows (two
// 16-row tiles) and a range of K; its four waves take interleaved 32-wide K
// steps. proj_down is R-contiguous while the instruction wants 8 consecutive
// k per lane, so each lane loads an 8 (k) x 8 (r) bf16 block with 16-byte
// loads and transposes it in registers with byte permutes; the 8 columns it
// then holds feed 8 instructions whose column sets are {8c + i}. The output
// lane layout gives every lane 8 consecutive r of one row, stored as 16 bytes.
//
// When the grid is split along K (few rows), each workgroup writes an fp32
// partial tile; the last workgroup to arrive for a row tile (arrival counter,
// zeroed by the quantisation kernel launched before this one) sums the
// partials in split order, so the result does not depend on timing.
#include "common.h"
#include "kernels.h"

namespace svdq {

namespace {

constexpr int kRows = 32;
constexpr int kThreads = 256;
constexpr int kRChunk = 128;

__device__ __forceinline__ uint32_t perm_lo(uint32_t lo_src, uint32_t hi_src) {
  // low 16 bits of lo_src | low 16 bits of hi_src << 16
  return __builtin_amdgcn_perm(hi_src, lo_src, 0x05040100u);
}
__device__ __forceinline__ uint32_t perm_hi(uint32_t lo_src, uint32_t hi_src) {
  // high 16 bits of lo_src | high 16 bits of hi_src << 16
  return __builtin_amdgcn_perm(hi_src, lo_src, 0x07060302u);
}

__global__ __launch_bounds__(kThreads) void lora_down_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ proj_down,
    uint16_t* __restrict__ lora_act, float* __restrict__ partials,
    unsigned* __restrict__ counters, int M, int K, int R, int splits) {
  __shared__ float s_red[4][kRows][kRChunk + 4];
  __shared__ unsigned s_last;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;       // k group of 8 within a 32-wide step
  const int c = lane & 15;       // column group of 8
  const int m_base = blockIdx.x * kRows;
  const int split = blockIdx.y;

  const int steps = (K + 31) / 32;
  const int s_begin = (int)((int64_t)steps * split / splits);
  const int s_end = (int)((int64_t)steps * (split + 1) / splits);

  for (int r_base = 0; r_base < R; r_base += kRChunk) {
    f32x4 acc[2][8];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[t][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int rc = r_base + 8 * c;           // first of this lane's 8 columns
    const bool r_in = rc < R;                // R % 16 == 0: all 8 in or all out

    for (int st = s_begin + wave; st < s_end; st += 4) {
      const int kg = st * 32 + 8 * g;        // first of this lane's 8 k
      // A fragments: x rows, 8 consecutive k
      bf16x8 a[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int m = m_base + 16 * t + c;
        u32x4 w = zero4();
        if (m < M && kg < K) w = *reinterpret_cast<const u32x4*>(x + (size_t)m * K + kg);
        a[t] = __builtin_bit_cast(bf16x8, w);
      }
      // 8 x 8 block of proj_down: rows kg .. kg+7, columns rc .. rc+7
      u32x4 p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[j] = zero4();
        if (r_in && kg + j < K) p[j] = *reinterpret_cast<const u32x4*>(proj_down + (size_t)(kg + j) * R + rc);
      }
      // transpose: f[i] holds column rc + i for k = kg .. kg+7
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        u32x4 f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f[q] = (i & 1) ? perm_hi(p[2 * q][i >> 1], p[2 * q + 1][i >> 1])
                         : perm_lo(p[2 * q][i >> 1], p[2 * q + 1][i >> 1]);
        }
        const bf16x8 b = __builtin_bit_cast(bf16x8, f);
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[t][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[t], b, acc[t][i], 0, 0, 0);
      }
    }

    // lane holds rows 16t + 4g + q, columns rc + i (i = 0..7)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 8; ++i) s_red[wave][16 * t + 4 * g + q][8 * c + i] = acc[t][i][q];
    __syncthreads();

    // 32 rows x 16 column groups = 512 items, 2 per thread
    const int rchunk = min(kRChunk, R - r_base);
    float sum[2][8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int item = tid + u * kThreads;
      const int row = item >> 4, cg = item & 15;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        sum[u][i] = ((s_red[0][row][8 * cg + i] + s_red[1][row][8 * cg + i]) +
                     s_red[2][row][8 * cg + i]) + s_red[3][row][8 * cg + i];
    }

    if (splits == 1) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int item = tid + u * kThreads;
        const int row = item >> 4, cg = item & 15;
        const int m = m_base + row;
        if (m < M && 8 * cg < rchunk) {
          u32x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(sum[u][2 * q], sum[u][2 * q + 1]);
          *reinterpret_cast<u32x4*>(lora_act + (size_t)m * R + r_base + 8 * cg) = o;
        }
      }
    } else {
      // partials: [splits][M][R] fp32
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int item = tid + u * kThreads;
        const int row = item >> 4, cg = item & 15;
        const int m = m_base + row;
        if (m < M && 8 * cg < rchunk) {
          float* dst = partials + ((size_t)split * M + m) * R + r_base + 8 * cg;
          *reinterpret_cast<f32x4*>(dst) = f32x4{sum[u][0], sum[u][1], sum[u][2], sum[u][3]};
          *reinterpret_cast<f32x4*>(dst + 4) = f32x4{sum[u][4], sum[u][5], sum[u][6], sum[u][7]};
        }
      }
    }
    __syncthreads();   // s_red is reused by the next R chunk
  }

  if (splits > 1) {
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const unsigned prev = __hip_atomic_fetch_add(counters + blockIdx.x, 1u, __ATOMIC_ACQ_REL,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      s_last = (prev == (unsigned)(splits - 1)) ? 1u : 0u;
    }
    __syncthreads();
    if (s_last) {
      __threadfence();
      // sum the partial tiles in split order and write bf16
      for (int item = tid; item < kRows * (R / 8); item += kThreads) {
        const int row = item / (R / 8);
        const int cg = item % (R / 8);
        const int m = m_base + row;
        if (m >= M) continue;
        float s8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) s8[i] = 0.0f;
        for (int sp = 0; sp < splits; ++sp) {
          const float* src = partials + ((size_t)sp * M + m) * R + 8 * cg;
          const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
          const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
          s8[0] += lo[0]; s8[1] += lo[1]; s8[2] += lo[2]; s8[3] += lo[3];
          s8[4] += hi[0]; s8[5] += hi[1]; s8[6] += hi[2]; s8[7] += hi[3];
        }
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(s8[2 * q], s8[2 * q + 1]);
        *reinterpret_cast<u32x4*>(lora_act + (size_t)m * R + 8 * cg) = o;
      }
    }
  }
}

}  // namespace

int lora_down_counters(int64_t M) { return (int)((M + kRows - 1) / kRows); }

int lora_down_splits(int64_t M, int64_t K, int64_t R) {
  if (R <= 0) return 1;
  const int64_t tiles = (M + kRows - 1) / kRows;
  const int64_t steps = (K + 31) / 32;
  int64_t s = 512 / (tiles > 0 ? tiles : 1);       // aim for ~2 workgroups per CU
  if (s > 8) s = 8;
  if (s > steps / 4) s = steps / 4;                  // keep every wave busy
  if (s < 1) s = 1;
  return (int)s;
}

size_t lora_down_workspace_bytes(int64_t M, int64_t K, int64_t R) {
  const int s = lora_down_splits(M, K, R);
  if (s <= 1) return 0;
  return lora_down_counter_offset(M, K, R) + sizeof(unsigned) * (size_t)lora_down_counters(M);
}

size_t lora_down_counter_offset(int64_t M, int64_t K, int64_t R) {
  const int s = lora_down_splits(M, K, R);
  const size_t part = sizeof(float) * (size_t)s * (size_t)M * (size_t)R;
  return (part + 255) & ~(size_t)255;
}

hipError_t launch_lora_down(const uint16_t* x, const uint16_t* proj_down, uint16_t* lora_act,
                            void* workspace, int64_t M, int64_t K, int64_t R,
                            hipStream_t stream) {
  const int s = lora_down_splits(M, K, R);
  float* partials = nullptr;
  unsigned* counters = nullptr;
  if (s > 1) {
    partials = static_cast<float*>(workspace);
    counters = reinterpret_cast<unsigned*>(static_cast<char*>(workspace) +
                                           lora_down_counter_offset(M, K, R));
  }
  dim3 grid((unsigned)lora_down_counters(M), (unsigned)s);
  hipLaunchKernelGGL(lora_down_kernel, grid, dim3(kThreads), 0, stream, x, proj_down, lora_act,
                     partials, counters, (int)M, (int)K, (int)R, s);
  return hipGetLastError();
}

}  // namespace svdq
