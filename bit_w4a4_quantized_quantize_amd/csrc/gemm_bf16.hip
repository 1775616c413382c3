// Plain bf16 GEMM for the linears a mixed-precision NVFP4 model keeps in bf16
// (blog page "Z-Image NVFP4 ...", variant table: the "Ultra" variant keeps
// attention qkv/out and every linear of blocks 0-4 and 25-29 in bf16):
//
//   y = bf16( x @ W^T + bias ),  x [M, K], W [N, K], bias [N], y [M, N], bf16,
//
// fp32 accumulation on v_mfma_f32_32x32x16_bf16.
//
// The workgroup structure is the NVFP4 GEMM's (gemm_lds.hip) without the
// dequantisation: 8 waves (4 x 2, two per SIMD), a 256 x (32*TN*2) tile, one
// 64-K panel per LDS stage, two stages. A panel is 32-row x 64-K chunks of x
// and W; each chunk lands in LDS as four 1 KB operand blocks (one per 16-K
// step, lane l at l*16 holding row l%32, k 8*(l/32)..+7: the matrix
// instruction's operand order, so the fragment reads are bank-conflict free).
// The blocks are copied by direct global-to-LDS loads (16 bytes per lane, no
// registers, no LDS write instructions): panel p+1 is requested when panel p
// starts multiplying, and one vmcnt wait plus one barrier per panel publish it.
// Rows beyond M or N read the last row (their results are never stored); a
// K that is not a multiple of 64 has its last panel copied through registers
// with the positions past K set to zero.
//
// Tile order and output: as in gemm_lds.hip (XCD-contiguous tile ranges,
// kGroupM row blocks per column sweep; bias add, bf16 round to nearest even,
// staged through LDS and stored as whole 16-byte row pieces).
#include "common.h"
#include "kernels.h"

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

namespace svdq {

namespace {

constexpr int kGroupM = 4;

// vmcnt(n) wait, other counters untouched (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 = 7, lgkmcnt 11:8 = 15).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

__device__ __forceinline__ void wait_lds_writes() { __builtin_amdgcn_s_waitcnt(0xC07F); }   // lgkmcnt(0)

// Workgroup barrier without a memory fence. A fence would wait for every
// outstanding load, including the direct-to-LDS copies of later panels; the
// waits this pipeline needs are explicit instead (vmcnt for a panel's copies,
// lgkmcnt for LDS writes). The empty asm statements keep the compiler from
// moving memory accesses across the barrier.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// TS 16-K steps per panel, S LDS stages (panels in flight: S - 1).
template <int WM, int WN, int TM, int TN, int TS, int S>
struct Bf16Cfg {
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BM = 32 * TM * WM;
  static constexpr int BN = 32 * TN * WN;
  static constexpr int kPanelK = 16 * TS;
  static constexpr int kChunksA = BM / 32;
  static constexpr int kChunksB = BN / 32;
  static constexpr int kChunks = kChunksA + kChunksB;
  static constexpr int kFull = kChunks / kWaves;           // chunks every wave copies
  static constexpr int kRest = kChunks - kFull * kWaves;   // waves 0..kRest-1 copy one more
  static constexpr int kPerWave = kFull + (kRest ? 1 : 0);
  static constexpr int kChunkBytes = TS * 1024;             // 32 rows x kPanelK bf16
  static constexpr int kPieces = kPanelK / 8;              // 16-byte pieces per row segment
  static constexpr int kRowsPerCopy = 64 / kPieces;        // rows per 1 KB copy instruction
  static constexpr int kCopies = 32 / kRowsPerCopy;        // copy instructions per chunk
  static constexpr int kStageBytes = kChunks * kChunkBytes;
  // Piece permutation of chunk row r. A fragment read has 32 rows x one
  // 16-byte piece; groups of 8 lanes (32 four-byte banks) or 16 lanes (64
  // banks) must land in distinct 16-byte bank slots, i.e. rows whose segments
  // start at the same slot need distinct swz values: 64-K panels (128-byte
  // rows): rows of equal parity among 16; 32-K panels (64-byte rows): rows of
  // equal r % 2 among 8 and of equal r % 4 among 16.
  __host__ __device__ static constexpr int swz(int r) {
    return TS == 4 ? ((r ^ (r >> 3)) & 7) : TS == 2 ? (((r >> 1) ^ (r >> 3)) & 3) : 0;
  }
  static constexpr int kOutBytes = kWaves * 32 * (32 * TN) * 2;   // output staging (epilogue)
  static constexpr int kLdsBytes = S * kStageBytes > kOutBytes ? S * kStageBytes : kOutBytes;
};

// PIPE: the software-pipelined loop (two LDS stages of 64-K panels only). Each 16-K
// step issues the next step's fragment reads between its own matrix instructions, one
// read after each of the first TM + TN, into a second register set; the panel barrier
// sits before the last step, whose instructions then cover the first reads of the next
// panel. Without the ordering hints the compiler issues each step's reads after the
// previous step's matrix instructions and waits for them at once, and the matrix pipe
// idles for about one LDS round trip per step. It needs 2 * (TM + TN) fragment
// registers, which fits 2 x 4 tiles per wave but not 2 x 5.
template <int WM, int WN, int TM, int TN, int TS, int S, bool PIPE>
__global__ __launch_bounds__(64 * WM * WN) void gemm_bf16_kernel(Bf16GemmArgs a) {
  using C = Bf16Cfg<WM, WN, TM, TN, TS, S>;
  static_assert(!PIPE || (S == 2 && TS == 4), "pipelined loop: two stages of 64-K panels");
  static_assert(S >= 2 && (S - 2) * C::kPerWave * C::kCopies < 64, "stage count");
  static_assert(TS == 2 || TS == 4, "panel depth");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int wave_m = wave % WM;
  const int wave_n = wave / WM;

  const int M = (int)a.M, N = (int)a.N;
  const int64_t K = a.K;
  const int KP = (int)((K + C::kPanelK - 1) / C::kPanelK);

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
  const int m0 = by * C::BM;
  const int n0 = bx * C::BN;

  // LDS layout of a chunk (32 rows x kPanelK of x or W): row-major, row r at
  // r * kPanelK * 2 bytes, its 16-byte pieces permuted by piece ^ swz(r). A
  // copy instruction moves kRowsPerCopy whole row segments (lane l: row
  // l / kPieces, LDS slot l % kPieces, so the global side reads full
  // contiguous row segments and the LDS side one contiguous 1 KB block), and
  // the fragment reads (32 rows, one piece each) hit distinct banks.
  // chunk c = wave + kWaves * s (A chunks first); rows clamped into the tensor.
  const uint16_t* src[C::kPerWave][C::kCopies];
#pragma unroll
  for (int s = 0; s < C::kPerWave; ++s) {
    const int c = min(wave + C::kWaves * s, C::kChunks - 1);
    const bool is_a = c < C::kChunksA;
#pragma unroll
    for (int i = 0; i < C::kCopies; ++i) {
      const int r = i * C::kRowsPerCopy + lane / C::kPieces;      // row within the chunk
      const int piece = (lane % C::kPieces) ^ C::swz(r);
      const int row = is_a ? min(m0 + 32 * c + r, M - 1) : min(n0 + 32 * (c - C::kChunksA) + r, N - 1);
      src[s][i] = (is_a ? a.x : a.w) + (size_t)row * (size_t)K + 8 * piece;
    }
  }
  const bool extra = C::kRest && wave < C::kRest;   // this wave copies kPerWave chunks

  auto stage_at = [&](int kp) { return smem + (kp % S) * C::kStageBytes; };
  auto copy_chunk = [&](int s, int kp, uint8_t* stage) {
    const int c = wave + C::kWaves * s;
#pragma unroll
    for (int i = 0; i < C::kCopies; ++i) {
      // (a pointer of non-dependent type: the host pass rejects this builtin
      // with a template-dependent argument)
      const uint16_t* g = src[s][i] + (size_t)kp * C::kPanelK;
      __builtin_amdgcn_global_load_lds(g, LDS_PTR(stage + c * C::kChunkBytes + i * 1024), 16, 0, 0);
    }
  };
  // a panel reaching past K (K % kPanelK != 0): through registers, zeros past K
  // (K % 16 == 0, so each 8-element piece is entirely before or past K)
  auto fill_chunk = [&](int s, int kp, uint8_t* stage) {
    const int c = wave + C::kWaves * s;
#pragma unroll
    for (int i = 0; i < C::kCopies; ++i) {
      const int r = i * C::kRowsPerCopy + lane / C::kPieces;
      const int piece = (lane % C::kPieces) ^ C::swz(r);
      const int64_t k = (int64_t)kp * C::kPanelK + 8 * piece;
      u32x4 v = zero4();
      if (k < K) v = *reinterpret_cast<const u32x4*>(src[s][i] + (size_t)kp * C::kPanelK);
      *reinterpret_cast<u32x4*>(stage + c * C::kChunkBytes + i * 1024 + lane * 16) = v;
    }
  };
  const bool k_tail = (K % C::kPanelK) != 0;
  auto load_panel = [&](int kp) {
    uint8_t* stage = stage_at(kp);
    if (k_tail && kp == KP - 1) {
#pragma unroll
      for (int s = 0; s < C::kFull; ++s) fill_chunk(s, kp, stage);
      if (extra) fill_chunk(C::kFull, kp, stage);
    } else {
#pragma unroll
      for (int s = 0; s < C::kFull; ++s) copy_chunk(s, kp, stage);
      if (extra) copy_chunk(C::kFull, kp, stage);
    }
  };
  // Wait until this wave's copies of panel kp have landed: the copies of the
  // `later` panels issued after it may stay in flight (loads complete in
  // order). The register-filled tail panel leaves nothing in flight.
  auto wait_panel = [&](int kp) {
    const int last_issued = min(kp + S - 2, KP - 1);
    const int later = last_issued - kp - ((k_tail && last_issued == KP - 1 && kp < KP - 1) ? 1 : 0);
    if (S == 2 || later <= 0) {
      wait_vm<0>();
    } else if (S == 3 || later == 1) {
      if (extra) wait_vm<C::kPerWave * C::kCopies>(); else wait_vm<C::kFull * C::kCopies>();
    } else if (S == 4 || later == 2) {
      if (extra) wait_vm<(S >= 4 ? 2 : 0) * C::kPerWave * C::kCopies>(); else wait_vm<(S >= 4 ? 2 : 0) * C::kFull * C::kCopies>();
    } else {
      if (extra) wait_vm<(S >= 5 ? 3 : 0) * C::kPerWave * C::kCopies>(); else wait_vm<(S >= 5 ? 3 : 0) * C::kFull * C::kCopies>();
    }
  };

  // bias of this lane's columns (0 without a bias)
  const int n_w = n0 + wave_n * TN * 32;
  float bias_v[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = n_w + 32 * j + l32;
    bias_v[j] = (a.bias != nullptr && col < N) ? bf16lo_to_f32(a.bias[col]) : 0.0f;
  }

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // this lane's fragment (row l32, piece 2t + h of 16-K step t) within a chunk
  int frag_off[TS];
#pragma unroll
  for (int t = 0; t < TS; ++t) frag_off[t] = l32 * C::kPanelK * 2 + (((2 * t + h) ^ C::swz(l32)) * 16);

  if constexpr (PIPE) {
    bf16x8 fr[2][TM + TN];
    auto read_set = [&](bf16x8 (&dst)[TM + TN], const uint8_t* st, int t) {
      const int off = frag_off[t];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        dst[i] = *reinterpret_cast<const bf16x8*>(st + (wave_m * TM + i) * C::kChunkBytes + off);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        dst[TM + j] = *reinterpret_cast<const bf16x8*>(st + (C::kChunksA + wave_n * TN + j) * C::kChunkBytes + off);
    };
    // one 16-K step: the matrix instructions of `cur`, with the reads of step `t` of
    // stage `st` into `nxt` (when rd) placed one after each of the first TM + TN of them
    auto step = [&](const bf16x8 (&cur)[TM + TN], bf16x8 (&nxt)[TM + TN], const uint8_t* st, int t, bool rd) {
      __builtin_amdgcn_sched_barrier(0);
      if (rd) read_set(nxt, st, t);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur[i], cur[TM + j], acc[i][j], 0, 0, 0);
      if (rd) {
#pragma unroll
        for (int q = 0; q < TM + TN; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one matrix instruction
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - (TM + TN), 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    load_panel(0);
    wait_panel(0);
    wait_lds_writes();
    barrier_no_fence();
    if (KP > 1) load_panel(1);
    read_set(fr[0], stage_at(0), 0);
    for (int kp = 0; kp + 1 < KP; ++kp) {
      const uint8_t* cur = stage_at(kp);
      step(fr[0], fr[1], cur, 1, true);
      step(fr[1], fr[0], cur, 2, true);
      step(fr[0], fr[1], cur, 3, true);
      // every wave has read this stage to the end (lgkmcnt) and panel kp+1 has landed:
      // publish it, then refill this stage with panel kp+2 while the last step multiplies
      wait_panel(kp + 1);
      wait_lds_writes();
      barrier_no_fence();
      if (kp + 2 < KP) load_panel(kp + 2);
      step(fr[1], fr[0], stage_at(kp + 1), 0, true);
    }
    const uint8_t* last = stage_at(KP - 1);
    step(fr[0], fr[1], last, 1, true);
    step(fr[1], fr[0], last, 2, true);
    step(fr[0], fr[1], last, 3, true);
    step(fr[1], fr[0], last, 0, false);
  } else {
#pragma unroll
  for (int p = 0; p < S - 1; ++p)
    if (p < KP) load_panel(p);

  for (int kp = 0; kp < KP; ++kp) {
    wait_panel(kp);
    wait_lds_writes();   // the register-filled tail panel
    barrier_no_fence();  // panel kp visible to all waves; panel kp-1's stage is free
    if (kp + S - 1 < KP) load_panel(kp + S - 1);
    const uint8_t* cur = stage_at(kp);
    bf16x8 fa[TM], fb[TN];
    auto read_frags = [&](int t) {
      const int off = frag_off[t];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(cur + (wave_m * TM + i) * C::kChunkBytes + off);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fb[j] = *reinterpret_cast<const bf16x8*>(cur + (C::kChunksA + wave_n * TN + j) * C::kChunkBytes + off);
    };
    read_frags(0);
#pragma unroll
    for (int t = 0; t < TS; ++t) {
      bf16x8 ca[TM], cb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) ca[i] = fa[i];
#pragma unroll
      for (int j = 0; j < TN; ++j) cb[j] = fb[j];
      if (t + 1 < TS) read_frags(t + 1);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ca[i], cb[j], acc[i][j], 0, 0, 0);
    }
  }
  }
  __syncthreads();   // every wave done with the stages: LDS reused for the output

  // bf16 output through LDS: each wave stages its 32-row slices row-major,
  // then stores whole 16-byte row pieces.
  constexpr int kCols = 32 * TN;
  constexpr int kPieces = kCols / 8;
  const int m_w = m0 + wave_m * TM * 32;
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
          uint16_t* dst = a.y + (size_t)m * (size_t)N + n;
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

template <int WM, int WN, int TM, int TN, int TS, int S, bool PIPE>
hipError_t launch_bf16_cfg(const Bf16GemmArgs& a, hipStream_t stream) {
  using C = Bf16Cfg<WM, WN, TM, TN, TS, S>;
  static_assert(C::kLdsBytes <= 160 * 1024, "LDS budget");
  const int64_t tiles = ((a.N + C::BN - 1) / C::BN) * ((a.M + C::BM - 1) / C::BM);
  const unsigned lds = C::kLdsBytes;
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(&gemm_bf16_kernel<WM, WN, TM, TN, TS, S, PIPE>),
                                    (int)lds, lds_set);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((tiles + 7) / 8 * 8));
  hipLaunchKernelGGL((gemm_bf16_kernel<WM, WN, TM, TN, TS, S, PIPE>), grid, dim3(C::kThreads), lds, stream, a);
  return hipGetLastError();
}

// 64-K panels (each copy instruction moves 8 whole 128-byte row segments),
// two stages; waves WM x WN, each TM x TN 32x32 tiles.
constexpr int kTS = 4;
constexpr int kStages = 2;
constexpr int kWM = 4, kWN = 2, kTM = 2;

}  // namespace

int64_t gemm_bf16_tiles(int64_t M, int64_t N) {
  return ((M + 255) / 256) * ((N + 255) / 256);
}

// Tile width 256 or 320 columns by a round-count estimate: one workgroup per CU,
// ceil(tiles / 256) rounds, a 256-wide tile (pipelined loop) costing about 75% of a
// 320-wide one (measured at K = 3840: 104.5 us for one round of 256-wide tiles against
// 287 us for two rounds of 320-wide ones).
hipError_t launch_gemm_bf16(const Bf16GemmArgs& a, hipStream_t stream) {
  const int64_t row_blocks = (a.M + 255) / 256;
  const int64_t tiles320 = row_blocks * ((a.N + 319) / 320);
  const int64_t tiles256 = row_blocks * ((a.N + 255) / 256);
  const double cost320 = (double)((tiles320 + 255) / 256);
  const double cost256 = 0.75 * (double)((tiles256 + 255) / 256);
  if (cost256 < cost320) return launch_bf16_cfg<kWM, kWN, kTM, 4, kTS, kStages, true>(a, stream);
  return launch_bf16_cfg<kWM, kWN, kTM, 5, kTS, kStages, false>(a, stream);
}

}  // namespace svdq
