// Internal launchers of the library's kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace svdq {

// Raise a kernel's dynamic LDS limit to `bytes`, once per device and process
// (`done` holds one bit per device ordinal), so that launches in a steady
// state (or under stream capture) make no attribute calls.
inline hipError_t set_lds_limit_once(const void* kernel, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = uint64_t(1) << (dev & 63);
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// a1: quant(x * smooth) -> qact [M, K/2], ascales [K/16, M] (canonical layout;
// the work is laid out for HBM streaming).
// gscale: NULL (dynamic scales) or the static global activation scale, bf16 [1] on
// the device (block scales relative to it; see common.h, BlockScale).
hipError_t launch_quant_act(const uint16_t* x, const uint16_t* smooth, uint8_t* qact,
                            uint8_t* ascales, int64_t M, int64_t K, hipStream_t stream,
                            const uint16_t* gscale = nullptr);

// a1 + a2 fused: one pass over x gives quant(x * smooth) and
// lora_act [M, R] = bf16(x @ proj_down) (R may be 0). Output codes/scales in the
// canonical layout or in the packed fragment layout read by gemm_lds.
// When R > 0 and M is small, K is split across workgroups: the fp32 partials
// go to `partial` (quant_lora_workspace_bytes(M, K, R) bytes, NULL if 0) and a
// second kernel adds them in split order.
size_t quant_lora_workspace_bytes(int64_t M, int64_t K, int64_t R);
hipError_t launch_quant_lora(const uint16_t* x, const uint16_t* smooth, const uint16_t* proj_down,
                             uint8_t* qact, uint8_t* ascales, uint16_t* lora_act, float* partial,
                             int64_t M, int64_t K, int64_t R, bool packed_out, hipStream_t stream,
                             const uint16_t* gscale = nullptr);

// Calibration of the static global activation scale: gscale [1] bf16 =
// bf16(max |x * smooth| / (6 * 448)), or 1 when that maximum is 0. workspace:
// calibrate_workspace_bytes(M, K) bytes of per-workgroup maxima.
size_t calibrate_workspace_bytes(int64_t M, int64_t K);
hipError_t launch_calibrate(const uint16_t* x, const uint16_t* smooth, int64_t M, int64_t K, uint16_t* gscale,
                            float* workspace, hipStream_t stream);

// a4 + a5: scaled GEMM, low-rank up-projection and epilogue.
struct GemmArgs {
  const uint8_t* qact;      // [M, K/2]
  const uint8_t* ascales;   // [K/16, M]
  const uint16_t* lora_act; // [M, R] bf16 (R > 0)
  const uint8_t* weight;    // canonical qweight [N, K/2] or packed buffer
  const uint8_t* wscales;   // canonical [K/16, N] (NULL when packed)
  const uint16_t* wcscales; // [N]
  const uint16_t* wtscale;  // [1]
  const uint16_t* proj_up;  // [N, R]
  const uint16_t* bias;     // [N] or NULL
  uint16_t* y;              // [M, N]
  int64_t M, N, K, R;
  int packed;
  int64_t gated_f;          // 0, or F: N = 2F and y = silu(y[:, :F]) * y[:, F:] is [M, F]
  const uint16_t* act_gscale = nullptr;  // static global activation scale bf16 [1], or NULL (= 1)
  // gated only: also quantise h for the next layer (w2), whose smooth is next_smooth [F],
  // into next_qact, the packed activation layout of [M, F] (F % 64 == 0), or NULL
  const uint16_t* next_smooth = nullptr;
  uint8_t* next_qact = nullptr;
  // launch_gemm_lds: activations in the canonical layout (qact [M, K/2], ascales [K/16, M])
  // instead of the packed buffer; only with the packed weight (canonical activations with
  // the canonical weight go to launch_gemm_w4a4)
  int act_canonical = 0;
};
// canonical activations (LDS-staged), canonical or packed weights
hipError_t launch_gemm_w4a4(const GemmArgs& a, hipStream_t stream);
// activations packed (qact holds the packed buffer) or canonical (act_canonical) and the
// weight packed or canonical (`packed`), not both canonical: each element dequantised once
// per workgroup into LDS
hipError_t launch_gemm_lds(const GemmArgs& a, hipStream_t stream);
// Process-wide tile shape of launch_gemm_lds: 0 automatic, 1 256 x 320, 2 256 x 256,
// 3 128 x 320, 4 128 x 160 (not gated: automatic there). Returns the previous value.
int set_gemm_tile(int tile);

// Linears kept in bf16: y = bf16(x @ w^T + bias), x [M, K], w [N, K], bias [N]
// or NULL, y [M, N]; K a multiple of 16, M and N below 2^24.
struct Bf16GemmArgs {
  const uint16_t* x;
  const uint16_t* w;
  const uint16_t* bias;
  uint16_t* y;
  int64_t M, N, K;
};
int64_t gemm_bf16_tiles(int64_t M, int64_t N);
hipError_t launch_gemm_bf16(const Bf16GemmArgs& a, hipStream_t stream);
// The same product through hipBLASLt (no workspace); *done stays false when no
// plan exists for the shape (first seen under stream capture) and nothing ran.
hipError_t blaslt_linear_bf16(const Bf16GemmArgs& a, hipStream_t stream, bool* done);

// Load-time SVDQuant weight preparation: the rank-R split of W / smooth by the
// randomized range finder (omega [K, R] fp32 from the caller; writes proj_down
// and proj_up, bf16), and the residual with its two-level scales and NVFP4
// codes. Both use one workspace of prep_workspace_bytes(N, K, R); R <= 128.
size_t prep_workspace_bytes(int64_t N, int64_t K, int64_t R);
hipError_t launch_prepare_lowrank(const uint16_t* W, const uint16_t* smooth, const float* omega, int64_t N,
                                  int64_t K, int64_t R, int iters, uint16_t* proj_down, uint16_t* proj_up,
                                  uint8_t* workspace, hipStream_t stream);
hipError_t launch_prepare_residual(const uint16_t* W, const uint16_t* smooth, const uint16_t* proj_down,
                                   const uint16_t* proj_up, int64_t N, int64_t K, int64_t R, uint8_t* qweight,
                                   uint8_t* wscales, uint16_t* wcscales, uint16_t* wtscale, uint8_t* workspace,
                                   hipStream_t stream);

// MXFP4 variant: E2M1 with one E8M0 scale per 32 K (codes in 32-row x 64-K
// chunks in the matrix-instruction order, mx_codes_bytes(rows, K) bytes; scales
// canonical [K/32, rows]). K % 128 == 0 for the GEMM.
size_t mx_codes_bytes(int64_t rows, int64_t K);
hipError_t launch_quant_act_mx(const uint16_t* x, const uint16_t* smooth, uint8_t* codes, uint8_t* scales,
                               int64_t M, int64_t K, hipStream_t stream);
hipError_t launch_reround_mx(const uint8_t* qweight, const uint8_t* wscales, uint8_t* codes, uint8_t* scales,
                             int64_t N, int64_t K, hipStream_t stream);
struct MxGemmArgs {
  const uint8_t* act_codes;
  const uint8_t* act_scales;
  const uint16_t* lora_act;
  const uint8_t* w_codes;
  const uint8_t* w_scales;
  const uint16_t* wcscales;
  const uint16_t* wtscale;
  const uint16_t* proj_up;
  const uint16_t* bias;
  uint16_t* y;
  int64_t M, N, K, R;
};
hipError_t launch_gemm_mx(const MxGemmArgs& a, hipStream_t stream);
// The variant's fused step: MX codes and scales of x * smooth (the layout above)
// and lora_act = bf16(x @ proj_down) in one pass over x (R = 0: the quantisation
// alone); partial as for launch_quant_lora. K % 128 == 0.
hipError_t launch_quant_lora_mx(const uint16_t* x, const uint16_t* smooth, const uint16_t* proj_down, uint8_t* codes,
                                uint8_t* scales, uint16_t* lora_act, float* partial, int64_t M, int64_t K, int64_t R,
                                hipStream_t stream);
// lora_act = bf16(x @ proj_down) alone (the quantiser's down-projection without
// the quantisation); partial as for launch_quant_lora
hipError_t launch_lowrank_down(const uint16_t* x, const uint16_t* proj_down, uint16_t* lora_act, float* partial,
                               int64_t M, int64_t K, int64_t R, hipStream_t stream);

// a3: load-time repack of qweight/wscales into the MFMA-order layout, and back.
// The same chunk layout holds packed activations (rows = tokens).
size_t packed_weight_bytes(int64_t N, int64_t K);
hipError_t launch_repack(const uint8_t* qweight, const uint8_t* wscales, uint8_t* packed,
                         int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_unpack(const uint8_t* packed, uint8_t* qweight, uint8_t* wscales,
                         int64_t N, int64_t K, hipStream_t stream);

// Measurement helpers (not part of the layer): sustained f16 matrix-instruction
// rate on a caller-filled operand table of calib_table_bytes() bytes, with the
// core-clock and constant-rate counters of each workgroup's start and end in
// clocks [workgroups][4] (c0, c1, w0, w1); out receives 512 floats per
// workgroup. And a plain device copy of `bytes` (a multiple of 16).
size_t calib_table_bytes();
int calib_waves_per_workgroup();
int64_t calib_flop_per_wave_iteration();
hipError_t launch_calib_mfma(const void* table, int64_t iters, int64_t workgroups, float* out, uint64_t* clocks,
                             hipStream_t stream);
// the block-scaled instruction (fmt 4: fp4 E2M1, 0: fp8 e4m3), unit scales, same table
int64_t calib_scaled_flop_per_wave_iteration();
hipError_t launch_calib_mfma_scaled(const void* table, int64_t iters, int64_t workgroups, int fmt, float* out,
                                    uint64_t* clocks, hipStream_t stream);
// LDS bandwidth (mode 0: 16-byte reads, 1: writes, 2: three reads to one write)
int64_t calib_lds_bytes_per_iteration(int64_t workgroups);
hipError_t launch_calib_lds(int64_t iters, int64_t workgroups, int mode, float* out, hipStream_t stream);
hipError_t launch_calib_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

}  // namespace svdq
