// Internal launchers of the library's kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace svdq {

// a1: quant(x * smooth) -> qact [M, K/2], ascales [K/16, M]. When `counters`
// is non-null the first workgroup also zeroes counters[0 .. n_counters) for
// the down-projection launched after it on the same stream.
hipError_t launch_quant_act(const uint16_t* x, const uint16_t* smooth, uint8_t* qact,
                            uint8_t* ascales, int64_t M, int64_t K, unsigned* counters,
                            int n_counters, hipStream_t stream);

// a2: lora_act [M, R] = bf16(x @ proj_down). Split over K across workgroups
// when M is small; then the workspace holds fp32 partial sums and one
// arrival counter per 32-row tile (zeroed by launch_quant_act).
int lora_down_splits(int64_t M, int64_t K, int64_t R);
int lora_down_counters(int64_t M);
size_t lora_down_workspace_bytes(int64_t M, int64_t K, int64_t R);
hipError_t launch_lora_down(const uint16_t* x, const uint16_t* proj_down, uint16_t* lora_act,
                            void* workspace, int64_t M, int64_t K, int64_t R,
                            hipStream_t stream);
// Offset of the counter array inside the down-projection workspace.
size_t lora_down_counter_offset(int64_t M, int64_t K, int64_t R);

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
};
hipError_t launch_gemm_w4a4(const GemmArgs& a, hipStream_t stream);

// a3: load-time repack of qweight/wscales into the MFMA-order layout, and back.
size_t packed_weight_bytes(int64_t N, int64_t K);
hipError_t launch_repack(const uint8_t* qweight, const uint8_t* wscales, uint8_t* packed,
                         int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_unpack(const uint8_t* packed, uint8_t* qweight, uint8_t* wscales,
                         int64_t N, int64_t K, hipStream_t stream);

}  // namespace svdq
