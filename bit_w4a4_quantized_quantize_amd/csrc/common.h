// Device-side helpers shared by the library's gfx950 kernels.
//
// NVFP4 = E2M1 codes with one float8_e4m3fn scale per 16 consecutive K
// elements (model card "nunchaku-z-image-turbo-svdq", header). The helpers
// below use gfx950 conversion instructions whose behaviour this library
// relies on (each checked exhaustively against exact arithmetic on the device):
//  * v_cvt_f32_fp8 decodes OCP e4m3fn exactly (all 256 codes, any byte select);
//  * v_cvt_pk_fp8_f32 rounds to nearest even but returns NaN above 464, so
//    inputs are clamped to 448 first (saturating encode);
//  * v_cvt_scalef32_pk_fp4_f32 with scale 1.0 is round-to-nearest-even onto
//    the E2M1 grid, saturating at 6, keeping the sign of zero; its scale
//    operand only contributes its power-of-two exponent;
//  * v_cvt_scalef32_pk_f16_fp4 with scale 1.0 decodes E2M1 exactly; an E2M1
//    value times any e4m3 value has at most 6 significant bits and lies in
//    [2^-10, 2688], so one f16 multiply by the decoded scale is exact.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even, by the hardware conversion
// (v_cvt_pk_bf16_f32). For every non-NaN input it equals the integer formula
// (u + 0x7FFF + ((u >> 16) & 1)) >> 16, denormals and ties included (checked on
// the device over 2^28 bit patterns); a NaN stays a NaN.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// e4m3fn byte (in the low byte of `b`) -> fp32, exact.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8((int)b, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8((int)b, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8((int)b, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8((int)b, 3);
  }
}

// s >= 0 -> e4m3fn code, round to nearest even, saturating at 448.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float s) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(s, 448.0f), 0.0f, 0, false) & 0xFFu;
}

// Block scale of a 16-block: e4m3(max|v| / 6). Multiplying by RN(1/6) gives the
// same code as the exact quotient: an exact e4m3 rounding midpoint mu (at most 5
// significant bits) comes out as mu * (1 + 2^-25), which rounds back to mu in
// fp32, and every other quotient is at least 2^-16 (relative) from a midpoint.
__device__ __forceinline__ uint32_t block_scale_code(float amax) {
  return f32_to_e4m3_sat(amax * (1.0f / 6.0f));
}

// 1 / s for a positive normal fp32 s (a decoded nonzero e4m3 scale, possibly times a
// global scale): hardware reciprocal plus one Newton step, within about 1 unit in
// the last place, which the 21-bit rounding of the quotients (below) tolerates.
__device__ __forceinline__ float scale_reciprocal(float sd) {
  const float r = __builtin_amdgcn_rcpf(sd);
  return __builtin_fmaf(__builtin_fmaf(-sd, r, 1.0f), r, r);
}

// Round a quotient v / s_d, computed as v * (1/s_d) within 3 units in the last
// place, to 21 significant bits: an exact E2M1 rounding midpoint (at most 3
// significant bits) is restored exactly, and every other quotient (at least
// 2^-16 relative away from any midpoint, since v has at most 16 significant
// bits and s_d at most 4) stays on its side of every midpoint.
__device__ __forceinline__ float snap21(float q) {
  return __uint_as_float((__float_as_uint(q) + 4u) & ~7u);
}

// Per-block scale rule, dynamic or relative to a static global activation scale g
// (a bf16 value: at most 8 significant bits, positive and normal).
//  dynamic: s = e4m3(max|v| * RN(1/6)), divisor dec(s);
//  static:  s = e4m3(round21(max|v| * r)) with r within about 1 unit of 1/(6 g),
//           divisor dec(s) * g (exact: 4 + 8 significant bits).
// Static exactness: max|v| (16 significant bits) against an e4m3 midpoint times
// 6 g (5 + 10 bits) is either equal or at least 2^-17 (relative) apart, so the
// product within 2 units of the quotient, rounded to 21 significant bits, lands
// exactly on a tie and on the right side otherwise; the code quotient v / (dec(s)
// g) keeps the same separation (3 + 12 bits against 16), as in the dynamic case.
template <bool STATIC>
struct BlockScale {
  float g = 1.0f, r6g = 0.0f;
  __device__ __forceinline__ void init(const uint16_t* gscale) {
    if (STATIC) {
      g = bf16lo_to_f32(gscale[0]);
      r6g = scale_reciprocal(6.0f * g);
    }
  }
  __device__ __forceinline__ uint32_t code(float amax) const {
    return STATIC ? f32_to_e4m3_sat(snap21(amax * r6g)) : block_scale_code(amax);
  }
  __device__ __forceinline__ float divisor(uint32_t sc) const {
    const float sd = e4m3_to_f32(sc, 0);
    return STATIC ? sd * g : sd;
  }
};

// Dequantise one dword of 8 E2M1 codes (low nibble first = lower k) times the
// block scale `s` (an exactly representable f16) into 8 f16 values, exactly.
__device__ __forceinline__ f16x8 dequant8_f16(uint32_t codes, _Float16 s) {
  const f16x2 ss = {s, s};
  f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * ss;
  f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * ss;
  f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * ss;
  f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * ss;
  f16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ u32x4 zero4() { u32x4 z = {0u, 0u, 0u, 0u}; return z; }

// Raw buffer resource over [base, base + bytes): loads at an offset at or past
// `bytes` return zero and stores there are dropped, so bounds checks become
// offset selects instead of branches. Every access in this library is either
// entirely inside or entirely outside the range.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

}  // namespace svdq
