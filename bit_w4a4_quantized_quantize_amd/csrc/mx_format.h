// The MX (OCP microscaling) E2M1 block rule shared by the MXFP4 kernels: a block
// of 32 consecutive K has the E8M0 exponent X = floor(log2 amax) - 2 clamped to
// [-127, 127] (byte X + 127; an all-zero block gets X = -127), and each value's
// code is the E2M1 nearest-even of v * 2^-X (exact power-of-two scaling, then the
// hardware conversion, which saturates at 6 and keeps the sign).
#pragma once

#include "common.h"

namespace svdq {

__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.0f)) return -127;
  int e;
  frexpf(amax, &e);   // amax = m 2^e, m in [0.5, 1): floor(log2 amax) = e - 1
  return min(127, max(-127, e - 1 - 2));
}

// 8 values of a block -> 4 bytes of E2M1 codes (value 2i in the low nibble of byte i)
__device__ __forceinline__ uint32_t mx_codes8(const float* v, int X) {
  uint32_t p = 0;
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, ldexpf(v[0], -X), ldexpf(v[1], -X), 1.0f, 0);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, ldexpf(v[2], -X), ldexpf(v[3], -X), 1.0f, 1);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, ldexpf(v[4], -X), ldexpf(v[5], -X), 1.0f, 2);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, ldexpf(v[6], -X), ldexpf(v[7], -X), 1.0f, 3);
  return p;
}

}  // namespace svdq
