// E4M3 block-scale rounding of the NVFP4-style path (OCP E4M3: bias 7, 3
// mantissa bits, subnormal step 2^-9, largest 448), shared by its kernels and
// by the convert check that pins it against the oracle on the device.
#pragma once
#include "device_common.h"

namespace sharq {

// E4M3 of a binary32 x >= 0, round to nearest even, saturating; returns the
// value and sets the byte.  Normal range: round the binary32 significand to 3
// bits (add half an ulp of the target minus one plus the kept LSB, then
// truncate).  Below 2^-6: the subnormal grid, rint(x * 2^9) * 2^-9 (v_rndne:
// half to even).
__device__ __forceinline__ float e4m3_round(float x, uint32_t& byte) {
  if (x >= 448.0f) {
    byte = 0x7Eu;
    return 448.0f;
  }
  if (x >= 0x1p-6f) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFFu + ((u >> 20) & 1u);
    u &= 0xFFF00000u;
    byte = ((((u >> 23) & 0xFFu) - 120u) << 3) | ((u >> 20) & 7u);
    return __uint_as_float(u);
  }
  const float n = __builtin_rintf(x * 512.0f);
  byte = (uint32_t)n;                  // 0..8; 8 is 2^-6, byte 0x08
  return n * 0x1p-9f;
}

// E4M3 byte (sign clear) -> binary32
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
}

}  // namespace sharq
