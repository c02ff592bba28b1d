// Operand, MFMA and output helpers shared by the GEMM kernels.
//
// MFMA 16x16x128 FP4 operand layout (pinned on the device bit for bit by
// tests/test_gpu_mfma.py through sharq_check_mfma_fp4): lane l holds row (or
// column) l%16 and K range [32*(l/16), 32*(l/16)+32) as 16 bytes, lower k in
// the low nibble; its scale byte is that row's E8M0 for the same 32-block; the
// accumulator of lane l holds D[4*(l/16)+i][l%16], i = 0..3.
#pragma once
#include "device_common.h"
#include "launch.h"

namespace sharq {

__device__ __forceinline__ v8i as_operand(uint4 q) {
  v8i r;
  r[0] = (int)q.x; r[1] = (int)q.y; r[2] = (int)q.z; r[3] = (int)q.w;
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

__device__ __forceinline__ v4f mfma_fp4(v8i a, v8i b, v4f c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

__device__ __forceinline__ uint32_t bf16_bits_rne(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// One output: fp32, or bf16 (nearest even) of the value -- plus the residual
// stream's bf16 element first when the layer adds one (one binary32 add).
__device__ __forceinline__ void store_out(const GemmArgs& g, int64_t row, int64_t col, float v) {
  if (g.out_bf16) {
    if (g.resid) v = __uint_as_float((uint32_t)g.resid[row * g.ld_resid + col] << 16) + v;
    reinterpret_cast<uint16_t*>(g.y)[row * g.ldy + col] = (uint16_t)bf16_bits_rne(v);
  } else {
    reinterpret_cast<float*>(g.y)[row * g.ldy + col] = v;
  }
}

// four consecutive outputs of one row (16-byte aligned for fp32, 8-byte for
// bf16 and the residual)
__device__ __forceinline__ void store_out4(const GemmArgs& g, int64_t row, int64_t col, v4f v) {
  if (g.out_bf16) {
    if (g.resid) {
      const uint2 x = *reinterpret_cast<const uint2*>(g.resid + row * g.ld_resid + col);
      v[0] = __uint_as_float(x.x << 16) + v[0];
      v[1] = __uint_as_float(x.x & 0xFFFF0000u) + v[1];
      v[2] = __uint_as_float(x.y << 16) + v[2];
      v[3] = __uint_as_float(x.y & 0xFFFF0000u) + v[3];
    }
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(g.y) + row * g.ldy + col) =
        make_uint2(bf16_bits_rne(v[0]) | bf16_bits_rne(v[1]) << 16, bf16_bits_rne(v[2]) | bf16_bits_rne(v[3]) << 16);
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(g.y) + row * g.ldy + col) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

}  // namespace sharq
