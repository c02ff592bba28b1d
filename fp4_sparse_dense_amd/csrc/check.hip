// The E2M1 converts of the SharQ kernels on caller-supplied values, used exactly
// as the preparation (fp4_enc / fp4_dec with the block scale inside the
// convert), the weight pack (a binary32 product by 2^-e, then fp4_pack2 with
// scale 1) and the NVFP4-style path (fp4_pack2 / fp4_unpack2 with scale 1) use
// them, so a test can compare every code and value with the rounding rule; the
// NVFP4-style path's E4M3 block-scale rounding and decoding; and one
// block-scaled FP4 MFMA issued as the GEMM kernels issue it, so a test can pin
// its operand, scale and accumulator lane layouts.
#include <hip/hip_runtime.h>

#include <cstring>

#include "sharq_check.h"
#include "device_common.h"
#include "e4m3.h"
#include "gemm_common.h"
#include "prep_common.h"

namespace sharq {

sharq_status record_error(sharq_status s, const char* msg);   // api.hip

__global__ __launch_bounds__(256) void check_e2m1_kernel(const float* __restrict__ x, const int32_t* __restrict__ exps,
                                                         int64_t n, int64_t groups, uint32_t* __restrict__ enc,
                                                         uint32_t* __restrict__ pack, float* __restrict__ dec,
                                                         float* __restrict__ unpack) {
  const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;   // group of 8 values
  if (gi >= groups) return;
  const int64_t per = n / 8;
  const int s = (int)(gi / per);
  const int e = exps[s];
  const float* xs = x + gi * 8;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = xs[i];
  // the preparation's way
  const float sc = pow2(e);
  uint32_t c = fp4_enc<0>(0u, v[0], v[1], sc);
  c = fp4_enc<1>(c, v[2], v[3], sc);
  c = fp4_enc<2>(c, v[4], v[5], sc);
  c = fp4_enc<3>(c, v[6], v[7], sc);
  float d[8];
  fp4_dec<0>(c, sc, d[0], d[1]);
  fp4_dec<1>(c, sc, d[2], d[3]);
  fp4_dec<2>(c, sc, d[4], d[5]);
  fp4_dec<3>(c, sc, d[6], d[7]);
  // the pack's way
  const float qs = pow2_neg(e);
  uint32_t p = fp4_pack2<0>(0u, v[0] * qs, v[1] * qs);
  p = fp4_pack2<1>(p, v[2] * qs, v[3] * qs);
  p = fp4_pack2<2>(p, v[4] * qs, v[5] * qs);
  p = fp4_pack2<3>(p, v[6] * qs, v[7] * qs);
  float u[8];
  fp4_unpack2<0>(p, u[0], u[1]);
  fp4_unpack2<1>(p, u[2], u[3]);
  fp4_unpack2<2>(p, u[4], u[5]);
  fp4_unpack2<3>(p, u[6], u[7]);
  enc[gi] = c;
  pack[gi] = p;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    dec[gi * 8 + i] = d[i];
    unpack[gi * 8 + i] = u[i];
  }
}

// E4M3 of each value as the NVFP4-style kernels round their block scales, and
// the byte decoded back as their GEMM decodes it.
__global__ __launch_bounds__(256) void check_e4m3_kernel(const float* __restrict__ x, int64_t n,
                                                         uint8_t* __restrict__ byte, float* __restrict__ value,
                                                         float* __restrict__ dec) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  uint32_t b = 0;
  value[i] = e4m3_round(x[i], b);
  byte[i] = (uint8_t)b;
  dec[i] = e4m3_value(b);
}

// One block-scaled FP4 MFMA per wave on operands in the tiled layout, issued
// through the GEMM kernels' own operand and MFMA helpers (as_operand,
// mfma_fp4): lane l brings the 16 code bytes and the scale byte of row l % 16,
// 32-element chunk l / 16, of each operand, and its accumulator holds
// D[4 * (l / 16) + i][l % 16], i = 0..3.
__global__ __launch_bounds__(256) void check_mfma_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ sa,
                                                         const uint8_t* __restrict__ b, const uint8_t* __restrict__ sb,
                                                         int n_blocks, float* __restrict__ d) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= n_blocks) return;   // wave-uniform
  const uint4 qa = *reinterpret_cast<const uint4*>(a + blk * 1024 + lane * 16);
  const uint4 qb = *reinterpret_cast<const uint4*>(b + blk * 1024 + lane * 16);
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  acc = mfma_fp4(as_operand(qa), as_operand(qb), acc, sa[blk * 64 + lane], sb[blk * 64 + lane]);
#pragma unroll
  for (int i = 0; i < 4; ++i) d[blk * 256 + (4 * (lane >> 4) + i) * 16 + (lane & 15)] = acc[i];
}

}  // namespace sharq

extern "C" {

sharq_status sharq_check_e2m1(const float* x_dev, const int32_t* exps_dev, int64_t n, int32_t n_scales,
                              uint32_t* enc_dev, uint32_t* pack_dev, float* dec_dev, float* unpack_dev, void* stream) {
  if (!x_dev || !exps_dev || !enc_dev || !pack_dev || !dec_dev || !unpack_dev)
    return sharq::record_error(SHARQ_ERR_INVALID_ARG, "null argument");
  if (n <= 0 || n % 8 || n_scales < 1 || (int64_t)n_scales * n >= ((int64_t)1 << 31))
    return sharq::record_error(SHARQ_ERR_INVALID_ARG, "n must be a positive multiple of 8, n_scales >= 1, n_scales*n < 2^31");
  if ((reinterpret_cast<uintptr_t>(x_dev) | reinterpret_cast<uintptr_t>(exps_dev) | reinterpret_cast<uintptr_t>(enc_dev) |
       reinterpret_cast<uintptr_t>(pack_dev) | reinterpret_cast<uintptr_t>(dec_dev) |
       reinterpret_cast<uintptr_t>(unpack_dev)) & 3)
    return sharq::record_error(SHARQ_ERR_INVALID_ARG, "buffers must be 4-byte aligned");
  int dev = 0;
  hipDeviceProp_t p;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&p, dev) != hipSuccess)
    return sharq::record_error(SHARQ_ERR_HIP, "device query failed");
  if (std::strncmp(p.gcnArchName, "gfx950", 6) != 0) return sharq::record_error(SHARQ_ERR_UNSUPPORTED, "not gfx950");
  const int64_t groups = (int64_t)n_scales * n / 8;
  hipLaunchKernelGGL(sharq::check_e2m1_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), x_dev, exps_dev, n, groups, enc_dev, pack_dev, dec_dev,
                     unpack_dev);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return sharq::record_error(SHARQ_ERR_HIP, hipGetErrorString(e));
  return SHARQ_OK;
}

sharq_status sharq_check_e4m3(const float* x_dev, int64_t n, uint8_t* byte_dev, float* value_dev, float* dec_dev,
                              void* stream) {
  if (!x_dev || !byte_dev || !value_dev || !dec_dev) return sharq::record_error(SHARQ_ERR_INVALID_ARG, "null argument");
  if (n < 1 || n > ((int64_t)1 << 31)) return sharq::record_error(SHARQ_ERR_INVALID_ARG, "n must be in 1 .. 2^31");
  if ((reinterpret_cast<uintptr_t>(x_dev) | reinterpret_cast<uintptr_t>(value_dev) | reinterpret_cast<uintptr_t>(dec_dev)) & 3)
    return sharq::record_error(SHARQ_ERR_INVALID_ARG, "float buffers must be 4-byte aligned");
  int dev = 0;
  hipDeviceProp_t p;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&p, dev) != hipSuccess)
    return sharq::record_error(SHARQ_ERR_HIP, "device query failed");
  if (std::strncmp(p.gcnArchName, "gfx950", 6) != 0) return sharq::record_error(SHARQ_ERR_UNSUPPORTED, "not gfx950");
  hipLaunchKernelGGL(sharq::check_e4m3_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), x_dev, n, byte_dev, value_dev, dec_dev);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return sharq::record_error(SHARQ_ERR_HIP, hipGetErrorString(e));
  return SHARQ_OK;
}

sharq_status sharq_check_mfma_fp4(const uint8_t* a_dev, const uint8_t* sa_dev, const uint8_t* b_dev,
                                  const uint8_t* sb_dev, int32_t n_blocks, float* d_dev, void* stream) {
  if (!a_dev || !sa_dev || !b_dev || !sb_dev || !d_dev) return sharq::record_error(SHARQ_ERR_INVALID_ARG, "null argument");
  if (n_blocks < 1 || n_blocks > (1 << 20)) return sharq::record_error(SHARQ_ERR_INVALID_ARG, "n_blocks must be in 1 .. 2^20");
  if ((reinterpret_cast<uintptr_t>(a_dev) | reinterpret_cast<uintptr_t>(b_dev)) & 15 ||
      reinterpret_cast<uintptr_t>(d_dev) & 3)
    return sharq::record_error(SHARQ_ERR_INVALID_ARG, "codes must be 16-byte aligned, outputs 4-byte aligned");
  int dev = 0;
  hipDeviceProp_t p;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&p, dev) != hipSuccess)
    return sharq::record_error(SHARQ_ERR_HIP, "device query failed");
  if (std::strncmp(p.gcnArchName, "gfx950", 6) != 0) return sharq::record_error(SHARQ_ERR_UNSUPPORTED, "not gfx950");
  hipLaunchKernelGGL(sharq::check_mfma_kernel, dim3((unsigned)((n_blocks + 3) / 4)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a_dev, sa_dev, b_dev, sb_dev, n_blocks, d_dev);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return sharq::record_error(SHARQ_ERR_HIP, hipGetErrorString(e));
  return SHARQ_OK;
}

}  // extern "C"
