// Fusion ablations of the SharQ layer (README page of the SharQ repository,
// section "Benchmarks": the RMSNorm fusion and the epilogue fusion can each be
// switched off to measure what they save).
//
//   unfused RMSNorm: a standalone normalisation writes the normalised row in
//     bf16 (round to nearest even); the preparation then runs without gamma on
//     that row.  The bf16 rounding is the numerical price of not fusing.
//   residual add (the synthetic decoder layer): bf16 + fp32 -> bf16.
//   unfused epilogue: the two GEMM paths run as separate launches into two
//     fp32 outputs, then one elementwise add.  (With the backbone stored as a
//     masked dense operand, either path alone is the plain FP4 GEMM pointed at
//     that operand's codes and scales.)
#include "device_common.h"
#include "launch.h"

namespace sharq {
namespace {

// One workgroup per row: 1/rms by the same pairwise tree as the fused
// preparation, then y = bf16((x * inv) * gamma) in 64-byte pieces.
__global__ __launch_bounds__(256) void rmsnorm_bf16_kernel(const uint16_t* __restrict__ x, int64_t ldx, int K,
                                                           const uint16_t* __restrict__ gamma, float eps,
                                                           uint16_t* __restrict__ y, int64_t ldy) {
  __shared__ float cs[1024];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * ldx;
  const float inv = row_inv_rms(xr, K, eps, cs);
  for (int c = threadIdx.x; c < K / 32; c += 256) {
    float v[32];
    load32(xr + 32 * c, v);
    apply_norm(v, gamma + 32 * c, inv);
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t lo = __float_as_uint(v[2 * i]), hi = __float_as_uint(v[2 * i + 1]);
      lo += 0x7FFFu + ((lo >> 16) & 1u);
      hi += 0x7FFFu + ((hi >> 16) & 1u);
      w[i] = (lo >> 16) | (hi & 0xFFFF0000u);
    }
    uint4* dst = reinterpret_cast<uint4*>(y + row * ldy + 32 * c);
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
  }
}

// y = a + b, four elements per thread where all three are 16-byte aligned
__global__ __launch_bounds__(256) void add_f32_kernel(const float* __restrict__ a, const float* __restrict__ b,
                                                      float* __restrict__ y, int64_t n, int vec) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  if (vec) {
    const int64_t n4 = n / 4;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
      const float4 p = reinterpret_cast<const float4*>(a)[i], q = reinterpret_cast<const float4*>(b)[i];
      reinterpret_cast<float4*>(y)[i] = make_float4(p.x + q.x, p.y + q.y, p.z + q.z, p.w + q.w);
    }
    for (int64_t i = n4 * 4 + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) y[i] = a[i] + b[i];
  } else {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) y[i] = a[i] + b[i];
  }
}

// out = bf16(x + y) (binary32 sum of a bf16 and an fp32 element, rounded to
// nearest even): the residual add of a decoder layer.  Four elements per
// thread when every pointer is 8-byte aligned for x/out and 16 for y.
__global__ __launch_bounds__(256) void add_bf16_f32_kernel(const uint16_t* __restrict__ x, const float* __restrict__ y,
                                                           uint16_t* __restrict__ out, int64_t n, int vec) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  auto one = [](uint16_t xb, float yv) -> uint16_t {
    uint32_t u = __float_as_uint(__uint_as_float((uint32_t)xb << 16) + yv);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
  };
  int64_t start = 0;
  if (vec) {
    const int64_t n4 = n / 4;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
      const uint2 xv = reinterpret_cast<const uint2*>(x)[i];
      const float4 yv = reinterpret_cast<const float4*>(y)[i];
      uint2 o;
      o.x = (uint32_t)one((uint16_t)xv.x, yv.x) | ((uint32_t)one((uint16_t)(xv.x >> 16), yv.y) << 16);
      o.y = (uint32_t)one((uint16_t)xv.y, yv.z) | ((uint32_t)one((uint16_t)(xv.y >> 16), yv.w) << 16);
      reinterpret_cast<uint2*>(out)[i] = o;
    }
    start = n4 * 4;
  }
  for (int64_t i = start + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) out[i] = one(x[i], y[i]);
}

}  // namespace

hipError_t launch_rmsnorm_bf16(const uint16_t* x, int64_t M, int K, int64_t ldx, const uint16_t* gamma, float eps,
                               uint16_t* y, int64_t ldy, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (M > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rmsnorm_bf16_kernel, dim3((unsigned)M), dim3(256), 0, stream, x, ldx, K, gamma, eps, y, ldy);
  return hipGetLastError();
}

hipError_t launch_add_bf16_f32(const uint16_t* x, const float* y, uint16_t* out, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int vec = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(out)) & 7) == 0 &&
                  (reinterpret_cast<uintptr_t>(y) & 15) == 0;
  int64_t blocks = (n / (vec ? 4 : 1) + 255) / 256;
  blocks = blocks < 1 ? 1 : (blocks > 8192 ? 8192 : blocks);
  hipLaunchKernelGGL(add_bf16_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, y, out, n, vec);
  return hipGetLastError();
}

hipError_t launch_add_f32(const float* a, const float* b, float* y, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int vec = ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) | reinterpret_cast<uintptr_t>(y)) & 15) == 0;
  int64_t blocks = (n / (vec ? 4 : 1) + 255) / 256;
  blocks = blocks < 1 ? 1 : (blocks > 8192 ? 8192 : blocks);
  hipLaunchKernelGGL(add_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, b, y, n, vec);
  return hipGetLastError();
}

}  // namespace sharq
