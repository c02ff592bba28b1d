// Measurement kernels: the FP4 MFMA rate and the streaming read bandwidth the
// chip reaches in practice (the layer's kernels are reported against these and
// against the published peaks).  Nothing here is part of the layer.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "sharq_peak.h"
#include "device_common.h"

namespace sharq {

constexpr int kPeakWaves = 4;          // per workgroup
constexpr int kPeakGroupsPerCu = 4;    // 16 waves per compute unit

__global__ __launch_bounds__(kPeakWaves * 64) void peak_fp4_kernel(const uint8_t* __restrict__ ops, int iters,
                                                                   float* sink) {
  const int lane = threadIdx.x & 63;
  // four A operands (bytes 0 .. 4095) and two B operands (4096 .. 6143),
  // 16 bytes per lane each
  v8i a[4], b[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 q = *reinterpret_cast<const uint4*>(ops + (size_t)(i * 64 + lane) * 16);
    a[i] = (v8i){(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint4 q = *reinterpret_cast<const uint4*>(ops + (size_t)((4 + i) * 64 + lane) * 16);
    b[i] = (v8i){(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
  }
  const uint32_t sa = 120u + ops[lane] % 15u, sb = 120u + ops[64 - 1 - lane] % 15u;
  v4f c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
  const int isa = (int)sa, isb = (int)sb;
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[0], b[0], c0, 4, 4, 0, isa, 0, isb);
    c1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[1], b[0], c1, 4, 4, 0, isa, 0, isb);
    c2 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[2], b[0], c2, 4, 4, 0, isa, 0, isb);
    c3 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[3], b[0], c3, 4, 4, 0, isa, 0, isb);
    c4 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[0], b[1], c4, 4, 4, 0, isa, 0, isb);
    c5 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[1], b[1], c5, 4, 4, 0, isa, 0, isb);
    c6 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[2], b[1], c6, 4, 4, 0, isa, 0, isb);
    c7 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[3], b[1], c7, 4, 4, 0, isa, 0, isb);
  }
  const v4f t = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
  const float s = (t[0] + t[1]) + (t[2] + t[3]);
  if (s == 1.2345678e-30f) sink[0] = s;
}

constexpr int kReadThreads = 256;
constexpr int kReadGroupsPerCu = 8;

__global__ __launch_bounds__(kReadThreads) void peak_read_kernel(const uint4* __restrict__ buf, size_t n16,
                                                                uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
  // four loads in flight per thread per trip
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 p = buf[i], q = buf[i + stride], r = buf[i + 2 * stride], t = buf[i + 3 * stride];
    acc ^= p.x ^ p.y ^ p.z ^ p.w ^ q.x ^ q.y ^ q.z ^ q.w ^ r.x ^ r.y ^ r.z ^ r.w ^ t.x ^ t.y ^ t.z ^ t.w;
  }
  for (; i < n16; i += stride) {
    const uint4 p = buf[i];
    acc ^= p.x ^ p.y ^ p.z ^ p.w;
  }
  if (acc == 0x9E3779B9u && threadIdx.x == 0 && blockIdx.x == 0x7FFFFFFF) sink[0] = acc;
}

}  // namespace sharq

namespace sharq {
sharq_status record_error(sharq_status s, const char* msg);   // api.hip
}

namespace {

sharq_status peak_fail(sharq_status s, const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return sharq::record_error(s, buf);
}

// compute units of a gfx950 device, or an error status
sharq_status peak_device(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return peak_fail(SHARQ_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  hipDeviceProp_t p;
  e = hipGetDeviceProperties(&p, dev);
  if (e != hipSuccess) return peak_fail(SHARQ_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  if (std::strncmp(p.gcnArchName, "gfx950", 6) != 0) return peak_fail(SHARQ_ERR_UNSUPPORTED, "not gfx950");
  *cus = p.multiProcessorCount;
  return SHARQ_OK;
}

}  // namespace

extern "C" {

sharq_status sharq_peak_fp4_mfma(const void* operands_dev, size_t operand_bytes, int32_t iters, float* sink_dev,
                                 double* flops_out, void* stream) {
  if (!operands_dev || !sink_dev || !flops_out) return peak_fail(SHARQ_ERR_INVALID_ARG, "null argument");
  if (operand_bytes < 6144 || (reinterpret_cast<uintptr_t>(operands_dev) & 15))
    return peak_fail(SHARQ_ERR_INVALID_ARG, "operands must be >= 6144 bytes, 16-byte aligned");
  if (iters < 1 || iters > (1 << 20)) return peak_fail(SHARQ_ERR_INVALID_ARG, "iters out of range");
  int cus = 0;
  sharq_status st = peak_device(&cus);
  if (st != SHARQ_OK) return st;
  const int grid = cus * sharq::kPeakGroupsPerCu;
  hipLaunchKernelGGL(sharq::peak_fp4_kernel, dim3(grid), dim3(sharq::kPeakWaves * 64), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(operands_dev), iters, sink_dev);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return peak_fail(SHARQ_ERR_HIP, "launch: %s", hipGetErrorString(e));
  *flops_out = (double)grid * sharq::kPeakWaves * (double)iters * 8.0 * (2.0 * 16 * 16 * 128);
  return SHARQ_OK;
}

sharq_status sharq_peak_read(const void* buf_dev, size_t bytes, uint32_t* sink_dev, double* bytes_out, void* stream) {
  if (!buf_dev || !sink_dev || !bytes_out) return peak_fail(SHARQ_ERR_INVALID_ARG, "null argument");
  if (bytes < (1u << 20) || bytes % 16 || (reinterpret_cast<uintptr_t>(buf_dev) & 15))
    return peak_fail(SHARQ_ERR_INVALID_ARG, "bytes must be a multiple of 16, >= 1 MiB, 16-byte aligned");
  int cus = 0;
  sharq_status st = peak_device(&cus);
  if (st != SHARQ_OK) return st;
  const int grid = cus * sharq::kReadGroupsPerCu;
  hipLaunchKernelGGL(sharq::peak_read_kernel, dim3(grid), dim3(sharq::kReadThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(buf_dev), bytes / 16, sink_dev);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return peak_fail(SHARQ_ERR_HIP, "launch: %s", hipGetErrorString(e));
  *bytes_out = (double)bytes;
  return SHARQ_OK;
}

}  // extern "C"
