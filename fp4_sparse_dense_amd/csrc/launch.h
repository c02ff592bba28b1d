// Internal launchers (host side).  Arguments are validated by the C ABI layer
// before any of these run.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sharq {

struct PrepOut {
  uint8_t* s_codes;
  uint8_t* s_meta;
  uint8_t* s_scales;
  uint8_t* r_codes;
  uint8_t* r_scales;
};

hipError_t launch_prepare(const uint16_t* x, int64_t M, int K, int64_t ldx, const uint16_t* gamma,
                          float eps, PrepOut out, hipStream_t stream);

hipError_t launch_pack_weight(const uint16_t* w, int64_t N, int K, int64_t ldw, uint8_t* codes,
                              uint8_t* scales, hipStream_t stream);

struct GemmArgs {
  const uint8_t* s_codes;
  const uint8_t* s_meta;
  const uint8_t* s_scales;
  const uint8_t* r_codes;
  const uint8_t* r_scales;
  const uint8_t* w_codes;
  const uint8_t* w_scales_sparse;  // weight scale view of the sparse path
  const uint8_t* w_scales_dense;   // weight scale view of the dense path
  int64_t w_scales_ld;             // bytes between weight rows in both views
  void* y;
  int64_t ldy;
  int64_t M, N;
  int K;
  int out_bf16;
};

hipError_t launch_linear(const GemmArgs& a, hipStream_t stream);

}  // namespace sharq
