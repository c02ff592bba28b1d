// Decomposition of one MX block (32 consecutive elements of one row, one lane):
// the 2:4 mask, MXFP4 of the backbone, the residual against the quantised
// backbone and MXFP4 of the residual.  Shared by the preparation kernel and the
// fused small-M layer.
//
// SharQ paper page (mlsanity), Abstract: the backbone is an input-adaptive N:M
// mask of the row, quantised to FP4; the residual is taken against the
// quantised backbone and quantised for the dense path.
#pragma once
#include "device_common.h"

namespace sharq {

// ---------------------------------------------------------------------------
// One MX block (32 consecutive elements of one row) per lane.
// ---------------------------------------------------------------------------
struct Block32 {
  uint4 r_codes;     // 32 R nibbles
  uint4 s_codes;     // 32 S nibbles: the kept codes in place, zero codes at dropped positions
  uint32_t meta;     // 8 metadata nibbles
  uint32_t s_e8, r_e8;
};

// 2:4 mask of one group: element k is kept iff at most one other element
// beats it (larger magnitude, or equal magnitude and lower index).
//  * Element 0 wins every tie, so it is kept iff at most one of |a1|,|a2|,|a3|
//    exceeds |a0|, i.e. iff |a0| >= med3(|a1|,|a2|,|a3|).
//  * Element 3 loses every tie, so it is kept iff at most one of
//    |a0|,|a1|,|a2| reaches |a3|, i.e. iff med3(|a0|,|a1|,|a2|) < |a3|.
//  * Exactly two are kept.  If both or neither of elements 0 and 3 are kept,
//    elements 1 and 2 are both dropped or both kept; if exactly one is, the
//    other kept element is whichever of 1 and 2 beats the other
//    (|a1| >= |a2| for element 1).
// group_mask evaluates this with lane masks inside one asm block (no mask
// outlives the group), writes the masked group -- kept elements in place, +0
// at the dropped ones (a kept -0 stays -0) -- and shifts the group's metadata
// nibble i0 | i1 << 2 (the kept offsets in order) into `meta` most
// significant bit first (v_addc doubles and adds the carry-in mask).
__device__ __forceinline__ void group_mask(float a0, float a1, float a2, float a3, float& s0, float& s1, float& s2,
                                           float& s3, uint32_t& meta) {
  uint64_t k0, k1, k2, k3, b12, e, n, c;
  float m;
  asm volatile(
      "v_med3_f32 %[m], |%[a1]|, |%[a2]|, |%[a3]|\n\t"
      "v_cmp_ge_f32_e64 %[k0], |%[a0]|, %[m]\n\t"
      "v_med3_f32 %[m], |%[a0]|, |%[a1]|, |%[a2]|\n\t"
      "v_cmp_lt_f32_e64 %[k3], %[m], |%[a3]|\n\t"
      "v_cmp_ge_f32_e64 %[b12], |%[a1]|, |%[a2]|\n\t"
      // e = exactly one of k0, k3; n = neither
      "s_xor_b64 %[e], %[k0], %[k3]\n\t"
      "s_nor_b64 %[n], %[k0], %[k3]\n\t"
      "s_and_b64 %[c], %[e], %[b12]\n\t"
      "s_or_b64 %[k1], %[n], %[c]\n\t"
      "s_andn2_b64 %[c], %[e], %[b12]\n\t"
      "s_or_b64 %[k2], %[n], %[c]\n\t"
      "v_cndmask_b32_e64 %[s0], 0, %[a0], %[k0]\n\t"
      "v_cndmask_b32_e64 %[s1], 0, %[a1], %[k1]\n\t"
      "v_cndmask_b32_e64 %[s2], 0, %[a2], %[k2]\n\t"
      "v_cndmask_b32_e64 %[s3], 0, %[a3], %[k3]\n\t"
      // nibble bits, high to low: i1 = k3 ? 3 : (k2 ? 2 : 1), i0 = k0 ? 0 : (k1 ? 1 : 2)
      "s_or_b64 %[c], %[k3], %[k2]\n\t"
      "v_addc_co_u32_e64 %[meta], %[e], %[meta], %[meta], %[c]\n\t"
      "s_orn2_b64 %[c], %[k3], %[k2]\n\t"
      "v_addc_co_u32_e64 %[meta], %[e], %[meta], %[meta], %[c]\n\t"
      "s_nor_b64 %[c], %[k0], %[k1]\n\t"
      "v_addc_co_u32_e64 %[meta], %[e], %[meta], %[meta], %[c]\n\t"
      "s_andn2_b64 %[c], %[k1], %[k0]\n\t"
      "v_addc_co_u32_e64 %[meta], %[e], %[meta], %[meta], %[c]"
      : [s0] "=&v"(s0), [s1] "=&v"(s1), [s2] "=&v"(s2), [s3] "=&v"(s3), [meta] "+v"(meta), [m] "=&v"(m),
        [k0] "=&s"(k0), [k1] "=&s"(k1), [k2] "=&s"(k2), [k3] "=&s"(k3), [b12] "=&s"(b12), [e] "=&s"(e),
        [n] "=&s"(n), [c] "=&s"(c)
      : [a0] "v"(a0), [a1] "v"(a1), [a2] "v"(a2), [a3] "v"(a3)
      : "scc");
}

__device__ __forceinline__ float abs_max3(float m, float a, float b) {
  return fmaxf(fmaxf(m, fabsf(a)), fabsf(b));
}

// Encode two values as E2M1 into byte SEL of `old`, dividing by the power of
// two `scale` inside the convert, and decode byte SEL of `packed` multiplied
// by `scale`.  tests/test_gpu_fp4_convert.py checks both against the rounding
// rule and the exact values (through sharq_check_e2m1, which uses them as
// decompose32 does): every finite bf16 value and the 64 binary32 neighbours
// of every E2M1 grid point and midpoint times the scale, for every scale
// 2^-127 .. 2^125.
template <int SEL>
__device__ __forceinline__ uint32_t fp4_enc(uint32_t old, float lo, float hi, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, lo, hi, scale, SEL);
}
template <int SEL>
__device__ __forceinline__ void fp4_dec(uint32_t packed, float scale, float& lo, float& hi) {
  auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, scale, SEL);
  lo = v[0];
  hi = v[1];
}

// The whole decomposition of one MX block; v is replaced by the residual.
// DENSE (the plain FP4 linear, no backbone): the residual is v itself and
// only its MXFP4 codes are produced.
template <bool DENSE>
__device__ __forceinline__ Block32 decompose32(float (&v)[32]) {
  uint32_t sc[4] = {0u, 0u, 0u, 0u}, meta = 0;
  int es = -127;
  if constexpr (!DENSE) {
    // S block scale: the block maximum of v is always kept, so amax(S) == amax(v)
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; i += 2) am = abs_max3(am, v[i], v[i + 1]);
    es = mx_shared_exp(__float_as_uint(am));
    const float ss = pow2(es);

    // eight elements (two groups, one code word) at a time, last to first: the
    // metadata nibbles enter most significant first.  The masked group is
    // encoded in place (a dropped +0 gets code 0), decoded, and the residual is
    // v - deq(code): exact, and v itself where the element was dropped.
#pragma unroll
    for (int w = 3; w >= 0; --w) {
      float s8[8];
      group_mask(v[8 * w + 4], v[8 * w + 5], v[8 * w + 6], v[8 * w + 7], s8[4], s8[5], s8[6], s8[7], meta);
      group_mask(v[8 * w], v[8 * w + 1], v[8 * w + 2], v[8 * w + 3], s8[0], s8[1], s8[2], s8[3], meta);
      uint32_t c = fp4_enc<0>(0u, s8[0], s8[1], ss);
      c = fp4_enc<1>(c, s8[2], s8[3], ss);
      c = fp4_enc<2>(c, s8[4], s8[5], ss);
      c = fp4_enc<3>(c, s8[6], s8[7], ss);
      sc[w] = c;
      float d[8];
      fp4_dec<0>(c, ss, d[0], d[1]);
      fp4_dec<1>(c, ss, d[2], d[3]);
      fp4_dec<2>(c, ss, d[4], d[5]);
      fp4_dec<3>(c, ss, d[6], d[7]);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[8 * w + i] = v[8 * w + i] - d[i];
    }
  }

  float ar = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; i += 2) ar = abs_max3(ar, v[i], v[i + 1]);
  const int er = mx_shared_exp(__float_as_uint(ar));
  const float rs = pow2(er);
  uint32_t rc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t w = fp4_enc<0>(0u, v[8 * j], v[8 * j + 1], rs);
    w = fp4_enc<1>(w, v[8 * j + 2], v[8 * j + 3], rs);
    w = fp4_enc<2>(w, v[8 * j + 4], v[8 * j + 5], rs);
    rc[j] = fp4_enc<3>(w, v[8 * j + 6], v[8 * j + 7], rs);
  }

  Block32 o;
  o.r_codes = make_uint4(rc[0], rc[1], rc[2], rc[3]);
  o.s_codes = make_uint4(sc[0], sc[1], sc[2], sc[3]);
  o.meta = meta;
  o.s_e8 = (uint32_t)(es + 127);
  o.r_e8 = (uint32_t)(er + 127);
  return o;
}

}  // namespace sharq
