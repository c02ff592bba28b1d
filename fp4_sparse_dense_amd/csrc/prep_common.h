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
// group_keep evaluates this with lane masks in one asm block (so no mask
// outlives its group), selects the kept values in index order (s0 = first
// kept, s1 = second) and shifts the group's metadata nibble i0 | i1 << 2 into
// `meta` most significant bit first (v_addc doubles and adds the carry-in
// mask).  Its masks go to group_residual, which replaces a kept a_i by
// a_i - dq_i, dq the dequantised kept value (dlo for the first kept, dhi for
// the second); dropped elements keep a_i.
struct Keep { uint64_t k0, k1, k2, k3; };

__device__ __forceinline__ Keep group_keep(float a0, float a1, float a2, float a3, float& s0, float& s1,
                                           uint32_t& meta) {
  Keep k;
  uint64_t b12, e, n, c;
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
      // s0 = k0 ? a0 : (k1 ? a1 : a2);  s1 = k3 ? a3 : (k2 ? a2 : a1)
      "v_cndmask_b32_e64 %[s0], %[a2], %[a1], %[k1]\n\t"
      "v_cndmask_b32_e64 %[s0], %[s0], %[a0], %[k0]\n\t"
      "v_cndmask_b32_e64 %[s1], %[a1], %[a2], %[k2]\n\t"
      "v_cndmask_b32_e64 %[s1], %[s1], %[a3], %[k3]\n\t"
      // nibble bits, high to low: i1 = k3 ? 3 : (k2 ? 2 : 1), i0 = k0 ? 0 : (k1 ? 1 : 2)
      "s_or_b64 %[c], %[k3], %[k2]\n\t"
      "v_addc_co_u32_e64 %[meta], %[e], %[meta], %[meta], %[c]\n\t"
      "s_orn2_b64 %[c], %[k3], %[k2]\n\t"
      "v_addc_co_u32_e64 %[meta], %[e], %[meta], %[meta], %[c]\n\t"
      "s_nor_b64 %[c], %[k0], %[k1]\n\t"
      "v_addc_co_u32_e64 %[meta], %[e], %[meta], %[meta], %[c]\n\t"
      "s_andn2_b64 %[c], %[k1], %[k0]\n\t"
      "v_addc_co_u32_e64 %[meta], %[e], %[meta], %[meta], %[c]"
      : [s0] "=&v"(s0), [s1] "=&v"(s1), [meta] "+v"(meta), [m] "=&v"(m), [k0] "=&s"(k.k0), [k1] "=&s"(k.k1),
        [k2] "=&s"(k.k2), [k3] "=&s"(k.k3), [b12] "=&s"(b12), [e] "=&s"(e), [n] "=&s"(n), [c] "=&s"(c)
      : [a0] "v"(a0), [a1] "v"(a1), [a2] "v"(a2), [a3] "v"(a3)
      : "scc");
  return k;
}

__device__ __forceinline__ void group_residual(float& a0, float& a1, float& a2, float& a3, float dlo, float dhi,
                                               const Keep& k) {
  float t;
  asm volatile(
      "v_sub_f32_e32 %[t], %[a0], %[dlo]\n\t"
      "v_cndmask_b32_e64 %[a0], %[a0], %[t], %[k0]\n\t"
      "v_sub_f32_e32 %[t], %[a3], %[dhi]\n\t"
      "v_cndmask_b32_e64 %[a3], %[a3], %[t], %[k3]\n\t"
      "v_cndmask_b32_e64 %[t], %[dlo], %[dhi], %[k0]\n\t"
      "v_sub_f32_e32 %[t], %[a1], %[t]\n\t"
      "v_cndmask_b32_e64 %[a1], %[a1], %[t], %[k1]\n\t"
      "v_cndmask_b32_e64 %[t], %[dhi], %[dlo], %[k3]\n\t"
      "v_sub_f32_e32 %[t], %[a2], %[t]\n\t"
      "v_cndmask_b32_e64 %[a2], %[a2], %[t], %[k2]"
      : [a0] "+v"(a0), [a1] "+v"(a1), [a2] "+v"(a2), [a3] "+v"(a3), [t] "=&v"(t)
      : [dlo] "v"(dlo), [dhi] "v"(dhi), [k0] "s"(k.k0), [k1] "s"(k.k1), [k2] "s"(k.k2), [k3] "s"(k.k3));
}

__device__ __forceinline__ float abs_max3(float m, float a, float b) {
  return fmaxf(fmaxf(m, fabsf(a)), fabsf(b));
}

// Encode two values as E2M1 into byte SEL of `old`, dividing by the power of
// two `scale` inside the convert, and decode byte SEL of `packed` multiplied
// by `scale`.  Both were checked exact against the rounding rule (encode:
// every binary32 in a 2^17 window around each scale, scales 2^-127..2^125;
// decode: every code byte at the same scales).
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

// Group G of a block: mask, kept codes into byte G%4 of `codes`, metadata,
// residual in place.
template <int G>
__device__ __forceinline__ void group4(float (&v)[32], float s_scale, uint32_t& codes, uint32_t& meta) {
  float s0, s1, dlo, dhi;
  const Keep k = group_keep(v[4 * G], v[4 * G + 1], v[4 * G + 2], v[4 * G + 3], s0, s1, meta);
  codes = fp4_enc<G % 4>(codes, s0, s1, s_scale);
  fp4_dec<G % 4>(codes, s_scale, dlo, dhi);
  group_residual(v[4 * G], v[4 * G + 1], v[4 * G + 2], v[4 * G + 3], dlo, dhi, k);
}

// The whole decomposition of one MX block; v is replaced by the residual.
// DENSE (the plain FP4 linear, no backbone): the residual is v itself and
// only its MXFP4 codes are produced.
template <bool DENSE>
__device__ __forceinline__ Block32 decompose32(float (&v)[32]) {
  uint32_t lo = 0, hi = 0, meta = 0;
  int es = -127;
  if constexpr (!DENSE) {
    // S block scale: the block maximum of v is always kept, so amax(S) == amax(v)
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; i += 2) am = abs_max3(am, v[i], v[i + 1]);
    es = mx_shared_exp(__float_as_uint(am));
    const float ss = pow2(es);

    // groups last to first: the metadata nibbles enter most significant first
    group4<7>(v, ss, hi, meta);
    group4<6>(v, ss, hi, meta);
    group4<5>(v, ss, hi, meta);
    group4<4>(v, ss, hi, meta);
    group4<3>(v, ss, lo, meta);
    group4<2>(v, ss, lo, meta);
    group4<1>(v, ss, lo, meta);
    group4<0>(v, ss, lo, meta);
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
  o.s_codes = DENSE ? make_uint4(0, 0, 0, 0) : expand_chunk(lo, hi, meta);
  o.meta = meta;
  o.s_e8 = (uint32_t)(es + 127);
  o.r_e8 = (uint32_t)(er + 127);
  return o;
}

}  // namespace sharq
