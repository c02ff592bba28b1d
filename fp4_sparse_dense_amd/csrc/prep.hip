// Fused SharQ preparation and weight packing for gfx950.
//
// SharQ paper page (mlsanity), Abstract: one preparation operator absorbs the
// normalisation, the input-adaptive N:M mask that extracts the sparse
// backbone, the FP4 quantisation of that backbone, and the residual taken
// against the *quantised* backbone; the residual is then quantised for the
// dense FP4 path.  The README page (sections "Evaluation", "Benchmarks") names
// the fused normalisation RMSNorm.
//
// Outputs are written in the MFMA-tiled layout the GEMM copies with contiguous
// loads (16 rows x 128 K per tile, lane order; see include/sharq.h), padding
// rows and the K tail of the last tile as zeros.
//
// Mapping: one wavefront per activation row.  A row is covered in slots of
// 512 elements; in a slot lane l owns elements [8l, 8l+8) (one 16-byte load),
// so a wave load is 1 KiB contiguous, a 2:4 group never leaves a lane and a
// 32-element MX block spans an aligned quad of lanes.  Up to eight slots are
// loaded before any is processed (8 KiB in flight per wave).  All arithmetic is
// binary32 with no contraction (built with -ffp-contract=off).
#include "device_common.h"
#include "launch.h"

namespace sharq {

constexpr int kSlot = 512;
constexpr int kRegSlots = 8;
constexpr int kRowsPerBlock = 4;

// ss -> 1/sqrt(ss/K + eps), each step correctly rounded to binary32.  The
// quotient and the square root are taken in binary64 and rounded once more to
// binary32; with 53 >= 2*24+2 bits that second rounding equals direct
// correct rounding.
__device__ __forceinline__ float rms_inverse(float ss, int K, float eps) {
  float mean = (float)((double)ss / (double)K);
  float a = mean + eps;
  float root = (float)__dsqrt_rn((double)a);
  return (float)(1.0 / (double)root);
}

// x*x over the lane's eight elements, summed as the balanced tree of those eight.
__device__ __forceinline__ float sq_tree8(uint4 w) {
  float x0 = bf16_lo(w.x), x1 = bf16_hi(w.x), x2 = bf16_lo(w.y), x3 = bf16_hi(w.y);
  float x4 = bf16_lo(w.z), x5 = bf16_hi(w.z), x6 = bf16_lo(w.w), x7 = bf16_hi(w.w);
  return ((x0 * x0 + x1 * x1) + (x2 * x2 + x3 * x3)) + ((x4 * x4 + x5 * x5) + (x6 * x6 + x7 * x7));
}

// Kept offsets i0 < i1 of the two largest magnitudes of a group of four
// (magnitudes as binary32 bit patterns with the sign cleared, so +0 == -0);
// on equal magnitude the lower index wins.
__device__ __forceinline__ void top2of4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, int& i0,
                                        int& i1) {
  // element i beats element k (i < k) iff a_i >= a_k; rank = number of beaters
  int b01 = a0 >= a1, b02 = a0 >= a2, b03 = a0 >= a3;
  int b12 = a1 >= a2, b13 = a1 >= a3, b23 = a2 >= a3;
  int r0 = 3 - b01 - b02 - b03;
  int r1 = b01 + 2 - b12 - b13;
  int r2 = b02 + b12 + 1 - b23;
  int k0 = r0 < 2, k1 = r1 < 2, k2 = r2 < 2;
  i0 = k0 ? 0 : (k1 ? 1 : 2);
  i1 = (k0 + k1 + k2 == 2) ? (k2 ? 2 : 1) : 3;
}

struct Lane8 {
  uint32_t s_codes;  // 4 kept S nibbles (16 bits)
  uint32_t meta;     // 2 metadata nibbles (8 bits)
  uint32_t r_codes;  // 8 R nibbles
  uint32_t s_e8;     // E8M0 of the lane's S block
  uint32_t r_e8;     // E8M0 of the lane's R block
};

// Decompose eight consecutive normalised values of one lane.  Every lane of
// the wave must call this (quad exchanges for the 32-element block maxima).
__device__ __forceinline__ Lane8 decompose8(const float (&v)[8]) {
  uint32_t a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = __float_as_uint(v[i]) & 0x7FFFFFFFu;

  // 2:4 mask
  int ia0, ia1, ib0, ib1;
  top2of4(a[0], a[1], a[2], a[3], ia0, ia1);
  top2of4(a[4], a[5], a[6], a[7], ib0, ib1);

  // S block scale: the block maximum of v is always kept, so amax(S) == amax(v)
  uint32_t am = max(max(max(a[0], a[1]), max(a[2], a[3])), max(max(a[4], a[5]), max(a[6], a[7])));
  am = quad_max_u32(am);
  const int es = mx_shared_exp(am);
  const float qs = pow2_neg(es), ds = pow2(es);

  // kept values in k order
  float sa0 = ia0 == 0 ? v[0] : (ia0 == 1 ? v[1] : v[2]);
  float sa1 = ia1 == 3 ? v[3] : (ia1 == 2 ? v[2] : v[1]);
  float sb0 = ib0 == 0 ? v[4] : (ib0 == 1 ? v[5] : v[6]);
  float sb1 = ib1 == 3 ? v[7] : (ib1 == 2 ? v[6] : v[5]);
  uint32_t sc = fp4_pack2<0>(0u, sa0 * qs, sa1 * qs);
  sc = fp4_pack2<1>(sc, sb0 * qs, sb1 * qs);

  // backbone dequantised (exact) and the residual against it
  float da0, da1, db0, db1;
  fp4_unpack2<0>(sc, da0, da1);
  fp4_unpack2<1>(sc, db0, db1);
  da0 *= ds; da1 *= ds; db0 *= ds; db1 *= ds;
  float r[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    r[k] = k == ia0 ? v[k] - da0 : (k == ia1 ? v[k] - da1 : v[k]);
    r[4 + k] = k == ib0 ? v[4 + k] - db0 : (k == ib1 ? v[4 + k] - db1 : v[4 + k]);
  }

  // R block scale and codes
  uint32_t ar = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) ar = max(ar, __float_as_uint(r[i]) & 0x7FFFFFFFu);
  ar = quad_max_u32(ar);
  const int er = mx_shared_exp(ar);
  const float qr = pow2_neg(er);
  uint32_t rc = fp4_pack2<0>(0u, r[0] * qr, r[1] * qr);
  rc = fp4_pack2<1>(rc, r[2] * qr, r[3] * qr);
  rc = fp4_pack2<2>(rc, r[4] * qr, r[5] * qr);
  rc = fp4_pack2<3>(rc, r[6] * qr, r[7] * qr);

  Lane8 o;
  o.s_codes = sc & 0xFFFFu;
  o.meta = (uint32_t)(ia0 | (ia1 << 2)) | ((uint32_t)(ib0 | (ib1 << 2)) << 4);
  o.r_codes = rc;
  o.s_e8 = (uint32_t)(es + 127);
  o.r_e8 = (uint32_t)(er + 127);
  return o;
}

__device__ __forceinline__ uint4 load16_or_zero(const uint16_t* p, bool ok) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  if (ok) {
    u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
  }
  return make_uint4(0, 0, 0, 0);
}

template <bool NORM>
__global__ __launch_bounds__(256) void prep_kernel(const uint16_t* __restrict__ x, int64_t M, int K,
                                                   int64_t ldx, const uint16_t* __restrict__ gamma,
                                                   float eps, PrepOut o) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int64_t RB = (M + 15) / 16;
  if (row >= RB * 16) return;  // uniform per wave; rows M..RB*16 are zero padding
  const bool row_ok = row < M;
  const int KB = (K + 127) / 128, Kp = KB * 128;
  const int nslot = (K + kSlot - 1) / kSlot;
  const uint16_t* xr = x + (row_ok ? row : 0) * ldx;
  uint4 xb[kRegSlots];
  float inv = 1.0f;

  if (NORM && nslot > kRegSlots) {
    // Long rows: a first pass for the sum of squares.  Lane s keeps slot s's
    // 512-element tree sum; a final lane tree combines the slots in order
    // (lanes beyond the last slot hold +0, i.e. the zero padding).
    float mine = 0.0f;
    for (int c0 = 0; c0 < nslot; c0 += kRegSlots) {
#pragma unroll
      for (int s = 0; s < kRegSlots; ++s) {
        int k = (c0 + s) * kSlot + lane * 8;
        xb[s] = load16_or_zero(xr + k, row_ok && c0 + s < nslot && k < K);
      }
#pragma unroll
      for (int s = 0; s < kRegSlots; ++s) {
        if (c0 + s < nslot) {
          float t = wave_tree_sum(sq_tree8(xb[s]));
          if (lane == c0 + s) mine = t;
        }
      }
    }
    inv = rms_inverse(wave_tree_sum(mine), K, eps);
  }

  for (int c0 = 0; c0 < nslot; c0 += kRegSlots) {
#pragma unroll
    for (int s = 0; s < kRegSlots; ++s) {
      int k = (c0 + s) * kSlot + lane * 8;
      xb[s] = load16_or_zero(xr + k, row_ok && c0 + s < nslot && k < K);
    }
    if (NORM && nslot <= kRegSlots) {
      float mine = 0.0f;
#pragma unroll
      for (int s = 0; s < kRegSlots; ++s) {
        if (s < nslot) {
          float t = wave_tree_sum(sq_tree8(xb[s]));
          if (lane == s) mine = t;
        }
      }
      inv = rms_inverse(wave_tree_sum(mine), K, eps);
    }
#pragma unroll
    for (int s = 0; s < kRegSlots; ++s) {
      const int slot = c0 + s;
      if (slot >= nslot) break;  // uniform
      const int k = slot * kSlot + lane * 8;
      const bool active = k < K;          // real input
      const bool store = k < Kp;          // real input or zero padding of the last K tile
      const uint4 w = xb[s];
      float v[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                    bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
      if (NORM) {
        uint4 g = active ? *reinterpret_cast<const uint4*>(gamma + k) : make_uint4(0, 0, 0, 0);
        float gv[8] = {bf16_lo(g.x), bf16_hi(g.x), bf16_lo(g.y), bf16_hi(g.y),
                       bf16_lo(g.z), bf16_hi(g.z), bf16_lo(g.w), bf16_hi(g.w)};
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (v[i] * inv) * gv[i];
      }
      if (!active || !row_ok) {   // padding is exact zeros whatever inv is (eps = 0, zero row)
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
      }
      const Lane8 d = decompose8(v);
      if (store) {
        // tiled layout: tile (row/16, k/128), tile lane = 16*(32-chunk) + row%16,
        // this lane's 8 elements are quarter q of that tile lane's 32
        const int64_t tile = (row >> 4) * KB + (k >> 7);
        const int tl = ((k >> 5) & 3) * 16 + (int)(row & 15);
        const int q = (k >> 3) & 3;
        *reinterpret_cast<uint32_t*>(o.r_codes + tile * 1024 + tl * 16 + q * 4) = d.r_codes;
        *reinterpret_cast<uint16_t*>(o.s_codes + tile * 512 + (q >> 1) * 256 + tl * 4 + (q & 1) * 2) =
            (uint16_t)d.s_codes;
        o.s_meta[tile * 256 + tl * 4 + q] = (uint8_t)d.meta;
        if (q == 0) {
          const int64_t sc = ((int64_t)(k >> 7) * RB + (row >> 4)) * 64 + tl;
          o.s_scales[sc] = (uint8_t)d.s_e8;
          o.r_scales[sc] = (uint8_t)d.r_e8;
        }
      }
    }
  }
}

// Weight payload: MXFP4 over each 32-block of a row of W, no mask, no norm.
__global__ __launch_bounds__(256) void pack_weight_kernel(const uint16_t* __restrict__ w, int64_t N, int K,
                                                          int64_t ldw, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int64_t NB = (N + 15) / 16;
  if (row >= NB * 16) return;  // rows N..NB*16 are zero padding
  const bool row_ok = row < N;
  const int KB = (K + 127) / 128, Kp = KB * 128;
  const uint16_t* wr = w + (row_ok ? row : 0) * ldw;
  const int nslot = (K + kSlot - 1) / kSlot;
  for (int slot = 0; slot < nslot; ++slot) {
    const int k = slot * kSlot + lane * 8;
    const bool active = row_ok && k < K;
    const uint4 q = active ? *reinterpret_cast<const uint4*>(wr + k) : make_uint4(0, 0, 0, 0);
    float v[8] = {bf16_lo(q.x), bf16_hi(q.x), bf16_lo(q.y), bf16_hi(q.y),
                  bf16_lo(q.z), bf16_hi(q.z), bf16_lo(q.w), bf16_hi(q.w)};
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = max(am, __float_as_uint(v[i]) & 0x7FFFFFFFu);
    am = quad_max_u32(am);
    const int e = mx_shared_exp(am);
    const float qs = pow2_neg(e);
    uint32_t c = fp4_pack2<0>(0u, v[0] * qs, v[1] * qs);
    c = fp4_pack2<1>(c, v[2] * qs, v[3] * qs);
    c = fp4_pack2<2>(c, v[4] * qs, v[5] * qs);
    c = fp4_pack2<3>(c, v[6] * qs, v[7] * qs);
    if (k < Kp) {
      const int64_t tile = (row >> 4) * KB + (k >> 7);
      const int tl = ((k >> 5) & 3) * 16 + (int)(row & 15);
      const int qq = (k >> 3) & 3;
      *reinterpret_cast<uint32_t*>(codes + tile * 1024 + tl * 16 + qq * 4) = c;
      if (qq == 0) scales[((int64_t)(k >> 7) * NB + (row >> 4)) * 64 + tl] = (uint8_t)(e + 127);
    }
  }
}

hipError_t launch_prepare(const uint16_t* x, int64_t M, int K, int64_t ldx, const uint16_t* gamma,
                          float eps, PrepOut out, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int64_t rows = (M + 15) / 16 * 16;   // includes the zero padding rows
  dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(256);
  if (gamma)
    hipLaunchKernelGGL(prep_kernel<true>, grid, block, 0, stream, x, M, K, ldx, gamma, eps, out);
  else
    hipLaunchKernelGGL(prep_kernel<false>, grid, block, 0, stream, x, M, K, ldx, gamma, eps, out);
  return hipGetLastError();
}

hipError_t launch_pack_weight(const uint16_t* w, int64_t N, int K, int64_t ldw, uint8_t* codes,
                              uint8_t* scales, hipStream_t stream) {
  const int64_t rows = (N + 15) / 16 * 16;
  dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(256);
  hipLaunchKernelGGL(pack_weight_kernel, grid, block, 0, stream, w, N, K, ldw, codes, scales);
  return hipGetLastError();
}

}  // namespace sharq
