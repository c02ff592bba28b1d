// SharQ layer in the NVFP4-style format for gfx950: preparation, weight
// packing and the dual GEMM.
//
// SharQ paper page (mlsanity), Abstract: the method is reported under NVFP4 as
// well as MXFP4 and HiF4.  The pages do not define NVFP4; this file follows
// the public two-level NVFP4 description: E2M1 elements in 16-element blocks,
// an OCP E4M3 block scale, and one binary32 scale per tensor
//   g = amax(tensor) / 2688   (2688 = 6 * 448; g = 1 for an all-zero tensor)
//   s = E4M3(amax(block) / (6 g)), round to nearest even, saturating at 448
//   code = E2M1(u / (s g))  (the signed zero code when s = 0)
// with every step one binary32 operation, rounded once (built with
// -ffp-contract=off and IEEE division).  Backbone S, residual R and weight W
// each have their own tensor scale; R's depends on Q(S), so the preparation
// runs as three launches: per-row statistics, the backbone (and max |R|), the
// residual.
//
// gfx950's block-scaled MFMA takes E8M0 scales per 32 elements, which cannot
// carry an E4M3 scale per 16.  The GEMM therefore expands each code to
// val(code) * s -- at most 6 significant bits in [2^-10, 2688], so exact in
// fp16 -- and runs the fp16 MFMA with one fp32 accumulator per path; the
// tensor scales enter once, in the epilogue: y = g_S g_W acc_S + g_R g_W acc_R.
#include <atomic>

#include "device_common.h"
#include "e4m3.h"
#include "launch.h"

namespace sharq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

constexpr float kNvTensorDiv = 2688.0f;
constexpr int kNvWaves = 4;          // one K tile per wave, 4 per workgroup

__device__ __forceinline__ float tensor_scale(float amax) { return amax > 0.0f ? amax / kNvTensorDiv : 1.0f; }

// E2M1 nibble of binary32 q (round to nearest even, saturating at 6, sign of
// zero kept): the convert instruction with unit scale.
__device__ __forceinline__ uint32_t e2m1_pair(float lo, float hi) { return fp4_pack2<0>(0u, lo, hi) & 0xFFu; }

// Element quotient u / (s g) (IEEE division), or a signed zero when the block
// scale is zero.  Both sides are computed and selected, so the lanes of a wave
// never diverge around the division.
__device__ __forceinline__ float nv_quot(float u, float tq, float s) {
  const float q = u / tq;
  return s > 0.0f ? q : u * 0.0f;
}

struct NvPrepArgs {
  const uint16_t* x;
  int64_t M, ldx;
  int K;
  const uint16_t* gamma;
  float eps;
  int64_t RB;
  int KB, WX;
  PrepOut o;
  float* g_s;       // tensor scale of S (s_scales record)
  float* g_r;       // tensor scale of R (r_scales record)
  float* rowamax;   // [RB*16] max |v| of each row
  float* inv;       // [RB*16] 1/rms of each row
  float* rparts;    // [RB*WX] max |r| of each workgroup
};

// ---------------------------------------------------------------------------
// Phase 1: one workgroup per row.  With RMSNorm, the sum of squares follows
// the pairwise tree over the row zero-padded to a power of two: aligned
// 32-element chunks are subtrees, and the chunk sums are combined pairwise in
// LDS.  Writes 1/rms (when normalising) and max |v| of the row.
// ---------------------------------------------------------------------------
template <bool NORM>
__global__ __launch_bounds__(256) void nv_rowstats_kernel(NvPrepArgs a) {
  __shared__ float cs[1024];
  __shared__ float red[4];
  const int t = threadIdx.x;
  const int64_t row = blockIdx.x;
  const uint16_t* xr = a.x + row * a.ldx;
  const int KC = a.K / 32;
  const float inv = NORM ? row_inv_rms(xr, a.K, a.eps, cs) : 1.0f;
  float am = 0.0f;
  for (int c = t; c < KC; c += 256) {
    float v[32];
    load32(xr + 32 * c, v);
    if (NORM) apply_norm(v, a.gamma + 32 * c, inv);
#pragma unroll
    for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(v[i]));
  }
  am = block_max<4>(am, red);
  if (t == 0) {
    a.rowamax[row] = am;
    if (NORM) a.inv[row] = inv;
  }
}

// 2:4 mask of one group a0..a3: element i is kept iff at most one other
// element beats it (larger magnitude, or equal magnitude and lower index).
// The first kept element is i0 (never 3), the second i1 (never 0); the
// metadata nibble is i0 | i1 << 2.  Only fixed register indices are used.
struct Keep24 {
  bool f1, f2;       // element 1 / 2 is the first kept one (element 0 is iff k0)
  bool s1, s2;       // element 1 / 2 is the second kept one (element 3 is iff k3)
  bool k0, k3;
  uint32_t nib;
};
__device__ __forceinline__ Keep24 keep24(float a0, float a1, float a2, float a3) {
  const float m0 = fabsf(a0), m1 = fabsf(a1), m2 = fabsf(a2), m3 = fabsf(a3);
  const int b01 = m0 >= m1, b02 = m0 >= m2, b03 = m0 >= m3, b12 = m1 >= m2, b13 = m1 >= m3, b23 = m2 >= m3;
  Keep24 k;
  k.k0 = (3 - b01 - b02 - b03) <= 1;
  const bool k1 = (b01 + 2 - b12 - b13) <= 1;
  const bool k2 = (b02 + b12 + 1 - b23) <= 1;
  k.k3 = (b03 + b13 + b23) <= 1;
  k.f1 = !k.k0 && k1;
  k.f2 = !k.k0 && !k1;
  k.s1 = !k.k3 && !k2;
  k.s2 = !k.k3 && k2;
  const uint32_t i0 = k.k0 ? 0u : (k1 ? 1u : 2u);
  const uint32_t i1 = k.k3 ? 3u : (k2 ? 2u : 1u);
  k.nib = i0 | (i1 << 2);
  return k;
}

// One lane's 32 elements (two 16-element blocks) of v: the 2:4 mask, the
// E4M3 block scales and the kept codes of the backbone (tensor scale g_s); v
// is replaced by the residual r = v - deq(Q(S)).
// One 16-element block v[0..16) of the backbone: its E4M3 scale byte, the 8
// kept codes (first kept element of group g in bits 8g..8g+3, second in
// 8g+4..8g+7), the 4 groups' metadata nibbles (bits 4g..4g+3); v becomes the
// residual.
__device__ __forceinline__ void nv_backbone_block(float* v, float g_s, uint32_t& scode, uint32_t& meta16,
                                                  uint32_t& sbyte) {
  const float six_g = 6.0f * g_s;
  float bm = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) bm = fmaxf(bm, fabsf(v[i]));
  const float s = e4m3_round(bm / six_g, sbyte);
  const float tq = s * g_s;
  scode = 0u;
  meta16 = 0u;
#pragma unroll
  for (int gq = 0; gq < 4; ++gq) {
    float& a0 = v[4 * gq];
    float& a1 = v[4 * gq + 1];
    float& a2 = v[4 * gq + 2];
    float& a3 = v[4 * gq + 3];
    const Keep24 k = keep24(a0, a1, a2, a3);
    meta16 |= k.nib << (4 * gq);
    const float x0 = k.k0 ? a0 : (k.f1 ? a1 : a2);
    const float x1 = k.k3 ? a3 : (k.s2 ? a2 : a1);
    const float q0 = nv_quot(x0, tq, s), q1 = nv_quot(x1, tq, s);
    const uint32_t c = e2m1_pair(q0, q1);
    scode |= c << (8 * gq);
    float d0, d1;
    fp4_unpack2<0>(c, d0, d1);
    d0 = (d0 * s) * g_s;
    d1 = (d1 * s) * g_s;
    const float r0 = x0 - d0, r1 = x1 - d1;
    a0 = k.k0 ? r0 : a0;
    a1 = k.f1 ? r0 : (k.s1 ? r1 : a1);
    a2 = k.f2 ? r0 : (k.s2 ? r1 : a2);
    a3 = k.k3 ? r1 : a3;
  }
}

// The backbone of a 32-element chunk: its two 16-element blocks.
__device__ __forceinline__ void nv_backbone(float (&v)[32], float g_s, uint32_t (&scodes)[2], uint32_t& meta,
                                            uint32_t& sbytes) {
  meta = 0u;
  sbytes = 0u;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    uint32_t m16, byte;
    nv_backbone_block(v + 16 * b, g_s, scodes[b], m16, byte);
    meta |= m16 << (16 * b);
    sbytes |= byte << (8 * b);
  }
}

// One 16-element block of the residual: its E4M3 scale byte and 16 codes
// (element i in bits 4(i % 8).. of word i / 8).
__device__ __forceinline__ void nv_residual_block(const float* v, float g_r, uint32_t (&rc)[2], uint32_t& rbyte) {
  const float six_r = 6.0f * g_r;
  float bm = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) bm = fmaxf(bm, fabsf(v[i]));
  const float s = e4m3_round(bm / six_r, rbyte);
  const float tq = s * g_r;
  rc[0] = rc[1] = 0u;
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    const float q0 = nv_quot(v[i], tq, s), q1 = nv_quot(v[i + 1], tq, s);
    rc[i / 8] |= e2m1_pair(q0, q1) << (4 * (i % 8));
  }
}

__device__ __forceinline__ void nv_residual(const float (&v)[32], float g_r, uint32_t (&rc)[4], uint32_t& rbytes) {
  rbytes = 0u;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    uint32_t w[2], byte;
    nv_residual_block(v + 16 * b, g_r, w, byte);
    rc[2 * b] = w[0];
    rc[2 * b + 1] = w[1];
    rbytes |= byte << (8 * b);
  }
}

// ---------------------------------------------------------------------------
// Quarter-chunk forms of the two steps: one lane per 8 consecutive elements
// of a 32-element chunk (half of a 16-element block; the chunk's quarters in
// lanes 4j .. 4j+3 of one wave, so a block's two halves sit in lanes l and
// l ^ 1).  The arithmetic is nv_backbone's and nv_residual's; a block maximum
// is the larger of the two halves' maxima, exchanged between the two lanes,
// and a lane's dependent chain is a quarter as long.  Every lane of a wave
// must call them (the exchange).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float pair_max(float v) { return fmaxf(v, __shfl_xor(v, 1)); }

// The backbone of a quarter: dense = its 8 S codes in the masked dense layout
// (the kept codes in place, zero codes at the dropped positions; element i in
// bits 4i..4i+3), meta8 = its two groups' metadata nibbles (group g in bits
// 4g..4g+3), sbyte = the block's E4M3 scale byte; v becomes the residual.
__device__ __forceinline__ void nv_backbone_q(float (&v)[8], float g_s, uint32_t& dense, uint32_t& meta8,
                                              uint32_t& sbyte) {
  const float six_g = 6.0f * g_s;
  float bm = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) bm = fmaxf(bm, fabsf(v[i]));
  bm = pair_max(bm);
  const float s = e4m3_round(bm / six_g, sbyte);
  const float tq = s * g_s;
  dense = 0u;
  meta8 = 0u;
#pragma unroll
  for (int gq = 0; gq < 2; ++gq) {
    float& a0 = v[4 * gq];
    float& a1 = v[4 * gq + 1];
    float& a2 = v[4 * gq + 2];
    float& a3 = v[4 * gq + 3];
    const Keep24 k = keep24(a0, a1, a2, a3);
    meta8 |= k.nib << (4 * gq);
    const float x0 = k.k0 ? a0 : (k.f1 ? a1 : a2);
    const float x1 = k.k3 ? a3 : (k.s2 ? a2 : a1);
    const float q0 = nv_quot(x0, tq, s), q1 = nv_quot(x1, tq, s);
    const uint32_t c = e2m1_pair(q0, q1);
    const uint32_t i0 = k.nib & 3u, i1 = k.nib >> 2;
    dense |= ((c & 0xFu) << (16 * gq + 4 * i0)) | ((c >> 4) << (16 * gq + 4 * i1));
    float d0, d1;
    fp4_unpack2<0>(c, d0, d1);
    d0 = (d0 * s) * g_s;
    d1 = (d1 * s) * g_s;
    const float r0 = x0 - d0, r1 = x1 - d1;
    a0 = k.k0 ? r0 : a0;
    a1 = k.f1 ? r0 : (k.s1 ? r1 : a1);
    a2 = k.f2 ? r0 : (k.s2 ? r1 : a2);
    a3 = k.k3 ? r1 : a3;
  }
}

// The residual codes of a quarter (element i in bits 4i..4i+3) and its
// block's E4M3 scale byte.
__device__ __forceinline__ void nv_residual_q(const float (&v)[8], float g_r, uint32_t& rc, uint32_t& rbyte) {
  const float six_r = 6.0f * g_r;
  float bm = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) bm = fmaxf(bm, fabsf(v[i]));
  bm = pair_max(bm);
  const float s = e4m3_round(bm / six_r, rbyte);
  const float tq = s * g_r;
  rc = 0u;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const float q0 = nv_quot(v[i], tq, s), q1 = nv_quot(v[i + 1], tq, s);
    rc |= e2m1_pair(q0, q1) << (4 * i);
  }
}

// 8 bf16 -> binary32
__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    v[2 * h] = bf16_lo(w[h]);
    v[2 * h + 1] = bf16_hi(w[h]);
  }
}

// ---------------------------------------------------------------------------
// Phases 2 and 3: one workgroup of 16 waves per 4 tiles (16 rows x 128 K
// each) of one row block; the four quarters of a chunk in four consecutive
// lanes, chunk lane l = (t % 256) / 4 owning row 16 rb + l%16 and K
// [128 kb + 32 (l/16), +32) -- the lane order of the tiled layout.  Both
// phases rebuild v, the mask, Q(S) and the residual; phase 2 stores the
// backbone and each workgroup's max |r|, phase 3 quantises R with the tensor
// scale those maxima give.
// ---------------------------------------------------------------------------
constexpr int kNvPrepThreads = 256 * kNvWaves;
constexpr int64_t kNvSelfScanElems = 65536;   // X small enough for every phase-2 workgroup to scan

// SELF (phase 2 without RMSNorm, small tensors): max |v| = max |x| is taken
// over the whole of X by every workgroup itself, with no per-row phase before.
template <bool NORM, bool RESID, bool SELF = false>
__global__ __launch_bounds__(kNvPrepThreads) void nv_decompose_kernel(NvPrepArgs a) {
  static_assert(!SELF || (!NORM && !RESID), "the whole-tensor scan stands in for phase 1 without RMSNorm");
  __shared__ float red[kNvPrepThreads / 64];
  constexpr int NW = kNvPrepThreads / 64;
  const int t = threadIdx.x, u = t & 255, l = u >> 2, h = u & 3;
  const int64_t rb = blockIdx.y;
  const int kb = blockIdx.x * kNvWaves + (t >> 8);

  // tensor scales: g_S from max |v| (max |S| = max |v|: the mask keeps each
  // group's largest magnitude) -- phase 2 reduces the rows' maxima (or scans
  // X), phase 3 reads the g_S phase 2 stored -- and g_R from phase 2's maxima
  float g_s;
  if constexpr (RESID) {
    g_s = *a.g_s;
  } else {
    float am = 0.0f;
    if constexpr (SELF) {
      const int k8 = a.K / 8;
      for (int64_t j = t; j < a.M * k8; j += kNvPrepThreads) {
        float v8[8];
        load8(a.x + (j / k8) * a.ldx + 8 * (j % k8), v8);
#pragma unroll
        for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v8[i]));
      }
    } else {
      for (int64_t i = t; i < a.M; i += kNvPrepThreads) am = fmaxf(am, a.rowamax[i]);
    }
    g_s = tensor_scale(block_max<NW>(am, red));
  }
  float g_r = 1.0f;
  if (RESID) {
    float ar = 0.0f;
    for (int64_t i = t; i < a.RB * a.WX; i += kNvPrepThreads) ar = fmaxf(ar, a.rparts[i]);
    g_r = tensor_scale(block_max<NW>(ar, red));
  }

  const int64_t row = rb * 16 + (l & 15);
  const int k0 = kb * 128 + 32 * (l >> 4) + 8 * h;
  const bool valid = kb < a.KB && row < a.M && k0 < a.K;
  float v[8];
  if (valid) {
    load8(a.x + row * a.ldx + k0, v);
    if (NORM) {
      const float iv = a.inv[row];
      float gm[8];
      load8(a.gamma + k0, gm);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (v[i] * iv) * gm[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }

  // backbone: mask, per-16 block scale, kept codes; residual in place
  uint32_t dense, meta8, sbyte;
  nv_backbone_q(v, g_s, dense, meta8, sbyte);
  const int64_t tile = rb * a.KB + kb;
  const int64_t sc = ((int64_t)kb * a.RB + rb) * 128 + 2 * l + (h >> 1);

  if (!RESID) {
    if (kb < a.KB) {
      *reinterpret_cast<uint32_t*>(a.o.s_codes + tile * 1024 + l * 16 + h * 4) = dense;
      a.o.s_meta[tile * 256 + l * 4 + h] = (uint8_t)meta8;
      if (!(h & 1)) a.o.s_scales[sc] = (uint8_t)sbyte;
    }
    float ar = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ar = fmaxf(ar, fabsf(v[i]));
    ar = block_max<NW>(ar, red);
    if (t == 0) a.rparts[rb * a.WX + blockIdx.x] = ar;
    if (t == 0 && blockIdx.x == 0 && blockIdx.y == 0) *a.g_s = g_s;
  } else {
    uint32_t rc, rbyte;
    nv_residual_q(v, g_r, rc, rbyte);
    if (kb < a.KB) {
      *reinterpret_cast<uint32_t*>(a.o.r_codes + tile * 1024 + l * 16 + h * 4) = rc;
      if (!(h & 1)) a.o.r_scales[sc] = (uint8_t)rbyte;
    }
    if (t == 0 && blockIdx.x == 0 && blockIdx.y == 0) *a.g_r = g_r;
  }
}

// ---------------------------------------------------------------------------
// Weight packing: max |w| per workgroup, the tensor scale, then the codes.
// Same tile / lane mapping as the preparation (16 weight rows per tile).
// ---------------------------------------------------------------------------
struct NvWeightArgs {
  const uint16_t* w;
  int64_t N, ldw;
  int K;
  int64_t NB;
  int KB, WX;
  uint8_t* codes;
  uint8_t* scales;
  float* g;
  float* parts;
};

__global__ __launch_bounds__(256) void nv_weight_amax_kernel(NvWeightArgs a) {
  __shared__ float red[4];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t nb = blockIdx.y;
  const int kb = blockIdx.x * kNvWaves + wave;
  const int64_t row = nb * 16 + (lane & 15);
  const int k0 = kb * 128 + 32 * (lane >> 4);
  float am = 0.0f;
  if (kb < a.KB && row < a.N && k0 < a.K) {
    float v[32];
    load32(a.w + row * a.ldw + k0, v);
#pragma unroll
    for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(v[i]));
  }
  am = block_max<4>(am, red);
  if (t == 0) a.parts[nb * a.WX + blockIdx.x] = am;
}

__global__ __launch_bounds__(256) void nv_weight_scale_kernel(NvWeightArgs a) {
  __shared__ float red[4];
  float am = 0.0f;
  for (int64_t i = threadIdx.x; i < a.NB * a.WX; i += 256) am = fmaxf(am, a.parts[i]);
  am = block_max<4>(am, red);
  if (threadIdx.x == 0) *a.g = tensor_scale(am);
}

__global__ __launch_bounds__(256) void nv_pack_weight_kernel(NvWeightArgs a) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t nb = blockIdx.y;
  const int kb = blockIdx.x * kNvWaves + wave;
  if (kb >= a.KB) return;
  const int64_t row = nb * 16 + (lane & 15);
  const int k0 = kb * 128 + 32 * (lane >> 4);
  float v[32];
  if (row < a.N && k0 < a.K) {
    load32(a.w + row * a.ldw + k0, v);
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = 0.0f;
  }
  const float g = *a.g, six_g = 6.0f * g;
  uint32_t c[4] = {0u, 0u, 0u, 0u}, bytes = 0u;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float bm = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) bm = fmaxf(bm, fabsf(v[16 * b + i]));
    uint32_t byte;
    const float s = e4m3_round(bm / six_g, byte);
    bytes |= byte << (8 * b);
    const float tq = s * g;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float x0 = v[16 * b + i], x1 = v[16 * b + i + 1];
      const float q0 = nv_quot(x0, tq, s), q1 = nv_quot(x1, tq, s);
      const int e = 16 * b + i;
      c[e / 8] |= e2m1_pair(q0, q1) << (4 * (e % 8));
    }
  }
  const int64_t tile = nb * a.KB + kb;
  *reinterpret_cast<uint4*>(a.codes + tile * 1024 + lane * 16) = make_uint4(c[0], c[1], c[2], c[3]);
  *reinterpret_cast<uint16_t*>(a.scales + ((int64_t)kb * a.NB + nb) * 128 + 2 * lane) = (uint16_t)bytes;
}

// ---------------------------------------------------------------------------
// Dual GEMM (small M: decode).  As the MXFP4 small-M kernel: one workgroup per
// CBG 16-column blocks of the weight (and per group of RBG 16-row activation
// blocks), NW waves split K, operands read straight from the tiled layout.
// Each lane's 32 codes of a K tile are expanded to val * s in fp16 and feed
// four 16x16x32 fp16 MFMAs; MFMA j takes elements [8j, 8j+8) of every lane
// for both operands, so A and B see the same K order.  The expansion is
// exact: val (E2M1) has at most 2 significant bits and s (E4M3) at most 4, so
// val * s has at most 6 and lies in [2^-10, 2688] or is a signed zero -- all
// fp16 normals.  The convert yields the fp16 pair of codes and one packed
// fp16 multiply applies s.
// ---------------------------------------------------------------------------
template <int SEL>
__device__ __forceinline__ f16x2 deq_pair(uint32_t codes, f16x2 s) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, SEL) * s;
}

__device__ __forceinline__ f16x8 deq8(uint32_t codes, f16x2 s) {
  const f16x2 p0 = deq_pair<0>(codes, s), p1 = deq_pair<1>(codes, s);
  const f16x2 p2 = deq_pair<2>(codes, s), p3 = deq_pair<3>(codes, s);
  const auto lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  const auto hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// 32 codes (uint4) + two E4M3 bytes -> four MFMA operands
__device__ __forceinline__ void deq32(uint4 q, uint32_t sb, f16x8 (&o)[4]) {
  const _Float16 h0 = (_Float16)e4m3_value(sb & 0xFFu), h1 = (_Float16)e4m3_value((sb >> 8) & 0xFFu);
  const f16x2 s0 = {h0, h0}, s1 = {h1, h1};
  o[0] = deq8(q.x, s0);
  o[1] = deq8(q.y, s0);
  o[2] = deq8(q.z, s1);
  o[3] = deq8(q.w, s1);
}

__device__ __forceinline__ v4f mfma_f16(f16x8 a, f16x8 b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void store_y(const GemmArgs& g, int64_t row, int64_t col, float v) {
  if (g.out_bf16) {
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFu + ((u >> 16) & 1u);
    reinterpret_cast<uint16_t*>(g.y)[row * g.ldy + col] = (uint16_t)(u >> 16);
  } else {
    reinterpret_cast<float*>(g.y)[row * g.ldy + col] = v;
  }
}

template <int RBG, int NW, int CBG = 1>
__global__ __launch_bounds__(64 * NW) void nv_dual_gemm_kernel(GemmArgs g) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & (NW - 1);
  const int64_t RB = g.a_blocks, NB = (g.N + 15) / 16;
  const int KT = (g.K + 127) / 128;
  const int64_t nb0 = (int64_t)blockIdx.x * CBG;
  const int64_t rb0 = (int64_t)blockIdx.y * RBG;

  v4f acs[CBG][RBG], acr[CBG][RBG];
#pragma unroll
  for (int n = 0; n < CBG; ++n)
#pragma unroll
    for (int r = 0; r < RBG; ++r) acs[n][r] = acr[n][r] = (v4f){0.f, 0.f, 0.f, 0.f};

  constexpr int CH = (RBG == 1 ? 8 : (RBG == 2 ? 4 : 2)) * 4 / NW;
  for (int base = 0; base < KT; base += NW * CH) {
    uint4 wq[CH][CBG], rq[CH][RBG], sq[CH][RBG];
    uint32_t wsb[CH][CBG], ssb[CH][RBG], rsb[CH][RBG];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      // clamped tile index; a tile past K gets a zero weight fragment
      const int kt = base + wave + NW * c;
      const int ktc = kt < KT ? kt : KT - 1;
#pragma unroll
      for (int n = 0; n < CBG; ++n) {
        const int64_t nb = nb0 + n < NB ? nb0 + n : NB - 1;   // past N: only feeds columns never stored
        wq[c][n] = *reinterpret_cast<const uint4*>(g.w_codes + (nb * KT + ktc) * 1024 + lane * 16);
        wsb[c][n] = *reinterpret_cast<const uint16_t*>(g.w_scales_dense + ((int64_t)ktc * NB + nb) * 128 + 2 * lane);
        if (kt >= KT) { wq[c][n] = make_uint4(0, 0, 0, 0); wsb[c][n] = 0u; }
      }
#pragma unroll
      for (int r = 0; r < RBG; ++r) {
        const int64_t rb = rb0 + r < RB ? rb0 + r : RB - 1;
        const int64_t tile = rb * KT + ktc;
        const int64_t sc = ((int64_t)ktc * RB + rb) * 128 + 2 * lane;
        rq[c][r] = *reinterpret_cast<const uint4*>(g.r_codes + tile * 1024 + lane * 16);
        sq[c][r] = *reinterpret_cast<const uint4*>(g.s_codes + tile * 1024 + lane * 16);
        ssb[c][r] = *reinterpret_cast<const uint16_t*>(g.s_scales + sc);
        rsb[c][r] = *reinterpret_cast<const uint16_t*>(g.r_scales + sc);
      }
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if constexpr (RBG == 1 && NW == 16) {
        // one row block on 16 waves: both paths' operands expanded once, then
        // each weight block in turn (fewer live registers than every weight
        // block at once, for four waves per SIMD; every accumulator sees its
        // MFMAs in the same order)
        f16x8 xs[4], xr[4];
        deq32(sq[c][0], ssb[c][0], xs);
        deq32(rq[c][0], rsb[c][0], xr);
#pragma unroll
        for (int n = 0; n < CBG; ++n) {
          f16x8 b[4];
          deq32(wq[c][n], wsb[c][n], b);
#pragma unroll
          for (int j = 0; j < 4; ++j) acs[n][0] = mfma_f16(xs[j], b[j], acs[n][0]);
#pragma unroll
          for (int j = 0; j < 4; ++j) acr[n][0] = mfma_f16(xr[j], b[j], acr[n][0]);
        }
        continue;
      }
      f16x8 b[CBG][4];
#pragma unroll
      for (int n = 0; n < CBG; ++n) deq32(wq[c][n], wsb[c][n], b[n]);
#pragma unroll
      for (int r = 0; r < RBG; ++r) {
        f16x8 x[4];
        deq32(sq[c][r], ssb[c][r], x);
#pragma unroll
        for (int n = 0; n < CBG; ++n)
#pragma unroll
          for (int j = 0; j < 4; ++j) acs[n][r] = mfma_f16(x[j], b[n][j], acs[n][r]);
        deq32(rq[c][r], rsb[c][r], x);
#pragma unroll
        for (int n = 0; n < CBG; ++n)
#pragma unroll
          for (int j = 0; j < 4; ++j) acr[n][r] = mfma_f16(x[j], b[n][j], acr[n][r]);
      }
    }
  }

  // tensor scales once per path, then the waves' partial sums in wave order
  // (column block n of the group by wave n mod NW)
  const float gw = *g.g_w;
  const float fs = *g.g_s * gw, fr = *g.g_r * gw;
  __shared__ v4f part[NW][CBG][RBG][64];
#pragma unroll
  for (int n = 0; n < CBG; ++n)
#pragma unroll
    for (int r = 0; r < RBG; ++r) {
      v4f p;
#pragma unroll
      for (int q = 0; q < 4; ++q) p[q] = fs * acs[n][r][q] + fr * acr[n][r][q];
      part[wave][n][r][lane] = p;
    }
  __syncthreads();
#pragma unroll
  for (int n = 0; n < CBG; ++n) {
    if (wave != n % NW) continue;
    const int64_t col = (nb0 + n) * 16 + (lane & 15);
#pragma unroll
    for (int r = 0; r < RBG; ++r) {
      v4f v = part[0][n][r][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) v = v + part[w][n][r][lane];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = (rb0 + r) * 16 + 4 * (lane >> 4) + q;
        if (row < g.M && col < g.N) store_y(g, row, col, v[q]);
      }
    }
  }
}


// ---------------------------------------------------------------------------
// The NVFP4-style layer in one launch for small M (decode: M <= 16).  The
// activation tensor is the M rows, so every workgroup of the weight-streaming
// GEMM can compute its tensor scales itself: it prepares the rows into LDS --
// the RMSNorm tree, max |v| (g_S), the backbone and max |r| (g_R), the
// residual codes, the three phases of the preparation above with the same
// arithmetic -- and then runs the small-M GEMM's split-K loop (one row block,
// eight waves) on those operands.  Outputs are identical to the preparation
// followed by the GEMM.
// ---------------------------------------------------------------------------
constexpr int kNvFusedWaves = 8;
constexpr int kNvFusedThreads = 64 * kNvFusedWaves;

struct NvFusedArgs {
  const uint16_t* x;
  int64_t ldx;
  int M, K;
  const uint16_t* gamma;   // nullptr: no RMSNorm
  float eps;
  GemmArgs g;              // weight (codes, scales, g_w), output, N
  PrepOut out;             // the preparation alone: the prepared activation (one row block)
  float *g_s_out, *g_r_out;
};

struct NvFusedLds {
  uint32_t s, r, ss, rs, inv, red, total;   // byte offsets (the RMSNorm tree uses the R region first)
  int KT, KC, P;
};

__host__ __device__ inline NvFusedLds nv_fused_lds(int K, int waves = kNvFusedWaves) {
  NvFusedLds L;
  L.KT = (K + 127) / 128;
  L.KC = K / 32;
  L.P = 1;
  while (L.P < L.KC) L.P *= 2;
  L.s = 0;
  L.r = L.s + (uint32_t)L.KT * 1024;
  L.ss = L.r + (uint32_t)L.KT * 1024;
  L.rs = L.ss + (uint32_t)L.KT * 128;
  L.inv = L.rs + (uint32_t)L.KT * 128;
  L.red = L.inv + 16 * 4;
  L.total = L.red + waves * 4;
  // after the GEMM loop the waves' partial sums (8 x 64 x 16 B) reuse the LDS from offset 0
  const uint32_t parts = (uint32_t)kNvFusedWaves * 64u * 16u;
  if (L.total < parts) L.total = parts;
  return L;
}

// SMALL (at most kNvSmallChunks 32-element chunks of the rows per thread):
// each thread loads its chunks of X and gamma once, then requests the weight's
// first split-K pass (loads retire in issue order: the rows first), and keeps
// v and then the residual in registers across the phases; otherwise every
// phase re-reads its chunks and rebuilds the backbone.  Same arithmetic.
constexpr int kNvSmallChunks = 2;

// PREP: the preparation alone (one workgroup; M <= 16, so one row block): the
// same three phases into LDS, then the tiles, the metadata and the tensor
// scales go to the activation's buffers instead of feeding the GEMM.
template <bool NORM, bool SMALL, bool PREP = false, int NT = kNvFusedThreads>
__global__ __launch_bounds__(NT) void nv_fused_layer_kernel(NvFusedArgs a) {
  constexpr int kNvFusedThreads = NT, kNvFusedWaves = NT / 64;   // this instantiation's workgroup
  extern __shared__ __align__(16) uint8_t smem[];
  const NvFusedLds L = nv_fused_lds(a.K, kNvFusedWaves);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6) & (kNvFusedWaves - 1);
  float* inv = reinterpret_cast<float*>(smem + L.inv);
  float* red = reinterpret_cast<float*>(smem + L.red);
  const int nq = a.M * L.KC;   // 32-element chunks of the rows
  const GemmArgs& g = a.g;
  const int KT = L.KT;
  const int64_t NB = (g.N + 15) / 16, nb = blockIdx.x;
  constexpr int CH = 8 * 4 / kNvFusedWaves;
  // weight fragments of one split-K pass (a tile past K gets zeros)
  auto load_w = [&](int base, uint4 (&wq)[CH], uint32_t (&wsb)[CH]) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int kt = base + wave + kNvFusedWaves * c;
      const int ktc = kt < KT ? kt : KT - 1;
      wq[c] = *reinterpret_cast<const uint4*>(g.w_codes + (nb * KT + ktc) * 1024 + lane * 16);
      wsb[c] = *reinterpret_cast<const uint16_t*>(g.w_scales_dense + ((int64_t)ktc * NB + nb) * 128 + 2 * lane);
      if (kt >= KT) { wq[c] = make_uint4(0, 0, 0, 0); wsb[c] = 0u; }
    }
  };
  uint4 wq0[CH];
  uint32_t wsb0[CH];
  float g_s, g_r;

  if constexpr (SMALL) {
    // ---- chunk q = t + kNvFusedThreads * i: X and gamma as loaded, then the weight
    uint4 xr[kNvSmallChunks][4], gr[kNvSmallChunks][4];
#pragma unroll
    for (int i = 0; i < kNvSmallChunks; ++i) {
      const int q = t + kNvFusedThreads * i;
      if (q < nq) {
        const int r = q / L.KC, c = q % L.KC;
        const uint4* px = reinterpret_cast<const uint4*>(a.x + (int64_t)r * a.ldx + 32 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) xr[i][e] = px[e];
        if (NORM) {
          const uint4* pg = reinterpret_cast<const uint4*>(a.gamma + 32 * c);
#pragma unroll
          for (int e = 0; e < 4; ++e) gr[i][e] = pg[e];
        }
      }
    }
    if constexpr (!PREP) load_w(0, wq0, wsb0);
    auto widen32 = [&](const uint4 (&q4)[4], float (&v)[32]) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w[4] = {q4[e].x, q4[e].y, q4[e].z, q4[e].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          v[8 * e + 2 * h] = bf16_lo(w[h]);
          v[8 * e + 2 * h + 1] = bf16_hi(w[h]);
        }
      }
    };
    float v[kNvSmallChunks][32];
#pragma unroll
    for (int i = 0; i < kNvSmallChunks; ++i) widen32(xr[i], v[i]);
    if (NORM) {
      float* cs = reinterpret_cast<float*>(smem + L.r);
#pragma unroll
      for (int i = 0; i < kNvSmallChunks; ++i) {
        const int q = t + kNvFusedThreads * i;
        if (q < nq) cs[(q / L.KC) * L.P + q % L.KC] = chunk_sumsq(v[i]);
      }
      for (int it = t; it < a.M * L.P; it += kNvFusedThreads)
        if (it % L.P >= L.KC) cs[it] = 0.0f;   // the zero padding of the tree
      __syncthreads();
      for (int n = L.P; n > 1; n >>= 1) {
        const int h = n >> 1;
        float tmp[4];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int it = t + qq * kNvFusedThreads;
          tmp[qq] = it < a.M * h ? cs[(it / h) * L.P + 2 * (it % h)] + cs[(it / h) * L.P + 2 * (it % h) + 1] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int it = t + qq * kNvFusedThreads;
          if (it < a.M * h) cs[(it / h) * L.P + (it % h)] = tmp[qq];
        }
        __syncthreads();
      }
      if (t < a.M) inv[t] = rms_inverse(cs[t * L.P], a.K, a.eps);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kNvSmallChunks; ++i) {
        const int q = t + kNvFusedThreads * i;
        if (q < nq) {
          float gm[32];
          widen32(gr[i], gm);
          const float iv = inv[q / L.KC];
#pragma unroll
          for (int e = 0; e < 32; ++e) v[i][e] = (v[i][e] * iv) * gm[e];
        }
      }
    }
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < kNvSmallChunks; ++i)
      if (t + kNvFusedThreads * i < nq) {
#pragma unroll
        for (int e = 0; e < 32; ++e) am = fmaxf(am, fabsf(v[i][e]));
      }
    g_s = tensor_scale(block_max<kNvFusedWaves>(am, red));
    float ar = 0.0f;
#pragma unroll
    for (int i = 0; i < kNvSmallChunks; ++i) {
      const int q = t + kNvFusedThreads * i;
      if (q < nq) {
        uint32_t scodes[2], meta, sbytes;
        nv_backbone(v[i], g_s, scodes, meta, sbytes);   // v[i] becomes the residual
        const int r = q / L.KC, c = q % L.KC, kt = c >> 2, tl = (c & 3) * 16 + r;
        *reinterpret_cast<uint4*>(smem + L.s + kt * 1024 + tl * 16) = expand_chunk(scodes[0], scodes[1], meta);
        *reinterpret_cast<uint16_t*>(smem + L.ss + kt * 128 + 2 * tl) = (uint16_t)sbytes;
        if constexpr (PREP) *reinterpret_cast<uint32_t*>(a.out.s_meta + kt * 256 + tl * 4) = meta;
#pragma unroll
        for (int e = 0; e < 32; ++e) ar = fmaxf(ar, fabsf(v[i][e]));
      }
    }
    g_r = tensor_scale(block_max<kNvFusedWaves>(ar, red));   // its barriers also end the tree's use of R
#pragma unroll
    for (int i = 0; i < kNvSmallChunks; ++i) {
      const int q = t + kNvFusedThreads * i;
      if (q < nq) {
        uint32_t rc[4], rbytes;
        nv_residual(v[i], g_r, rc, rbytes);
        const int r = q / L.KC, c = q % L.KC, kt = c >> 2, tl = (c & 3) * 16 + r;
        *reinterpret_cast<uint4*>(smem + L.r + kt * 1024 + tl * 16) = make_uint4(rc[0], rc[1], rc[2], rc[3]);
        *reinterpret_cast<uint16_t*>(smem + L.rs + kt * 128 + 2 * tl) = (uint16_t)rbytes;
      }
    }
  } else {

  // ---- RMSNorm: per row the pairwise tree over 32-element chunk subtrees
  // (M * P * 4 <= 4K bytes fit the R region, written only later)
  if (NORM) {
    float* cs = reinterpret_cast<float*>(smem + L.r);
    for (int it = t; it < a.M * L.P; it += kNvFusedThreads) {
      const int r = it / L.P, c = it % L.P;
      float s = 0.0f;
      if (c < L.KC) {
        float v[32];
        load32(a.x + (int64_t)r * a.ldx + 32 * c, v);
        s = chunk_sumsq(v);
      }
      cs[r * L.P + c] = s;
    }
    __syncthreads();
    for (int n = L.P; n > 1; n >>= 1) {
      const int h = n >> 1;
      float tmp[4];   // a.M * h <= 16 * 128 = 4 * kNvFusedThreads items
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int it = t + q * kNvFusedThreads;
        tmp[q] = it < a.M * h ? cs[(it / h) * L.P + 2 * (it % h)] + cs[(it / h) * L.P + 2 * (it % h) + 1] : 0.0f;
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int it = t + q * kNvFusedThreads;
        if (it < a.M * h) cs[(it / h) * L.P + (it % h)] = tmp[q];
      }
      __syncthreads();
    }
    if (t < a.M) inv[t] = rms_inverse(cs[t * L.P], a.K, a.eps);
    __syncthreads();
  }
  auto load_v = [&](int q, float (&v)[32]) {
    const int r = q / L.KC, c = q % L.KC;
    load32(a.x + (int64_t)r * a.ldx + 32 * c, v);
    if (NORM) apply_norm(v, a.gamma + 32 * c, inv[r]);
  };

  // ---- g_S from max |v| (the mask keeps each group's largest magnitude)
  float am = 0.0f;
  for (int q = t; q < nq; q += kNvFusedThreads) {
    float v[32];
    load_v(q, v);
#pragma unroll
    for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(v[i]));
  }
  g_s = tensor_scale(block_max<kNvFusedWaves>(am, red));

  // ---- backbone into LDS (tile c/4, lane (c%4)*16 + r), g_R from max |r|
  float ar = 0.0f;
  for (int q = t; q < nq; q += kNvFusedThreads) {
    float v[32];
    load_v(q, v);
    uint32_t scodes[2], meta, sbytes;
    nv_backbone(v, g_s, scodes, meta, sbytes);
    const int r = q / L.KC, c = q % L.KC, kt = c >> 2, tl = (c & 3) * 16 + r;
    *reinterpret_cast<uint4*>(smem + L.s + kt * 1024 + tl * 16) = expand_chunk(scodes[0], scodes[1], meta);
    *reinterpret_cast<uint16_t*>(smem + L.ss + kt * 128 + 2 * tl) = (uint16_t)sbytes;
    if constexpr (PREP) *reinterpret_cast<uint32_t*>(a.out.s_meta + kt * 256 + tl * 4) = meta;
#pragma unroll
    for (int i = 0; i < 32; ++i) ar = fmaxf(ar, fabsf(v[i]));
  }
  g_r = tensor_scale(block_max<kNvFusedWaves>(ar, red));   // its barriers also end the tree's use of R

  // ---- residual codes into LDS
  for (int q = t; q < nq; q += kNvFusedThreads) {
    float v[32];
    load_v(q, v);
    uint32_t scodes[2], meta, sbytes, rc[4], rbytes;
    nv_backbone(v, g_s, scodes, meta, sbytes);
    nv_residual(v, g_r, rc, rbytes);
    const int r = q / L.KC, c = q % L.KC, kt = c >> 2, tl = (c & 3) * 16 + r;
    *reinterpret_cast<uint4*>(smem + L.r + kt * 1024 + tl * 16) = make_uint4(rc[0], rc[1], rc[2], rc[3]);
    *reinterpret_cast<uint16_t*>(smem + L.rs + kt * 128 + 2 * tl) = (uint16_t)rbytes;
  }
  }   // !SMALL

  // rows past M and chunks past K: zero codes and scale bytes
  for (int b = t; b < 16 * L.KT * 4; b += kNvFusedThreads) {
    const int r = b / (L.KT * 4), c = b % (L.KT * 4);
    if (r < a.M && c < L.KC) continue;
    const int kt = c >> 2, tl = (c & 3) * 16 + r;
    *reinterpret_cast<uint4*>(smem + L.s + kt * 1024 + tl * 16) = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(smem + L.r + kt * 1024 + tl * 16) = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint16_t*>(smem + L.ss + kt * 128 + 2 * tl) = 0;
    *reinterpret_cast<uint16_t*>(smem + L.rs + kt * 128 + 2 * tl) = 0;
    if constexpr (PREP) *reinterpret_cast<uint32_t*>(a.out.s_meta + kt * 256 + tl * 4) = 0x44444444u;   // zero groups
  }
  __syncthreads();
  if constexpr (PREP) {
    // the prepared tiles (row block 0: tile kt at kt * 1024, scales at kt * 128)
    for (int i = t; i < KT * 64; i += kNvFusedThreads) {
      *reinterpret_cast<uint4*>(a.out.s_codes + i * 16) = *reinterpret_cast<const uint4*>(smem + L.s + i * 16);
      *reinterpret_cast<uint4*>(a.out.r_codes + i * 16) = *reinterpret_cast<const uint4*>(smem + L.r + i * 16);
    }
    for (int i = t; i < KT * 8; i += kNvFusedThreads) {
      *reinterpret_cast<uint4*>(a.out.s_scales + i * 16) = *reinterpret_cast<const uint4*>(smem + L.ss + i * 16);
      *reinterpret_cast<uint4*>(a.out.r_scales + i * 16) = *reinterpret_cast<const uint4*>(smem + L.rs + i * 16);
    }
    if (t == 0) {
      *a.g_s_out = g_s;
      *a.g_r_out = g_r;
    }
    return;
  }

  // ---- split-K GEMM: nv_dual_gemm_kernel<1, 8>'s loop with A from LDS
  v4f acs = (v4f){0.f, 0.f, 0.f, 0.f}, acr = acs;
  for (int base = 0; base < KT; base += kNvFusedWaves * CH) {
    uint4 wq[CH], rq[CH], sq[CH];
    uint32_t wsb[CH], ssb[CH], rsb[CH];
    if (SMALL && base == 0) {
#pragma unroll
      for (int c = 0; c < CH; ++c) { wq[c] = wq0[c]; wsb[c] = wsb0[c]; }
    } else {
      load_w(base, wq, wsb);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int kt = base + wave + kNvFusedWaves * c;
      const int ktc = kt < KT ? kt : KT - 1;
      rq[c] = *reinterpret_cast<const uint4*>(smem + L.r + ktc * 1024 + lane * 16);
      sq[c] = *reinterpret_cast<const uint4*>(smem + L.s + ktc * 1024 + lane * 16);
      ssb[c] = *reinterpret_cast<const uint16_t*>(smem + L.ss + ktc * 128 + 2 * lane);
      rsb[c] = *reinterpret_cast<const uint16_t*>(smem + L.rs + ktc * 128 + 2 * lane);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      f16x8 b[4], x[4];
      deq32(wq[c], wsb[c], b);
      deq32(sq[c], ssb[c], x);
#pragma unroll
      for (int j = 0; j < 4; ++j) acs = mfma_f16(x[j], b[j], acs);
      deq32(rq[c], rsb[c], x);
#pragma unroll
      for (int j = 0; j < 4; ++j) acr = mfma_f16(x[j], b[j], acr);
    }
  }

  // tensor scales once per path, then the waves' partial sums in wave order
  // (all LDS is free once every wave has left the loop)
  const float gw = *g.g_w;
  const float fs = g_s * gw, fr = g_r * gw;
  __syncthreads();
  v4f* part = reinterpret_cast<v4f*>(smem + L.s);
  v4f p;
#pragma unroll
  for (int q = 0; q < 4; ++q) p[q] = fs * acs[q] + fr * acr[q];
  part[wave * 64 + lane] = p;
  __syncthreads();
  if (wave == 0) {
    const int64_t col = nb * 16 + (lane & 15);
    v4f v = part[lane];
#pragma unroll
    for (int w = 1; w < kNvFusedWaves; ++w) v = v + part[w * 64 + lane];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t row = 4 * (lane >> 4) + q;
      if (row < a.M && col < g.N) store_y(g, row, col, v[q]);
    }
  }
}

}  // namespace

hipError_t launch_prepare_nv(const uint16_t* x, int64_t M, int K, int64_t ldx, const uint16_t* gamma, float eps,
                             PrepOut out, hipStream_t stream) {
  const NvActLayout L = nv_act_layout(M, K);
  NvPrepArgs a;
  a.x = x;
  a.M = M;
  a.ldx = ldx;
  a.K = K;
  a.gamma = gamma;
  a.eps = eps;
  a.RB = (M + 15) / 16;
  a.KB = (K + 127) / 128;
  a.WX = L.wx;
  a.o = out;
  a.g_s = reinterpret_cast<float*>(out.s_scales + L.g);
  a.g_r = reinterpret_cast<float*>(out.r_scales + L.g);
  a.rowamax = reinterpret_cast<float*>(out.r_scales + L.rowamax);
  a.inv = reinterpret_cast<float*>(out.r_scales + L.inv);
  a.rparts = reinterpret_cast<float*>(out.r_scales + L.rparts);
  if (M > 0x7FFFFFFF || a.RB > 65535) return hipErrorInvalidValue;
  constexpr int kNvPrepOneWgThreads = kNvFusedThreads;
  if (M >= 1 && M <= 16 && M * (K / 32) <= kNvPrepOneWgThreads &&
      nv_fused_lds(K, kNvPrepOneWgThreads / 64).total <= 160 * 1024) {
    // at most one 32-element chunk per thread of one 512-thread workgroup:
    // that workgroup runs the three phases (the one-launch layer's
    // preparation) instead of three dependent launches (K = 4096: M = 1
    // 11.1 -> 6.9 us).  One compute unit's VALU then carries the whole
    // preparation, which stops paying with more rows: at M = 8 it took
    // 14.3 us with two chunks per thread and 13.5 us with 1024 threads,
    // against 11.6 us for the three launches.
    NvFusedArgs f{};
    f.x = x;
    f.ldx = ldx;
    f.M = (int)M;
    f.K = K;
    f.gamma = gamma;
    f.eps = eps;
    f.out = out;
    f.g_s_out = a.g_s;
    f.g_r_out = a.g_r;
    auto kern = gamma ? nv_fused_layer_kernel<true, true, true, kNvPrepOneWgThreads>
                      : nv_fused_layer_kernel<false, true, true, kNvPrepOneWgThreads>;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    static std::atomic<bool> attr_set[64][2];
    const int which = gamma ? 1 : 0;
    if (!attr_set[dev][which].load(std::memory_order_acquire)) {
      e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      if (e != hipSuccess) return e;
      attr_set[dev][which].store(true, std::memory_order_release);
    }
    hipLaunchKernelGGL(kern, dim3(1), dim3(kNvPrepOneWgThreads), nv_fused_lds(K, kNvPrepOneWgThreads / 64).total,
                       stream, f);
    return hipGetLastError();
  }
  const dim3 rows((unsigned)M), tiles((unsigned)a.WX, (unsigned)a.RB), blk(256), blk_q(kNvPrepThreads);
  if (gamma) {
    hipLaunchKernelGGL((nv_rowstats_kernel<true>), rows, blk, 0, stream, a);
    hipLaunchKernelGGL((nv_decompose_kernel<true, false>), tiles, blk_q, 0, stream, a);
    hipLaunchKernelGGL((nv_decompose_kernel<true, true>), tiles, blk_q, 0, stream, a);
  } else if (M * (int64_t)K <= kNvSelfScanElems) {
    // small tensors without RMSNorm: phase 2 scans X itself (two launches;
    // M = 8, K = 4096: 11.4 -> 10.2 us)
    hipLaunchKernelGGL((nv_decompose_kernel<false, false, true>), tiles, blk_q, 0, stream, a);
    hipLaunchKernelGGL((nv_decompose_kernel<false, true>), tiles, blk_q, 0, stream, a);
  } else {
    hipLaunchKernelGGL((nv_rowstats_kernel<false>), rows, blk, 0, stream, a);
    hipLaunchKernelGGL((nv_decompose_kernel<false, false>), tiles, blk_q, 0, stream, a);
    hipLaunchKernelGGL((nv_decompose_kernel<false, true>), tiles, blk_q, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_pack_weight_nv(const uint16_t* w, int64_t N, int K, int64_t ldw, uint8_t* codes, uint8_t* scales,
                                 hipStream_t stream) {
  const NvWeightLayout L = nv_weight_layout(N, K);
  NvWeightArgs a;
  a.w = w;
  a.N = N;
  a.ldw = ldw;
  a.K = K;
  a.NB = (N + 15) / 16;
  a.KB = (K + 127) / 128;
  a.WX = L.wx;
  a.codes = codes;
  a.scales = scales;
  a.g = reinterpret_cast<float*>(scales + L.g);
  a.parts = reinterpret_cast<float*>(scales + L.parts);
  if (a.NB > 65535) return hipErrorInvalidValue;
  const dim3 tiles((unsigned)a.WX, (unsigned)a.NB), blk(256);
  hipLaunchKernelGGL(nv_weight_amax_kernel, tiles, blk, 0, stream, a);
  hipLaunchKernelGGL(nv_weight_scale_kernel, dim3(1), blk, 0, stream, a);
  hipLaunchKernelGGL(nv_pack_weight_kernel, tiles, blk, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_linear_nv(const GemmArgs& a, hipStream_t stream) {
  const int64_t NB = (a.N + 15) / 16, RB = a.a_blocks;
  if (NB > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (RB > 4) {
    // past the decode sizes: four row blocks per workgroup
    const int64_t groups = (RB + 3) / 4;
    if (groups > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL((nv_dual_gemm_kernel<4, 4>), dim3((unsigned)NB, (unsigned)groups), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  // one row block and CBG 16-column blocks per workgroup, CBG the largest of
  // 4, 2, 1 that still gives every compute unit a workgroup: each workgroup
  // expands its row block's codes once for CBG weight blocks (K = N = 4096 at
  // M = 64: CBG 4)
  const int cus = compute_units();
  if (cus <= 0) return hipErrorInvalidDevice;
  const int cbg = (NB + 3) / 4 * RB >= cus ? 4 : (NB + 1) / 2 * RB >= cus ? 2 : 1;
  const dim3 grid((unsigned)((NB + cbg - 1) / cbg), (unsigned)RB);
  // two column blocks: 16 waves, two K tiles each (M = 32: 8.25 -> 7.85 us);
  // with four the 16-wave form spills or, at two blocks, doubles the
  // activation's reads (M = 64: 11.8 against 14.8 and 13.1 us), and one
  // block keeps 8 waves
  if (cbg == 4) hipLaunchKernelGGL((nv_dual_gemm_kernel<1, 8, 4>), grid, dim3(512), 0, stream, a);
  else if (cbg == 2) hipLaunchKernelGGL((nv_dual_gemm_kernel<1, 16, 2>), grid, dim3(1024), 0, stream, a);
  else hipLaunchKernelGGL((nv_dual_gemm_kernel<1, 8, 1>), grid, dim3(512), 0, stream, a);
  return hipGetLastError();
}


size_t nv_fused_layer_lds_bytes(int K) { return nv_fused_lds(K).total; }

hipError_t launch_linear_fused_nv(const uint16_t* x, int M, int K, int64_t ldx, const uint16_t* gamma, float eps,
                                  const GemmArgs& g, hipStream_t stream) {
  if (M == 0 || g.N == 0) return hipSuccess;
  const int64_t NB = (g.N + 15) / 16;
  const NvFusedLds L = nv_fused_lds(K);
  if (M > 16 || NB > 0x7FFFFFFF || L.total > 160 * 1024) return hipErrorInvalidValue;
  NvFusedArgs a;
  a.x = x;
  a.ldx = ldx;
  a.M = M;
  a.K = K;
  a.gamma = gamma;
  a.eps = eps;
  a.g = g;
  const bool norm = gamma != nullptr;
  const bool small = (int64_t)M * (K / 32) <= (int64_t)kNvSmallChunks * kNvFusedThreads;
  auto kern = norm ? (small ? nv_fused_layer_kernel<true, true> : nv_fused_layer_kernel<true, false>)
                   : (small ? nv_fused_layer_kernel<false, true> : nv_fused_layer_kernel<false, false>);
  // the LDS limit is a per-function attribute: set it once per device
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  static std::atomic<bool> attr_set[64][4];
  const int which = (norm ? 2 : 0) + (small ? 1 : 0);
  if (!attr_set[dev][which].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set[dev][which].store(true, std::memory_order_release);
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)NB), dim3(kNvFusedThreads), L.total, stream, a);
  return hipGetLastError();
}

}  // namespace sharq
