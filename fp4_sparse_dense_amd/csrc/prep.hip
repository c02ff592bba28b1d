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


// ---------------------------------------------------------------------------
// One MX block (32 consecutive elements of one row) per lane.
// ---------------------------------------------------------------------------
struct Block32 {
  uint4 r_codes;     // 32 R nibbles
  uint2 s_codes;     // 16 kept S nibbles: groups 0-3, groups 4-7
  uint32_t meta;     // 8 metadata nibbles
  uint32_t s_e8, r_e8;
};

// 2:4 mask of one group: element k is kept iff at most one other element
// beats it (larger magnitude, or equal magnitude and lower index).  With
// bij = |a_i| >= |a_j| for i < j, "at most one beater" is a majority of three
// comparisons; ranks are a permutation, so exactly two are kept.
struct Keep4 { bool k0, k1, k2, k3; };
__device__ __forceinline__ Keep4 keep_2of4(float a0, float a1, float a2, float a3) {
  const bool b01 = fabsf(a0) >= fabsf(a1), b02 = fabsf(a0) >= fabsf(a2), b03 = fabsf(a0) >= fabsf(a3);
  const bool b12 = fabsf(a1) >= fabsf(a2), b13 = fabsf(a1) >= fabsf(a3), b23 = fabsf(a2) >= fabsf(a3);
  Keep4 k;
  k.k0 = (b01 && b02) || (b01 && b03) || (b02 && b03);
  k.k1 = (!b01 && b12) || (!b01 && b13) || (b12 && b13);
  k.k2 = (!b02 && !b12) || (!b02 && b23) || (!b12 && b23);
  k.k3 = (!b03 && !b13) || (!b03 && !b23) || (!b13 && !b23);
  return k;
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

// One group of four: mask, kept codes into byte SEL of *codes, metadata
// nibble, and the residual of the four elements against the dequantised
// backbone.  Returns the nibble.
template <int SEL>
__device__ __forceinline__ uint32_t group4(const float* a, float s_scale, uint32_t& codes, float* r) {
  const Keep4 k = keep_2of4(a[0], a[1], a[2], a[3]);
  const float s0 = k.k0 ? a[0] : (k.k1 ? a[1] : a[2]);   // kept values in k order
  const float s1 = k.k3 ? a[3] : (k.k2 ? a[2] : a[1]);
  codes = fp4_enc<SEL>(codes, s0, s1, s_scale);
  float dlo, dhi;
  fp4_dec<SEL>(codes, s_scale, dlo, dhi);
  // a kept position is the group's first kept offset or its second;
  // dropped positions keep v (v - (+0) == v for every v)
  r[0] = a[0] - (k.k0 ? dlo : 0.0f);
  r[1] = a[1] - (k.k1 ? (k.k0 ? dhi : dlo) : 0.0f);
  r[2] = a[2] - (k.k2 ? ((k.k0 || k.k1) ? dhi : dlo) : 0.0f);
  r[3] = a[3] - (k.k3 ? dhi : 0.0f);
  const uint32_t i0 = k.k0 ? 0u : (k.k1 ? 1u : 2u), i1 = k.k3 ? 3u : (k.k2 ? 2u : 1u);
  return i0 | (i1 << 2);
}

__device__ __forceinline__ Block32 decompose32(const float (&v)[32]) {
  // S block scale: the block maximum of v is always kept, so amax(S) == amax(v)
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; i += 2) am = abs_max3(am, v[i], v[i + 1]);
  const float ss = pow2(mx_shared_exp(__float_as_uint(am)));

  uint32_t lo = 0, hi = 0, meta = 0;
  float r[32];
  meta |= group4<0>(v + 0, ss, lo, r + 0);
  meta |= group4<1>(v + 4, ss, lo, r + 4) << 4;
  meta |= group4<2>(v + 8, ss, lo, r + 8) << 8;
  meta |= group4<3>(v + 12, ss, lo, r + 12) << 12;
  meta |= group4<0>(v + 16, ss, hi, r + 16) << 16;
  meta |= group4<1>(v + 20, ss, hi, r + 20) << 20;
  meta |= group4<2>(v + 24, ss, hi, r + 24) << 24;
  meta |= group4<3>(v + 28, ss, hi, r + 28) << 28;

  float ar = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; i += 2) ar = abs_max3(ar, r[i], r[i + 1]);
  const int er = mx_shared_exp(__float_as_uint(ar));
  const float rs = pow2(er);
  uint32_t rc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t w = fp4_enc<0>(0u, r[8 * j], r[8 * j + 1], rs);
    w = fp4_enc<1>(w, r[8 * j + 2], r[8 * j + 3], rs);
    w = fp4_enc<2>(w, r[8 * j + 4], r[8 * j + 5], rs);
    rc[j] = fp4_enc<3>(w, r[8 * j + 6], r[8 * j + 7], rs);
  }

  Block32 o;
  o.r_codes = make_uint4(rc[0], rc[1], rc[2], rc[3]);
  o.s_codes = make_uint2(lo, hi);
  o.meta = meta;
  o.s_e8 = (uint32_t)(mx_shared_exp(__float_as_uint(am)) + 127);
  o.r_e8 = (uint32_t)(er + 127);
  return o;
}

// ---------------------------------------------------------------------------
// Prep kernel.  A workgroup owns 8 rows (one half of a 16-row tile) and all of
// K, in chunks of up to 4096 elements staged in LDS.  Rows arrive by 1 KiB
// contiguous global -> LDS copies; inside each 256-byte window the 16-byte
// units of row r are XOR-permuted by sw(r) so that the block reads below hit
// 16 distinct bank groups per 16-lane phase (64 banks x 4 bytes).
//
// A wave's 64 lanes cover 8 rows x 2 K tiles: lane l takes row l%8, 32-chunk
// (l/8)%4 and tile l/32, i.e. one MX block, and writes it in tile-lane order
// (chunk*16 + half*8 + row), so every output store is a contiguous run.
//
// RMSNorm: the sum of squares of a block is a pairwise tree of its 32 squares
// (the leaf pairs as fma(x0,x0,x1*x1), exact since bf16 squares are exact in
// binary32), the blocks of a 256-element unit combine by lane exchanges in K
// order, units by a 16-leaf tree in LDS, chunks by an 8-leaf tree: all of it
// is the balanced tree of the zero-padded row.
// ---------------------------------------------------------------------------
constexpr int kPrepRows = 8;
constexpr int kPrepThreads = 512;
constexpr int kPrepChunk = 4096;                 // K elements per LDS stage
constexpr int kPrepUnits = kPrepChunk / 256;     // 256-element units per chunk (16)
constexpr int kPrepMaxChunks = 8;                // K <= 32768 with RMSNorm

__device__ __forceinline__ uint32_t prep_swz(int r) { return (uint32_t)((r & 3) | ((r & 4) << 1)); }

struct PrepLds {
  uint32_t row_bytes;   // LDS bytes per staged row (multiple of 1 KiB)
  uint32_t off_g;       // gamma, binary32
  uint32_t off_us;      // unit sums [16][8]
  uint32_t off_cs;      // chunk sums [8][8]
  uint32_t total;
};
__host__ __device__ inline PrepLds prep_lds_layout(int K) {
  PrepLds L;
  const int kc = K < kPrepChunk ? ((K + 511) / 512) * 512 : kPrepChunk;
  L.row_bytes = (uint32_t)kc * 2;
  L.off_g = L.row_bytes * kPrepRows;
  L.off_us = L.off_g + (uint32_t)kc * 4;
  L.off_cs = L.off_us + kPrepUnits * kPrepRows * 4;
  L.total = L.off_cs + kPrepMaxChunks * kPrepRows * 4;
  return L;
}

__device__ __forceinline__ float tree16(const float* p, int stride) {
  float t[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) t[i] = p[i * stride];
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) t[i] = t[2 * i] + t[2 * i + 1];
  return t[0];
}

template <bool NORM>
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(const uint16_t* __restrict__ x, int64_t M, int K,
                                                            int64_t ldx, const uint16_t* __restrict__ gamma,
                                                            float eps, PrepOut o) {
  extern __shared__ __align__(1024) uint8_t smem[];
  const PrepLds L = prep_lds_layout(K);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // workgroup -> (16-row block, half); the two halves of a block are 8 blocks
  // apart in launch order, i.e. on the same XCD, so their L2 merges the writes
  const int64_t RB = (M + 15) / 16, nwg = RB * 2, w = blockIdx.x;
  const int64_t full = nwg / 16 * 16;
  int64_t rb, half;
  if (w < full) { rb = (w / 16) * 8 + (w % 8); half = (w % 16) / 8; }
  else { rb = w / 2; half = w % 2; }
  const int64_t row0 = rb * 16 + half * 8;

  const int KB = (K + 127) / 128;
  const int nchunk = (K + kPrepChunk - 1) / kPrepChunk;
  const int r8 = lane & 7, c4 = (lane >> 3) & 3, t2 = lane >> 5;
  const int64_t my_row = row0 + r8;
  const bool row_ok = my_row < M;
  const uint32_t lds0 = lds_addr(smem);
  const uint32_t sw_me = prep_swz(r8);
  float* gs = reinterpret_cast<float*>(smem + L.off_g);
  float* us = reinterpret_cast<float*>(smem + L.off_us);
  float* cs = reinterpret_cast<float*>(smem + L.off_cs);
  const int segs = (int)(L.row_bytes / 1024);

  // stage chunk ch: rows by 1 KiB copies (wave-strided), gamma widened by every thread
  auto stage = [&](int ch) {
    const uint32_t kbyte0 = (uint32_t)ch * kPrepChunk * 2;
    for (int j = wave; j < kPrepRows * segs; j += 8) {
      const int r = j / segs, sg = j % segs;
      const int64_t row = row0 + r;
      const u32x4 d = make_desc(x + (row < M ? row : 0) * ldx, row < M ? (uint64_t)K * 2 : 0);
      const uint32_t unit = (uint32_t)sg * 64 + ((uint32_t)lane ^ prep_swz(r));
      lds_dma16(d, lds0 + (uint32_t)r * L.row_bytes + (uint32_t)sg * 1024, kbyte0 + unit * 16, 0);
    }
    if (NORM) {
      const int kc = (int)(L.row_bytes / 2);
      for (int e = tid * 8; e < kc; e += kPrepThreads * 8) {
        const int k = ch * kPrepChunk + e;
        uint4 q = k < K ? *reinterpret_cast<const uint4*>(gamma + k) : make_uint4(0, 0, 0, 0);
        float4 lo = make_float4(bf16_lo(q.x), bf16_hi(q.x), bf16_lo(q.y), bf16_hi(q.y));
        float4 hi = make_float4(bf16_lo(q.z), bf16_hi(q.z), bf16_lo(q.w), bf16_hi(q.w));
        *reinterpret_cast<float4*>(gs + e) = lo;
        *reinterpret_cast<float4*>(gs + e + 4) = hi;
      }
    }
    wait_vm_lgkm<0, 0>();
    __syncthreads();
  };

  // the lane's 32 bf16 of unit u (chunk-local), read back through the swizzle
  auto load_block = [&](int u, uint32_t (&xw)[16]) {
    const uint32_t g0 = (uint32_t)(2 * u + t2) * 16 + c4 * 4;   // first 16-byte unit
    const uint8_t* rowp = smem + (uint32_t)r8 * L.row_bytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t g = g0 + i;
      const uint4 q = *reinterpret_cast<const uint4*>(rowp + (((g & ~15u) | ((g & 15u) ^ sw_me)) * 16));
      xw[4 * i] = q.x; xw[4 * i + 1] = q.y; xw[4 * i + 2] = q.z; xw[4 * i + 3] = q.w;
    }
  };

  // balanced tree of the 32 squares of a block
  auto block_ss = [&](const uint32_t (&xw)[16]) {
    float p[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float a = bf16_lo(xw[j]), b = bf16_hi(xw[j]);
      p[j] = __builtin_fmaf(a, a, b * b);
    }
#pragma unroll
    for (int w2 = 8; w2 >= 1; w2 >>= 1)
#pragma unroll
      for (int j = 0; j < w2; ++j) p[j] = p[2 * j] + p[2 * j + 1];
    return p[0];
  };

  const int nunit_tot = (KB + 1) / 2;

  // ---- RMSNorm denominators
  float inv = 1.0f;
  if (NORM) {
    for (int ch = 0; ch < nchunk; ++ch) {
      if (nchunk > 1 || ch == 0) stage(ch);
      const int nu = min(kPrepUnits, nunit_tot - ch * kPrepUnits);
      for (int u = wave; u < kPrepUnits; u += 8) {
        float t = 0.0f;
        if (u < nu) {
          uint32_t xw[16];
          load_block(u, xw);
          t = block_ss(xw);
          t = t + __shfl_xor(t, 8, 64);    // blocks of a tile, in K order
          t = t + __shfl_xor(t, 16, 64);
          t = t + __shfl_xor(t, 32, 64);   // the two tiles of the unit
        }
        if (lane < 8) us[u * kPrepRows + lane] = t;
      }
      __syncthreads();
      if (tid < kPrepRows) cs[ch * kPrepRows + tid] = tree16(us + tid, kPrepRows);
      __syncthreads();
    }
    float c8[kPrepMaxChunks];
#pragma unroll
    for (int i = 0; i < kPrepMaxChunks; ++i) c8[i] = i < nchunk ? cs[i * kPrepRows + r8] : 0.0f;
#pragma unroll
    for (int w2 = 4; w2 >= 1; w2 >>= 1)
#pragma unroll
      for (int i = 0; i < w2; ++i) c8[i] = c8[2 * i] + c8[2 * i + 1];
    inv = rms_inverse(c8[0], K, eps);
  }

  // ---- decomposition, chunk by chunk
  for (int ch = 0; ch < nchunk; ++ch) {
    if (!NORM || nchunk > 1) {
      if (ch > 0 || NORM) __syncthreads();   // previous chunk fully read
      stage(ch);
    }
    const int nu = min(kPrepUnits, nunit_tot - ch * kPrepUnits);
    for (int u = wave; u < nu; u += 8) {
      const int kt = ch * (kPrepChunk / 128) + 2 * u + t2;     // global K tile of this lane
      if (kt >= KB) continue;
      const int kloc = (2 * u + t2) * 128 + c4 * 32;           // chunk-local first element
      const bool live = row_ok && ch * kPrepChunk + kloc < K;  // real input (else zero padding)
      uint32_t xw[16];
      load_block(u, xw);
      float v[32];
#pragma unroll
      for (int j = 0; j < 16; ++j) { v[2 * j] = bf16_lo(xw[j]); v[2 * j + 1] = bf16_hi(xw[j]); }
      if (NORM) {
#pragma unroll
        for (int i = 0; i < 32; i += 4) {
          const float4 gv = *reinterpret_cast<const float4*>(gs + kloc + i);
          v[i] = (v[i] * inv) * gv.x;
          v[i + 1] = (v[i + 1] * inv) * gv.y;
          v[i + 2] = (v[i + 2] * inv) * gv.z;
          v[i + 3] = (v[i + 3] * inv) * gv.w;
        }
      }
      if (!live) {
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = 0.0f;
      }
      const Block32 b = decompose32(v);
      const int64_t tile = rb * KB + kt;
      const int tl = c4 * 16 + (int)half * 8 + r8;
      *reinterpret_cast<uint4*>(o.r_codes + tile * 1024 + tl * 16) = b.r_codes;
      *reinterpret_cast<uint2*>(o.s_codes + tile * 512 + tl * 8) = b.s_codes;
      *reinterpret_cast<uint32_t*>(o.s_meta + tile * 256 + tl * 4) = b.meta;
      const int64_t sc = ((int64_t)kt * RB + rb) * 64 + tl;
      o.s_scales[sc] = (uint8_t)b.s_e8;
      o.r_scales[sc] = (uint8_t)b.r_e8;
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
  const PrepLds L = prep_lds_layout(K);
  const int64_t nwg = (M + 15) / 16 * 2;
  auto kn = gamma ? prep_kernel<true> : prep_kernel<false>;
  static bool attr_set[2] = {false, false};
  if (!attr_set[gamma ? 1 : 0]) {
    hipError_t e = hipFuncSetAttribute((const void*)kn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       prep_lds_layout(kPrepChunk).total);
    if (e != hipSuccess) return e;
    attr_set[gamma ? 1 : 0] = true;
  }
  hipLaunchKernelGGL(kn, dim3((unsigned)nwg), dim3(kPrepThreads), L.total, stream, x, M, K, ldx, gamma, eps, out);
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
