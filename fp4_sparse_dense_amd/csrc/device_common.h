// Device helpers shared by the SharQ kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sharq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------- DPP lane exchange
// Row-local permutes; every lane of the wave must be active.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Sum over the 64 lanes whose partial results equal a balanced pairwise tree
// in lane order: at every step each lane adds the sum of the neighbouring
// aligned lane group of the same size (x + y == y + x bit for bit, so the
// mirrors used once groups are uniform give exactly T[left] + T[right]).
__device__ __forceinline__ float wave_tree_sum(float s) {
  s = s + dpp_f32<kQuadXor1>(s);
  s = s + dpp_f32<kQuadXor2>(s);
  s = s + dpp_f32<kRowHalfMirror>(s);
  s = s + dpp_f32<kRowMirror>(s);
  s = s + __shfl_xor(s, 16, kWave);
  s = s + __shfl_xor(s, 32, kWave);
  return s;
}

// max over the 4 lanes of an aligned quad
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kQuadXor1>(v));
  v = max(v, dpp_u32<kQuadXor2>(v));
  return v;
}

// ---------------------------------------------------------------- MXFP4 scale
// Shared exponent of a block with largest magnitude `amax_bits` (binary32 bits,
// sign cleared): e = clamp(floor(log2 amax) - 2, -127, 127); 0 -> -127.
// floor(log2) comes from the bit pattern: biased exponent - 127 for normals,
// top mantissa bit position - 149 for subnormals.
__device__ __forceinline__ int mx_shared_exp(uint32_t amax_bits) {
  int fl;
  uint32_t ex = amax_bits >> 23;
  if (ex != 0) fl = (int)ex - 127;
  else fl = (31 - __clz((int)amax_bits)) - 149;   // amax_bits == 0 -> very negative
  int e = fl - 2;
  e = e < -127 ? -127 : e;
  return e;   // finite inputs give e <= 125
}
// 2^-e as binary32 (normal for every e in [-127, 125])
__device__ __forceinline__ float pow2_neg(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }
// 2^e as binary32 (subnormal 2^-127 for e == -127)
__device__ __forceinline__ float pow2(int e) {
  return e >= -126 ? __uint_as_float((uint32_t)(127 + e) << 23) : __uint_as_float(0x00400000u);
}

// ---------------------------------------------------------------- RMSNorm
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

// ---------------------------------------------------------------- row helpers
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// max over the workgroup of non-negative v (all threads must call)
template <int NWAVES>
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int i = 1; i < NWAVES; ++i) m = fmaxf(m, red[i]);
  return m;
}

// 32 bf16 of one row -> binary32
__device__ __forceinline__ void load32(const uint16_t* p, float (&v)[32]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 d = *reinterpret_cast<const uint4*>(p + 8 * q);
    const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      v[8 * q + 2 * h] = bf16_lo(w[h]);
      v[8 * q + 2 * h + 1] = bf16_hi(w[h]);
    }
  }
}

// v = (x * inv) * gamma, elementwise, two roundings
__device__ __forceinline__ void apply_norm(float (&v)[32], const uint16_t* gamma, float inv) {
  float g[32];
  load32(gamma, g);
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = (v[i] * inv) * g[i];
}

// Pairwise tree of squares over 32 consecutive elements: leaves x0^2 + x1^2
// (squares of bf16 values are exact), then halving in index order.
__device__ __forceinline__ float chunk_sumsq(const float (&v)[32]) {
  float p[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) p[i] = v[2 * i] * v[2 * i] + v[2 * i + 1] * v[2 * i + 1];
#pragma unroll
  for (int n = 8; n >= 1; n >>= 1)
#pragma unroll
    for (int i = 0; i < n; ++i) p[i] = p[2 * i] + p[2 * i + 1];
  return p[0];
}

// 1/rms of one row of K bf16 values (K % 32 == 0, K <= 32768), computed by a
// whole workgroup of 256 threads (all must call): the sum of squares is the
// balanced pairwise tree over the row zero-padded to a power of two -- aligned
// 32-element chunks are subtrees (chunk_sumsq), their sums are combined
// pairwise in LDS (cs: 1024 floats).
__device__ __forceinline__ float row_inv_rms(const uint16_t* xr, int K, float eps, float* cs) {
  const int t = threadIdx.x;
  const int KC = K / 32;
  int P = 1;
  while (P < KC) P *= 2;
  for (int c = t; c < P; c += 256) {
    float s = 0.0f;
    if (c < KC) {
      float v[32];
      load32(xr + 32 * c, v);
      s = chunk_sumsq(v);
    }
    cs[c] = s;
  }
  __syncthreads();
  for (int n = P; n > 1; n >>= 1) {
    const int h = n >> 1;
    const float s0 = t < h ? cs[2 * t] + cs[2 * t + 1] : 0.0f;
    const float s1 = t + 256 < h ? cs[2 * (t + 256)] + cs[2 * (t + 256) + 1] : 0.0f;
    __syncthreads();
    if (t < h) cs[t] = s0;
    if (t + 256 < h) cs[t + 256] = s1;
    __syncthreads();
  }
  return rms_inverse(cs[0], K, eps);
}

// ---------------------------------------------------------------- E2M1
// Two binary32 values -> two E2M1 nibbles placed in byte SEL of `old`.
// v_cvt_scalef32_pk_fp4_f32 with scale 1.0 rounds to nearest, ties to even,
// saturates at 6 and keeps the sign of zero: tests/test_gpu_fp4_convert.py
// checks it against that rule (through sharq_check_e2m1) on every finite bf16
// value and the 64 binary32 neighbours of every grid point and midpoint, at
// every power-of-two scale the kernels use.
template <int SEL>
__device__ __forceinline__ uint32_t fp4_pack2(uint32_t old, float lo, float hi) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, lo, hi, 1.0f, SEL);
}
// E2M1 nibbles of byte SEL of `packed` -> two binary32 values (exact).
template <int SEL>
__device__ __forceinline__ void fp4_unpack2(uint32_t packed, float& lo, float& hi) {
  auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, SEL);
  lo = v[0];
  hi = v[1];
}

// ---------------------------------------------------------------- 2:4 expansion
// The kept codes of 32 logical K positions (8 groups) are 16 nibbles (group g
// in byte g, lower offset in the low nibble) plus 8 metadata nibbles (group g:
// i0 | i1<<2 in nibble g); codes_lo holds groups 0-3, codes_hi groups 4-7.
// The result is the 32 dense nibbles, zero codes at dropped positions.  Two
// groups are handled per dword, one in each 16-bit half, with byte permutes
// and packed 16-bit shifts.
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

template <int H>
__device__ __forceinline__ uint32_t expand_dword(uint32_t cw, uint32_t mb4, int j) {
  // code bytes 2H and 2H+1 of cw -> low byte of half 0 and half 1
  constexpr uint32_t sel = H == 0 ? 0x0C010C00u : 0x0C030C02u;
  const uint32_t d = __builtin_amdgcn_perm(0u, cw, sel);
  const uint32_t lo = d & 0x000F000Fu, hi = d & 0x00F000F0u;
  // metadata byte j -> both halves; the second half keeps the upper nibble
  const uint32_t msel = 0x0C000C00u | (uint32_t)j | ((uint32_t)j << 16);
  u16x2 tv = __builtin_bit_cast(u16x2, __builtin_amdgcn_perm(0u, mb4, msel));
  tv = tv >> (u16x2){0, 4};
  const uint32_t t = __builtin_bit_cast(uint32_t, tv);
  const uint32_t sl = (t << 2) & 0x000C000Cu;            // 4*i0 per half
  const uint32_t sh = (t & 0x000C000Cu) - 0x00040004u;   // 4*i1 - 4 per half (i1 >= 1)
  const u16x2 los = __builtin_bit_cast(u16x2, lo) << __builtin_bit_cast(u16x2, sl);
  const u16x2 his = __builtin_bit_cast(u16x2, hi) << __builtin_bit_cast(u16x2, sh);
  return __builtin_bit_cast(uint32_t, los) | __builtin_bit_cast(uint32_t, his);
}

__device__ __forceinline__ uint4 expand_chunk(uint32_t codes_lo, uint32_t codes_hi, uint32_t meta) {
  uint4 d;
  d.x = expand_dword<0>(codes_lo, meta, 0);
  d.y = expand_dword<1>(codes_lo, meta, 1);
  d.z = expand_dword<0>(codes_hi, meta, 2);
  d.w = expand_dword<1>(codes_hi, meta, 3);
  return d;
}

// ---------------------------------------------------------------- buffer copies
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource for a raw byte buffer (stride 0, offsets checked against
// num_records: reads past the end return zero).
__device__ __forceinline__ u32x4 make_desc(const void* p, uint64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t n = bytes >= 0x7FFFFFFFull ? 0x7FFFFFFFu : (uint32_t)bytes;
  return (u32x4){(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, n, 0x00020000u};
}

// Global -> LDS copies (buffer_load ... lds): lane l's bytes land at
// lds_off + l*size.  They are issued from inline asm so that the compiler does
// not make every later LDS access wait for them; the kernel waits for them
// itself (vmcnt) before the barrier that publishes a stage.  They have no
// register results.  M0 (the LDS base) needs one wait state between its SALU
// write and the copy that reads it, hence the s_nop.
__device__ __forceinline__ void lds_dma16(u32x4 rsrc, uint32_t lds_off, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds_off), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}
__device__ __forceinline__ void lds_dma4(u32x4 rsrc, uint32_t lds_off, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds_off), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}
// The same 16-byte copy for the lanes set in `lanes` only.  EXEC is switched
// inside the asm and restored before it ends, so no branch is generated and
// the copy stays in the caller's basic block.
__device__ __forceinline__ void lds_dma16_lanes(u32x4 rsrc, uint32_t lds_off, uint32_t voff, uint32_t soff,
                                                uint64_t lanes) {
  uint64_t saved;
  asm volatile("s_mov_b64 %0, exec\n\ts_mov_b64 exec, %1\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
               "buffer_load_dwordx4 %3, %4, %5 offen lds\n\ts_mov_b64 exec, %0"
               : "=&s"(saved) : "s"(lanes), "s"(lds_off), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

constexpr uint32_t kOOB = 0x80000000u;   // buffer offset past every buffer: reads as zero

// s_waitcnt vmcnt(VM): at most VM vector memory operations of this wave still
// in flight.  Inline asm with a memory clobber, so the compiler keeps every
// memory access on its side of the wait.
template <int VM>
__device__ __forceinline__ void wait_vm() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(VM) : "memory");
}

}  // namespace sharq
