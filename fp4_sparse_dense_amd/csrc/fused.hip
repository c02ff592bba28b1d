// The whole SharQ layer in one launch for small M (decode: M <= 16 rows; it
// beats the two-launch path up to M = 8 -- 5.1 against 10.0 us at M = 1 for
// K = N = 4096 -- and loses at 16, where the per-workgroup preparation of 16
// rows costs more than the launch it saves).
//
// SharQ paper page (mlsanity), Abstract: the preparation (normalisation, the
// input-adaptive N:M mask, FP4 of the backbone, the residual against the
// quantised backbone, FP4 of the residual) is one fused operator feeding a
// sparse and a dense FP4 GEMM over one weight payload; README page, section
// "Benchmarks": the epilogue sums the two paths.
//
// At decode sizes the preparation is a few thousand elements, far less work
// than one launch costs, and the GEMM streams the weight once.  So every
// workgroup of the weight-streaming kernel prepares the (at most 16) activation
// rows itself into LDS, in the tiled lane order the MFMA reads, and then runs
// exactly the split-K loop of the two-launch path on those operands.  The
// activation never goes to HBM, and the arithmetic -- the preparation and the
// accumulation order -- is the two-launch path's, so the outputs are identical
// bit for bit.
#include <atomic>

#include "device_common.h"
#include "gemm_common.h"
#include "launch.h"
#include "prep_common.h"

namespace sharq {
namespace {

constexpr int kFusedWaves = 8;
constexpr int kFusedThreads = kFusedWaves * 64;

struct FusedArgs {
  const uint16_t* x;
  int64_t ldx;
  int M, K;
  const uint16_t* gamma;   // nullptr: no RMSNorm
  float eps;
  GemmArgs g;              // weight, output, N (activation fields unused)
};

struct FusedLds {
  uint32_t s, r, ss, rs, cs, inv, total;   // byte offsets
  int KT, KC, P;
};

__host__ __device__ inline FusedLds fused_lds(int K, bool norm) {
  FusedLds L;
  L.KT = (K + 127) / 128;
  L.KC = K / 32;
  L.P = 1;
  while (L.P < L.KC) L.P *= 2;
  L.s = 0;
  L.r = L.s + (uint32_t)L.KT * 1024;
  L.ss = L.r + (uint32_t)L.KT * 1024;
  L.rs = L.ss + (uint32_t)L.KT * 64;
  L.cs = (L.rs + (uint32_t)L.KT * 64 + 15) / 16 * 16;
  // the chunk sums of the RMSNorm tree, later the waves' partial outputs
  const uint32_t sums = norm ? 16u * (uint32_t)L.P * 4u : 0u;
  const uint32_t parts = (uint32_t)kFusedWaves * 64u * 16u;
  L.inv = L.cs + (sums > parts ? sums : parts);
  L.total = L.inv + 16 * 4;   // all LDS is dynamic: the kernel's attribute allows 160 KiB of it
  return L;
}

// 32 bf16 held as loaded (16 VGPRs) and widened to binary32 where used
struct Raw32 { uint4 q[4]; };
__device__ __forceinline__ void load_raw(const uint16_t* p, Raw32& r) {
#pragma unroll
  for (int i = 0; i < 4; ++i) r.q[i] = reinterpret_cast<const uint4*>(p)[i];
}
__device__ __forceinline__ void widen(const Raw32& r, float (&v)[32]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {r.q[i].x, r.q[i].y, r.q[i].z, r.q[i].w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      v[8 * i + 2 * h] = bf16_lo(w[h]);
      v[8 * i + 2 * h + 1] = bf16_hi(w[h]);
    }
  }
}

// SMALL (at most kSmallChunks 32-element chunks of the M rows per thread):
// every thread loads its chunks of X (and of gamma) into registers first, then
// issues the weight fragments of the first split-K pass, and prepares the rows
// from registers while the weight is in flight.  Loads retire in issue order,
// so the activation must be requested before the weight for its arithmetic
// not to wait for the weight.  Otherwise the rows are read in the preparation
// loops and the weight afterwards.  The arithmetic is the same either way.
constexpr int kSmallChunks = 2;

template <bool NORM, bool SMALL>
__global__ __launch_bounds__(kFusedThreads) void fused_layer_kernel(FusedArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const FusedLds L = fused_lds(a.K, NORM);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6) & (kFusedWaves - 1);
  float* cs = reinterpret_cast<float*>(smem + L.cs);
  float* inv = reinterpret_cast<float*>(smem + L.inv);

  const GemmArgs& g = a.g;
  const int KT = L.KT;
  const int64_t nb = blockIdx.x;
  constexpr int CH = 8 * 4 / kFusedWaves;
  // weight fragments of one split-K pass (clamped indices; a tile past K gets
  // a zero fragment)
  auto load_w = [&](int base, v8i (&b)[CH], uint32_t (&sw)[CH]) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int kt = base + wave + kFusedWaves * c;
      const int ktc = kt < KT ? kt : KT - 1;
      uint4 wq = *reinterpret_cast<const uint4*>(g.w_codes + (nb * KT + ktc) * 1024 + lane * 16);
      if (kt >= KT) wq = make_uint4(0, 0, 0, 0);
      b[c] = as_operand(wq);
      sw[c] = g.w_scales_dense[(int64_t)ktc * g.w_scales_ld + nb * 64 + lane];
    }
  };
  v8i b0[CH];
  uint32_t sw0[CH];

  if constexpr (SMALL) {
    // ---- chunk q = t + kFusedThreads * i of the M x KC grid, held as bf16
    Raw32 xr[kSmallChunks], gr[kSmallChunks];
    const int nq = a.M * L.KC;
#pragma unroll
    for (int i = 0; i < kSmallChunks; ++i) {
      const int q = t + kFusedThreads * i;
      if (q < nq) {
        const int r = q / L.KC, c = q % L.KC;
        load_raw(a.x + (int64_t)r * a.ldx + 32 * c, xr[i]);
        if (NORM) load_raw(a.gamma + 32 * c, gr[i]);
      }
    }
    load_w(0, b0, sw0);   // requested after the rows: the rows' arithmetic does not wait for it
    if (NORM) {
#pragma unroll
      for (int i = 0; i < kSmallChunks; ++i) {
        const int q = t + kFusedThreads * i;
        if (q < nq) {
          float v[32];
          widen(xr[i], v);
          cs[(q / L.KC) * L.P + q % L.KC] = chunk_sumsq(v);
        }
      }
      for (int it = t; it < a.M * L.P; it += kFusedThreads)
        if (it % L.P >= L.KC) cs[it] = 0.0f;   // the zero padding of the tree
      __syncthreads();
      for (int n = L.P; n > 1; n >>= 1) {
        const int h = n >> 1;
        float tmp[8];
#pragma unroll
        for (int qq = 0; qq < 8; ++qq) {
          const int it = t + qq * kFusedThreads;
          tmp[qq] = it < a.M * h ? cs[(it / h) * L.P + 2 * (it % h)] + cs[(it / h) * L.P + 2 * (it % h) + 1] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int qq = 0; qq < 8; ++qq) {
          const int it = t + qq * kFusedThreads;
          if (it < a.M * h) cs[(it / h) * L.P + (it % h)] = tmp[qq];
        }
        __syncthreads();
      }
      if (t < a.M) inv[t] = rms_inverse(cs[t * L.P], a.K, a.eps);
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < kSmallChunks; ++i) {
      const int q = t + kFusedThreads * i;
      if (q < nq) {
        const int r = q / L.KC, c = q % L.KC;
        float v[32];
        widen(xr[i], v);
        if (NORM) {
          float gm[32];
          widen(gr[i], gm);
          const float iv = inv[r];
#pragma unroll
          for (int e = 0; e < 32; ++e) v[e] = (v[e] * iv) * gm[e];
        }
        const Block32 o = decompose32<false>(v);
        const int kt = c >> 2, tl = (c & 3) * 16 + r;
        *reinterpret_cast<uint4*>(smem + L.s + kt * 1024 + tl * 16) = o.s_codes;
        *reinterpret_cast<uint4*>(smem + L.r + kt * 1024 + tl * 16) = o.r_codes;
        smem[L.ss + kt * 64 + tl] = (uint8_t)o.s_e8;
        smem[L.rs + kt * 64 + tl] = (uint8_t)o.r_e8;
      }
    }
    // rows past M and chunks past K: the outputs of zero input (zero codes and
    // scale bytes)
    for (int bq = t; bq < 16 * L.KT * 4; bq += kFusedThreads) {
      const int r = bq / (L.KT * 4), c = bq % (L.KT * 4);
      if (r < a.M && c < L.KC) continue;
      const int kt = c >> 2, tl = (c & 3) * 16 + r;
      *reinterpret_cast<uint4*>(smem + L.s + kt * 1024 + tl * 16) = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(smem + L.r + kt * 1024 + tl * 16) = make_uint4(0, 0, 0, 0);
      smem[L.ss + kt * 64 + tl] = 0;
      smem[L.rs + kt * 64 + tl] = 0;
    }
    __syncthreads();
  }

  // ---- RMSNorm: per row the pairwise tree over 32-element chunk subtrees
  if (NORM && !SMALL) {
    for (int it = t; it < a.M * L.P; it += kFusedThreads) {
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
      float tmp[8];   // a.M * h <= 16 * 128 = 4 * kFusedThreads items
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int it = t + q * kFusedThreads;
        tmp[q] = it < a.M * h ? cs[(it / h) * L.P + 2 * (it % h)] + cs[(it / h) * L.P + 2 * (it % h) + 1] : 0.0f;
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int it = t + q * kFusedThreads;
        if (it < a.M * h) cs[(it / h) * L.P + (it % h)] = tmp[q];
      }
      __syncthreads();
    }
    if (t < a.M) inv[t] = rms_inverse(cs[t * L.P], a.K, a.eps);
    __syncthreads();
  }

  // ---- decomposition into LDS: block (row r, 32-chunk c) -> tile c/4, lane
  // (c%4)*16 + r.  Rows past M and chunks past K hold zero input's outputs
  // (zero codes, zero scale bytes).  (Issuing several blocks' loads before
  // their arithmetic measured slower: with two waves per SIMD the dependent
  // arithmetic of a block, not the load, sets the pace.)
  if constexpr (!SMALL) {
    for (int b = t; b < 16 * L.KT * 4; b += kFusedThreads) {
      const int r = b / (L.KT * 4), c = b % (L.KT * 4);
      const int kt = c >> 2, tl = (c & 3) * 16 + r;
      uint4 sc = make_uint4(0, 0, 0, 0), rc = make_uint4(0, 0, 0, 0);
      uint32_t se = 0, re = 0;
      if (r < a.M && c < L.KC) {
        float v[32];
        load32(a.x + (int64_t)r * a.ldx + 32 * c, v);
        if (NORM) apply_norm(v, a.gamma + 32 * c, inv[r]);
        const Block32 o = decompose32<false>(v);
        sc = o.s_codes;
        rc = o.r_codes;
        se = o.s_e8;
        re = o.r_e8;
      }
      *reinterpret_cast<uint4*>(smem + L.s + kt * 1024 + tl * 16) = sc;
      *reinterpret_cast<uint4*>(smem + L.r + kt * 1024 + tl * 16) = rc;
      smem[L.ss + kt * 64 + tl] = (uint8_t)se;
      smem[L.rs + kt * 64 + tl] = (uint8_t)re;
    }
    __syncthreads();
  }

  // ---- the split-K weight stream (as the two-launch small-M kernel with one
  // row block and eight waves): K tiles in chunks of CH per wave, clamped
  // indices, a tile past K gets a zero weight fragment
  v4f acs = (v4f){0.f, 0.f, 0.f, 0.f}, acr = acs;
  for (int base = 0; base < KT; base += kFusedWaves * CH) {
    v8i b[CH], as[CH], ar[CH];
    uint32_t sw[CH], ss[CH], sr[CH];
    if (SMALL && base == 0) {
#pragma unroll
      for (int c = 0; c < CH; ++c) { b[c] = b0[c]; sw[c] = sw0[c]; }
    } else {
      load_w(base, b, sw);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int kt = base + wave + kFusedWaves * c;
      const int ktc = kt < KT ? kt : KT - 1;
      ar[c] = as_operand(*reinterpret_cast<const uint4*>(smem + L.r + ktc * 1024 + lane * 16));
      as[c] = as_operand(*reinterpret_cast<const uint4*>(smem + L.s + ktc * 1024 + lane * 16));
      sr[c] = smem[L.rs + ktc * 64 + lane];
      ss[c] = smem[L.ss + ktc * 64 + lane];
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      acs = mfma_fp4(as[c], b[c], acs, ss[c], sw[c]);
      acr = mfma_fp4(ar[c], b[c], acr, sr[c], sw[c]);
    }
  }

  // partial sums of the waves in wave order (the chunk-sum area is free now)
  __syncthreads();
  v4f* part = reinterpret_cast<v4f*>(smem + L.cs);
  part[wave * 64 + lane] = acs + acr;
  __syncthreads();
  if (wave == 0) {
    const int64_t col = nb * 16 + (lane & 15);
    v4f v = part[lane];
#pragma unroll
    for (int w = 1; w < kFusedWaves; ++w) v = v + part[w * 64 + lane];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t row = 4 * (lane >> 4) + q;
      if (row < a.M && col < g.N) store_out(g, row, col, v[q]);
    }
  }
}

}  // namespace

size_t fused_layer_lds_bytes(int K, bool norm) { return fused_lds(K, norm).total; }

hipError_t launch_linear_fused(const uint16_t* x, int M, int K, int64_t ldx, const uint16_t* gamma, float eps,
                               const GemmArgs& g, hipStream_t stream) {
  if (M == 0 || g.N == 0) return hipSuccess;
  const int64_t NB = (g.N + 15) / 16;
  if (M > 16 || NB > 0x7FFFFFFF) return hipErrorInvalidValue;
  const bool norm = gamma != nullptr;
  const FusedLds L = fused_lds(K, norm);
  if (L.total > 160 * 1024) return hipErrorInvalidValue;
  FusedArgs a;
  a.x = x;
  a.ldx = ldx;
  a.M = M;
  a.K = K;
  a.gamma = gamma;
  a.eps = eps;
  a.g = g;
  const bool small = (int64_t)M * (K / 32) <= (int64_t)kSmallChunks * kFusedThreads;
  auto kern = norm ? (small ? fused_layer_kernel<true, true> : fused_layer_kernel<true, false>)
                   : (small ? fused_layer_kernel<false, true> : fused_layer_kernel<false, false>);
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
  hipLaunchKernelGGL(kern, dim3((unsigned)NB), dim3(kFusedThreads), L.total, stream, a);
  return hipGetLastError();
}

}  // namespace sharq
