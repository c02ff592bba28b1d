// The whole SharQ layer in one launch for small M (decode: M <= 16 rows; it
// beats the two-launch path up to M = 8 -- 6.1 against 10.0 us at M = 1 for
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

template <bool NORM>
__global__ __launch_bounds__(kFusedThreads) void fused_layer_kernel(FusedArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const FusedLds L = fused_lds(a.K, NORM);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6) & (kFusedWaves - 1);
  float* cs = reinterpret_cast<float*>(smem + L.cs);
  float* inv = reinterpret_cast<float*>(smem + L.inv);

  // ---- RMSNorm: per row the pairwise tree over 32-element chunk subtrees
  if (NORM) {
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

  // ---- the split-K weight stream (as the two-launch small-M kernel with one
  // row block and eight waves): K tiles in chunks of CH per wave, clamped
  // indices, a tile past K gets a zero weight fragment
  const GemmArgs& g = a.g;
  const int KT = L.KT;
  const int64_t nb = blockIdx.x;
  v4f acs = (v4f){0.f, 0.f, 0.f, 0.f}, acr = acs;
  constexpr int CH = 8 * 4 / kFusedWaves;
  for (int base = 0; base < KT; base += kFusedWaves * CH) {
    v8i b[CH], as[CH], ar[CH];
    uint32_t sw[CH], ss[CH], sr[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int kt = base + wave + kFusedWaves * c;
      const int ktc = kt < KT ? kt : KT - 1;
      uint4 wq = *reinterpret_cast<const uint4*>(g.w_codes + (nb * KT + ktc) * 1024 + lane * 16);
      if (kt >= KT) wq = make_uint4(0, 0, 0, 0);
      b[c] = as_operand(wq);
      sw[c] = g.w_scales_dense[(int64_t)ktc * g.w_scales_ld + nb * 64 + lane];
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
  auto kern = norm ? fused_layer_kernel<true> : fused_layer_kernel<false>;
  // the LDS limit is a per-function attribute: set it once per device
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  static std::atomic<bool> attr_set[64][2];
  if (!attr_set[dev][norm].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set[dev][norm].store(true, std::memory_order_release);
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)NB), dim3(kFusedThreads), L.total, stream, a);
  return hipGetLastError();
}

}  // namespace sharq
