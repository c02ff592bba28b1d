// SharQ dual FP4 GEMM for gfx950: Y = deq(Q(S)) deq(W)^T + deq(Q(R)) deq(W)^T.
//
// SharQ paper page (mlsanity), Abstract: a sparse FP4 GEMM processes the
// backbone, a dense FP4 GEMM compensates with the residual, both read one FP4
// weight payload through path-specific scale views.  README page, section
// "Benchmarks": an epilogue fusion sums the two paths.
//
// gfx950 has block-scaled FP4 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4) but no
// sparse FP4 MFMA, so the sparse path is a packed-K scheme: Q(S) stays
// compressed in memory (K/2 codes + 2-bit offsets) and is expanded to dense
// 4-bit codes on chip right before the MFMA.  Both paths then issue the same
// instruction against the same weight fragment into one fp32 accumulator, and
// one store writes the sum.
//
// MFMA 16x16x128 FP4 operand layout (measured): lane l holds row (or column)
// l%16 and K range [32*(l/16), 32*(l/16)+32) as 16 bytes, lower k in the low
// nibble; its scale byte is that row's E8M0 for the same 32-block; the
// accumulator of lane l holds D[4*(l/16)+i][l%16], i = 0..3.
#include "device_common.h"
#include "launch.h"

namespace sharq {

// Expand the compressed 2:4 operand of 32 logical K positions (8 groups):
// codes = 16 kept nibbles (8 bytes, group g in byte g, lower offset in the low
// nibble), meta = 8 nibbles (group g: i0 | i1<<2 at nibble g).  Result: 32
// dense nibbles with zero codes at dropped positions.
__device__ __forceinline__ uint32_t expand_pair(uint32_t cbytes, uint32_t mbyte) {
  uint32_t b0 = cbytes & 0xFFu, b1 = (cbytes >> 8) & 0xFFu;
  uint32_t m0 = mbyte & 0xFu, m1 = (mbyte >> 4) & 0xFu;
  uint32_t o = ((b0 & 0xFu) << ((m0 & 3u) * 4u)) | ((b0 >> 4) << ((m0 >> 2) * 4u));
  o |= (((b1 & 0xFu) << ((m1 & 3u) * 4u)) | ((b1 >> 4) << ((m1 >> 2) * 4u))) << 16;
  return o;
}
__device__ __forceinline__ uint4 expand32(uint2 codes, uint32_t meta) {
  uint4 d;
  d.x = expand_pair(codes.x & 0xFFFFu, meta & 0xFFu);
  d.y = expand_pair(codes.x >> 16, (meta >> 8) & 0xFFu);
  d.z = expand_pair(codes.y & 0xFFFFu, (meta >> 16) & 0xFFu);
  d.w = expand_pair(codes.y >> 16, meta >> 24);
  return d;
}

__device__ __forceinline__ v8i as_operand(uint4 q) {
  v8i r;
  r[0] = (int)q.x; r[1] = (int)q.y; r[2] = (int)q.z; r[3] = (int)q.w;
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

__device__ __forceinline__ v4f mfma_fp4(v8i a, v8i b, v4f c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

// Reference-simple tiling: each wave owns WM x WN MFMA tiles (16x16 each) and
// reads its fragments straight from global memory.  Block = 4 waves as 2x2.
template <int WM, int WN>
__global__ __launch_bounds__(256) void dual_gemm_direct(GemmArgs g) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t m_base = (int64_t)blockIdx.y * (2 * WM * 16) + (wave >> 1) * WM * 16;
  const int64_t n_base = (int64_t)blockIdx.x * (2 * WN * 16) + (wave & 1) * WN * 16;
  const int K = g.K;
  const int64_t K2 = K / 2, K4 = K / 4, K8 = K / 8, K32 = K / 32;
  const int r16 = lane & 15, chunk = lane >> 4;

  v4f acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < K; k0 += 128) {
    const int kk = k0 + 32 * chunk;
    const bool kin = kk < K;
    v8i as[WM], ar[WM], b[WN];
    uint32_t ss[WM], sr[WM], sw_s[WN], sw_d[WN];
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      const int64_t row = m_base + 16 * i + r16;
      const bool ok = kin && row < g.M;
      uint4 rq = ok ? *reinterpret_cast<const uint4*>(g.r_codes + row * K2 + kk / 2) : make_uint4(0, 0, 0, 0);
      uint2 sq = ok ? *reinterpret_cast<const uint2*>(g.s_codes + row * K4 + kk / 4) : make_uint2(0, 0);
      uint32_t mq = ok ? *reinterpret_cast<const uint32_t*>(g.s_meta + row * K8 + kk / 8) : 0u;
      ar[i] = as_operand(rq);
      as[i] = as_operand(expand32(sq, mq));
      ss[i] = ok ? g.s_scales[row * K32 + kk / 32] : 0u;
      sr[i] = ok ? g.r_scales[row * K32 + kk / 32] : 0u;
    }
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int64_t col = n_base + 16 * j + r16;
      const bool ok = kin && col < g.N;
      uint4 wq = ok ? *reinterpret_cast<const uint4*>(g.w_codes + col * K2 + kk / 2) : make_uint4(0, 0, 0, 0);
      b[j] = as_operand(wq);
      sw_s[j] = ok ? g.w_scales_sparse[col * g.w_scales_ld + kk / 32] : 0u;
      sw_d[j] = ok ? g.w_scales_dense[col * g.w_scales_ld + kk / 32] : 0u;
    }
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        acc[i][j] = mfma_fp4(as[i], b[j], acc[i][j], ss[i], sw_s[j]);
        acc[i][j] = mfma_fp4(ar[i], b[j], acc[i][j], sr[i], sw_d[j]);
      }
  }

  // single epilogue store of Y_S + Y_R
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int64_t col = n_base + 16 * j + r16;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int64_t row = m_base + 16 * i + 4 * chunk + t;
        if (row < g.M && col < g.N) {
          if (g.out_bf16) {
            float f = acc[i][j][t];
            uint32_t u = __float_as_uint(f);
            u += 0x7FFFu + ((u >> 16) & 1u);
            reinterpret_cast<uint16_t*>(g.y)[row * g.ldy + col] = (uint16_t)(u >> 16);
          } else {
            reinterpret_cast<float*>(g.y)[row * g.ldy + col] = acc[i][j][t];
          }
        }
      }
    }
}

hipError_t launch_linear(const GemmArgs& a, hipStream_t stream) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  constexpr int WM = 2, WN = 4;
  dim3 grid((unsigned)((a.N + 2 * WN * 16 - 1) / (2 * WN * 16)), (unsigned)((a.M + 2 * WM * 16 - 1) / (2 * WM * 16)));
  hipLaunchKernelGGL((dual_gemm_direct<WM, WN>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sharq
