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

// ---------------------------------------------------------------------------
// Tiled dual GEMM (M > 64, K % 128 == 0).
//
// LDS holds each 16-row x 128-K operand block as 1 KiB in MFMA lane order
// (16 bytes for lane l = row l%16, K chunk l/16), so every fragment read is a
// contiguous 16-byte-per-lane read.  The dense residual codes, the weight
// codes and all scale dwords are copied global -> LDS by buffer loads with the
// LDS destination (no register staging); a lane fetches exactly the 16 bytes
// its LDS slot needs.  The compressed backbone is loaded to registers,
// expanded to dense 4-bit codes and written in the same layout.  Rows past M
// or N are given an out-of-range buffer offset, which the hardware turns into
// zeros.  Each weight fragment feeds the sparse and the dense MFMA of the same
// output tile; all products accumulate in one register tile.
// ---------------------------------------------------------------------------
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Expand two 2:4 groups (code bytes at bits [8h, 8h+16) of cw, metadata byte
// mb) into one dword of 8 dense nibbles, using 16-bit halves for the groups.
template <int H>
__device__ __forceinline__ uint32_t expand_dword(uint32_t cw, uint32_t mb4, int j) {
  // codes: group 2j' byte to half 0, next byte to half 1 (zero-extended)
  constexpr uint32_t sel = H == 0 ? 0x0C010C00u : 0x0C030C02u;
  const uint32_t d = __builtin_amdgcn_perm(0u, cw, sel);
  const uint32_t lo = d & 0x000F000Fu, hi = d & 0x00F000F0u;
  // metadata byte j of mb4 to both halves, then the second half's nibble down
  const uint32_t msel = 0x0C000C00u | (uint32_t)j | ((uint32_t)j << 16);
  uint32_t t = __builtin_amdgcn_perm(0u, mb4, msel);
  t = t >> (uint32_t)0 ;  // keep as dword; halves: (mb, mb)
  u16x2 tv = __builtin_bit_cast(u16x2, t);
  tv = tv >> (u16x2){0, 4};
  t = __builtin_bit_cast(uint32_t, tv);
  const uint32_t sl = (t << 2) & 0x000C000Cu;            // 4*i0 per half
  const uint32_t sh = (t & 0x000C000Cu) - 0x00040004u;   // 4*i1 - 4 per half (i1 >= 1)
  const u16x2 los = __builtin_bit_cast(u16x2, lo) << __builtin_bit_cast(u16x2, sl);
  const u16x2 his = __builtin_bit_cast(u16x2, hi) << __builtin_bit_cast(u16x2, sh);
  return __builtin_bit_cast(uint32_t, los) | __builtin_bit_cast(uint32_t, his);
}

__device__ __forceinline__ uint4 expand_chunk(uint2 codes, uint32_t meta) {
  uint4 d;
  d.x = expand_dword<0>(codes.x, meta, 0);
  d.y = expand_dword<1>(codes.x, meta, 1);
  d.z = expand_dword<0>(codes.y, meta, 2);
  d.w = expand_dword<1>(codes.y, meta, 3);
  return d;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void lds_copy4(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 4, voff, soff, 0, 0);
}

constexpr uint32_t kOOB = 0x80000000u;   // buffer offset past every buffer: reads as zero

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint64_t bytes) {
  const int n = bytes >= 0x7FFFFFFFull ? 0x7FFFFFFF : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}

template <int BM, int BN, int NWM, int NWN>
struct TileCfg {
  static constexpr int kWaves = NWM * NWN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kMB = BM / 16, kNB = BN / 16;     // 16-row blocks
  static constexpr int kWMT = kMB / NWM, kWNT = kNB / NWN; // MFMA tiles per wave
  static constexpr int kOffAS = 0;
  static constexpr int kOffAR = kMB * 1024;
  static constexpr int kOffB = 2 * kMB * 1024;
  static constexpr int kOffSS = kOffB + kNB * 1024;       // scale dword per row (4 K-blocks)
  static constexpr int kOffSR = kOffSS + BM * 4;
  static constexpr int kOffSW = kOffSR + BM * 4;
  static constexpr int kStage = kOffSW + ((BN + 63) / 64) * 256;  // W scale groups of 64 rows
  static_assert(BM % 64 == 0 && BN % 16 == 0, "tile");
  static_assert(kMB % NWM == 0 && kNB % NWN == 0, "wave split");
};

template <int BM, int BN, int NWM, int NWN>
__global__ __launch_bounds__(64 * NWM * NWN) void dual_gemm_tiled(GemmArgs g) {
  using C = TileCfg<BM, BN, NWM, NWN>;
  extern __shared__ __align__(1024) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS targets go to M0
  const int K = g.K;
  const uint32_t K2 = K / 2, K4 = K / 4, K8 = K / 8, K32 = K / 32;
  const int KT = K / 128;

  // ---- tile selection: blocks on one XCD (block id mod 8) take a contiguous
  // range of tiles, walked M-fastest, so they share weight and activation rows in L2
  const int tiles_m = (int)((g.M + BM - 1) / BM);
  const int tiles_n = (int)((g.N + BN - 1) / BN);
  const int T = tiles_m * tiles_n;
  int t = blockIdx.x;
  if (T % 8 == 0) t = (t % 8) * (T / 8) + t / 8;
  const int64_t m0 = (int64_t)(t % tiles_m) * BM;
  const int64_t n0 = (int64_t)(t / tiles_m) * BN;

  const __amdgpu_buffer_rsrc_t rs_sc = make_rsrc(g.s_codes, (uint64_t)g.M * K4);
  const __amdgpu_buffer_rsrc_t rs_sm = make_rsrc(g.s_meta, (uint64_t)g.M * K8);
  const __amdgpu_buffer_rsrc_t rs_ss = make_rsrc(g.s_scales, (uint64_t)g.M * K32);
  const __amdgpu_buffer_rsrc_t rs_rc = make_rsrc(g.r_codes, (uint64_t)g.M * K2);
  const __amdgpu_buffer_rsrc_t rs_rs = make_rsrc(g.r_scales, (uint64_t)g.M * K32);
  const __amdgpu_buffer_rsrc_t rs_wc = make_rsrc(g.w_codes, (uint64_t)g.N * K2);
  const __amdgpu_buffer_rsrc_t rs_ws = make_rsrc(g.w_scales_dense, (uint64_t)g.N * (uint64_t)g.w_scales_ld);

  const int r16 = lane & 15, c4 = lane >> 4;

  // ---- per-lane buffer offsets at K step 0 (invalid rows -> kOOB), hoisted out of the K loop
  // S/R blocks and W blocks are dealt to waves round-robin; scale rows go in
  // groups of 64 (one lane per row): S groups, then R groups, then W groups.
  constexpr int kSB = (C::kMB + C::kWaves - 1) / C::kWaves;
  constexpr int kWB = (C::kNB + C::kWaves - 1) / C::kWaves;
  constexpr int kScA = BM / 64, kScW = (BN + 63) / 64, kNQ = 2 * kScA + kScW;
  constexpr int kQB = (kNQ + C::kWaves - 1) / C::kWaves;

  uint32_t offR[kSB], offC[kSB], offM[kSB];
#pragma unroll
  for (int i = 0; i < kSB; ++i) {
    const int64_t row = m0 + (int64_t)(wave + i * C::kWaves) * 16 + r16;
    const bool ok = row < g.M;
    offR[i] = ok ? (uint32_t)row * K2 + c4 * 16 : kOOB;
    offC[i] = ok ? (uint32_t)row * K4 + c4 * 8 : kOOB;
    offM[i] = ok ? (uint32_t)row * K8 + c4 * 4 : kOOB;
  }
  uint32_t offW[kWB];
#pragma unroll
  for (int i = 0; i < kWB; ++i) {
    const int64_t row = n0 + (int64_t)(wave + i * C::kWaves) * 16 + r16;
    offW[i] = row < g.N ? (uint32_t)row * K2 + c4 * 16 : kOOB;
  }
  uint32_t offQ[kQB];
  int kindQ[kQB], ldsQ[kQB];
#pragma unroll
  for (int j = 0; j < kQB; ++j) {
    const int q = wave + j * C::kWaves;
    kindQ[j] = 3;
    offQ[j] = kOOB;
    ldsQ[j] = 0;
    if (q < kScA) {
      const int64_t row = m0 + q * 64 + lane;
      kindQ[j] = 0; ldsQ[j] = C::kOffSS + q * 256;
      offQ[j] = row < g.M ? (uint32_t)row * K32 : kOOB;
    } else if (q < 2 * kScA) {
      const int64_t row = m0 + (q - kScA) * 64 + lane;
      kindQ[j] = 1; ldsQ[j] = C::kOffSR + (q - kScA) * 256;
      offQ[j] = row < g.M ? (uint32_t)row * K32 : kOOB;
    } else if (q < kNQ) {
      const int qq = q - 2 * kScA;
      const int64_t row = n0 + qq * 64 + lane;
      kindQ[j] = 2; ldsQ[j] = C::kOffSW + qq * 256;
      offQ[j] = (row < g.N && qq * 64 + lane < BN) ? (uint32_t)row * (uint32_t)g.w_scales_ld : kOOB;
    }
  }

  uint2 scode[kSB];
  uint32_t smeta[kSB];

  auto issue = [&](int ks, uint8_t* st) {
    const uint32_t so2 = (uint32_t)ks * 64, so4 = (uint32_t)ks * 32, so8 = (uint32_t)ks * 16, so32 = (uint32_t)ks * 4;
#pragma unroll
    for (int i = 0; i < kSB; ++i) {
      const int b = wave + i * C::kWaves;
      if (b < C::kMB) {
        lds_copy16(rs_rc, st + C::kOffAR + b * 1024, offR[i], so2);
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b32(rs_sc, offC[i], so4, 0);
        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b32(rs_sc, offC[i] + 4, so4, 0);
        scode[i] = make_uint2(lo, hi);
        smeta[i] = __builtin_amdgcn_raw_buffer_load_b32(rs_sm, offM[i], so8, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < kWB; ++i) {
      const int b = wave + i * C::kWaves;
      if (b < C::kNB) lds_copy16(rs_wc, st + C::kOffB + b * 1024, offW[i], so2);
    }
#pragma unroll
    for (int j = 0; j < kQB; ++j) {
      if (kindQ[j] == 0) lds_copy4(rs_ss, st + ldsQ[j], offQ[j], so32);
      else if (kindQ[j] == 1) lds_copy4(rs_rs, st + ldsQ[j], offQ[j], so32);
      else if (kindQ[j] == 2) lds_copy4(rs_ws, st + ldsQ[j], offQ[j], so32);
    }
  };
  auto expand_store = [&](uint8_t* st) {
#pragma unroll
    for (int i = 0; i < kSB; ++i) {
      const int b = wave + i * C::kWaves;
      if (b < C::kMB) {
        const uint4 d = expand_chunk(scode[i], smeta[i]);
        *reinterpret_cast<uint4*>(st + C::kOffAS + b * 1024 + lane * 16) = d;
      }
    }
  };

  const int wm = wave / NWN, wn = wave % NWN;
  v4f acc[C::kWMT][C::kWNT];
#pragma unroll
  for (int i = 0; i < C::kWMT; ++i)
#pragma unroll
    for (int j = 0; j < C::kWNT; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  issue(0, smem);
  expand_store(smem);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int ks = 0; ks < KT; ++ks) {
    uint8_t* cur = smem + (ks & 1) * C::kStage;
    uint8_t* nxt = smem + ((ks + 1) & 1) * C::kStage;
    if (ks + 1 < KT) issue(ks + 1, nxt);

    v8i fs[C::kWMT], fr[C::kWMT], fb[C::kWNT];
    uint32_t ss[C::kWMT], sr[C::kWMT], sw[C::kWNT];
#pragma unroll
    for (int i = 0; i < C::kWMT; ++i) {
      const int blk = wm * C::kWMT + i;
      fs[i] = as_operand(*reinterpret_cast<const uint4*>(cur + C::kOffAS + blk * 1024 + lane * 16));
      fr[i] = as_operand(*reinterpret_cast<const uint4*>(cur + C::kOffAR + blk * 1024 + lane * 16));
      ss[i] = cur[C::kOffSS + (blk * 16 + r16) * 4 + c4];
      sr[i] = cur[C::kOffSR + (blk * 16 + r16) * 4 + c4];
    }
#pragma unroll
    for (int j = 0; j < C::kWNT; ++j) {
      const int blk = wn * C::kWNT + j;
      fb[j] = as_operand(*reinterpret_cast<const uint4*>(cur + C::kOffB + blk * 1024 + lane * 16));
      sw[j] = cur[C::kOffSW + (blk * 16 + r16) * 4 + c4];
    }
#pragma unroll
    for (int i = 0; i < C::kWMT; ++i)
#pragma unroll
      for (int j = 0; j < C::kWNT; ++j) acc[i][j] = mfma_fp4(fs[i], fb[j], acc[i][j], ss[i], sw[j]);
#pragma unroll
    for (int i = 0; i < C::kWMT; ++i)
#pragma unroll
      for (int j = 0; j < C::kWNT; ++j) acc[i][j] = mfma_fp4(fr[i], fb[j], acc[i][j], sr[i], sw[j]);

    if (ks + 1 < KT) expand_store(nxt);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // single epilogue store of Y_S + Y_R
#pragma unroll
  for (int i = 0; i < C::kWMT; ++i)
#pragma unroll
    for (int j = 0; j < C::kWNT; ++j) {
      const int64_t col = n0 + (wn * C::kWNT + j) * 16 + r16;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = m0 + (wm * C::kWMT + i) * 16 + 4 * c4 + q;
        if (row < g.M && col < g.N) {
          if (g.out_bf16) {
            uint32_t u = __float_as_uint(acc[i][j][q]);
            u += 0x7FFFu + ((u >> 16) & 1u);
            reinterpret_cast<uint16_t*>(g.y)[row * g.ldy + col] = (uint16_t)(u >> 16);
          } else {
            reinterpret_cast<float*>(g.y)[row * g.ldy + col] = acc[i][j][q];
          }
        }
      }
    }
}

template <int BM, int BN, int NWM, int NWN>
static hipError_t launch_tiled(const GemmArgs& a, hipStream_t stream) {
  using C = TileCfg<BM, BN, NWM, NWN>;
  auto kern = dual_gemm_tiled<BM, BN, NWM, NWN>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 2 * C::kStage);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(C::kThreads), 2 * C::kStage, stream, a);
  return hipGetLastError();
}

hipError_t launch_linear(const GemmArgs& a, hipStream_t stream) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  // the tiled kernel addresses every operand with 31-bit buffer offsets
  const bool fits = (uint64_t)a.M * (a.K / 2) < 0x7FFFFFFFull && (uint64_t)a.N * (a.K / 2) < 0x7FFFFFFFull;
  if (a.K % 128 == 0 && a.M > 64 && fits) return launch_tiled<256, 192, 4, 2>(a, stream);
  constexpr int WM = 2, WN = 4;
  dim3 grid((unsigned)((a.N + 2 * WN * 16 - 1) / (2 * WN * 16)), (unsigned)((a.M + 2 * WM * 16 - 1) / (2 * WM * 16)));
  hipLaunchKernelGGL((dual_gemm_direct<WM, WN>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sharq
