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

__device__ __forceinline__ v8i as_operand(uint4 q) {
  v8i r;
  r[0] = (int)q.x; r[1] = (int)q.y; r[2] = (int)q.z; r[3] = (int)q.w;
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

__device__ __forceinline__ v4f mfma_fp4(v8i a, v8i b, v4f c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

// ---------------------------------------------------------------------------
// 2:4 expansion.  The compressed operand of 32 logical K positions (8 groups)
// is 16 kept nibbles (group g in byte g, lower offset in the low nibble) plus
// 8 metadata nibbles (group g: i0 | i1<<2 in nibble g); codes_lo holds groups
// 0-3, codes_hi groups 4-7.  The result is 32
// dense nibbles with zero codes at dropped positions.  Two groups are handled
// per dword, one in each 16-bit half, with byte permutes and packed shifts.
// ---------------------------------------------------------------------------
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

__device__ __forceinline__ void store_out(const GemmArgs& g, int64_t row, int64_t col, float v) {
  if (g.out_bf16) {
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFu + ((u >> 16) & 1u);
    reinterpret_cast<uint16_t*>(g.y)[row * g.ldy + col] = (uint16_t)(u >> 16);
  } else {
    reinterpret_cast<float*>(g.y)[row * g.ldy + col] = v;
  }
}

// ---------------------------------------------------------------------------
// Direct kernel (small M): each wave owns WM x WN MFMA tiles (16 x 16) and
// reads its fragments straight from global memory.  In the tiled layout a
// fragment is 64 contiguous lanes, so these reads are contiguous too.
// ---------------------------------------------------------------------------
template <int WM, int WN>
__global__ __launch_bounds__(256) void dual_gemm_direct(GemmArgs g) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t RB = (g.M + 15) / 16, NB = (g.N + 15) / 16;
  const int KB = (g.K + 127) / 128;
  const int64_t rb_base = (int64_t)blockIdx.y * (2 * WM) + (wave >> 1) * WM;
  const int64_t nb_base = (int64_t)blockIdx.x * (2 * WN) + (wave & 1) * WN;
  const int r16 = lane & 15, chunk = lane >> 4;

  v4f acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  for (int ks = 0; ks < KB; ++ks) {
    v8i as[WM], ar[WM], b[WN];
    uint32_t ss[WM], sr[WM], sw_s[WN], sw_d[WN];
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      const int64_t rb = rb_base + i;
      const bool ok = rb < RB;
      const int64_t tile = rb * KB + ks;
      uint4 rq = ok ? *reinterpret_cast<const uint4*>(g.r_codes + tile * 1024 + lane * 16) : make_uint4(0, 0, 0, 0);
      const uint2 sq = ok ? *reinterpret_cast<const uint2*>(g.s_codes + tile * 512 + lane * 8) : make_uint2(0, 0);
      const uint32_t lo = sq.x, hi = sq.y;
      uint32_t mq = ok ? *reinterpret_cast<const uint32_t*>(g.s_meta + tile * 256 + lane * 4) : 0x44444444u;
      ar[i] = as_operand(rq);
      as[i] = as_operand(expand_chunk(lo, hi, mq));
      ss[i] = ok ? g.s_scales[((int64_t)ks * RB + rb) * 64 + lane] : 0u;
      sr[i] = ok ? g.r_scales[((int64_t)ks * RB + rb) * 64 + lane] : 0u;
    }
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int64_t nb = nb_base + j;
      const bool ok = nb < NB;
      uint4 wq = ok ? *reinterpret_cast<const uint4*>(g.w_codes + (nb * KB + ks) * 1024 + lane * 16) : make_uint4(0, 0, 0, 0);
      b[j] = as_operand(wq);
      sw_s[j] = ok ? g.w_scales_sparse[(int64_t)ks * g.w_scales_ld + nb * 64 + lane] : 0u;
      sw_d[j] = ok ? g.w_scales_dense[(int64_t)ks * g.w_scales_ld + nb * 64 + lane] : 0u;
    }
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j) acc[i][j] = mfma_fp4(as[i], b[j], acc[i][j], ss[i], sw_s[j]);
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j) acc[i][j] = mfma_fp4(ar[i], b[j], acc[i][j], sr[i], sw_d[j]);
  }

  // single epilogue store of Y_S + Y_R
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int64_t col = (nb_base + j) * 16 + r16;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int64_t row = (rb_base + i) * 16 + 4 * chunk + t;
        if (row < g.M && col < g.N) store_out(g, row, col, acc[i][j][t]);
      }
    }
}

// ---------------------------------------------------------------------------
// Tiled kernel (M > 64).
//
// Operands arrive in the MFMA-tiled layout (16 rows x 128 K per tile, lane
// order), so every global -> LDS copy is a contiguous run: one 1 KiB dense
// tile per instruction, the 512-byte compressed tile and its 256-byte
// metadata, and the scale bytes of a whole tile edge in one go.  Copies are
// buffer loads with an LDS destination (no register staging).  Tiles past the
// padded row count get an out-of-range buffer offset, which reads as zero.
// The compressed backbone of a tile lands in the first 768 bytes of the 1 KiB
// slot it will become, and the wave that copied it expands it in place.  Each
// weight fragment feeds the sparse and the dense MFMA of the same output tile.
// ---------------------------------------------------------------------------
template <int BM, int BN, int NWM, int NWN, int NST>
struct TileCfg {
  static constexpr int kWaves = NWM * NWN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kMB = BM / 16, kNB = BN / 16;       // 16-row blocks
  static constexpr int kWMT = kMB / NWM, kWNT = kNB / NWN;  // MFMA tiles per wave
  static constexpr int kOffAS = 0;
  static constexpr int kOffAR = kMB * 1024;
  static constexpr int kOffB = 2 * kMB * 1024;
  static constexpr int kOffSS = kOffB + kNB * 1024;         // scale bytes, 64 per 16-row block (lane order)
  static constexpr int kOffSR = kOffSS + kMB * 64;
  static constexpr int kOffSW = kOffSR + kMB * 64;
  static constexpr int kStage = kOffSW + kNB * 64;
  static constexpr int kStages = NST;                // LDS ring depth; copies run NST-1 steps ahead
  static_assert(BM % 16 == 0 && BN % 16 == 0 && BM <= 256 && BN <= 256, "tile (scale edge copied by one instruction)");
  static_assert(kMB % NWM == 0 && kNB % NWN == 0, "wave split");
};

template <int BM, int BN, int NWM, int NWN, int NST>
__global__ __launch_bounds__(64 * NWM * NWN) void dual_gemm_tiled(GemmArgs g) {
  using C = TileCfg<BM, BN, NWM, NWN, NST>;
  extern __shared__ __align__(1024) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS targets go to M0
  const int KT = (g.K + 127) / 128;                       // K tiles (zero padded)
  const int64_t RB = (g.M + 15) / 16, NB = (g.N + 15) / 16; // padded 16-row blocks

  // tile selection: blocks on one XCD (block id mod 8) take a contiguous
  // range of tiles, walked M-fastest, so they share weight and activation rows in L2
  const int tiles_m = (int)((g.M + BM - 1) / BM);
  const int tiles_n = (int)((g.N + BN - 1) / BN);
  const int T = tiles_m * tiles_n;
  int t = blockIdx.x;
  if (T % 8 == 0) t = (t % 8) * (T / 8) + t / 8;
  const int64_t rb0 = (int64_t)(t % tiles_m) * C::kMB;      // first 16-row block of the tile
  const int64_t nb0 = (int64_t)(t / tiles_m) * C::kNB;

  const u32x4 rs_sc = make_desc(g.s_codes, (uint64_t)RB * KT * 512);
  const u32x4 rs_sm = make_desc(g.s_meta, (uint64_t)RB * KT * 256);
  const u32x4 rs_ss = make_desc(g.s_scales, (uint64_t)RB * KT * 64);
  const u32x4 rs_rc = make_desc(g.r_codes, (uint64_t)RB * KT * 1024);
  const u32x4 rs_rs = make_desc(g.r_scales, (uint64_t)RB * KT * 64);
  const u32x4 rs_wc = make_desc(g.w_codes, (uint64_t)NB * KT * 1024);
  const u32x4 rs_ws = make_desc(g.w_scales_dense, (uint64_t)KT * (uint64_t)g.w_scales_ld);
  const uint32_t lds0 = lds_addr(smem);
  const int r16 = lane & 15, c4 = lane >> 4;

  // ---- per-lane buffer offsets at K tile 0 (blocks past the padding -> kOOB),
  // hoisted out of the K loop.  A-side blocks and W blocks are dealt to waves
  // round-robin; waves 0, 1, 2 copy the S, R and W scale edges.
  constexpr int kSB = (C::kMB + C::kWaves - 1) / C::kWaves;
  constexpr int kWB = (C::kNB + C::kWaves - 1) / C::kWaves;
  static_assert(C::kWaves >= 3, "scale copies need three waves");

  uint32_t offR[kSB], offC[kSB], offM[kSB];
#pragma unroll
  for (int i = 0; i < kSB; ++i) {
    const int64_t rb = rb0 + wave + i * C::kWaves;
    const bool ok = rb < RB;
    offR[i] = ok ? (uint32_t)(rb * KT) * 1024u + lane * 16 : kOOB;
    offC[i] = ok ? (uint32_t)(rb * KT) * 512u + lane * 16 : kOOB;   // lanes 0..31
    offM[i] = ok ? (uint32_t)(rb * KT) * 256u + lane * 16 : kOOB;   // lanes 0..15
  }
  uint32_t offW[kWB];
#pragma unroll
  for (int i = 0; i < kWB; ++i) {
    const int64_t nb = nb0 + wave + i * C::kWaves;
    offW[i] = nb < NB ? (uint32_t)(nb * KT) * 1024u + lane * 16 : kOOB;
  }
  // scale edge: 16 lanes per 64-byte block; lanes past the tile edge are masked
  const int eb = lane >> 2;   // block of the edge this lane copies
  const uint32_t offScA = rb0 + eb < RB ? (uint32_t)((rb0 + eb) * 64 + (lane & 3) * 16) : kOOB;
  const uint32_t offScW = nb0 + eb < NB ? (uint32_t)((nb0 + eb) * 64 + (lane & 3) * 16) : kOOB;
  const uint32_t strideScA = (uint32_t)RB * 64, strideScW = (uint32_t)g.w_scales_ld;

  // Copy K tile ks into the LDS stage at byte offset st.
  auto issue = [&](int ks, uint32_t st) {
    const uint32_t so1k = (uint32_t)ks * 1024, so512 = (uint32_t)ks * 512, so256 = (uint32_t)ks * 256;
#pragma unroll
    for (int i = 0; i < kSB; ++i) {
      const int b = wave + i * C::kWaves;
      if (b < C::kMB) {
        lds_dma16(rs_rc, st + C::kOffAR + b * 1024, offR[i], so1k);
        const uint32_t as = st + C::kOffAS + b * 1024;
        if (lane < 32) lds_dma16(rs_sc, as, offC[i], so512);
        if (lane < 16) lds_dma16(rs_sm, as + 512, offM[i], so256);
      }
    }
#pragma unroll
    for (int i = 0; i < kWB; ++i) {
      const int b = wave + i * C::kWaves;
      if (b < C::kNB) lds_dma16(rs_wc, st + C::kOffB + b * 1024, offW[i], so1k);
    }
    if (wave == 0 && lane < C::kMB * 4) lds_dma16(rs_ss, st + C::kOffSS, offScA, ks * strideScA);
    if (wave == 1 && lane < C::kMB * 4) lds_dma16(rs_rs, st + C::kOffSR, offScA, ks * strideScA);
    if (wave == 2 && lane < C::kNB * 4) lds_dma16(rs_ws, st + C::kOffSW, offScW, ks * strideScW);
  };

  // Expand this wave's backbone blocks of the stage at st in place: every lane
  // reads its 12 compressed bytes (8 code bytes at 8*lane, 4 metadata bytes at
  // 512 + 4*lane), the wave waits for all of its reads, then
  // every lane writes its 16 dense bytes (a block belongs to one wave).
  auto expand_store = [&](uint8_t* st) {
    uint32_t lo[kSB], hi[kSB], mt[kSB];
#pragma unroll
    for (int i = 0; i < kSB; ++i) {
      const int b = wave + i * C::kWaves;
      if (b < C::kMB) {
        const uint8_t* blk = st + C::kOffAS + b * 1024;
        const uint2 sq = *reinterpret_cast<const uint2*>(blk + lane * 8);
        lo[i] = sq.x;
        hi[i] = sq.y;
        mt[i] = *reinterpret_cast<const uint32_t*>(blk + 512 + lane * 4);
      }
    }
    wait_vm_lgkm<63, 0>();
#pragma unroll
    for (int i = 0; i < kSB; ++i) {
      const int b = wave + i * C::kWaves;
      if (b < C::kMB)
        *reinterpret_cast<uint4*>(st + C::kOffAS + b * 1024 + lane * 16) = expand_chunk(lo[i], hi[i], mt[i]);
    }
  };

  const int wm = wave / NWN, wn = wave % NWN;
  v4f acc[C::kWMT][C::kWNT];
#pragma unroll
  for (int i = 0; i < C::kWMT; ++i)
#pragma unroll
    for (int j = 0; j < C::kWNT; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint8_t* cur) {
    v8i fs[C::kWMT], fr[C::kWMT], fb[C::kWNT];
    uint32_t ss[C::kWMT], sr[C::kWMT], sw[C::kWNT];
#pragma unroll
    for (int i = 0; i < C::kWMT; ++i) {
      const int blk = wm * C::kWMT + i;
      fs[i] = as_operand(*reinterpret_cast<const uint4*>(cur + C::kOffAS + blk * 1024 + lane * 16));
      fr[i] = as_operand(*reinterpret_cast<const uint4*>(cur + C::kOffAR + blk * 1024 + lane * 16));
      ss[i] = cur[C::kOffSS + blk * 64 + lane];
      sr[i] = cur[C::kOffSR + blk * 64 + lane];
    }
#pragma unroll
    for (int j = 0; j < C::kWNT; ++j) {
      const int blk = wn * C::kWNT + j;
      fb[j] = as_operand(*reinterpret_cast<const uint4*>(cur + C::kOffB + blk * 1024 + lane * 16));
      sw[j] = cur[C::kOffSW + blk * 64 + lane];
    }
#pragma unroll
    for (int i = 0; i < C::kWMT; ++i)
#pragma unroll
      for (int j = 0; j < C::kWNT; ++j) acc[i][j] = mfma_fp4(fs[i], fb[j], acc[i][j], ss[i], sw[j]);
#pragma unroll
    for (int i = 0; i < C::kWMT; ++i)
#pragma unroll
      for (int j = 0; j < C::kWNT; ++j) acc[i][j] = mfma_fp4(fr[i], fb[j], acc[i][j], sr[i], sw[j]);
  };

  // Pipeline: an LDS ring of NST stages; copies run D = NST-1 K steps ahead.
  // Before expanding stage ks+1 a wave waits until only the copies of the
  // stages after it are outstanding (vmcnt retires in issue order; every wave
  // issues at least kLoadsMin copies per stage), then all waves meet at a
  // barrier before the stage is read.
  constexpr int D = NST - 1;
  constexpr int kLoadsMin = C::kMB / C::kWaves * 3 + C::kNB / C::kWaves;
  static_assert(kLoadsMin >= 1 && kLoadsMin * (D > 1 ? D - 1 : 1) < 64, "vmcnt range");
  auto stage_off = [&](int ks) { return (uint32_t)((ks % NST) * C::kStage); };
  // wait until at most `newer` stages' copies are still in flight
  auto wait_stages = [&](int newer) {
    static_assert(D <= 5, "wait table");
    switch (newer) {
      case 0: wait_vm_lgkm<0, 15>(); break;
      case 1: wait_vm_lgkm<kLoadsMin, 15>(); break;
      case 2: wait_vm_lgkm<(2 * kLoadsMin < 64 ? 2 * kLoadsMin : 63), 15>(); break;
      case 3: wait_vm_lgkm<(3 * kLoadsMin < 64 ? 3 * kLoadsMin : 63), 15>(); break;
      default: wait_vm_lgkm<(4 * kLoadsMin < 64 ? 4 * kLoadsMin : 63), 15>(); break;
    }
  };

  const int pre = KT < D ? KT : D;     // stages copied before the loop
  for (int s = 0; s < pre; ++s) issue(s, lds0 + stage_off(s));
  wait_stages(pre - 1);
  expand_store(smem + stage_off(0));
  __syncthreads();

  for (int ks = 0; ks < KT; ++ks) {
    if (ks + D < KT) issue(ks + D, lds0 + stage_off(ks + D));
    compute(smem + stage_off(ks));
    if (ks + 1 < KT) {
      const int last = ks + D < KT ? ks + D : KT - 1;   // newest stage copied so far
      wait_stages(last - (ks + 1));
      expand_store(smem + stage_off(ks + 1));
      __syncthreads();
    }
  }

  // single epilogue store of Y_S + Y_R
#pragma unroll
  for (int i = 0; i < C::kWMT; ++i)
#pragma unroll
    for (int j = 0; j < C::kWNT; ++j) {
      const int64_t col = (nb0 + wn * C::kWNT + j) * 16 + r16;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = (rb0 + wm * C::kWMT + i) * 16 + 4 * c4 + q;
        if (row < g.M && col < g.N) store_out(g, row, col, acc[i][j][q]);
      }
    }
}

template <int BM, int BN, int NWM, int NWN, int NST>
static hipError_t launch_tiled(const GemmArgs& a, hipStream_t stream) {
  using C = TileCfg<BM, BN, NWM, NWN, NST>;
  auto kern = dual_gemm_tiled<BM, BN, NWM, NWN, NST>;
  constexpr int lds = C::kStages * C::kStage;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(C::kThreads), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_linear(const GemmArgs& a, hipStream_t stream) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  // the tiled kernel addresses every operand with 31-bit buffer offsets
  const uint64_t kb = (a.K + 127) / 128;
  const bool fits = (uint64_t)((a.M + 15) / 16) * kb * 1024 < 0x7FFFFFFFull &&
                    (uint64_t)((a.N + 15) / 16) * kb * 1024 < 0x7FFFFFFFull;
  if (a.M > 64 && fits) return launch_tiled<256, 192, 4, 2, 3>(a, stream);
  constexpr int WM = 2, WN = 4;
  dim3 grid((unsigned)((a.N + 2 * WN * 16 - 1) / (2 * WN * 16)), (unsigned)((a.M + 2 * WM * 16 - 1) / (2 * WM * 16)));
  hipLaunchKernelGGL((dual_gemm_direct<WM, WN>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sharq
