// SharQ dual FP4 GEMM for gfx950: Y = deq(Q(S)) deq(W)^T + deq(Q(R)) deq(W)^T.
//
// SharQ paper page (mlsanity), Abstract: a sparse FP4 GEMM processes the
// backbone, a dense FP4 GEMM compensates with the residual, both read one FP4
// weight payload, each through its own view of the scales.  README page, section
// "Benchmarks": an epilogue fusion sums the two paths.
//
// gfx950 has block-scaled FP4 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4) but no
// sparse FP4 MFMA, so the backbone Q(S) is a masked dense operand: its kept
// codes in place and zero codes at the dropped positions (the preparation
// writes it so, beside the 2:4 metadata).  Both paths then issue the same
// instruction against the same weight fragment into one fp32 accumulator, and
// one store writes the sum.
//
// MFMA 16x16x128 FP4 operand layout (measured): lane l holds row (or column)
// l%16 and K range [32*(l/16), 32*(l/16)+32) as 16 bytes, lower k in the low
// nibble; its scale byte is that row's E8M0 for the same 32-block; the
// accumulator of lane l holds D[4*(l/16)+i][l%16], i = 0..3.
#include <atomic>

#include "device_common.h"
#include "gemm_common.h"
#include "launch.h"
#include "prep_common.h"

namespace sharq {

// ---------------------------------------------------------------------------
// Small-M kernel (decode, M <= 64): the weight is streamed once and the work
// is HBM-bound on it.  One workgroup per CBG 16-column blocks of W and RBG
// 16-row blocks; its NW waves split K (wave w takes K tiles w, w+NW, ...) and
// read their fragments straight from global memory -- in the tiled layout a
// fragment is 64 lanes x 16 contiguous bytes, so each read is one contiguous
// KiB.  With MASK, lanes of rows past M load no codes (zeros instead).  The
// NW partial sums meet in LDS and are added in wave order.  Both paths read
// the weight scales through one load: the API admits only views of one scale
// array.
// ---------------------------------------------------------------------------
template <int RBG, int NW, bool DENSE, int CBG = 1, bool MASK = false>
__global__ __launch_bounds__(64 * NW) void dual_gemm_splitk(GemmArgs g) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & (NW - 1);
  const int64_t RB = (g.M + 15) / 16;
  const int64_t NBt = (g.N + 15) / 16;
  const int KT = (g.K + 127) / 128;
  const int64_t nb0 = (int64_t)blockIdx.x * CBG;      // first 16-column block
  const int64_t rb0 = (int64_t)blockIdx.y * RBG;      // first 16-row block
  const int r16 = lane & 15, c4 = lane >> 4;

  // one accumulator per path (shorter dependent MFMA chains); Y_S + Y_R is
  // formed once, before the cross-wave sum
  v4f acs[CBG][RBG], acr[CBG][RBG];
#pragma unroll
  for (int n = 0; n < CBG; ++n)
#pragma unroll
    for (int r = 0; r < RBG; ++r) acs[n][r] = acr[n][r] = (v4f){0.f, 0.f, 0.f, 0.f};

  // K tiles in chunks of CH per wave, all loads of a chunk issued before its
  // MFMAs (K = 4096 with eight waves: every K tile of a wave in one chunk, one
  // memory round trip).  Indices are clamped into range: a tile past K gets a
  // zero weight fragment (it adds exactly zero) and a row block past the
  // padding only feeds output rows that are never stored.
  constexpr int CH = 32 / NW;
  for (int base = 0; base < KT; base += NW * CH) {
    v8i b[CH][CBG], as[CH][RBG], ar[CH][RBG];
    uint32_t sw[CH][CBG], ss[CH][RBG], sr[CH][RBG];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int kt = base + wave + NW * c;
      const int ktc = kt < KT ? kt : KT - 1;
#pragma unroll
      for (int n = 0; n < CBG; ++n) {
        const int64_t nb = nb0 + n < NBt ? nb0 + n : NBt - 1;   // past N: only feeds columns never stored
        uint4 wq = *reinterpret_cast<const uint4*>(g.w_codes + (nb * KT + ktc) * 1024 + lane * 16);
        if (kt >= KT) wq = make_uint4(0, 0, 0, 0);
        b[c][n] = as_operand(wq);
        sw[c][n] = g.w_scales_dense[(int64_t)ktc * g.w_scales_ld + nb * 64 + lane];   // both views (one array)
      }
#pragma unroll
      for (int r = 0; r < RBG; ++r) {
        const int64_t rb = rb0 + r < RB ? rb0 + r : RB - 1;
        const int64_t tile = rb * KT + ktc;
        const bool live = !MASK || (rb * 16 + r16 < g.M);
        uint4 rq = make_uint4(0, 0, 0, 0);
        if (live) rq = *reinterpret_cast<const uint4*>(g.r_codes + tile * 1024 + lane * 16);
        sr[c][r] = g.r_scales[((int64_t)ktc * RB + rb) * 64 + lane];
        ar[c][r] = as_operand(rq);
        if constexpr (!DENSE) {
          uint4 sq = make_uint4(0, 0, 0, 0);
          if (live) sq = *reinterpret_cast<const uint4*>(g.s_codes + tile * 1024 + lane * 16);
          ss[c][r] = g.s_scales[((int64_t)ktc * RB + rb) * 64 + lane];
          as[c][r] = as_operand(sq);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int n = 0; n < CBG; ++n)
#pragma unroll
        for (int r = 0; r < RBG; ++r) {
          if constexpr (!DENSE) acs[n][r] = mfma_fp4(as[c][r], b[c][n], acs[n][r], ss[c][r], sw[c][n]);
          acr[n][r] = mfma_fp4(ar[c][r], b[c][n], acr[n][r], sr[c][r], sw[c][n]);
        }
  }

  // partial sums of the waves, added in wave order; one store of Y_S + Y_R
  // (column block n of the group by wave n mod NW)
  __shared__ v4f part[NW][CBG][RBG][64];
#pragma unroll
  for (int n = 0; n < CBG; ++n)
#pragma unroll
    for (int r = 0; r < RBG; ++r) part[wave][n][r][lane] = acs[n][r] + acr[n][r];
  __syncthreads();
#pragma unroll
  for (int n = 0; n < CBG; ++n) {
    if (wave != n % NW) continue;
    const int64_t col = (nb0 + n) * 16 + r16;
#pragma unroll
    for (int r = 0; r < RBG; ++r) {
      v4f v = part[0][n][r][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) v = v + part[w][n][r][lane];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = (rb0 + r) * 16 + 4 * c4 + q;
        if (row < g.M && col < g.N) store_out(g, row, col, v[q]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Tiled kernel (M > 64).
//
// Operands arrive in the MFMA-tiled layout (16 rows x 128 K per tile, lane
// order), so every global -> LDS copy is a contiguous run: one 1 KiB tile
// (backbone, residual or weight) per instruction and the scale bytes of a
// whole tile edge in one go.  Copies are buffer loads with an LDS destination
// (no register staging).  Tiles past the padded row count get an out-of-range
// buffer offset, which reads as zero.  Each weight fragment feeds the sparse
// and the dense MFMA of the same output tile.
// ---------------------------------------------------------------------------
template <bool B> struct BoolTag { static constexpr bool value = B; };
// lane mask of lanes 0 .. n-1 (n <= 64)
constexpr uint64_t low_lanes(int n) { return n >= 64 ? ~0ull : ((1ull << n) - 1); }

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

// One 16x16 output block of the tiled kernel, computed transposed: the weight
// fragment is the MFMA's first operand and the activation fragment its second,
// so lane (c4 = lane / 16, r16 = lane % 16) accumulates output row r16, columns
// 4*c4 .. 4*c4+3 of the block -- four consecutive outputs of one row, stored
// with one 16-byte (fp32) or 8-byte (bf16) write.
__device__ __forceinline__ v4f mfma_yt(v8i act, v8i w, v4f c, uint32_t s_act, uint32_t s_w) {
  return mfma_fp4(w, act, c, s_w, s_act);
}

// SWIGLU: 0 = store Y; 1 = store H = bf16(SiLU(gate) * up) of the column
// pairs; 2 = prepare H for the next layer (2:4, MXFP4, no RMSNorm) straight
// from the tile, H never stored.
template <int BM, int BN, int NWM, int NWN, int NST, bool GROUPED, bool DENSE, int SWIGLU>
__global__ __launch_bounds__(64 * NWM * NWN) void dual_gemm_tiled(GemmArgs g) {
  using C = TileCfg<BM, BN, NWM, NWN, NST>;
  extern __shared__ __align__(1024) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  static_assert((C::kWaves & (C::kWaves - 1)) == 0, "wave count is a power of two");
  // uniform (LDS targets go to M0); the mask tells the compiler wave < kWaves
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (C::kWaves - 1);
  const int KT = (g.K + 127) / 128;                       // K tiles (zero padded)
  const int64_t RB = g.a_blocks, NB = (g.N + 15) / 16;   // padded 16-row blocks

  // Tile of this workgroup: activation row blocks [rb0, rb0 + kMB) (valid below
  // rb_end), weight column blocks [nb0, nb0 + kNB) (valid below nb_end); output
  // row of activation block rb, row r: y_row0 + (rb - rb_first) * 16 + r, valid
  // below y_rows; output column of weight block nb, column c:
  // (nb - nb_first) * 16 + c, valid below y_cols.
  int64_t rb0, nb0, rb_end, nb_end, rb_first, nb_first, y_row0, y_rows, y_cols;
  if constexpr (!GROUPED) {
    // Workgroups on one XCD (block id mod 8) take one region of xcd_bm M tiles
    // x bn N tiles, so the activation and weight tiles they share stay in that
    // XCD's L2 (the host picks the region shape with the fewest bytes per XCD);
    // without a region shape the tiles are dealt in plain order.
    const int tiles_m = (int)((g.M + BM - 1) / BM);
    const int tiles_n = (int)((g.N + BN - 1) / BN);
    const int T = tiles_m * tiles_n;
    const int t = blockIdx.x;
    int tm, tn;
    if (g.xcd_bm > 0) {
      const int bm = g.xcd_bm, bn = T / 8 / bm;
      const int x = t % 8, i = t / 8;                  // XCD, index on it
      const int regions_m = tiles_m / bm;
      tm = (x % regions_m) * bm + i % bm;
      tn = (x / regions_m) * bn + i / bm;
    } else {
      tm = t % tiles_m;
      tn = t / tiles_m;
    }
    rb0 = (int64_t)tm * C::kMB;
    nb0 = (int64_t)tn * C::kNB;
    rb_end = RB; nb_end = NB; rb_first = 0; nb_first = 0;
    y_row0 = 0; y_rows = g.M; y_cols = g.N;
  } else {
    // (expert, M tile, N tile): M tiles of all experts are numbered through
    // tprefix; the weight holds the experts' column blocks one after another
    // The T = (M tiles) x tiles_n units, numbered M tile major, are cut into 8
    // contiguous runs of `per`, one per XCD (workgroup b runs on XCD b mod 8,
    // as its b / 8-th): an M tile's N tiles then run side by side on one XCD
    // and share its activation tile in that L2, and an expert's M tiles stay
    // together, sharing its weight.  (Dealt in plain order, N tile j of every M
    // tile went to one XCD and each XCD read the whole activation.)  The grid
    // is a multiple of 8 holding at least T units; the rest return.
    const int64_t NBe = (uint32_t)NB / (uint32_t)g.E;            // 32-bit division (NB < 2^31)
    const int tiles_n = (int)((NBe + C::kNB - 1) / C::kNB);
    const int64_t T = (int64_t)g.tprefix[g.E] * tiles_n;
    const int64_t per = (T + 7) / 8;
    const int64_t i_x = blockIdx.x / 8;
    const int64_t u = (int64_t)(blockIdx.x % 8) * per + i_x;
    if (i_x >= per || u >= T) return;               // the whole workgroup: past the last unit
    const int nt = (int)((uint32_t)u % (uint32_t)tiles_n);     // u < 2^31: 32-bit division
    const int mtg = (int)((uint32_t)u / (uint32_t)tiles_n);
    const int e = g.texp[mtg];                       // tprefix[e] <= mtg < tprefix[e+1]
    rb_first = g.pseg[e];
    rb0 = rb_first + (int64_t)(mtg - g.tprefix[e]) * C::kMB;
    rb_end = g.pseg[e + 1];
    nb_first = (int64_t)e * NBe;
    nb0 = nb_first + (int64_t)nt * C::kNB;
    nb_end = nb_first + NBe;
    y_row0 = g.seg[e];
    y_rows = g.seg[e + 1] - g.seg[e];
    y_cols = NBe * 16;                              // N_e (a multiple of 16)
  }

  const int64_t RBc = GROUPED && g.gather ? g.src_blocks : RB;   // blocks of the code buffers
  const u32x4 rs_sc = make_desc(g.s_codes, (uint64_t)RBc * KT * 1024);
  const u32x4 rs_ss = make_desc(g.s_scales, (uint64_t)RB * KT * 64);
  const u32x4 rs_rc = make_desc(g.r_codes, (uint64_t)RBc * KT * 1024);
  const u32x4 rs_rs = make_desc(g.r_scales, (uint64_t)RB * KT * 64);
  const u32x4 rs_wc = make_desc(g.w_codes, (uint64_t)NB * KT * 1024);
  const u32x4 rs_ws = make_desc(g.w_scales_dense, (uint64_t)KT * (uint64_t)g.w_scales_ld);
  const uint32_t lds0 = lds_addr(smem);
  const int r16 = lane & 15, c4 = lane >> 4;

  // ---- copies.  A-side blocks and weight blocks are dealt to waves round
  // robin; a wave whose share of weight blocks runs past the tile copies one
  // of the first blocks again, and the three scale edges go to waves w % 3, so
  // that every wave issues the same kItems copies per K step with no branch
  // (identical data written twice to one place is harmless).  Per-lane buffer
  // offsets are taken at K tile 0 (blocks past the padding -> kOOB) and
  // hoisted out of the K loop.
  static_assert(C::kMB % C::kWaves == 0, "A-side blocks split evenly over the waves");
  static_assert(!(DENSE && GROUPED), "the grouped layer runs both paths");
  constexpr int kSB = C::kMB / C::kWaves;
  constexpr int kWB = (C::kNB + C::kWaves - 1) / C::kWaves;
  constexpr int kPerA = DENSE ? 1 : 2;                 // copies per A-side block
  constexpr int kEdges = DENSE ? 2 : 3;                // scale edges
  constexpr int kItems = kPerA * kSB + kWB + 1;
  static_assert(C::kWaves >= kEdges, "one wave per scale edge");

  uint32_t offA[kSB];   // both A-side operands: 1 KiB tiles, rb-major then K
#pragma unroll
  for (int i = 0; i < kSB; ++i) {
    const int64_t rb = rb0 + wave + i * C::kWaves;
    offA[i] = rb < rb_end ? (uint32_t)(rb * KT) * 1024u + lane * 16 : kOOB;
    if constexpr (GROUPED) {
      if (g.gather) {
        // this lane's piece (row r16, 32-element chunk c4) of routed row lr of
        // the expert, taken from its source row's piece; rows past the expert
        // or out of range read as zero
        const int64_t lr = (rb - rb_first) * 16 + r16;
        int64_t src = -1;
        if (rb < rb_end && lr < y_rows) src = g.row_index ? (int64_t)g.row_index[y_row0 + lr] : y_row0 + lr;
        offA[i] = src >= 0 && src < g.src_rows
                      ? (uint32_t)((src >> 4) * KT) * 1024u + (uint32_t)(c4 * 16 + (int)(src & 15)) * 16u
                      : kOOB;
      }
    }
  }
  int wblk[kWB];
  uint32_t offW[kWB];
#pragma unroll
  for (int i = 0; i < kWB; ++i) {
    const int b = wave + i * C::kWaves;
    wblk[i] = b < C::kNB ? b : b - C::kNB;
    const int64_t nb = nb0 + wblk[i];
    offW[i] = nb < nb_end ? (uint32_t)(nb * KT) * 1024u + lane * 16 : kOOB;
  }
  // scale edge of this wave: 0 = backbone, 1 = residual, 2 = weight (without
  // a backbone: 1 or 2); 16 lanes per 64-byte block
  const int edge = DENSE ? 1 + wave % 2 : wave % 3;
  const int eb = lane >> 2;   // block of the edge this lane copies
  const uint32_t offScA = rb0 + eb < rb_end ? (uint32_t)((rb0 + eb) * 64 + (lane & 3) * 16) : kOOB;
  const uint32_t offScW = nb0 + eb < nb_end ? (uint32_t)((nb0 + eb) * 64 + (lane & 3) * 16) : kOOB;
  const u32x4 rs_edge = edge == 0 ? rs_ss : (edge == 1 ? rs_rs : rs_ws);
  const uint32_t off_edge = edge == 2 ? offScW : offScA;
  const uint32_t stride_edge = edge == 2 ? (uint32_t)g.w_scales_ld : (uint32_t)RB * 64;
  const uint32_t lds_edge = edge == 0 ? C::kOffSS : (edge == 1 ? C::kOffSR : C::kOffSW);
  const uint64_t lanes_edge = edge == 2 ? low_lanes(C::kNB * 4) : low_lanes(C::kMB * 4);

  // copy item `it` of K step ks into the LDS stage at st: per A-side block the
  // residual tile and (with a backbone) the backbone tile, one per weight
  // block, then the scale edge
  auto issue_item = [&](int it, int ks, uint32_t st) {
    if (it < kPerA * kSB) {
      const int i = it / kPerA, kind = it % kPerA;
      const int b = wave + i * C::kWaves;
      if (kind == 0) lds_dma16(rs_rc, st + C::kOffAR + b * 1024, offA[i], (uint32_t)ks * 1024);
      else lds_dma16(rs_sc, st + C::kOffAS + b * 1024, offA[i], (uint32_t)ks * 1024);
    } else if (it < kPerA * kSB + kWB) {
      const int i = it - kPerA * kSB;
      lds_dma16(rs_wc, st + C::kOffB + wblk[i] * 1024, offW[i], (uint32_t)ks * 1024);
    } else {
      lds_dma16_lanes(rs_edge, st + lds_edge, off_edge, (uint32_t)ks * stride_edge, lanes_edge);
    }
  };
  auto issue = [&](int ks, uint32_t st) {
#pragma unroll
    for (int it = 0; it < kItems; ++it) issue_item(it, ks, st);
  };

  const int wm = wave / NWN, wn = wave % NWN;
  v4f acc[C::kWMT][C::kWNT];
#pragma unroll
  for (int i = 0; i < C::kWMT; ++i)
#pragma unroll
    for (int j = 0; j < C::kWNT; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  // operand fragments of one K step (lane order: one 16-byte load per block)
  auto frag = [&](const uint8_t* st, int off, int blk) {
    return as_operand(*reinterpret_cast<const uint4*>(st + off + blk * 1024 + lane * 16));
  };
  v8i fs[C::kWMT], fr[C::kWMT], fb[C::kWNT];
  uint32_t ss[C::kWMT], sr[C::kWMT], sw[C::kWNT];
  auto read_all = [&](const uint8_t* st) {
#pragma unroll
    for (int i = 0; i < C::kWMT; ++i) {
      const int blk = wm * C::kWMT + i;
      if constexpr (!DENSE) {
        fs[i] = frag(st, C::kOffAS, blk);
        ss[i] = st[C::kOffSS + blk * 64 + lane];
      }
      fr[i] = frag(st, C::kOffAR, blk);
      sr[i] = st[C::kOffSR + blk * 64 + lane];
    }
#pragma unroll
    for (int j = 0; j < C::kWNT; ++j) {
      const int blk = wn * C::kWNT + j;
      fb[j] = frag(st, C::kOffB, blk);
      sw[j] = st[C::kOffSW + blk * 64 + lane];
    }
  };

  // Pipeline: an LDS ring of NST stages, one K step each.  The prologue copies
  // steps 0..NST-1; step ks waits until only this wave's copies of later steps
  // than ks+1 are outstanding (loads retire in issue order; each step is
  // kItems copies), runs the backbone MFMAs of ks (fragments already in
  // registers), meets the other waves at one barrier -- after it step ks+1 is
  // in LDS and nobody reads step ks's slot any more -- then runs the residual
  // MFMAs of ks while it issues the copy of step ks+NST into that slot and
  // reads the fragments of step ks+1.
  static_assert(kItems * (NST > 2 ? NST - 2 : 1) < 64, "vmcnt range");
  auto stage_off = [&](int ks) { return (uint32_t)((ks % NST) * C::kStage); };
  auto wait_stages = [&](int newer) {
    static_assert(NST <= 6, "wait table");
    switch (newer) {
      case 0: wait_vm<0>(); break;
      case 1: wait_vm<kItems>(); break;
      case 2: wait_vm<(2 * kItems < 64 ? 2 * kItems : 63)>(); break;
      case 3: wait_vm<(3 * kItems < 64 ? 3 * kItems : 63)>(); break;
      default: wait_vm<(4 * kItems < 64 ? 4 * kItems : 63)>(); break;
    }
  };

  const int pre = KT < NST ? KT : NST;   // steps copied before the loop
  for (int s = 0; s < pre; ++s) issue(s, lds0 + stage_off(s));
  wait_stages(pre - 1);
  __syncthreads();
  read_all(smem + stage_off(0));

  // one K step (not the last); COPY: issue the copy of step ks+NST
  auto step = [&](int ks, int newer, auto copy_tag) {
    constexpr bool kCopy = decltype(copy_tag)::value;
    wait_stages(newer);
#pragma unroll
    for (int i = 0; i < C::kWMT; ++i)
#pragma unroll
      for (int j = 0; j < C::kWNT; ++j) acc[i][j] = mfma_yt(fs[i], fb[j], acc[i][j], ss[i], sw[j]);
    __builtin_amdgcn_sched_barrier(0);
    // the residual fragments of step ks were read from its slot at the end of
    // the previous step: those reads must be complete before the barrier
    // after which the slot is refilled (long done by now: no wait in practice)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();
    const uint32_t cst = lds0 + stage_off(ks);   // slot of step ks, free after the barrier
    const uint8_t* nx = smem + stage_off(ks + 1);
    // the backbone fragments are free: refill them first
#pragma unroll
    for (int i = 0; i < C::kWMT; ++i) {
      const int blk = wm * C::kWMT + i;
      fs[i] = frag(nx, C::kOffAS, blk);
      ss[i] = nx[C::kOffSS + blk * 64 + lane];
    }
    // residual MFMAs column by column; a weight fragment is refilled right
    // after its last use, the residual fragments after the last column; the
    // copies are spread over the columns
#pragma unroll
    for (int j = 0; j < C::kWNT; ++j) {
#pragma unroll
      for (int i = 0; i < C::kWMT; ++i) acc[i][j] = mfma_yt(fr[i], fb[j], acc[i][j], sr[i], sw[j]);
      __builtin_amdgcn_sched_barrier(0);   // keep the refill after the column's last use
      const int blk = wn * C::kWNT + j;
      fb[j] = frag(nx, C::kOffB, blk);
      sw[j] = nx[C::kOffSW + blk * 64 + lane];
      if constexpr (kCopy) {
#pragma unroll
        for (int it = j * kItems / C::kWNT; it < (j + 1) * kItems / C::kWNT; ++it) issue_item(it, ks + NST, cst);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < C::kWMT; ++i) {
      const int blk = wm * C::kWMT + i;
      fr[i] = frag(nx, C::kOffAR, blk);
      sr[i] = nx[C::kOffSR + blk * 64 + lane];
    }
  };
  // one K step without a backbone: the first half of the columns runs on the
  // fragments already in registers before the barrier, the rest after it;
  // every weight fragment is refilled after its column, the residual
  // fragments after the last column, the copies spread over the columns
  auto step_dense = [&](int ks, int newer, auto copy_tag) {
    constexpr bool kCopy = decltype(copy_tag)::value;
    constexpr int JH = C::kWNT / 2;
    wait_stages(newer);
#pragma unroll
    for (int j = 0; j < JH; ++j)
#pragma unroll
      for (int i = 0; i < C::kWMT; ++i) acc[i][j] = mfma_yt(fr[i], fb[j], acc[i][j], sr[i], sw[j]);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // every read of step ks's slot is complete
    __syncthreads();
    const uint32_t cst = lds0 + stage_off(ks);
    const uint8_t* nx = smem + stage_off(ks + 1);
#pragma unroll
    for (int j = 0; j < C::kWNT; ++j) {
      if (j >= JH) {
#pragma unroll
        for (int i = 0; i < C::kWMT; ++i) acc[i][j] = mfma_yt(fr[i], fb[j], acc[i][j], sr[i], sw[j]);
      }
      __builtin_amdgcn_sched_barrier(0);
      const int blk = wn * C::kWNT + j;
      fb[j] = frag(nx, C::kOffB, blk);
      sw[j] = nx[C::kOffSW + blk * 64 + lane];
      if constexpr (kCopy) {
#pragma unroll
        for (int it = j * kItems / C::kWNT; it < (j + 1) * kItems / C::kWNT; ++it) issue_item(it, ks + NST, cst);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < C::kWMT; ++i) {
      const int blk = wm * C::kWMT + i;
      fr[i] = frag(nx, C::kOffAR, blk);
      sr[i] = nx[C::kOffSR + blk * 64 + lane];
    }
  };

  int ks = 0;
  // steady state: copies issued so far end at step ks+NST-1, so NST-2 steps
  // are newer than ks+1
  if constexpr (DENSE) {
    for (; ks + NST < KT; ++ks) step_dense(ks, NST - 2, BoolTag<true>{});
    for (; ks + 1 < KT; ++ks) step_dense(ks, KT - 2 - ks, BoolTag<false>{});
  } else {
    for (; ks + NST < KT; ++ks) step(ks, NST - 2, BoolTag<true>{});
    for (; ks + 1 < KT; ++ks) step(ks, KT - 2 - ks, BoolTag<false>{});
  }
  // last step
  if constexpr (!DENSE) {
#pragma unroll
    for (int i = 0; i < C::kWMT; ++i)
#pragma unroll
      for (int j = 0; j < C::kWNT; ++j) acc[i][j] = mfma_yt(fs[i], fb[j], acc[i][j], ss[i], sw[j]);
  }
#pragma unroll
  for (int j = 0; j < C::kWNT; ++j)
#pragma unroll
    for (int i = 0; i < C::kWMT; ++i) acc[i][j] = mfma_yt(fr[i], fb[j], acc[i][j], sr[i], sw[j]);

  // single epilogue store of Y_S + Y_R
  if constexpr (SWIGLU != 0) {
    static_assert(!DENSE && (SWIGLU == 2 || !GROUPED), "the SwiGLU epilogue follows the 2:4 layer");
    // the wave's column blocks pair up as (gate, up): the tile starts at an
    // even block (BN/16 is even) and so does each wave's share
    static_assert(C::kWNT % 2 == 0 && C::kNB % 2 == 0, "gate/up pairs inside a wave");
    const int64_t hcols = y_cols / 2;
    auto h_bits = [&](int i, int j, uint32_t (&hb)[4]) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float gt = acc[i][j][q], up = acc[i][j + 1][q];
        hb[q] = bf16_bits_rne(gt / (1.0f + expf(-gt)) * up);
      }
    };
    if constexpr (SWIGLU == 1) {
      const bool vec = ((uintptr_t)g.y & 7) == 0 && (g.ldy & 3) == 0;
#pragma unroll
      for (int i = 0; i < C::kWMT; ++i)
#pragma unroll
        for (int j = 0; j < C::kWNT; j += 2) {
          const int64_t row = (rb0 + wm * C::kWMT + i) * 16 + r16;
          const int64_t col = (nb0 + wn * C::kWNT + j) / 2 * 16 + 4 * c4;
          uint32_t hb[4];
          h_bits(i, j, hb);
          if (row >= y_rows) continue;
          uint16_t* dst = reinterpret_cast<uint16_t*>(g.y) + row * g.ldy + col;
          if (vec && col + 3 < hcols) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(hb[0] | hb[1] << 16, hb[2] | hb[3] << 16);
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (col + q < hcols) dst[q] = (uint16_t)hb[q];
          }
        }
    } else {
      // H of the tile (BM rows x BN/2 columns, bf16) goes to LDS -- rows
      // padded to an odd number of 16-byte units so the block reads below hit
      // distinct banks -- then every thread prepares whole 32-column blocks of
      // it as sharq_prepare does (no RMSNorm: v = H) and writes them into the
      // next activation's tiled layout.  F = N/2 is a multiple of 128, so the
      // next layer's K tiles hold no padding; its padding rows (past M, below
      // the last 16-row block) come from zero activation rows and so hold the
      // outputs of zero input, as the preparation writes them.
      constexpr int kHCols = BN / 2, kHStride = kHCols + 8;       // bf16 elements per LDS row
      static_assert(kHCols % 32 == 0 && ((kHStride * 2 / 16) & 1) == 1, "H staging layout");
      static_assert(BM * kHStride * 2 <= C::kStages * C::kStage, "H fits the LDS ring");
      __syncthreads();   // every wave has consumed its last fragments: the ring is free
      uint16_t* hs = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
      for (int i = 0; i < C::kWMT; ++i)
#pragma unroll
        for (int j = 0; j < C::kWNT; j += 2) {
          uint32_t hb[4];
          h_bits(i, j, hb);
          const int lrow = (wm * C::kWMT + i) * 16 + r16, lcol = (wn * C::kWNT + j) / 2 * 16 + 4 * c4;
          *reinterpret_cast<uint2*>(hs + lrow * kHStride + lcol) = make_uint2(hb[0] | hb[1] << 16, hb[2] | hb[3] << 16);
        }
      __syncthreads();
      //
      // Grouped: the tile's rows are an expert's padded routed rows and H goes
      // to routed row y_row0 + (row within the expert), so the next activation
      // holds the routed rows in order, unpadded, as sharq_prepare lays out
      // the rows of H.  The expert's padding rows are not written (that row
      // of the next activation belongs to the next expert, or is its own
      // padding, which the host fills).
      const PrepOut& o = g.next;
      const int64_t RBn = GROUPED ? (g.M + 15) / 16 : g.a_blocks, KTn = hcols / 128;
      const int64_t kb0 = (nb0 - nb_first) / 4;                   // the tile's first 32-column block of H
      constexpr int kBlk = BM * kHCols / 32;
      for (int t = tid; t < kBlk; t += C::kThreads) {
        const int rl = t & 15, rbl = (t >> 4) % C::kMB, b = t / (16 * C::kMB);
        const int64_t kb = kb0 + b;
        int64_t rb = rb0 + rbl;
        int r = rl;
        if constexpr (GROUPED) {
          const int64_t lr = (rb0 - rb_first + rbl) * 16 + rl, yr = y_row0 + lr;
          if (lr >= y_rows) continue;
          rb = yr >> 4;
          r = (int)(yr & 15);
        }
        if (rb >= RBn || kb * 32 >= hcols) continue;
        const uint4* src = reinterpret_cast<const uint4*>(hs + (rbl * 16 + rl) * kHStride + b * 32);
        float v[32];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 w4 = src[q];
          const uint32_t wd[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[8 * q + 2 * e] = __uint_as_float(wd[e] << 16);
            v[8 * q + 2 * e + 1] = __uint_as_float(wd[e] & 0xFFFF0000u);
          }
        }
        const Block32 d = decompose32<false>(v);
        const int64_t kt = kb / 4, c = kb % 4, tile = rb * KTn + kt, tl = c * 16 + r;
        *reinterpret_cast<uint4*>(o.r_codes + tile * 1024 + tl * 16) = d.r_codes;
        *reinterpret_cast<uint4*>(o.s_codes + tile * 1024 + tl * 16) = d.s_codes;
        *reinterpret_cast<uint32_t*>(o.s_meta + tile * 256 + tl * 4) = d.meta;
        const int64_t sc = (kt * RBn + rb) * 64 + tl;
        o.s_scales[sc] = (uint8_t)d.s_e8;
        o.r_scales[sc] = (uint8_t)d.r_e8;
      }
    }
    return;
  }
  // Staged epilogue.  The lanes hold 64- (fp32) or 32-byte (bf16) pieces of
  // rows, which the memory system writes at a fraction of its line rate, so
  // each wave stages its blocks in LDS and writes whole 16-byte pieces in row
  // order, consecutive lanes along a row.  The pieces go out as non-temporal
  // stores: nothing here reads Y back, and keeping it out of the caches leaves
  // them to the operand tiles (QKV-shaped GEMM 53.9 -> 52.2 us, the grouped
  // K = 768 expert layer 138 -> 117 us).
  //
  // The grouped layer's ring (two stages) holds one 16-row block per wave at a
  // time, and its tiles are ragged (an expert's last rows, a last N tile past
  // N_e): each wave stages its blocks one by one and skips the pieces outside
  // Y.  N_e is a multiple of 16, so a 16-byte piece is wholly in or out.
  if constexpr (GROUPED) {
    constexpr int kSt = C::kWNT * 16 + 4;                 // floats per staged row (+4: banks)
    static_assert(C::kWaves * 16 * kSt * 4 <= C::kStages * C::kStage, "staging fits the LDS ring");
    const int eb = g.out_bf16 ? 2 : 4;
    const bool al = ((uintptr_t)g.y & 15) == 0 && ((g.ldy * eb) & 15) == 0 && y_cols % 8 == 0 && !g.resid;
    if (al) {
      __syncthreads();   // every wave has consumed its last fragments: the ring is free
      float* st = reinterpret_cast<float*>(smem) + wave * 16 * kSt;
      const int64_t col0 = (nb0 - nb_first + wn * C::kWNT) * 16;
#pragma unroll
      for (int i = 0; i < C::kWMT; ++i) {
#pragma unroll
        for (int j = 0; j < C::kWNT; ++j)
          *reinterpret_cast<v4f*>(st + r16 * kSt + 16 * j + 4 * c4) = acc[i][j];
        const int64_t row0 = (rb0 - rb_first + wm * C::kWMT + i) * 16;
        if (g.out_bf16) {
          constexpr int kPpr = C::kWNT * 2;                 // 8-element pieces per row
          static_assert(16 * kPpr % 64 == 0, "whole lanes per block");
#pragma unroll
          for (int k = 0; k < 16 * kPpr / 64; ++k) {
            const int pc = lane + 64 * k, r = pc / kPpr, c = (pc % kPpr) * 8;
            const v4f a = *reinterpret_cast<const v4f*>(st + r * kSt + c);
            const v4f b = *reinterpret_cast<const v4f*>(st + r * kSt + c + 4);
            const int64_t row = row0 + r, col = col0 + c;
            if (row < y_rows && col < y_cols)
              __builtin_nontemporal_store(
                  (u32x4){bf16_bits_rne(a[0]) | bf16_bits_rne(a[1]) << 16, bf16_bits_rne(a[2]) | bf16_bits_rne(a[3]) << 16,
                        bf16_bits_rne(b[0]) | bf16_bits_rne(b[1]) << 16, bf16_bits_rne(b[2]) | bf16_bits_rne(b[3]) << 16},
                  reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(g.y) + (y_row0 + row) * g.ldy + col));
          }
        } else {
          constexpr int kPpr = C::kWNT * 4;                 // 4-element pieces per row
          static_assert(16 * kPpr % 64 == 0, "whole lanes per block");
#pragma unroll
          for (int k = 0; k < 16 * kPpr / 64; ++k) {
            const int pc = lane + 64 * k, r = pc / kPpr, c = (pc % kPpr) * 4;
            const v4f a = *reinterpret_cast<const v4f*>(st + r * kSt + c);
            const int64_t row = row0 + r, col = col0 + c;
            if (row < y_rows && col < y_cols)
              __builtin_nontemporal_store(a, reinterpret_cast<v4f*>(reinterpret_cast<float*>(g.y) + (y_row0 + row) * g.ldy + col));
          }
        }
      }
      return;
    }
  }
  // A single problem's tile goes out this way when it lies wholly inside Y
  // with 16-byte-aligned rows, in rounds of kRB 16-row blocks per wave; the
  // residual add and the rounding are those of store_out.
  if constexpr (!GROUPED) {
    constexpr int kSt = C::kWNT * 16 + 4;                 // floats per staged row (+4: banks)
    // rounds of kRB 16-row blocks per wave: two where 32 rows fit the ring, else one
    constexpr int kRB = C::kWMT % 2 == 0 && C::kWaves * 32 * kSt * 4 <= C::kStages * C::kStage ? 2 : 1;
    static_assert(C::kWaves * 16 * kRB * kSt * 4 <= C::kStages * C::kStage, "staging fits the LDS ring");
    const int eb = g.out_bf16 ? 2 : 4;
    const bool full = (rb0 + C::kMB) * 16 <= y_rows && (nb0 + C::kNB) * 16 <= y_cols;
    const bool al = ((uintptr_t)g.y & 15) == 0 && ((g.ldy * eb) & 15) == 0 &&
                    (!g.resid || (((uintptr_t)g.resid & 15) == 0 && (g.ld_resid & 7) == 0));
    if (full && al) {
      __syncthreads();   // every wave has consumed its last fragments: the ring is free
      float* st = reinterpret_cast<float*>(smem) + wave * 16 * kRB * kSt;
      const int64_t col0 = (nb0 + wn * C::kWNT) * 16;
#pragma unroll
      for (int h = 0; h < C::kWMT / kRB; ++h) {
#pragma unroll
        for (int ii = 0; ii < kRB; ++ii)
#pragma unroll
          for (int j = 0; j < C::kWNT; ++j)
            *reinterpret_cast<v4f*>(st + (ii * 16 + r16) * kSt + 16 * j + 4 * c4) = acc[kRB * h + ii][j];
        const int64_t row0 = (rb0 + wm * C::kWMT + kRB * h) * 16;
        if (g.out_bf16) {
          constexpr int kPpr = C::kWNT * 2;                 // 8-element pieces per row
#pragma unroll
          for (int k = 0; k < 16 * kRB * kPpr / 64; ++k) {
            const int pc = lane + 64 * k, r = pc / kPpr, c = (pc % kPpr) * 8;
            v4f a = *reinterpret_cast<const v4f*>(st + r * kSt + c);
            v4f b = *reinterpret_cast<const v4f*>(st + r * kSt + c + 4);
            const int64_t row = y_row0 + row0 + r, col = col0 + c;
            if (g.resid) {
              const uint4 x = *reinterpret_cast<const uint4*>(g.resid + row * g.ld_resid + col);
              a[0] = __uint_as_float(x.x << 16) + a[0];
              a[1] = __uint_as_float(x.x & 0xFFFF0000u) + a[1];
              a[2] = __uint_as_float(x.y << 16) + a[2];
              a[3] = __uint_as_float(x.y & 0xFFFF0000u) + a[3];
              b[0] = __uint_as_float(x.z << 16) + b[0];
              b[1] = __uint_as_float(x.z & 0xFFFF0000u) + b[1];
              b[2] = __uint_as_float(x.w << 16) + b[2];
              b[3] = __uint_as_float(x.w & 0xFFFF0000u) + b[3];
            }
            __builtin_nontemporal_store(
                (u32x4){bf16_bits_rne(a[0]) | bf16_bits_rne(a[1]) << 16, bf16_bits_rne(a[2]) | bf16_bits_rne(a[3]) << 16,
                      bf16_bits_rne(b[0]) | bf16_bits_rne(b[1]) << 16, bf16_bits_rne(b[2]) | bf16_bits_rne(b[3]) << 16},
                reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(g.y) + row * g.ldy + col));
          }
        } else {
          constexpr int kPpr = C::kWNT * 4;                 // 4-element pieces per row
#pragma unroll
          for (int k = 0; k < 16 * kRB * kPpr / 64; ++k) {
            const int pc = lane + 64 * k, r = pc / kPpr, c = (pc % kPpr) * 4;
            const v4f a = *reinterpret_cast<const v4f*>(st + r * kSt + c);
            __builtin_nontemporal_store(a, reinterpret_cast<v4f*>(reinterpret_cast<float*>(g.y) + (y_row0 + row0 + r) * g.ldy + col0 + c));
          }
        }
      }
      return;
    }
  }
  // four consecutive outputs per lane and block: one 16-byte (fp32) or 8-byte
  // (bf16) store where the row stride and base allow it and all four columns
  // exist, else element by element
  const bool vec = ((uintptr_t)g.y & 15) == 0 && (g.ldy & 3) == 0 &&
                   (!g.resid || (((uintptr_t)g.resid & 7) == 0 && (g.ld_resid & 3) == 0));
#pragma unroll
  for (int i = 0; i < C::kWMT; ++i)
#pragma unroll
    for (int j = 0; j < C::kWNT; ++j) {
      const int64_t row = (rb0 - rb_first + wm * C::kWMT + i) * 16 + r16;
      const int64_t col = (nb0 - nb_first + wn * C::kWNT + j) * 16 + 4 * c4;
      if (row >= y_rows) continue;
      if (vec && col + 3 < y_cols) {
        store_out4(g, y_row0 + row, col, acc[i][j]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (col + q < y_cols) store_out(g, y_row0 + row, col + q, acc[i][j][q]);
      }
    }
}

template <int BM, int BN, int NWM, int NWN, int NST, bool GROUPED, bool DENSE, int SWIGLU = 0>
static hipError_t launch_tiled(const GemmArgs& a, int64_t tiles, hipStream_t stream) {
  using C = TileCfg<BM, BN, NWM, NWN, NST>;
  auto kern = dual_gemm_tiled<BM, BN, NWM, NWN, NST, GROUPED, DENSE, SWIGLU>;
  constexpr int lds = C::kStages * C::kStage;
  // the LDS limit is a per-function attribute: set it once per device
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  static std::atomic<bool> attr_set[64];
  if (!attr_set[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_set[dev].store(true, std::memory_order_release);
  }
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(C::kThreads), lds, stream, a);
  return hipGetLastError();
}

// tile shape of the tiled kernel
constexpr int kTileM = 256, kTileN = 192, kTileNarrowM = 128, kTileNarrowN = 256;
// The grouped (expert) layer runs 128-row tiles with a two-stage LDS ring
// (61 KiB): two workgroups share a CU, so one's prologue and output stores
// overlap the other's MFMAs -- the experts' K is short (768 to 2048) -- and a
// small expert wastes fewer padded rows.  (Qwen3-30B-A3B-shaped MoE: gate/up
// 240 -> 219 us, down 181 -> 160 us; the same tile with three stages, one
// workgroup per CU, is slower than 256-row tiles.)
constexpr int kGroupedTileM = 128;
int grouped_tile_m() { return kGroupedTileM; }

// compute units of the current device (cached per device), <= 0 on error
int compute_units() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  static std::atomic<int> cached[64];
  int n = cached[dev].load(std::memory_order_acquire);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return -1;
  cached[dev].store(n, std::memory_order_release);
  return n;
}

// M tiles per XCD region for a tm x tn tile grid split into 8 equal regions of
// bm x bn tiles: the shape that minimises the operand bytes one XCD reads
// (bm activation tiles at 1.0625 B/elem, bn weight tiles at 0.53125 B/elem);
// 0 when no such split exists.
static int xcd_region_m(int64_t tm, int64_t tn, int bm_rows, int bn_cols) {
  const int64_t T = tm * tn;
  if (T % 8 != 0) return 0;
  const int64_t per = T / 8;
  int best = 0;
  double best_cost = 0.0;
  for (int64_t bm = 1; bm <= tm && bm <= per; ++bm) {
    if (tm % bm || per % bm) continue;
    const int64_t bn = per / bm;
    if (tn % bn) continue;
    const double cost = (double)bm * bm_rows * 1.0625 + (double)bn * bn_cols * 0.53125;
    if (best == 0 || cost < best_cost) { best = (int)bm; best_cost = cost; }
  }
  return best;
}

hipError_t launch_linear_grouped_gemm(const GemmArgs& a, int64_t max_mtiles, hipStream_t stream) {
  const int64_t NBe = (a.N / a.E + 15) / 16;
  const int64_t tiles_n = (NBe + kTileN / 16 - 1) / (kTileN / 16);
  // a multiple of 8 workgroups: each XCD's run of units fits its share of the grid
  const int64_t grid = (max_mtiles * tiles_n + 7) / 8 * 8;
  return a.next.r_codes ? launch_tiled<kGroupedTileM, kTileN, 4, 2, 2, true, false, 2>(a, grid, stream)
                        : launch_tiled<kGroupedTileM, kTileN, 4, 2, 2, true, false>(a, grid, stream);
}

template <bool DENSE>
static hipError_t launch_linear_t(const GemmArgs& a, hipStream_t stream) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  // the tiled kernel addresses every operand with 31-bit buffer offsets
  const uint64_t kb = (a.K + 127) / 128;
  const bool fits = (uint64_t)((a.M + 15) / 16) * kb * 1024 < 0x7FFFFFFFull &&
                    (uint64_t)((a.N + 15) / 16) * kb * 1024 < 0x7FFFFFFFull;
  if (a.M > 64 && fits) {
    // 256 x 192 tiles, or 128 x 256 ones (a third fewer outputs) when those
    // need no more waves of one workgroup per compute unit: a grid that already
    // fits in the waves the wider tile needs then runs the smaller one (N =
    // 4096 at M = 2048: 256 tiles fill the chip once where 176 of 256 x 192
    // leave a third of it idle).  128 x 256 rather than 256 x 128: 17% fewer
    // copied bytes per flop (N = 4096 down projection 118.6 -> 114.5 us); its
    // epilogue stages one 16-row block per round.
    const int cus = compute_units();
    if (cus <= 0) return hipErrorInvalidDevice;
    const int64_t tm = (a.M + kTileM - 1) / kTileM, tn_wide = (a.N + kTileN - 1) / kTileN;
    const int64_t tm_n = (a.M + kTileNarrowM - 1) / kTileNarrowM, tn_n = (a.N + kTileNarrowN - 1) / kTileNarrowN;
    const bool narrow = (tm_n * tn_n + cus - 1) / cus <= (tm * tn_wide + cus - 1) / cus;
    GemmArgs b = a;
    if (narrow) {
      b.xcd_bm = xcd_region_m(tm_n, tn_n, kTileNarrowM, kTileNarrowN);
      return launch_tiled<kTileNarrowM, kTileNarrowN, 4, 2, 3, false, DENSE>(b, tm_n * tn_n, stream);
    }
    b.xcd_bm = xcd_region_m(tm, tn_wide, kTileM, kTileN);
    return launch_tiled<kTileM, kTileN, 4, 2, 3, false, DENSE>(b, tm * tn_wide, stream);
  }
  const int64_t RB = (a.M + 15) / 16, NB = (a.N + 15) / 16;
  if (NB > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (a.M > 64) {
    // operands past 31-bit buffer offsets: two row blocks per workgroup
    const int64_t groups = (RB + 1) / 2;
    if (groups > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL((dual_gemm_splitk<2, 8, DENSE>), dim3((unsigned)NB, (unsigned)groups), dim3(512), 0, stream, a);
    return hipGetLastError();
  }
  // M <= 64: split-K weight streaming, eight waves per workgroup of one 16-row
  // block and CBG 16-column blocks, a wave issuing all its K tiles of a K =
  // 4096 row in one chunk.  The kernel is bound by the bytes each compute unit
  // pulls (every workgroup re-reads its row block's activation tiles), so CBG
  // is the largest of 4, 2, 1 that still gives every compute unit a workgroup:
  // K = N = 4096 at M = 32 runs CBG 2 (6.33 -> 5.50 us against one column
  // block and two row blocks per workgroup), at M = 64 CBG 4 (8.46 -> 6.66 us).
  // A partial row block loads only its live rows' codes (the padding rows feed
  // outputs that are never stored), which halves the activation lines read at
  // M <= 8 (M = 1: 4.82 -> 4.47 us); full blocks skip the per-lane test.
  const int cus = compute_units();
  if (cus <= 0) return hipErrorInvalidDevice;
  const int cbg = (NB + 3) / 4 * RB >= cus ? 4 : (NB + 1) / 2 * RB >= cus ? 2 : 1;
  const dim3 grid((unsigned)((NB + cbg - 1) / cbg), (unsigned)RB);
  if (a.M % 16 != 0) {
    if (cbg == 4) hipLaunchKernelGGL((dual_gemm_splitk<1, 8, DENSE, 4, true>), grid, dim3(512), 0, stream, a);
    else if (cbg == 2) hipLaunchKernelGGL((dual_gemm_splitk<1, 8, DENSE, 2, true>), grid, dim3(512), 0, stream, a);
    else hipLaunchKernelGGL((dual_gemm_splitk<1, 8, DENSE, 1, true>), grid, dim3(512), 0, stream, a);
  } else {
    if (cbg == 4) hipLaunchKernelGGL((dual_gemm_splitk<1, 8, DENSE, 4>), grid, dim3(512), 0, stream, a);
    else if (cbg == 2) hipLaunchKernelGGL((dual_gemm_splitk<1, 8, DENSE, 2>), grid, dim3(512), 0, stream, a);
    else hipLaunchKernelGGL((dual_gemm_splitk<1, 8, DENSE, 1>), grid, dim3(512), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_linear(const GemmArgs& a, hipStream_t stream) { return launch_linear_t<false>(a, stream); }

hipError_t launch_linear_swiglu(const GemmArgs& a, hipStream_t stream) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  const uint64_t kb = (a.K + 127) / 128;
  if ((uint64_t)((a.M + 15) / 16) * kb * 1024 >= 0x7FFFFFFFull || (uint64_t)((a.N + 15) / 16) * kb * 1024 >= 0x7FFFFFFFull)
    return hipErrorInvalidValue;
  const int64_t tm = (a.M + kTileM - 1) / kTileM, tn = (a.N + kTileN - 1) / kTileN;
  GemmArgs b = a;
  b.xcd_bm = xcd_region_m(tm, tn, kTileM, kTileN);
  return b.next.r_codes ? launch_tiled<kTileM, kTileN, 4, 2, 3, false, false, 2>(b, tm * tn, stream)
                        : launch_tiled<kTileM, kTileN, 4, 2, 3, false, false, 1>(b, tm * tn, stream);
}

hipError_t launch_linear_dense(const GemmArgs& a, hipStream_t stream) { return launch_linear_t<true>(a, stream); }

}  // namespace sharq
