// Fused SharQ preparation and weight packing for gfx950.
//
// SharQ paper page (mlsanity), Abstract: one preparation operator computes the
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
// All arithmetic is binary32 with no contraction (built with -ffp-contract=off),
// one rounding per operation, in the order the CPU reference states.
#include <atomic>

#include "device_common.h"
#include "launch.h"
#include "prep_common.h"

namespace sharq {

// weight packing: one wave per row, slots of 512 elements, lane l owns
// elements [8l, 8l+8) of a slot (a 32-element block spans an aligned quad)
constexpr int kSlot = 512;
constexpr int kRowsPerBlock = 4;



// ---------------------------------------------------------------------------
// Prep kernel.  A workgroup owns 8 rows (one half of a 16-row tile block) and
// all of K, or one K slice of them without RMSNorm.  K is cut into units of
// 256 elements (two K tiles); wave w of the 16 (or of 4 or 8 for short rows)
// owns the slice's units w, w+16, w+32, ... and streams them through a private ring of LDS
// slots (8 rows x 512 bytes = 4 KiB each) filled by its own global -> LDS
// copies, so no other wave ever waits for them.  The one workgroup-wide step
// is the RMSNorm sum of squares.
//
// Slot layout: copy c (0..3) of a unit fills bytes [1024c, 1024c+1024); its
// lane l brings 16 bytes of row l/8 from unit bytes 128c + 16*((l%8) ^ sw(l/8)).
// A reader lane takes row r8 = l%8, chunk c4 = (l/8)%4 and tile t2 = l/32 (one
// MX block): copy 2*t2 + c4/2, 16-byte pieces (c4%2)*4 + i.  The XOR by
// sw(r) = (r/2)%4 makes each 16-lane phase of those reads touch 16 distinct
// 16-byte bank groups (64 banks x 4 bytes).  Output lane order inside a tile
// is chunk*16 + row, so the 8 lanes of one chunk store one contiguous run.
//
// A wave waits for a unit with a vmcnt equal to the copies it issued after
// that unit (loads complete in order).  A unit's stores are issued one
// iteration late -- after the next unit's copy, before a block of arithmetic --
// so a wait seldom has to cover stores that were just issued.
//
// RMSNorm: the sum of squares of a row is the balanced pairwise tree of its
// zero-padded squares: per block a 32-leaf tree (each square rounded on its
// own, as a square below 2^-126 is not exact), per unit the 8
// blocks by lane exchanges in K order, then the units by an in-place tree in
// LDS over the next power of two.
// ---------------------------------------------------------------------------
constexpr int kPrepRows = 8;
constexpr int kPrepWaves = 16;
constexpr int kUnitK = 256;
constexpr int kSlotBytes = kPrepRows * kUnitK * 2;
constexpr uint32_t kPrepLdsMax = 160 * 1024;
constexpr int kMaxSlots = 4;
// gamma in LDS: each 32-element block padded to 36 binary32 (or 40 bf16)
// words, so the 16-byte reads of the eight distinct blocks a wave touches at
// once (two K tiles x four chunks) fall into eight different bank groups
constexpr uint32_t kGammaBlockF32 = 36, kGammaBlockBf16 = 40;

struct PrepPlan {
  int nunits;      // units of 256 along K
  int ups;         // units per K slice (one slice per workgroup; all units with RMSNorm)
  int units_p2;    // next power of two (RMSNorm tree width)
  int slots;       // LDS slots per wave
  int single;      // RMSNorm rows staged once (every unit of the wave resident)
  int gamma_f32;   // gamma held as binary32 (else bf16 words)
  uint32_t off_gamma, off_sums, total;
};

static PrepPlan prep_plan(int K, bool norm, int waves, int ksplit) {
  PrepPlan p{};
  p.nunits = (K + kUnitK - 1) / kUnitK;
  p.ups = (p.nunits + ksplit - 1) / ksplit;
  p.units_p2 = 1;
  while (p.units_p2 < p.nunits) p.units_p2 *= 2;
  const int per_wave = (p.ups + waves - 1) / waves;
  const uint32_t kp = (uint32_t)p.nunits * kUnitK;
  const uint32_t sums = norm ? (uint32_t)p.units_p2 * kPrepRows * 4 : 0;
  for (int f32 = norm ? 1 : 0; f32 >= 0; --f32) {
    const uint32_t gbytes = norm ? kp / 32u * (f32 ? kGammaBlockF32 * 4u : kGammaBlockBf16 * 2u) : 0;
    const int64_t avail = (int64_t)kPrepLdsMax - gbytes - sums;
    int s = avail > 0 ? (int)(avail / ((int64_t)waves * kSlotBytes)) : 0;
    s = s < kMaxSlots ? s : kMaxSlots;
    p.gamma_f32 = f32;
    p.single = norm && per_wave <= s;
    // a single staging needs one slot per unit; a stream keeps one unit in
    // flight per slot and gains nothing past the wave's units
    const int want = per_wave > 0 ? per_wave : 1;
    p.slots = p.single ? (per_wave > 0 ? per_wave : 1) : (want < s ? want : s);
    p.off_gamma = (uint32_t)p.slots * (uint32_t)waves * kSlotBytes;
    p.off_sums = p.off_gamma + gbytes;
    p.total = p.off_sums + sums;
    if (!norm || p.single || f32 == 0) break;
  }
  return p;
}

// s_waitcnt vmcnt(4n): at most n units (4 copies each) still in flight
__device__ __forceinline__ void wait_units(int n) {
  if (n <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if (n == 1) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if (n == 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
}

template <int W, bool NORM, bool GF32, bool DENSE>
__global__ __launch_bounds__(W * 64) void prep_kernel(const uint16_t* __restrict__ x, int64_t M, int K,
                                                            int64_t ldx, const uint16_t* __restrict__ gamma,
                                                            float eps, PrepPlan P, PrepOut o) {
  extern __shared__ __align__(1024) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // workgroup -> (K slice, 16-row block, half); the two halves of a block are
  // 8 blocks apart in launch order, i.e. on the same XCD, so their L2 merges
  // the writes.  Slice ks holds units [ks * ups, ks * ups + ups) of K.
  const int64_t RB = (M + 15) / 16, nwg = RB * 2;
  const int64_t w = blockIdx.x % (uint32_t)nwg;                  // the grid is < 2^31: 32-bit division
  const int ubase = (int)(blockIdx.x / (uint32_t)nwg) * P.ups;
  const int nunits_here = P.nunits - ubase < P.ups ? P.nunits - ubase : P.ups;
  const int64_t full = nwg / 16 * 16;
  int64_t rb, half;
  if (w < full) { rb = (w / 16) * 8 + (w % 8); half = (w % 16) / 8; }
  else { rb = w / 2; half = w % 2; }
  const int64_t row0 = rb * 16 + half * 8;

  const int KB = (K + 127) / 128;
  const int r8 = lane & 7, c4 = (lane >> 3) & 3, t2 = lane >> 5;
  const bool row_ok = row0 + r8 < M;
  const bool pad_rows = row0 + kPrepRows > M;

  // copy lanes: row lane/8, source piece (lane%8) ^ sw(row)
  const int crow = lane >> 3;
  const int cpiece = (lane & 7) ^ ((crow >> 1) & 3);
  const bool crow_ok = row0 + crow < M;
  const uint32_t clane_off = (uint32_t)crow * (uint32_t)ldx * 2u + (uint32_t)cpiece * 16u;
  const int clane_k = cpiece * 8;
  const int64_t rows_here = M - row0 < kPrepRows ? (M - row0 > 0 ? M - row0 : 0) : kPrepRows;
  const u32x4 desc = make_desc(x + (rows_here > 0 ? row0 : 0) * ldx, (uint64_t)rows_here * (uint64_t)ldx * 2u);

  const uint32_t ring_off = (uint32_t)wave * P.slots * kSlotBytes;
  const uint32_t ring = lds_addr(smem) + ring_off;
  const int nu_w = nunits_here > wave ? (nunits_here - wave + W - 1) / W : 0;
  // streaming look-ahead: one unit per slot.  A slot is refilled as soon as
  // its block reads have returned (the copies need no registers), so all
  // slots can be in flight while a block is being decomposed.
  const int D = P.slots;

  auto issue = [&](int j) {
    const int u = ubase + wave + W * j;
    const uint32_t slot = ring + (uint32_t)(j % P.slots) * kSlotBytes;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int k = u * kUnitK + c * 64 + clane_k;
      const uint32_t off = (crow_ok && k < K) ? clane_off + (uint32_t)u * 512u + (uint32_t)c * 128u : kOOB;
      lds_dma16(desc, slot + (uint32_t)c * 1024u, off, 0);
    }
  };

  const uint32_t rsw = (uint32_t)((r8 >> 1) & 3);
  auto read_block = [&](int j, uint32_t (&xw)[16]) {
    const uint8_t* base = smem + ring_off + (uint32_t)(j % P.slots) * kSlotBytes +
                          (uint32_t)(2 * t2 + (c4 >> 1)) * 1024u + (uint32_t)r8 * 128u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t p = (uint32_t)((c4 & 1) * 4 + i) ^ rsw;
      const uint4 q = *reinterpret_cast<const uint4*>(base + p * 16u);
      xw[4 * i] = q.x; xw[4 * i + 1] = q.y; xw[4 * i + 2] = q.z; xw[4 * i + 3] = q.w;
    }
  };

  // ---- RMSNorm denominator of row r8
  float inv = 1.0f;
  if (NORM) {
    float* sums = reinterpret_cast<float*>(smem + P.off_sums);
    // gamma into LDS (binary32, or bf16 words for long rows), zero past K
    const int kp = P.nunits * kUnitK;
    for (int e = tid * 8; e < kp; e += (W * 64) * 8) {
      const uint4 q = e < K ? *reinterpret_cast<const uint4*>(gamma + e) : make_uint4(0, 0, 0, 0);
      if (GF32) {
        float* gs = reinterpret_cast<float*>(smem + P.off_gamma) + e + (kGammaBlockF32 - 32) * (e / 32);
        *reinterpret_cast<float4*>(gs) = make_float4(bf16_lo(q.x), bf16_hi(q.x), bf16_lo(q.y), bf16_hi(q.y));
        *reinterpret_cast<float4*>(gs + 4) = make_float4(bf16_lo(q.z), bf16_hi(q.z), bf16_lo(q.w), bf16_hi(q.w));
      } else {
        *reinterpret_cast<uint4*>(smem + P.off_gamma + (e + (kGammaBlockBf16 - 32) * (e / 32)) * 2) = q;
      }
    }
    for (int i = P.nunits * kPrepRows + tid; i < P.units_p2 * kPrepRows; i += (W * 64)) sums[i] = 0.0f;

    auto unit_ss = [&](const uint32_t (&xw)[16], int j) {
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float a = bf16_lo(xw[i]), b = bf16_hi(xw[i]);
        p[i] = a * a + b * b;
      }
#pragma unroll
      for (int w2 = 8; w2 >= 1; w2 >>= 1)
#pragma unroll
        for (int i = 0; i < w2; ++i) p[i] = p[2 * i] + p[2 * i + 1];
      float t = p[0];
      t = t + __shfl_xor(t, 8, 64);    // blocks of a tile, in K order
      t = t + __shfl_xor(t, 16, 64);
      t = t + __shfl_xor(t, 32, 64);   // the two tiles of the unit
      if (lane < 8) sums[(ubase + wave + W * j) * kPrepRows + lane] = t;
    };

    if (P.single) {
      for (int j = 0; j < nu_w; ++j) issue(j);
      for (int j = 0; j < nu_w; ++j) {
        wait_units(nu_w - 1 - j);
        uint32_t xw[16];
        read_block(j, xw);
        unit_ss(xw, j);
      }
    } else {
      for (int j = 0; j < D && j < nu_w; ++j) issue(j);
      for (int j = 0; j < nu_w; ++j) {
        wait_units(min(D - 1, nu_w - 1 - j));
        uint32_t xw[16];
        read_block(j, xw);
        if (j + D < nu_w) {
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // slot j % D read back
          issue(j + D);
        }
        unit_ss(xw, j);
      }
    }
    for (int s = 1; s < P.units_p2; s *= 2) {
      __syncthreads();
      const int pairs = P.units_p2 / (2 * s);
      for (int i = tid; i < pairs * kPrepRows; i += (W * 64)) {
        const int a = (i / kPrepRows) * 2 * s, r = i % kPrepRows;
        sums[a * kPrepRows + r] = sums[a * kPrepRows + r] + sums[(a + s) * kPrepRows + r];
      }
    }
    __syncthreads();
    inv = rms_inverse(sums[r8], K, eps);
  }

  // ---- decomposition
  auto compute = [&](const uint32_t (&xw)[16], int j) {
    float v[32];
#pragma unroll
    for (int i = 0; i < 16; ++i) { v[2 * i] = bf16_lo(xw[i]); v[2 * i + 1] = bf16_hi(xw[i]); }
    const int u = ubase + wave + W * j;
    const int kb = (2 * u + t2) * 128 + c4 * 32;   // first element of the block
    if (NORM) {
      if (GF32) {
        const float* gs = reinterpret_cast<const float*>(smem + P.off_gamma) + kb / 32 * kGammaBlockF32;
#pragma unroll
        for (int i = 0; i < 32; i += 4) {
          const float4 g = *reinterpret_cast<const float4*>(gs + i);
          v[i] = (v[i] * inv) * g.x;
          v[i + 1] = (v[i + 1] * inv) * g.y;
          v[i + 2] = (v[i + 2] * inv) * g.z;
          v[i + 3] = (v[i + 3] * inv) * g.w;
        }
      } else {
        const uint8_t* gb = smem + P.off_gamma + kb / 32 * kGammaBlockBf16 * 2;
#pragma unroll
        for (int i = 0; i < 32; i += 8) {
          const uint4 g = *reinterpret_cast<const uint4*>(gb + i * 2);
          const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            v[i + 2 * h] = (v[i + 2 * h] * inv) * bf16_lo(gw[h]);
            v[i + 2 * h + 1] = (v[i + 2 * h + 1] * inv) * bf16_hi(gw[h]);
          }
        }
      }
      // positions past K or rows past M are zero input (x reads as zero, but
      // x * inv may not be zero when inv is not finite)
      if (pad_rows || (u + 1) * kUnitK > K) {
        if (!(row_ok && kb < K)) {
#pragma unroll
          for (int i = 0; i < 32; ++i) v[i] = 0.0f;
        }
      }
    }
    return decompose32<DENSE>(v);
  };

  const int tl = c4 * 16 + (int)half * 8 + r8;
  auto store = [&](const Block32& b, int j) {
    const int kt = 2 * (ubase + wave + W * j) + t2;
    if (kt < KB) {
      const int64_t tile = rb * KB + kt;
      *reinterpret_cast<uint4*>(o.r_codes + tile * 1024 + tl * 16) = b.r_codes;
      const int64_t sc = ((int64_t)kt * RB + rb) * 64 + tl;
      o.r_scales[sc] = (uint8_t)b.r_e8;
      if constexpr (!DENSE) {
        *reinterpret_cast<uint4*>(o.s_codes + tile * 1024 + tl * 16) = b.s_codes;
        *reinterpret_cast<uint32_t*>(o.s_meta + tile * 256 + tl * 4) = b.meta;
        o.s_scales[sc] = (uint8_t)b.s_e8;
      }
    }
  };

  Block32 prev;
  if (NORM && P.single) {
    for (int j = 0; j < nu_w; ++j) {
      uint32_t xw[16];
      read_block(j, xw);
      if (j > 0) store(prev, j - 1);
      prev = compute(xw, j);
    }
  } else {
    for (int j = 0; j < D && j < nu_w; ++j) issue(j);
    for (int j = 0; j < nu_w; ++j) {
      wait_units(min(D - 1, nu_w - 1 - j));
      uint32_t xw[16];
      read_block(j, xw);
      if (j + D < nu_w) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // slot j % D read back
        issue(j + D);
      }
      if (j > 0) store(prev, j - 1);
      prev = compute(xw, j);
    }
  }
  if (nu_w > 0) store(prev, nu_w - 1);
}

// ---------------------------------------------------------------------------
// Prep kernel for RMSNorm rows of at most 8192 elements.
//
// The streaming kernel above stages its 8-row group through per-wave LDS
// rings, sums the squares with a workgroup-wide tree and only then starts
// the arithmetic.  Here a workgroup (16 waves) still owns the 8 rows of half
// a 16-row tile block, but each row belongs to two waves (one half of its
// blocks each), which load their blocks straight into registers (buffer
// loads: reads past K or past the last row return zeros) and meet only
// through a pair of LDS slots for the row's sum of squares, so a row's
// arithmetic starts as soon as its own two halves have arrived.  (QKV shape
// 2048 x 4096: 12.1 -> 10.2 us.  Per-wave clock stamps put the loads at
// about 3 us of the launch, the arithmetic of 16 waves at about 2.2 us once
// their rows are in, and the stores of the codes at about 2 us more; issuing
// the four row pairs' loads at staggered times, a wave per two rows with
// 32-byte store runs, or all 8 rows per wave with whole-line stores were no
// faster.)
//
// Lane l of wave (row r, half h) holds blocks h*64*NB + 64*j + l, j < NB (one
// MX block of 32 elements each).  Its sum of squares is the balanced pairwise
// tree of the row zero-padded to 4096*NB elements, which equals the tree over
// the next power of two of K (the extra leaves are +0): per block the 32-leaf
// tree (chunk_sumsq), across the 64 lanes the butterfly of wave_tree_sum
// (blocks in lane order), then the NB slots, then the two halves, which meet
// through a pair of LDS slots (each wave publishes its half and waits for the
// other's; both always publish, and the wait is bounded).
//
// Codes go out as 16-byte stores straight from the registers; metadata and
// scale bytes (4- and 1-byte pieces per lane) are collected in LDS and
// written after the last block in runs of the 8 rows (32 and 8 bytes).
// ---------------------------------------------------------------------------
constexpr int kRowsWaves = 16;
constexpr int kRowsMaxK = 8192;
constexpr uint32_t kRowsSpinLimit = 1u << 20;   // bound of the pair wait (never reached)

struct RowsPlan {
  int KB;                                     // K tiles (K padded to 128)
  uint32_t off_sync, off_meta, off_ssc, off_rsc, total;
};

static RowsPlan rows_plan(int K) {
  RowsPlan p{};
  p.KB = (K + 127) / 128;
  p.off_sync = ((uint32_t)p.KB * 4u + 1u) * kGammaBlockF32 * 4u;   // gamma: binary32, 36 words per block, then a zero block
  p.off_meta = p.off_sync + 8u * 2u * 8u;                     // 8 rows x 2 halves x {sum, flag}
  p.off_ssc = p.off_meta + (uint32_t)p.KB * 128u;             // [kt][chunk][row] words
  p.off_rsc = p.off_ssc + (uint32_t)p.KB * 32u;               // [kt][chunk][row] bytes
  p.total = p.off_rsc + (uint32_t)p.KB * 32u;
  return p;
}

template <int NB, bool DENSE>
__global__ __launch_bounds__(kRowsWaves * 64) void prep_norm_rows_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                                         int K, int64_t ldx,
                                                                         const uint16_t* __restrict__ gamma, float eps,
                                                                         RowsPlan P, PrepOut o) {
  extern __shared__ __align__(1024) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rl = wave >> 1;                        // row among the workgroup's 8
  const int hf = wave & 1;                         // half of the row's blocks

  // workgroup -> (16-row block, half): the two halves of a block are 8 apart
  // in launch order, i.e. on one XCD, so their L2 merges the writes
  const int64_t RB = (M + 15) / 16, nwg = RB * 2;
  const int64_t w = blockIdx.x;
  const int64_t full = nwg / 16 * 16;
  int64_t rb, half;
  if (w < full) { rb = (w / 16) * 8 + (w % 8); half = (w % 16) / 8; }
  else { rb = w / 2; half = w % 2; }
  const int64_t row = rb * 16 + half * 8 + rl;
  const int r16 = (int)half * 8 + rl;
  const bool row_ok = row < M;
  const int KB = P.KB, nblk = KB * 4;

  // gamma: one 16-byte piece per thread (K <= 8192), zeros past K
  const __amdgpu_buffer_rsrc_t grs = __builtin_amdgcn_make_buffer_rsrc((void*)gamma, (short)0, K * 2, 0x00020000);
  const int ge = tid * 8;
  const u32x4 gq = __builtin_amdgcn_raw_buffer_load_b128(grs, ge * 2, 0, 0);

  // this wave's blocks of the row
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(x + (row_ok ? row : 0) * ldx), (short)0, row_ok ? K * 2 : 0, 0x00020000);
  const int b0 = hf * 64 * NB + lane;
  u32x4 xq[NB][4];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) xq[j][q] = __builtin_amdgcn_raw_buffer_load_b128(xrs, (b0 + 64 * j) * 64 + 16 * q, 0, 0);

  // gamma into LDS as binary32, blocks padded to 36 words (the 16-byte reads
  // of 16 consecutive blocks then hit 16 distinct bank groups); pair slots cleared
  float* gs = reinterpret_cast<float*>(smem);
  if (ge < nblk * 32) {
    float* d = gs + (ge / 32) * kGammaBlockF32 + (ge % 32);
    *reinterpret_cast<float4*>(d) = make_float4(bf16_lo(gq[0]), bf16_hi(gq[0]), bf16_lo(gq[1]), bf16_hi(gq[1]));
    *reinterpret_cast<float4*>(d + 4) = make_float4(bf16_lo(gq[2]), bf16_hi(gq[2]), bf16_lo(gq[3]), bf16_hi(gq[3]));
  }
  if (tid < 32) gs[nblk * kGammaBlockF32 + tid] = 0.0f;
  uint2* slots = reinterpret_cast<uint2*>(smem + P.off_sync);
  if (tid < 16) slots[tid] = make_uint2(0u, 0u);
  __syncthreads();
  // nothing that needs this wave's rows moves above the barrier (each wave
  // reaches it before its own rows have arrived)
  __builtin_amdgcn_sched_barrier(0);

  // sum of squares of this half, then of the row
  float xf[NB][32];
  float th = 0.0f;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        xf[j][8 * i + 2 * h] = bf16_lo(xq[j][i][h]);
        xf[j][8 * i + 2 * h + 1] = bf16_hi(xq[j][i][h]);
      }
    const float t = wave_tree_sum(chunk_sumsq(xf[j]));
    th = j == 0 ? t : th + t;
  }
  if (lane == 0) slots[rl * 2 + hf] = make_uint2(__float_as_uint(th), 1u);
  float tother = 0.0f;
  {
    volatile __attribute__((address_space(3))) uint32_t* other =
        (volatile __attribute__((address_space(3))) uint32_t*)(slots + rl * 2 + (hf ^ 1));
    for (uint32_t it = 0; it < kRowsSpinLimit; ++it) {
      // the flag first, then the sum (LDS accesses of one wave are done in order)
      if (__builtin_amdgcn_readfirstlane(other[1]) != 0u) {
        tother = __uint_as_float(__builtin_amdgcn_readfirstlane(other[0]));
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  const float inv = rms_inverse(th + tother, K, eps);   // the halves' sum (x + y == y + x exactly)

  // decomposition; codes stored now, metadata and scales staged
  uint32_t* meta_st = reinterpret_cast<uint32_t*>(smem + P.off_meta);
  uint8_t* ssc_st = smem + P.off_ssc;
  uint8_t* rsc_st = smem + P.off_rsc;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int b = b0 + 64 * j;
    if (b < nblk) {
      // rows past M and blocks past K are zero input: x reads as +0 there; a
      // factor +0 in place of inv (which may not be finite) and gamma +0 (the
      // table is zero past K; rows past M read the zero block after it) keep
      // v = +0 with its sign
      const float invb = row_ok && 32 * b < K ? inv : 0.0f;
      float v[32];
      const float* gb = gs + (row_ok ? b : nblk) * kGammaBlockF32;
#pragma unroll
      for (int i = 0; i < 32; i += 4) {
        const float4 g = *reinterpret_cast<const float4*>(gb + i);
        v[i] = (xf[j][i] * invb) * g.x;
        v[i + 1] = (xf[j][i + 1] * invb) * g.y;
        v[i + 2] = (xf[j][i + 2] * invb) * g.z;
        v[i + 3] = (xf[j][i + 3] * invb) * g.w;
      }
      const Block32 d = decompose32<DENSE>(v);
      const int kt = b >> 2, c = b & 3;
      const int64_t tile = rb * KB + kt;
      const int tl = c * 16 + r16;
      *reinterpret_cast<uint4*>(o.r_codes + tile * 1024 + tl * 16) = d.r_codes;
      const int st = kt * 32 + c * 8 + rl;
      rsc_st[st] = (uint8_t)d.r_e8;
      if constexpr (!DENSE) {
        *reinterpret_cast<uint4*>(o.s_codes + tile * 1024 + tl * 16) = d.s_codes;
        meta_st[st] = d.meta;
        ssc_st[st] = (uint8_t)d.s_e8;
      }
    }
  }
  __syncthreads();

  // metadata and scales of the 8 rows: per (K tile, chunk) 32 contiguous
  // bytes of metadata and 8 of each scale
  for (int i = tid; i < nblk; i += kRowsWaves * 64) {
    const int kt = i >> 2, c = i & 3, st = kt * 32 + c * 8;
    const int64_t sc = ((int64_t)kt * RB + rb) * 64 + c * 16 + half * 8;
    *reinterpret_cast<uint2*>(o.r_scales + sc) = *reinterpret_cast<const uint2*>(rsc_st + st);
    if constexpr (!DENSE) {
      *reinterpret_cast<uint2*>(o.s_scales + sc) = *reinterpret_cast<const uint2*>(ssc_st + st);
      uint8_t* md = o.s_meta + (rb * KB + kt) * 256 + (c * 16 + half * 8) * 4;
      *reinterpret_cast<uint4*>(md) = *reinterpret_cast<const uint4*>(meta_st + st);
      *reinterpret_cast<uint4*>(md + 16) = *reinterpret_cast<const uint4*>(meta_st + st + 4);
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

// K slices per row group: rows without RMSNorm need nothing across K, so long
// rows of a short grid are cut into up to four slices, each its own
// workgroup, until the grid reaches 1024 workgroups (2048 x 14336: 24.8 ->
// 23.9 us; 2048 x 4096: 11.2 -> 10.2 us).  Rows of fewer than 16 units gain
// nothing and stay whole.
static int prep_ksplit(int64_t nwg, int units, bool norm) {
  if (norm || units < 16 || nwg >= 1024) return 1;
  const int64_t want = (1024 + nwg - 1) / nwg;
  return (int)(want < 4 ? want : 4);
}

template <bool DENSE>
static hipError_t launch_prepare_rows(const uint16_t* x, int64_t M, int K, int64_t ldx, const uint16_t* gamma,
                                     float eps, PrepOut out, hipStream_t stream) {
  const RowsPlan P = rows_plan(K);
  const int64_t grid = (M + 15) / 16 * 2;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (K <= 4096)
    hipLaunchKernelGGL((prep_norm_rows_kernel<1, DENSE>), dim3((unsigned)grid), dim3(kRowsWaves * 64), P.total,
                       stream, x, M, K, ldx, gamma, eps, P, out);
  else
    hipLaunchKernelGGL((prep_norm_rows_kernel<2, DENSE>), dim3((unsigned)grid), dim3(kRowsWaves * 64), P.total,
                       stream, x, M, K, ldx, gamma, eps, P, out);
  return hipGetLastError();
}

template <bool DENSE>
static hipError_t launch_prepare_t(const uint16_t* x, int64_t M, int K, int64_t ldx, const uint16_t* gamma,
                                   float eps, PrepOut out, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (gamma && K <= kRowsMaxK)
    return launch_prepare_rows<DENSE>(x, M, K, ldx, gamma, eps, out, stream);
  // Short rows without RMSNorm (at most eight 256-element units: K <= 2048,
  // the expert layers) run 4- or 8-wave workgroups: with 16 waves most would
  // have no unit, and the CU would hold only two workgroups' few busy waves.
  const int units = (K + kUnitK - 1) / kUnitK;
  const int64_t nwg = (M + 15) / 16 * 2;
  const int ksplit = prep_ksplit(nwg, units, gamma != nullptr);
  const int sunits = (units + ksplit - 1) / ksplit;
  const int waves = gamma ? kPrepWaves : (sunits <= 4 ? 4 : (sunits <= 8 ? 8 : kPrepWaves));
  const PrepPlan P = prep_plan(K, gamma != nullptr, waves, ksplit);
  if (P.slots < 1 || P.total > kPrepLdsMax) return hipErrorInvalidValue;
  auto kn = waves == 4 ? prep_kernel<4, false, false, DENSE>
            : waves == 8 ? prep_kernel<8, false, false, DENSE>
            : (!gamma ? prep_kernel<kPrepWaves, false, false, DENSE>
                      : (P.gamma_f32 ? prep_kernel<kPrepWaves, true, true, DENSE>
                                     : prep_kernel<kPrepWaves, true, false, DENSE>));
  // the LDS limit is a per-function attribute: set it once per device
  const int which = waves == 4 ? 3 : (waves == 8 ? 4 : (!gamma ? 0 : (P.gamma_f32 ? 1 : 2)));
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  static std::atomic<bool> attr_set[64][5];
  if (!attr_set[dev][which].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute((const void*)kn, hipFuncAttributeMaxDynamicSharedMemorySize, kPrepLdsMax);
    if (e != hipSuccess) return e;
    attr_set[dev][which].store(true, std::memory_order_release);
  }
  const int64_t grid = nwg * ((units + P.ups - 1) / P.ups);
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kn, dim3((unsigned)grid), dim3(waves * 64), P.total, stream, x, M, K, ldx, gamma, eps, P, out);
  return hipGetLastError();
}

hipError_t launch_prepare(const uint16_t* x, int64_t M, int K, int64_t ldx, const uint16_t* gamma,
                          float eps, PrepOut out, hipStream_t stream) {
  return launch_prepare_t<false>(x, M, K, ldx, gamma, eps, out, stream);
}

hipError_t launch_prepare_dense(const uint16_t* x, int64_t M, int K, int64_t ldx, const uint16_t* gamma,
                                float eps, PrepOut out, hipStream_t stream) {
  return launch_prepare_t<true>(x, M, K, ldx, gamma, eps, out, stream);
}

hipError_t launch_pack_weight(const uint16_t* w, int64_t N, int K, int64_t ldw, uint8_t* codes,
                              uint8_t* scales, hipStream_t stream) {
  const int64_t rows = (N + 15) / 16 * 16;
  dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(256);
  hipLaunchKernelGGL(pack_weight_kernel, grid, block, 0, stream, w, N, K, ldw, codes, scales);
  return hipGetLastError();
}

}  // namespace sharq
