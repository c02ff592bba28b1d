// Grouped expert layer (mixture-of-experts) on top of the tiled dual GEMM.
//
// SharQ paper page (mlsanity), Abstract: the method is evaluated on mixture-of-
// experts models as well as dense ones; each expert is an ordinary SharQ
// linear layer over the tokens routed to it.  Prep is row-local, so each token
// is prepared once and its prepared row is reused by every expert it is routed
// to (the result is identical to preparing it per expert).
//
// Three launches on the caller's stream:
//   1. setup   (one wave): clamps the caller's segment offsets into a
//      nondecreasing sequence in [0, rows], and tabulates, per expert, its
//      first 16-row block in the gathered activation (segments padded to whole
//      blocks) and the number of M tiles (grouped_tile_m() rows) before it;
//   2. gather  (one wave per gathered 16-row block): copies each routed row's
//      backbone and residual codes and scales (the GEMM does not read the
//      metadata) from the source activation (row row_index[i]) into expert
//      order, writing zero codes and scales for the padding rows.  Without a
//      row index the rows are already in expert order and only the scales are
//      copied: the GEMM reads the codes from the source rows itself;
//   3. the tiled dual GEMM with one workgroup per (expert, M tile, N tile).
// The SwiGLU-prep form (gate and up rows of each expert interleaved in 16-row
// blocks) replaces Y by the down projection's prepared activation: each tile
// applies h = SiLU(gate) * up, rounds h to bf16 and prepares it in its
// epilogue, writing the routed rows in order; a fourth small launch (before
// the GEMM) fills that activation's padding rows.
#include <atomic>

#include "device_common.h"
#include "launch.h"

namespace sharq {

namespace {

constexpr int kMaxExperts = 1024;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct WsLayout {
  int64_t blocks;        // 16-row blocks of the gathered activation (upper bound)
  int64_t tiles;         // M tiles (upper bound)
  size_t r_codes, s_codes, s_scales, r_scales, seg, pseg, tprefix, bexp, texp, total;
};

WsLayout ws_layout(int64_t rows, int E, int K) {
  WsLayout L;
  const int64_t KT = (K + 127) / 128;
  L.blocks = (rows + 15 * (int64_t)E + 15) / 16;
  size_t o = 0;
  L.r_codes = o;  o = align_up(o + (size_t)L.blocks * KT * 1024);
  L.s_codes = o;  o = align_up(o + (size_t)L.blocks * KT * 1024);
  L.s_scales = o; o = align_up(o + (size_t)L.blocks * KT * 64);
  L.r_scales = o; o = align_up(o + (size_t)L.blocks * KT * 64);
  L.seg = o;      o = align_up(o + (size_t)(E + 1) * 8);
  L.pseg = o;     o = align_up(o + (size_t)(E + 1) * 8);
  L.tprefix = o;  o = align_up(o + (size_t)(E + 1) * 4);
  L.tiles = (rows + grouped_tile_m() - 1) / grouped_tile_m() + E;
  L.bexp = o;     o = align_up(o + (size_t)L.blocks * 4);
  L.texp = o;     o = align_up(o + (size_t)L.tiles * 4);
  L.total = o;
  return L;
}

// Setup, one workgroup: wave 0's lane l owns the kSetupPer-or-fewer consecutive entries
// [l * per, l * per + per) of the E + 1 offsets.  The sanitised offsets are
// the running maximum of the clamped inputs with seg[0] = 0 and seg[E] = rows
// (every value is <= rows, so the sequence ends at rows); each expert's
// 16-row blocks and M tiles are then summed inclusively (entry e + 1 belongs
// to expert e).  Both scans run inside each lane's entries and then across
// the lanes by shuffles.  The block and tile prefixes also go to LDS; after
// one barrier every thread of the workgroup fills the block -> expert and
// tile -> expert maps by binary search there (empty experts own nothing: the
// search finds the last expert whose range starts at or before the entry).
constexpr int kSetupPer = (kMaxExperts + 1 + 63) / 64;   // entries per lane at most
constexpr int kSetupThreads = 1024;

__device__ __forceinline__ int64_t shfl_up64(int64_t v, int d) {
  const int lo = __shfl_up((int)(uint32_t)v, d, 64), hi = __shfl_up((int)(v >> 32), d, 64);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

__global__ __launch_bounds__(kSetupThreads) void grouped_setup_kernel(const int64_t* __restrict__ seg_in, int E, int64_t rows,
                                                           int tile_shift, int64_t* __restrict__ seg,
                                                           int64_t* __restrict__ pseg, int32_t* __restrict__ tprefix,
                                                           int32_t* __restrict__ bexp, int32_t* __restrict__ texp) {
  __shared__ int64_t lb[kMaxExperts + 1];
  __shared__ int32_t lt[kMaxExperts + 1];
  const int lane = threadIdx.x & 63;
  const int n = E + 1;
  if (threadIdx.x < 64) {   // wave 0: the scans
    const int per = (n + 63) / 64;
    const int e0 = lane * per;
    // clamped offsets, running maximum inside the lane (entries past n carry
    // it); every load is issued before the first is used (in-range indices)
    int64_t a[kSetupPer];
#pragma unroll
    for (int k = 0; k < kSetupPer; ++k) a[k] = seg_in[e0 + k < n ? e0 + k : n - 1];
#pragma unroll
    for (int k = 0; k < kSetupPer; ++k) {
      const int e = e0 + k;
      int64_t v = 0;
      if (k < per && e < n) {
        v = e == 0 ? 0 : (e == E ? rows : a[k]);
        v = v < 0 ? 0 : (v > rows ? rows : v);
      }
      a[k] = k > 0 && a[k - 1] > v ? a[k - 1] : v;
    }
    // exclusive running maximum of the lanes before this one
    int64_t m = a[kSetupPer - 1];
#pragma unroll
    for (int d = 1; d < 64; d *= 2) {
      const int64_t y = shfl_up64(m, d);
      if (lane >= d && y > m) m = y;
    }
    int64_t before = shfl_up64(m, 1);
    if (lane == 0) before = 0;
#pragma unroll
    for (int k = 0; k < kSetupPer; ++k) a[k] = a[k] > before ? a[k] : before;
    // per entry e >= 1 (expert e - 1): blocks and tiles of its length
    int64_t prev = before;   // the offset before this lane's first entry
    int64_t nb[kSetupPer], nt[kSetupPer];
#pragma unroll
    for (int k = 0; k < kSetupPer; ++k) {
      const int e = e0 + k;
      const int64_t len = (k < per && e < n && e > 0) ? a[k] - prev : 0;
      prev = a[k];
      nb[k] = (len + 15) / 16 + (k > 0 ? nb[k - 1] : 0);
      nt[k] = ((len + (1 << tile_shift) - 1) >> tile_shift) + (k > 0 ? nt[k - 1] : 0);   // M tiles of 2^shift rows
    }
    // exclusive sums of the lanes before this one
    int64_t sb = nb[kSetupPer - 1], st = nt[kSetupPer - 1];
#pragma unroll
    for (int d = 1; d < 64; d *= 2) {
      const int64_t yb = shfl_up64(sb, d), yt = shfl_up64(st, d);
      if (lane >= d) { sb += yb; st += yt; }
    }
    int64_t bb = shfl_up64(sb, 1), bt = shfl_up64(st, 1);
    if (lane == 0) bb = bt = 0;
#pragma unroll
    for (int k = 0; k < kSetupPer; ++k) {
      const int e = e0 + k;
      if (k < per && e < n) {
        seg[e] = a[k];
        pseg[e] = bb + nb[k];
        tprefix[e] = (int32_t)(bt + nt[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < kSetupPer; ++k) {
      const int e = e0 + k;
      if (k < per && e < n) {
        lb[e] = bb + nb[k];
        lt[e] = (int32_t)(bt + nt[k]);
      }
    }
  }
  __syncthreads();
  // the expert of every gathered 16-row block and of every M tile, so that the
  // gather and the GEMM find theirs with one load instead of a search
  const int64_t nblk = lb[E], ntil = lt[E];
  for (int64_t b = threadIdx.x; b < nblk; b += kSetupThreads) {
    int lo = 0, hi = E;                               // lb[lo] <= b < lb[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (lb[mid] <= b) lo = mid; else hi = mid;
    }
    bexp[b] = lo;
  }
  for (int64_t t = threadIdx.x; t < ntil; t += kSetupThreads) {
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (lt[mid] <= t) lo = mid; else hi = mid;
    }
    texp[t] = lo;
  }
}

struct GatherArgs {
  const uint8_t *s_codes, *s_scales, *r_codes, *r_scales;   // source activation
  uint8_t *g_s_codes, *g_s_scales, *g_r_codes, *g_r_scales;
  const int32_t* row_index;
  const int64_t *seg, *pseg;
  const int32_t* bexp;
  int64_t src_rows, src_blocks, dst_blocks;
  int KT, E;
};

__global__ __launch_bounds__(256) void grouped_gather_kernel(GatherArgs a) {
  const int lane = threadIdx.x & 63;
  // blocks x K tiles < 2^21 (the GEMM's 31-bit offsets): 32-bit division
  const uint32_t w = blockIdx.x * 4u + (threadIdx.x >> 6);
  const int64_t rbp = w / (uint32_t)a.KT;
  const int kt = (int)(w % (uint32_t)a.KT);
  if (rbp >= a.pseg[a.E]) return;                     // wave-uniform
  const int e = a.bexp[rbp];                          // pseg[e] <= rbp < pseg[e+1]
  const int r = lane & 15, c4 = lane >> 4;
  const int64_t lr = (rbp - a.pseg[e]) * 16 + r;      // row within the expert
  const int64_t n = a.seg[e + 1] - a.seg[e];
  uint4 rc = make_uint4(0, 0, 0, 0), sc = make_uint4(0, 0, 0, 0);
  uint32_t ssc = 0, rsc = 0;
  if (lr < n) {
    const int64_t i = a.seg[e] + lr;
    const int64_t src = a.row_index ? (int64_t)a.row_index[i] : i;
    if (src >= 0 && src < a.src_rows) {               // a row index out of range reads as zero input
      const int64_t sb = src / 16, st = sb * a.KT + kt;
      const int sl = c4 * 16 + (int)(src % 16);
      rc = *reinterpret_cast<const uint4*>(a.r_codes + st * 1024 + sl * 16);
      sc = *reinterpret_cast<const uint4*>(a.s_codes + st * 1024 + sl * 16);
      ssc = a.s_scales[((int64_t)kt * a.src_blocks + sb) * 64 + sl];
      rsc = a.r_scales[((int64_t)kt * a.src_blocks + sb) * 64 + sl];
    }
  }
  const int64_t dt = rbp * a.KT + kt;
  *reinterpret_cast<uint4*>(a.g_r_codes + dt * 1024 + lane * 16) = rc;
  *reinterpret_cast<uint4*>(a.g_s_codes + dt * 1024 + lane * 16) = sc;
  a.g_s_scales[((int64_t)kt * a.dst_blocks + rbp) * 64 + lane] = (uint8_t)ssc;
  a.g_r_scales[((int64_t)kt * a.dst_blocks + rbp) * 64 + lane] = (uint8_t)rsc;
}


// Scale bytes only, for rows already in expert order (the GEMM reads their
// codes straight from the source rows): one wave per gathered 16-row block,
// every K tile, kGatherChunk K tiles of loads in flight before their stores.
constexpr int kGatherChunk = 4;

__global__ __launch_bounds__(256) void grouped_gather_scales_kernel(GatherArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t rbp = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rbp >= a.pseg[a.E]) return;                     // wave-uniform
  const int e = a.bexp[rbp];                          // pseg[e] <= rbp < pseg[e+1]
  const int r = lane & 15, c4 = lane >> 4;
  const int64_t lr = (rbp - a.pseg[e]) * 16 + r;      // row within the expert
  const int64_t n = a.seg[e + 1] - a.seg[e];
  int64_t src = -1;
  if (lr < n) {
    const int64_t i = a.seg[e] + lr;
    src = a.row_index ? (int64_t)a.row_index[i] : i;
    if (src >= a.src_rows) src = -1;                  // a row index out of range reads as zero input
  }
  const int64_t sb = src >= 0 ? src / 16 : 0;
  const int sl = c4 * 16 + (src >= 0 ? (int)(src % 16) : 0);
  for (int kt0 = 0; kt0 < a.KT; kt0 += kGatherChunk) {
    uint32_t ssc[kGatherChunk], rsc[kGatherChunk];
#pragma unroll
    for (int q = 0; q < kGatherChunk; ++q) {
      const int kt = kt0 + q;
      ssc[q] = rsc[q] = 0;
      if (kt < a.KT && src >= 0) {
        ssc[q] = a.s_scales[((int64_t)kt * a.src_blocks + sb) * 64 + sl];
        rsc[q] = a.r_scales[((int64_t)kt * a.src_blocks + sb) * 64 + sl];
      }
    }
#pragma unroll
    for (int q = 0; q < kGatherChunk; ++q) {
      const int kt = kt0 + q;
      if (kt >= a.KT) break;
      a.g_s_scales[((int64_t)kt * a.dst_blocks + rbp) * 64 + lane] = (uint8_t)ssc[q];
      a.g_r_scales[((int64_t)kt * a.dst_blocks + rbp) * 64 + lane] = (uint8_t)rsc[q];
    }
  }
}

// The padding rows of the last 16-row block of an activation written by the
// SwiGLU-prep epilogue (which writes routed rows only): the outputs of zero
// input -- zero codes and scale bytes, metadata 0x4 per group (offsets 0 and
// 1 kept).  One wave per K tile.
__global__ __launch_bounds__(64) void grouped_act_tail_kernel(PrepOut o, int64_t rows, int KT) {
  const int lane = threadIdx.x, r = lane & 15;
  const int kt = blockIdx.x;
  const int64_t rb = rows / 16, RB = (rows + 15) / 16;
  if (r < (int)(rows % 16)) return;
  const int64_t tile = rb * KT + kt;
  *reinterpret_cast<uint4*>(o.r_codes + tile * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
  *reinterpret_cast<uint4*>(o.s_codes + tile * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
  *reinterpret_cast<uint32_t*>(o.s_meta + tile * 256 + lane * 4) = 0x44444444u;
  o.s_scales[((int64_t)kt * RB + rb) * 64 + lane] = 0;
  o.r_scales[((int64_t)kt * RB + rb) * 64 + lane] = 0;
}

}  // namespace

size_t grouped_workspace_bytes(int64_t rows, int E, int K) { return ws_layout(rows, E, K).total; }

// Library-owned scratch of sharq_linear_grouped_noalloc: one copy per GPU,
// allocated when the code object is loaded there and held until the process
// ends.  Host code never uses the array's name as an address (it is a
// host-side stand-in): noalloc_scratch() asks the runtime for this device's
// address once and keeps it.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

uint8_t* noalloc_scratch(hipError_t* err) {
  constexpr int kMaxDev = 64;
  static std::atomic<uint8_t*> ptr[kMaxDev];
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDev) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  uint8_t* p = ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  *err = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
  if (*err != hipSuccess) return nullptr;
  p = static_cast<uint8_t*>(q);
  ptr[dev].store(p, std::memory_order_release);   // the same value for every thread that gets here
  return p;
}

hipError_t launch_linear_grouped(const GroupedArgs& a, hipStream_t stream) {
  const int E = a.gemm.E;
  if (E < 1 || E > kMaxExperts) return hipErrorInvalidValue;
  const WsLayout L = ws_layout(a.rows, E, a.gemm.K);
  const int KT = (a.gemm.K + 127) / 128;
  int64_t* seg = reinterpret_cast<int64_t*>(a.ws + L.seg);
  int64_t* pseg = reinterpret_cast<int64_t*>(a.ws + L.pseg);
  int32_t* tprefix = reinterpret_cast<int32_t*>(a.ws + L.tprefix);
  int32_t* bexp = reinterpret_cast<int32_t*>(a.ws + L.bexp);
  int32_t* texp = reinterpret_cast<int32_t*>(a.ws + L.texp);

  // M tiles are a power of two of rows: the kernel shifts (a 64-bit division
  // by a runtime value is a long software sequence per entry)
  int tile_shift = 0;
  while ((1 << tile_shift) < grouped_tile_m()) ++tile_shift;
  if ((1 << tile_shift) != grouped_tile_m()) return hipErrorInvalidValue;
  hipLaunchKernelGGL(grouped_setup_kernel, dim3(1), dim3(kSetupThreads), 0, stream, a.seg_in, E, a.rows,
                     tile_shift, seg, pseg, tprefix, bexp, texp);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  // Rows already in expert order (no row index) are read by the GEMM straight
  // from the source: each 16-row block of an expert spans at most two source
  // blocks, so its copies stay nearly contiguous.  Routed token rows are
  // gathered (codes too) into expert order first.
  const bool gather_in_gemm = a.row_index == nullptr;
  GatherArgs g;
  g.s_codes = a.gemm.s_codes; g.s_scales = a.gemm.s_scales;
  g.r_codes = a.gemm.r_codes; g.r_scales = a.gemm.r_scales;
  g.g_r_codes = a.ws + L.r_codes; g.g_s_codes = a.ws + L.s_codes;
  g.g_s_scales = a.ws + L.s_scales; g.g_r_scales = a.ws + L.r_scales;
  g.row_index = a.row_index;
  g.seg = seg; g.pseg = pseg; g.bexp = bexp;
  g.src_rows = a.gemm.M; g.src_blocks = a.src_blocks; g.dst_blocks = L.blocks;
  g.KT = KT; g.E = E;
  if (gather_in_gemm) {
    const int64_t wgs = (L.blocks + 3) / 4;            // one wave per gathered block (upper bound)
    if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(grouped_gather_scales_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, g);
  } else {
    const int64_t wgs = (L.blocks * KT + 3) / 4;       // one wave per gathered block and K tile
    if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(grouped_gather_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, g);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;

  GemmArgs m = a.gemm;
  m.s_meta = nullptr; m.s_scales = g.g_s_scales; m.r_scales = g.g_r_scales;
  if (gather_in_gemm) {
    m.gather = 1;
    m.row_index = a.row_index;
    m.src_rows = a.gemm.M;
    m.src_blocks = a.src_blocks;
  } else {
    m.gather = 0;
    m.s_codes = g.g_s_codes; m.r_codes = g.g_r_codes;
  }
  m.a_blocks = L.blocks;
  m.M = a.rows;
  m.seg = seg; m.pseg = pseg; m.tprefix = tprefix; m.texp = texp;
  if (m.next.r_codes && a.rows % 16) {
    // the next activation (K = N_e / 2) gets its padding rows before the GEMM
    // writes the routed ones
    const int KTn = (int)(a.gemm.N / E / 2 / 128);
    hipLaunchKernelGGL(grouped_act_tail_kernel, dim3((unsigned)KTn), dim3(64), 0, stream, m.next, a.rows, KTn);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return launch_linear_grouped_gemm(m, L.tiles, stream);
}

}  // namespace sharq
