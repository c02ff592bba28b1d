// Internal launchers (host side).  Arguments are validated by the C ABI layer
// before any of these run.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sharq {

struct PrepOut {
  uint8_t* s_codes;
  uint8_t* s_meta;
  uint8_t* s_scales;
  uint8_t* r_codes;
  uint8_t* r_scales;
};

hipError_t launch_prepare(const uint16_t* x, int64_t M, int K, int64_t ldx, const uint16_t* gamma,
                          float eps, PrepOut out, hipStream_t stream);

hipError_t launch_pack_weight(const uint16_t* w, int64_t N, int K, int64_t ldw, uint8_t* codes,
                              uint8_t* scales, hipStream_t stream);

struct GemmArgs {
  const uint8_t* s_codes;
  const uint8_t* s_meta;
  const uint8_t* s_scales;
  const uint8_t* r_codes;
  const uint8_t* r_scales;
  const uint8_t* w_codes;
  const uint8_t* w_scales_sparse;  // weight scale view of the sparse path
  const uint8_t* w_scales_dense;   // weight scale view of the dense path
  int64_t w_scales_ld;             // bytes between weight rows in both views
  void* y;
  int64_t ldy;
  int64_t M, N;
  int K;
  int out_bf16;
  // residual epilogue (bf16 output only): y = bf16(resid + Y); nullptr: none
  const uint16_t* resid;
  int64_t ld_resid;
  // SwiGLU epilogue preparing H for the next layer (r_codes == nullptr: store H)
  PrepOut next;
  int64_t a_blocks;                // 16-row blocks of the activation buffers (scale stride)
  int xcd_bm;                      // tiled kernel: M tiles per XCD region (0: plain XCD order)
  // grouped expert layer; seg == nullptr for a single problem
  const int64_t* seg;              // [E+1] first output row of each expert (sanitised)
  const int64_t* pseg;             // [E+1] first activation 16-row block of each expert
  const int32_t* tprefix;          // [E+1] M tiles of the experts before each expert
  const int32_t* texp;             // [M tiles] expert of each M tile
  int E;
  // grouped, gather != 0: the backbone and residual codes are read straight
  // from the source activation (src_blocks 16-row blocks, src_rows rows):
  // routed row i is source row row_index[i] (or i); the scale fields hold
  // the scales gathered into expert order (a_blocks blocks)
  int gather;
  const int32_t* row_index;
  int64_t src_rows, src_blocks;
  // NVFP4-style operands: binary32 tensor scales of S, R and W (device)
  const float* g_s;
  const float* g_r;
  const float* g_w;
};

hipError_t launch_linear(const GemmArgs& a, hipStream_t stream);

// Plain FP4 linear (no backbone): prep writes only the MXFP4 codes and scales
// of v into r_codes / r_scales; the GEMM runs the dense path alone.
hipError_t launch_prepare_dense(const uint16_t* x, int64_t M, int K, int64_t ldx, const uint16_t* gamma,
                                float eps, PrepOut out, hipStream_t stream);
hipError_t launch_linear_dense(const GemmArgs& a, hipStream_t stream);
// SwiGLU epilogue: the weight's 16-row blocks alternate gate and up, and
// y[m][16j + c] = bf16(SiLU(gate) * up) of the column pair (block 2j,
// block 2j + 1), column c; y is bf16 with row stride ldy.  The tiled kernel.
hipError_t launch_linear_swiglu(const GemmArgs& a, hipStream_t stream);

// The whole layer in one launch for M <= 16 (every workgroup prepares the rows
// into LDS); fused_layer_lds_bytes must be <= 160 KiB.
size_t fused_layer_lds_bytes(int K, bool norm);
// The NVFP4-style layer in one launch (M <= 16): g carries the NVFP4 weight
// (codes, tiled E4M3 scales, g_w) and the output.
size_t nv_fused_layer_lds_bytes(int K);
hipError_t launch_linear_fused_nv(const uint16_t* x, int M, int K, int64_t ldx, const uint16_t* gamma, float eps,
                                  const GemmArgs& g, hipStream_t stream);
hipError_t launch_linear_fused(const uint16_t* x, int M, int K, int64_t ldx, const uint16_t* gamma, float eps,
                               const GemmArgs& g, hipStream_t stream);

// Fusion ablations: standalone RMSNorm writing bf16; fp32 elementwise add.
hipError_t launch_rmsnorm_bf16(const uint16_t* x, int64_t M, int K, int64_t ldx, const uint16_t* gamma, float eps,
                               uint16_t* y, int64_t ldy, hipStream_t stream);
hipError_t launch_add_f32(const float* a, const float* b, float* y, int64_t n, hipStream_t stream);
hipError_t launch_add_bf16_f32(const uint16_t* x, const float* y, uint16_t* out, int64_t n, hipStream_t stream);

// Grouped expert layer: rows of a prepared activation gathered (or taken in
// order) into expert segments padded to whole 16-row blocks, then one tiled
// dual GEMM over every (expert, tile).  See sharq_linear_grouped.
struct GroupedArgs {
  GemmArgs gemm;                   // activation fields = the source activation
  const int32_t* row_index;        // [rows] source row of each routed row, or nullptr
  const int64_t* seg_in;           // [E+1] caller's segment offsets (device)
  int64_t rows;                    // routed rows (output rows)
  int64_t src_blocks;              // 16-row blocks of the source activation
  uint8_t* ws;                     // workspace (sharq_grouped_workspace_bytes)
};
size_t grouped_workspace_bytes(int64_t rows, int E, int K);
// the grouped layer's workspace for callers that cannot allocate: a
// library-owned device array per GPU (its address on the current device, or
// nullptr with *err set)
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
uint8_t* noalloc_scratch(hipError_t* err);
int grouped_tile_m();
hipError_t launch_linear_grouped_gemm(const GemmArgs& a, int64_t max_mtiles, hipStream_t stream);
hipError_t launch_linear_grouped(const GroupedArgs& a, hipStream_t stream);

// ---------------------------------------------------------------------------
// NVFP4-style format (E2M1 codes, E4M3 scale per 16 elements, binary32 scale
// per tensor).  Codes use the MX tiled layout; block scales are tiled
// [KB][RB][128]: lane l of tile (rb, kb) owns bytes 2l (its first 16
// elements) and 2l+1 (the next 16).  Each scale buffer continues, at the
// first 256-byte boundary after the block scales, with a 256-byte record
// whose first word is the tensor scale; the residual's and the weight's
// buffers then hold the scratch of the kernels that compute those scales.
// ---------------------------------------------------------------------------
constexpr size_t nv_round256(size_t b) { return (b + 255) / 256 * 256; }
struct NvActLayout {
  size_t g;                        // tensor-scale offset (both scale buffers)
  size_t s_bytes;                  // s_scales buffer size
  size_t rowamax, inv, rparts;     // r_scales: per-row max |v|, per-row 1/rms, per-workgroup max |r|
  size_t r_bytes;                  // r_scales buffer size
  int wx;                          // workgroups along K (4 K tiles each)
};
inline NvActLayout nv_act_layout(int64_t M, int64_t K) {
  const size_t RB = (size_t)((M + 15) / 16), KB = (size_t)((K + 127) / 128);
  NvActLayout l;
  l.wx = (int)((KB + 3) / 4);
  l.g = nv_round256(RB * KB * 128);
  l.s_bytes = l.g + 256;
  l.rowamax = l.g + 256;
  l.inv = l.rowamax + nv_round256(RB * 16 * 4);
  l.rparts = l.inv + nv_round256(RB * 16 * 4);
  l.r_bytes = l.rparts + nv_round256(RB * (size_t)l.wx * 4);
  return l;
}
struct NvWeightLayout {
  size_t g;                        // tensor-scale offset
  size_t parts;                    // per-workgroup max |w|
  size_t bytes;
  int wx;
};
inline NvWeightLayout nv_weight_layout(int64_t N, int64_t K) {
  const size_t NB = (size_t)((N + 15) / 16), KB = (size_t)((K + 127) / 128);
  NvWeightLayout l;
  l.wx = (int)((KB + 3) / 4);
  l.g = nv_round256(NB * KB * 128);
  l.parts = l.g + 256;
  l.bytes = l.parts + nv_round256(NB * (size_t)l.wx * 4);
  return l;
}

hipError_t launch_prepare_nv(const uint16_t* x, int64_t M, int K, int64_t ldx, const uint16_t* gamma,
                             float eps, PrepOut out, hipStream_t stream);
hipError_t launch_pack_weight_nv(const uint16_t* w, int64_t N, int K, int64_t ldw, uint8_t* codes,
                                 uint8_t* scales, hipStream_t stream);
// GemmArgs with the NVFP4-style tiled scales and g_s / g_r / g_w set
hipError_t launch_linear_nv(const GemmArgs& a, hipStream_t stream);
// compute units of the current device (cached per device), <= 0 on error
int compute_units();

}  // namespace sharq
