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
  int64_t a_blocks;                // 16-row blocks of the activation buffers (scale stride)
  int xcd_bm;                      // tiled kernel: M tiles per XCD region (0: plain XCD order)
  // grouped expert layer; seg == nullptr for a single problem
  const int64_t* seg;              // [E+1] first output row of each expert (sanitised)
  const int64_t* pseg;             // [E+1] first activation 16-row block of each expert
  const int32_t* tprefix;          // [E+1] M tiles of the experts before each expert
  int E;
};

hipError_t launch_linear(const GemmArgs& a, hipStream_t stream);

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
int grouped_tile_m();
hipError_t launch_linear_grouped_gemm(const GemmArgs& a, int64_t max_mtiles, hipStream_t stream);
hipError_t launch_linear_grouped(const GroupedArgs& a, hipStream_t stream);

}  // namespace sharq
