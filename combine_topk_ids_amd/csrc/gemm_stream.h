// Weight-streaming down GEMM for 64-row expert tiles (gemm_stream.hip): the host side.
#pragma once

#include "common.h"

namespace moe {

// Operands of the down GEMM over the 64-row tiles of the tile table (as the grouped GEMMs of
// gemm.hip take them): y[orow] = h[off[e] + m] W2_e^T.
struct StreamArgs {
  const bf16_t* a;       // packed h rows [P, I]: row off[e] + m
  const int32_t* counts;
  const int32_t* offsets;
  int64_t clamp;
  const bf16_t* w;       // [L, H, I]
  bf16_t* out;           // y: orow = out_slab ? e*out_slab + m : off[e] + m
  int64_t out_slab;      // EM slab layout rows per expert (0 = packed)
  const int2* tiles;     // 64-row tiles
  const int32_t* num_tiles;
  int32_t Kd;            // contraction length I, a multiple of 256
  int32_t H;
};

// The kernel takes the contraction in stages of 256.
bool gemm_stream_fits(int32_t Kd);

hipError_t launch_gemm_stream_down(const StreamArgs& a, hipStream_t stream);

}  // namespace moe
