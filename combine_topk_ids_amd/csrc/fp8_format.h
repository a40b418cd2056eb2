// FP8 row format helpers shared by the FP8 kernels (format: see fp8.hip).
#pragma once

#include "common.h"

namespace moe {

constexpr int kLanesPerBlock = 16;  // lanes that hold one 128-value block, 8 values each

// The block's scale exponent k: the smallest k with amax <= 448 * 2^k = 1.75 * 2^(k+8).
__device__ __forceinline__ int block_scale_k(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e;
  const float f = frexpf(amax, &e);  // amax = f * 2^e, f in [0.5, 1)
  const int k = (2.0f * f <= 1.75f) ? e - 9 : e - 8;
  return k < -127 ? -127 : (k > 127 ? 127 : k);
}

// Quantises one block held by 16 consecutive lanes (lane group of 16; `v` = this lane's 8 values).
// Returns this lane's 8 codes (little-endian in two words) and the block's k in *k.
__device__ __forceinline__ uint2 quant_block_lanes(const float (&v)[8], int* k) {
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
#pragma unroll
  for (int d = 1; d < kLanesPerBlock; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d, kLanesPerBlock));
  *k = block_scale_k(amax);
  // E4M3 codes of v * 2^-k (|v * 2^-k| <= 448: no overflow) by the hardware's round-to-nearest-even
  // conversion (v_cvt_pk_fp8_f32, OCP E4M3 on gfx950), two values per instruction.  Checked against
  // the software encoder of the format on every bf16 value up to 448, the exact midpoints between
  // codes and their neighbours, signed zeros and fp32 subnormals: identical codes.
  float s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = ldexpf(v[e], -*k);
  uint32_t w0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(s[0], s[1], 0, false);
  w0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(s[2], s[3], (int)w0, true);
  uint32_t w1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(s[4], s[5], 0, false);
  w1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(s[6], s[7], (int)w1, true);
  return make_uint2(w0, w1);
}

}  // namespace moe
