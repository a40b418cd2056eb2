// FP8 row format helpers shared by the FP8 kernels (format: see fp8.hip).
#pragma once

#include "common.h"

namespace moe {

constexpr int kLanesPerBlock = 16;  // lanes that hold one 128-value block, 8 values each

// E4M3 code of v (|v| <= 448, finite), round to nearest even.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a < 0x3C800000u) {  // |v| < 2^-6: subnormal codes m * 2^-9 (m = 8 is the smallest normal)
    const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);  // exact scaling; rint: ties to even
    return sign | (uint32_t)m;
  }
  int e = (int)(a >> 23) - 127;
  uint32_t q = (a >> 20) & 7u;
  const uint32_t rem = a & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;
  if (q == 8u) {
    q = 0;
    ++e;
  }
  return sign | ((uint32_t)(e + 7) << 3) | q;
}

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
  uint32_t c[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) c[e] = e4m3_rne(ldexpf(v[e], -*k));
  return make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24), c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
}

}  // namespace moe
