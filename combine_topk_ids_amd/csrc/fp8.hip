// FP8 rows: the format of the FP8 dispatch and of FP8 expert weights (Mooncake PG/EP guide,
// "Buffer.dispatch": with use_fp8 the receive buffer holds FP8 data plus scales; hidden is a
// multiple of 128).  Each row is cut into blocks of 128 values; a block whose largest magnitude
// is a gets the scale 2^k, k the smallest integer with a <= 448 * 2^k (0 for an all-zero block,
// clamped to [-127, 127]), stored as the byte k + 127 (the E8M0 exponent the gfx950 block-scaled
// MFMA takes); every value v is stored as the OCP FP8 E4M3 code of v * 2^-k, rounded to nearest
// even.  |v * 2^-k| <= 448, the largest finite E4M3 value, so nothing saturates, and the
// dequantised value code * 2^k is exact in bf16 and fp32.
//
// A row's scales are padded to a multiple of 4 bytes (fp8_scale_stride) so that the scales of
// four consecutive blocks are one aligned 32-bit word.
#include "fp8_format.h"

namespace moe {
namespace {

// rows x cols bf16 -> codes [rows, cols], scale bytes [rows, stride]; one 16-lane group per block.
__global__ __launch_bounds__(256) void k_quantize_rows(const uint4* __restrict__ x, int64_t rows, int32_t cols,
                                                       int32_t stride, uint2* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
  const int32_t nb = cols / 128;
  const int64_t nblocks = rows * nb;
  const int li = threadIdx.x % kLanesPerBlock;
  const int64_t g0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kLanesPerBlock;
  const int64_t ng = (int64_t)gridDim.x * blockDim.x / kLanesPerBlock;
  for (int64_t g = g0; g < nblocks; g += ng) {  // uniform across each 16-lane group
    const int64_t r = g / nb;
    const int32_t b = (int32_t)(g % nb);
    float v[8];
    unpack8(x[(r * cols + (int64_t)b * 128) / 8 + li], v);
    int k;
    const uint2 c = quant_block_lanes(v, &k);
    codes[(r * cols + (int64_t)b * 128) / 8 + li] = c;
    if (li == 0) scales[r * stride + b] = (uint8_t)(k + 127);
    if (li > 0 && b == nb - 1 && nb + li - 1 < stride) scales[r * stride + nb + li - 1] = 0;  // padding
  }
}

// FP8 dispatch, RANK_MAJOR / FLAT: source row t is quantised once and written to its receive row
// (codes [rows, H], scales [rows, stride]).  One workgroup of 128 threads per token; thread i holds
// pieces i, i + 128, ... (16 consecutive threads = one 128-value block).
__global__ __launch_bounds__(128) void k_permute_rows_fp8(const uint4* __restrict__ x,
                                                          const int32_t* __restrict__ row_of_token, int32_t N,
                                                          int32_t H, int32_t stride, uint2* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const int32_t cpr = H / 8;
  for (int32_t t = blockIdx.x; t < N; t += gridDim.x) {
    const int32_t row = row_of_token[t];
    if (row < 0) continue;
    for (int32_t c = threadIdx.x; c < cpr; c += blockDim.x) {  // cpr % 16 == 0: whole blocks per pass
      float v[8];
      unpack8(x[(int64_t)t * cpr + c], v);
      int k;
      const uint2 q = quant_block_lanes(v, &k);
      codes[(int64_t)row * cpr + c] = q;
      if (c % kLanesPerBlock == 0) scales[(int64_t)row * stride + c / kLanesPerBlock] = (uint8_t)(k + 127);
    }
  }
}

// FP8 dispatch, EXPERT_MAJOR: source row t is quantised once and written to every slot it got.
__global__ __launch_bounds__(128) void k_permute_em_fp8(const uint4* __restrict__ x, const int32_t* __restrict__ slot_of,
                                                        int32_t N, int32_t K, int32_t H, int32_t stride,
                                                        uint2* __restrict__ codes, uint8_t* __restrict__ scales,
                                                        LayoutRangeArgs lr) {
  layout_ranges(lr);
  const int32_t cpr = H / 8;
  for (int32_t t = blockIdx.x; t < N; t += gridDim.x) {
    const int32_t* so = slot_of + (int64_t)t * K;
    int any = 0;
    for (int k = 0; k < K; ++k) any |= so[k] >= 0;
    if (!any) continue;
    for (int32_t c = threadIdx.x; c < cpr; c += blockDim.x) {
      float v[8];
      unpack8(x[(int64_t)t * cpr + c], v);
      int kk;
      const uint2 q = quant_block_lanes(v, &kk);
      for (int k = 0; k < K; ++k) {
        const int32_t s = so[k];
        if (s < 0) continue;
        codes[(int64_t)s * cpr + c] = q;
        if (c % kLanesPerBlock == 0) scales[(int64_t)s * stride + c / kLanesPerBlock] = (uint8_t)(kk + 127);
      }
    }
  }
}

}  // namespace

hipError_t launch_permute_fp8(const Geom& g, const void* x, const int32_t* slot_of, const int32_t* row_of_token,
                              void* codes, void* scales, hipStream_t stream, const LayoutRangeArgs& lr) {
  if (g.N == 0) return hipSuccess;
  const unsigned grid = (unsigned)(g.N < (1 << 20) ? g.N : (1 << 20));
  const int32_t stride = fp8_scale_stride(g.H);
  if (g.layout == 0)
    hipLaunchKernelGGL(k_permute_em_fp8, dim3(grid), dim3(128), 0, stream, (const uint4*)x, slot_of, g.N, g.K, g.H,
                       stride, (uint2*)codes, (uint8_t*)scales, lr);
  else
    hipLaunchKernelGGL(k_permute_rows_fp8, dim3(grid), dim3(128), 0, stream, (const uint4*)x, row_of_token, g.N, g.H,
                       stride, (uint2*)codes, (uint8_t*)scales);
  return hipGetLastError();
}

int32_t fp8_scale_stride(int32_t cols) { return ((cols / 128) + 3) / 4 * 4; }

hipError_t launch_quantize_rows_fp8(const void* x, int64_t rows, int32_t cols, void* codes, void* scales,
                                    hipStream_t stream) {
  const int64_t groups = rows * (cols / 128);
  if (groups == 0) return hipSuccess;
  const int64_t blocks = (groups * kLanesPerBlock + 255) / 256;
  hipLaunchKernelGGL(k_quantize_rows, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, stream,
                     (const uint4*)x, rows, cols, fp8_scale_stride(cols), (uint2*)codes, (uint8_t*)scales);
  return hipGetLastError();
}

}  // namespace moe
