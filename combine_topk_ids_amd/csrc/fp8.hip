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

}  // namespace

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
