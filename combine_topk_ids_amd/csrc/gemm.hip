// Grouped expert GEMMs on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16), fp32
// accumulation.
//
// What is computed (FlashInfer "MoE-EP implementation & usage", section 2
// "Call stack": the expert GEMM is a pure per-expert grouped GEMM with no
// routing inside; section 4 "Usage walkthrough": w1 [E, 2I, H], w2 [E, H, I]):
// for local expert e with rows X_e (its received rows, in slot / pick order)
//     h = SiLU(X_e W1_e[0:I]^T) * (X_e W1_e[I:2I]^T)      (gate_up, fused SwiGLU)
//     y = h W2_e^T                                         (down)
// Both operands of both GEMMs are K-contiguous row-major ("NT"), which is the
// native operand layout of the MFMA: lane l of a 32x32x16 step holds 8
// consecutive k of row l % 32 of A and of row l % 32 of B^T.
//
// Tiling: 256 threads (4 waves as 2x2) per 128-row tile of one expert.  The
// grid is (tiles of the device-side tile table) x (column tiles); blocks past
// the table's length exit at once.  A/B tiles of 64 k are staged through LDS
// with a 16-byte row pad, double buffered: the next tile's global loads are
// issued before the current tile's MFMAs and written to LDS after them.
// gate_up puts the gate columns [n0, n0+64) and the matching up columns
// [I+n0, I+n0+64) in one B tile, so each lane ends with gate and up
// accumulators of the same (row, column) and applies SiLU(g)*u in registers.

#include "common.h"

namespace moe {
namespace {

constexpr int BM = kGemmBM;  // rows per tile
constexpr int BK = 64;       // k per LDS stage
constexpr int LDK = BK + 8;  // LDS row stride in bf16 (16-byte pad)
constexpr int kThreads = 256;

__device__ __forceinline__ floatx16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const floatx16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// One 128 x 64 bf16 tile = 128 rows x 8 pieces of 16 bytes; thread tid moves
// rows tid/8 + 32*i (i < 4), piece tid % 8.
struct TileLoad {
  const uint4* src[4];  // row start + piece, advanced by BK per stage; NULL = zero row
  uint4 v[4];
  __device__ __forceinline__ void load(int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = src[i] ? src[i][kt * (BK / 8)] : make_uint4(0, 0, 0, 0);
  }
  __device__ __forceinline__ void store(bf16_t* lds) const {
    const int r = threadIdx.x / 8, p = threadIdx.x % 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) *(uint4*)(lds + (r + 32 * i) * LDK + p * 8) = v[i];
  }
};

__device__ __forceinline__ bf16x8_t lds_frag(const bf16_t* lds, int row, int k) {
  return *(const bf16x8_t*)(lds + row * LDK + k);
}

// Row -> (tile row, column) of accumulator register r of a 32x32 MFMA tile for this lane.
__device__ __forceinline__ int acc_row(int r, int lane) { return (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2); }

// Resolve the tile of this block; false if the block has no work.
__device__ __forceinline__ bool tile_of(const int2* tiles, const int32_t* num_tiles, int32_t mt, int32_t* el,
                                        int32_t* m0) {
  if (mt >= *num_tiles) return false;
  const int2 t = tiles[mt];
  *el = t.x;
  *m0 = t.y;
  return true;
}

__global__ __launch_bounds__(kThreads) void k_gemm_gate_up(GemmRows rows, const int32_t* __restrict__ counts,
                                                           const int32_t* __restrict__ offsets, int64_t clamp,
                                                           const bf16_t* __restrict__ w1, bf16_t* __restrict__ h,
                                                           const int2* __restrict__ tiles,
                                                           const int32_t* __restrict__ num_tiles, int32_t H,
                                                           int32_t I) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BM * LDK];
  const int32_t ntn = I / 64;
  const int32_t mt = blockIdx.x / ntn, nt = blockIdx.x % ntn;
  int32_t el, m0;
  if (!tile_of(tiles, num_tiles, mt, &el, &m0)) return;
  const int32_t cnt = (int32_t)min((int64_t)counts[el], clamp);
  const int32_t valid = min(BM, cnt - m0);
  const int32_t n0 = nt * 64;
  const int32_t off = offsets[el];

  TileLoad la, lb;
  {
    const int r = threadIdx.x / 8, p = threadIdx.x % 8;
    const int32_t hp = H / 8;  // pieces per row
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = r + 32 * i;
      if (rr < valid) {
        int64_t src_row;
        if (rows.perm) src_row = rows.perm[off + m0 + rr] / rows.K;
        else src_row = el * rows.slab + m0 + rr;
        la.src[i] = (const uint4*)rows.a + src_row * hp + p;
      } else {
        la.src[i] = nullptr;
      }
      const int64_t wrow = (int64_t)el * 2 * I + (rr < 64 ? n0 + rr : I + n0 + (rr - 64));
      lb.src[i] = (const uint4*)w1 + wrow * hp + p;
    }
  }

  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int wm = wave >> 1, wn = wave & 1;
  floatx16_t g0 = {0}, g1 = {0}, u0 = {0}, u1 = {0};

  const int nk = H / BK;
  la.load(0);
  lb.load(0);
  la.store(As[0]);
  lb.store(Bs[0]);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      la.load(kt + 1);
      lb.load(kt + 1);
    }
    const bf16_t* a_s = As[cur];
    const bf16_t* b_s = Bs[cur];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int k = ks * 16 + (lane >> 5) * 8;
      const bf16x8_t a0 = lds_frag(a_s, wm * 64 + (lane & 31), k);
      const bf16x8_t a1 = lds_frag(a_s, wm * 64 + 32 + (lane & 31), k);
      const bf16x8_t bg = lds_frag(b_s, wn * 32 + (lane & 31), k);
      const bf16x8_t bu = lds_frag(b_s, 64 + wn * 32 + (lane & 31), k);
      g0 = mfma32(a0, bg, g0);
      g1 = mfma32(a1, bg, g1);
      u0 = mfma32(a0, bu, u0);
      u1 = mfma32(a1, bu, u1);
    }
    if (kt + 1 < nk) {
      la.store(As[cur ^ 1]);
      lb.store(Bs[cur ^ 1]);
    }
    __syncthreads();
  }

  // epilogue: h = SiLU(g) * u, bf16, rows below `valid`
  const int32_t col = n0 + wn * 32 + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row0 = wm * 64 + acc_row(r, lane);
    const int row1 = row0 + 32;
    if (row0 < valid) {
      const float g = g0[r], u = u0[r];
      h[(int64_t)(off + m0 + row0) * I + col] = (bf16_t)f32_to_bf16(g / (1.0f + __expf(-g)) * u);
    }
    if (row1 < valid) {
      const float g = g1[r], u = u1[r];
      h[(int64_t)(off + m0 + row1) * I + col] = (bf16_t)f32_to_bf16(g / (1.0f + __expf(-g)) * u);
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_gemm_down(const int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ offsets, int64_t clamp,
                                                        const bf16_t* __restrict__ h, const bf16_t* __restrict__ w2,
                                                        bf16_t* __restrict__ y, int64_t out_slab,
                                                        const int2* __restrict__ tiles,
                                                        const int32_t* __restrict__ num_tiles, int32_t H, int32_t I) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BM * LDK];
  const int32_t ntn = H / 128;
  const int32_t mt = blockIdx.x / ntn, nt = blockIdx.x % ntn;
  int32_t el, m0;
  if (!tile_of(tiles, num_tiles, mt, &el, &m0)) return;
  const int32_t cnt = (int32_t)min((int64_t)counts[el], clamp);
  const int32_t valid = min(BM, cnt - m0);
  const int32_t n0 = nt * 128;
  const int32_t off = offsets[el];

  TileLoad la, lb;
  {
    const int r = threadIdx.x / 8, p = threadIdx.x % 8;
    const int32_t ip = I / 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = r + 32 * i;
      la.src[i] = rr < valid ? (const uint4*)h + (int64_t)(off + m0 + rr) * ip + p : nullptr;
      lb.src[i] = (const uint4*)w2 + ((int64_t)el * H + n0 + rr) * ip + p;
    }
  }

  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int wm = wave >> 1, wn = wave & 1;
  floatx16_t c00 = {0}, c01 = {0}, c10 = {0}, c11 = {0};

  const int nk = I / BK;
  la.load(0);
  lb.load(0);
  la.store(As[0]);
  lb.store(Bs[0]);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      la.load(kt + 1);
      lb.load(kt + 1);
    }
    const bf16_t* a_s = As[cur];
    const bf16_t* b_s = Bs[cur];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int k = ks * 16 + (lane >> 5) * 8;
      const bf16x8_t a0 = lds_frag(a_s, wm * 64 + (lane & 31), k);
      const bf16x8_t a1 = lds_frag(a_s, wm * 64 + 32 + (lane & 31), k);
      const bf16x8_t b0 = lds_frag(b_s, wn * 64 + (lane & 31), k);
      const bf16x8_t b1 = lds_frag(b_s, wn * 64 + 32 + (lane & 31), k);
      c00 = mfma32(a0, b0, c00);
      c01 = mfma32(a0, b1, c01);
      c10 = mfma32(a1, b0, c10);
      c11 = mfma32(a1, b1, c11);
    }
    if (kt + 1 < nk) {
      la.store(As[cur ^ 1]);
      lb.store(Bs[cur ^ 1]);
    }
    __syncthreads();
  }

  const int32_t col0 = n0 + wn * 64 + (lane & 31);
  const int64_t rbase = out_slab ? (int64_t)el * out_slab + m0 : (int64_t)off + m0;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row0 = wm * 64 + acc_row(r, lane);
    const int row1 = row0 + 32;
    if (row0 < valid) {
      y[(rbase + row0) * H + col0] = (bf16_t)f32_to_bf16(c00[r]);
      y[(rbase + row0) * H + col0 + 32] = (bf16_t)f32_to_bf16(c01[r]);
    }
    if (row1 < valid) {
      y[(rbase + row1) * H + col0] = (bf16_t)f32_to_bf16(c10[r]);
      y[(rbase + row1) * H + col0 + 32] = (bf16_t)f32_to_bf16(c11[r]);
    }
  }
}

}  // namespace

hipError_t launch_gemm_gate_up(const Geom& g, GemmRows rows, const int32_t* counts, const int32_t* offsets,
                               int64_t count_clamp, const bf16_t* w_gate_up, bf16_t* h, const int2* tiles,
                               const int32_t* num_tiles, int32_t max_tiles_, hipStream_t stream) {
  const int64_t blocks = (int64_t)max_tiles_ * (g.I / 64);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_gemm_gate_up, dim3((unsigned)blocks), dim3(kThreads), 0, stream, rows, counts, offsets,
                     count_clamp, w_gate_up, h, tiles, num_tiles, g.H, g.I);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const Geom& g, const int32_t* counts, const int32_t* offsets, int64_t count_clamp,
                            const bf16_t* h, const bf16_t* w_down, bf16_t* y, int64_t out_slab, const int2* tiles,
                            const int32_t* num_tiles, int32_t max_tiles_, hipStream_t stream) {
  const int64_t blocks = (int64_t)max_tiles_ * (g.H / 128);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_gemm_down, dim3((unsigned)blocks), dim3(kThreads), 0, stream, counts, offsets, count_clamp, h,
                     w_down, y, out_slab, tiles, num_tiles, g.H, g.I);
  return hipGetLastError();
}

}  // namespace moe
