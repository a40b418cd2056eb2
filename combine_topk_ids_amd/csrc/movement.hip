// Row movement kernels: the permute half of dispatch, the RANK_MAJOR / FLAT
// weighting of expert outputs, and combine.  All are HBM-bound: a row is
// moved as 16-byte pieces (8 bf16), one piece per lane, consecutive lanes on
// consecutive pieces, one source token (or received row) per workgroup
// iteration so that its routing metadata is wave-uniform.
//
// Semantics (FlashInfer "MoE-EP implementation & usage", section 3 "Algorithm
// / layout contracts"; Mooncake PG/EP guide, "Buffer.dispatch" /
// "Buffer.combine"):
//  - EXPERT_MAJOR: source row t is copied to every slot it was given; combine
//    re-weights on receive: out[t] = sum_k w[t,k] * y(slot of pick k).
//  - RANK_MAJOR / FLAT: source row t is copied once, to its receive row;
//    compute applies the real top_k with non-local picks weighted 0, and
//    combine is an unweighted sum over contributing ranks (one rank here).

#include "common.h"

namespace moe {
namespace {

// Threads per block for a row of `cpr` 16-byte pieces: a divisor of cpr when possible.
int row_threads(int32_t cpr) {
  if (cpr % 256 == 0) return 256;
  if (cpr % 128 == 0) return 128;
  return 64;
}

unsigned grid_for(int64_t items) {
  const int64_t cap = 1 << 20;
  return (unsigned)(items < 1 ? 1 : (items > cap ? cap : items));
}

// EXPERT_MAJOR permute: x[t] -> recv[slot] for every local pick of t.
__global__ void k_permute_em(const uint4* __restrict__ x, const int32_t* __restrict__ slot_of, int32_t N, int32_t K,
                             int32_t cpr, uint4* __restrict__ recv) {
  for (int32_t t = blockIdx.x; t < N; t += gridDim.x) {
    const int32_t* so = slot_of + (int64_t)t * K;
    int any = 0;
    for (int k = 0; k < K; ++k) any |= so[k] >= 0;
    if (!any) continue;
    for (int32_t c = threadIdx.x; c < cpr; c += blockDim.x) {
      const uint4 v = x[(int64_t)t * cpr + c];
      for (int k = 0; k < K; ++k) {
        const int32_t s = so[k];
        if (s >= 0) recv[(int64_t)s * cpr + c] = v;
      }
    }
  }
}

// RANK_MAJOR / FLAT permute: x[t] -> recv[row_of_token[t]].
__global__ void k_permute_rows(const uint4* __restrict__ x, const int32_t* __restrict__ row_of_token, int32_t N,
                               int32_t cpr, uint4* __restrict__ recv) {
  for (int32_t t = blockIdx.x; t < N; t += gridDim.x) {
    const int32_t row = row_of_token[t];
    if (row < 0) continue;
    for (int32_t c = threadIdx.x; c < cpr; c += blockDim.x) recv[(int64_t)row * cpr + c] = x[(int64_t)t * cpr + c];
  }
}

// EXPERT_MAJOR identity expert: expert_out[slot] = recv[slot] for every used slot.
__global__ void k_copy_slots(const int32_t* __restrict__ slot_of, int32_t N, int32_t K, int32_t cpr,
                             const uint4* __restrict__ recv, uint4* __restrict__ out) {
  for (int32_t t = blockIdx.x; t < N; t += gridDim.x) {
    const int32_t* so = slot_of + (int64_t)t * K;
    for (int k = 0; k < K; ++k) {
      const int32_t s = so[k];
      if (s < 0) continue;
      for (int32_t c = threadIdx.x; c < cpr; c += blockDim.x) out[(int64_t)s * cpr + c] = recv[(int64_t)s * cpr + c];
    }
  }
}

// EXPERT_MAJOR combine: out[t] = bf16(sum_k w[t,k] * Y[row(slot_of[t,k])]), k ascending, fp32.
__global__ void k_combine_em(const int32_t* __restrict__ slot_of, const float* __restrict__ w, int32_t N, int32_t K,
                             int32_t cpr, int64_t cap, const int32_t* __restrict__ offsets_packed,
                             const uint4* __restrict__ Y, uint4* __restrict__ out) {
  for (int32_t t = blockIdx.x; t < N; t += gridDim.x) {
    const int32_t* so = slot_of + (int64_t)t * K;
    const float* wt = w + (int64_t)t * K;
    for (int32_t c = threadIdx.x; c < cpr; c += blockDim.x) {
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int k = 0; k < K; ++k) {
        const int32_t s = so[k];
        if (s < 0) continue;
        const int64_t row = offsets_packed ? (int64_t)offsets_packed[s / cap] + s % cap : (int64_t)s;
        float f[8];
        unpack8(Y[row * cpr + c], f);
        const float wk = wt[k];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += wk * f[j];
      }
      out[(int64_t)t * cpr + c] = pack8(acc);
    }
  }
}

// RANK_MAJOR / FLAT: value of a received row = sum_k wmask[row,k] * y(pick k), fp32, k ascending.
// Token-major mode writes out[t] for every token (0 without a local pick); row mode writes z[row].
__global__ void k_finalize_rows(const int32_t* __restrict__ row_of_token, const int32_t* __restrict__ pick_slot,
                                const float* __restrict__ wmask, int32_t N, int32_t K, int32_t cpr,
                                const uint4* __restrict__ y, const uint4* __restrict__ recv_x,
                                uint4* __restrict__ dst, int token_major) {
  for (int32_t t = blockIdx.x; t < N; t += gridDim.x) {
    const int32_t row = row_of_token[t];
    if (row < 0) {
      if (token_major)
        for (int32_t c = threadIdx.x; c < cpr; c += blockDim.x) dst[(int64_t)t * cpr + c] = make_uint4(0, 0, 0, 0);
      continue;
    }
    const int32_t* ps = pick_slot + (int64_t)row * K;
    const float* wm = wmask + (int64_t)row * K;
    const int64_t drow = token_major ? t : row;
    for (int32_t c = threadIdx.x; c < cpr; c += blockDim.x) {
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int k = 0; k < K; ++k) {
        const int32_t p = ps[k];
        if (p < 0) continue;
        float f[8];
        unpack8(y ? y[(int64_t)p * cpr + c] : recv_x[(int64_t)row * cpr + c], f);
        const float wk = wm[k];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += wk * f[j];
      }
      dst[drow * cpr + c] = pack8(acc);
    }
  }
}

// RANK_MAJOR / FLAT combine: out[t] = z[row_of_token[t]] (0 without a local pick).
__global__ void k_combine_rows(const int32_t* __restrict__ row_of_token, int32_t N, int32_t cpr,
                               const uint4* __restrict__ z, uint4* __restrict__ out) {
  for (int32_t t = blockIdx.x; t < N; t += gridDim.x) {
    const int32_t row = row_of_token[t];
    for (int32_t c = threadIdx.x; c < cpr; c += blockDim.x)
      out[(int64_t)t * cpr + c] = row >= 0 ? z[(int64_t)row * cpr + c] : make_uint4(0, 0, 0, 0);
  }
}

}  // namespace

hipError_t launch_permute(const Geom& g, const void* x, const int32_t* slot_of, const int32_t* row_of_token,
                          void* recv_x, hipStream_t stream) {
  const int32_t cpr = g.H / 8;
  if (g.N == 0) return hipSuccess;
  if (g.layout == 0) {
    hipLaunchKernelGGL(k_permute_em, dim3(grid_for(g.N)), dim3(row_threads(cpr)), 0, stream, (const uint4*)x, slot_of,
                       g.N, g.K, cpr, (uint4*)recv_x);
  } else {
    hipLaunchKernelGGL(k_permute_rows, dim3(grid_for(g.N)), dim3(row_threads(cpr)), 0, stream, (const uint4*)x,
                       row_of_token, g.N, cpr, (uint4*)recv_x);
  }
  return hipGetLastError();
}

hipError_t launch_copy_slots(const Geom& g, const int32_t* slot_of, const void* recv_x, void* expert_out,
                             hipStream_t stream) {
  const int32_t cpr = g.H / 8;
  if (g.N == 0) return hipSuccess;
  hipLaunchKernelGGL(k_copy_slots, dim3(grid_for(g.N)), dim3(row_threads(cpr)), 0, stream, slot_of, g.N, g.K, cpr,
                     (const uint4*)recv_x, (uint4*)expert_out);
  return hipGetLastError();
}

hipError_t launch_combine_em(const Geom& g, const int32_t* slot_of, const float* topk_weights,
                             const int32_t* offsets_packed, const void* Y, void* out, hipStream_t stream) {
  const int32_t cpr = g.H / 8;
  if (g.N == 0) return hipSuccess;
  hipLaunchKernelGGL(k_combine_em, dim3(grid_for(g.N)), dim3(row_threads(cpr)), 0, stream, slot_of, topk_weights, g.N,
                     g.K, cpr, g.cap, offsets_packed, (const uint4*)Y, (uint4*)out);
  return hipGetLastError();
}

hipError_t launch_finalize_rows(const Geom& g, const int32_t* row_of_token, const int32_t* pick_slot,
                                const float* topk_wmask, const void* y_packed, const void* recv_x, void* dst,
                                bool out_token_major, hipStream_t stream) {
  const int32_t cpr = g.H / 8;
  if (g.N == 0) return hipSuccess;
  hipLaunchKernelGGL(k_finalize_rows, dim3(grid_for(g.N)), dim3(row_threads(cpr)), 0, stream, row_of_token, pick_slot,
                     topk_wmask, g.N, g.K, cpr, (const uint4*)y_packed, (const uint4*)recv_x, (uint4*)dst,
                     out_token_major ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_combine_rows(const Geom& g, const int32_t* row_of_token, const void* z, void* out,
                               hipStream_t stream) {
  const int32_t cpr = g.H / 8;
  if (g.N == 0) return hipSuccess;
  hipLaunchKernelGGL(k_combine_rows, dim3(grid_for(g.N)), dim3(row_threads(cpr)), 0, stream, row_of_token, g.N, cpr,
                     (const uint4*)z, (uint4*)out);
  return hipGetLastError();
}

}  // namespace moe
