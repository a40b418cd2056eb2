// Row movement kernels: the permute half of dispatch, the RANK_MAJOR / FLAT
// weighting of expert outputs, and combine.  All are HBM-bound.
//
// Semantics (FlashInfer "MoE-EP implementation & usage", section 3 "Algorithm
// / layout contracts"; Mooncake PG/EP guide, "Buffer.dispatch" /
// "Buffer.combine"):
//  - EXPERT_MAJOR: source row t is copied to every slot it was given; combine
//    re-weights on receive: out[t] = sum_k w[t,k] * y(slot of pick k).
//  - RANK_MAJOR / FLAT: source row t is copied once, to its receive row;
//    compute applies the real top_k with non-local picks weighted 0, and
//    combine is an unweighted sum over contributing ranks (one rank here).
//
// Layout of the work: a workgroup handles one token (or received row) per
// iteration, so the routing metadata of that row is wave-uniform (scalar
// loads).  A row of H bf16 is H/8 pieces of 16 bytes; thread i handles pieces
// i, i + T, i + 2T, ... (T threads), consecutive lanes on consecutive pieces.
// When H/8 = CPT * 128 for a small CPT the piece count per thread is a
// compile-time constant and every load of the row (CPT pieces x up to 8
// picks) is issued before the first use, so each thread keeps many 16-byte
// requests in flight; other widths take a generic loop.  Rows that are read
// once (source rows, expert outputs) and combined outputs use non-temporal
// loads / stores, so they do not evict data that is reused; receive rows are
// stored normally because the expert GEMM reads them next.

#include "common.h"

namespace moe {
namespace {

constexpr int kPickUnroll = 8;  // picks gathered per batch
// Word 3 of a gfx9 raw buffer resource (32-bit data format, no swizzle).
constexpr int kBufferRsrcWord3 = 0x00020000;

typedef unsigned int u4v_t __attribute__((ext_vector_type(4)));
// Streaming (non-temporal) 16-byte load / store: rows moved here are touched once.
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  const u4v_t v = __builtin_nontemporal_load((const u4v_t*)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st_nt(uint4* p, const uint4& v) {
  __builtin_nontemporal_store(u4v_t{v.x, v.y, v.z, v.w}, (u4v_t*)p);
}

unsigned grid_for(int64_t items) {
  const int64_t cap = 1 << 20;
  return (unsigned)(items < 1 ? 1 : (items > cap ? cap : items));
}

// EXPERT_MAJOR permute: x[t] -> recv[slot] for every local pick of t.
template <int CPT>
__global__ void k_permute_em(const uint4* __restrict__ x, const int32_t* __restrict__ slot_of, int32_t N, int32_t K,
                             int32_t cpr, uint4* __restrict__ recv, LayoutRangeArgs lr) {
  layout_ranges(lr);
  for (int32_t t = blockIdx.x; t < N; t += gridDim.x) {
    const int32_t* so = slot_of + (int64_t)t * K;
    int any = 0;
    for (int k = 0; k < K; ++k) any |= so[k] >= 0;
    if (!any) continue;
    if constexpr (CPT > 0) {
      uint4 v[CPT];
#pragma unroll
      for (int j = 0; j < CPT; ++j) v[j] = ld_nt(&x[(int64_t)t * cpr + threadIdx.x + j * blockDim.x]);
      for (int k = 0; k < K; ++k) {
        const int32_t s = so[k];
        if (s < 0) continue;
#pragma unroll
        for (int j = 0; j < CPT; ++j) recv[(int64_t)s * cpr + threadIdx.x + j * blockDim.x] = v[j];
      }
    } else {
      for (int32_t c = threadIdx.x; c < cpr; c += blockDim.x) {
        const uint4 v = x[(int64_t)t * cpr + c];
        for (int k = 0; k < K; ++k) {
          const int32_t s = so[k];
          if (s >= 0) recv[(int64_t)s * cpr + c] = v;
        }
      }
    }
  }
}

// RANK_MAJOR / FLAT permute: x[t] -> recv[row_of_token[t]].
template <int CPT>
__global__ void k_permute_rows(const uint4* __restrict__ x, const int32_t* __restrict__ row_of_token, int32_t N,
                               int32_t cpr, uint4* __restrict__ recv) {
  for (int32_t t = blockIdx.x; t < N; t += gridDim.x) {
    const int32_t row = row_of_token[t];
    if (row < 0) continue;
    if constexpr (CPT > 0) {
      uint4 v[CPT];
#pragma unroll
      for (int j = 0; j < CPT; ++j) v[j] = ld_nt(&x[(int64_t)t * cpr + threadIdx.x + j * blockDim.x]);
#pragma unroll
      for (int j = 0; j < CPT; ++j) recv[(int64_t)row * cpr + threadIdx.x + j * blockDim.x] = v[j];
    } else {
      for (int32_t c = threadIdx.x; c < cpr; c += blockDim.x)
        recv[(int64_t)row * cpr + c] = x[(int64_t)t * cpr + c];
    }
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

// Weighted sum of source rows into one output row: dst = bf16(sum_k w_k * Y[row_k]), fp32, picks
// in ascending k.  `pick(k, &row, &w)` returns false for picks that do not contribute.  Picks
// are taken in batches of kPickUnroll with a fixed register slot per pick of the batch, so that
// a piece's loads from all of the batch's picks are in flight before the first one is used.
template <int CPT, class Pick>
__device__ __forceinline__ void weighted_row(int32_t K, const Pick& pick, const uint4* __restrict__ Y, int32_t cpr,
                                             uint4* __restrict__ dst) {
  if constexpr (CPT > 0) {
    float acc[CPT][8];
#pragma unroll
    for (int j = 0; j < CPT; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] = 0.0f;
    for (int k0 = 0; k0 < K; k0 += kPickUnroll) {
      // One buffer resource per pick: base = its source row, size = one row, or size 0 for a
      // pick that does not contribute, whose loads then return zeros without touching memory.
      // Every load is unconditional, so a piece's loads from all picks are in flight together.
      __amdgpu_buffer_rsrc_t rs[kPickUnroll];
      float wk[kPickUnroll];
#pragma unroll
      for (int i = 0; i < kPickUnroll; ++i) {
        int64_t r = 0;
        float w = 0.0f;
        const bool ok = k0 + i < K && pick(k0 + i, &r, &w);
        wk[i] = ok ? w : 0.0f;
        rs[i] = __builtin_amdgcn_make_buffer_rsrc((void*)(Y + (ok ? r : 0) * cpr), 0, ok ? cpr * 16 : 0,
                                                  kBufferRsrcWord3);
      }
      // two pieces per step: 2 x kPickUnroll loads in flight
#pragma unroll
      for (int j0 = 0; j0 < CPT; j0 += 2) {
        constexpr int kPair = 2;
        uint4 v[kPair][kPickUnroll];
#pragma unroll
        for (int jj = 0; jj < kPair; ++jj) {
          if (j0 + jj >= CPT) break;
          const int32_t ofs = (threadIdx.x + (j0 + jj) * blockDim.x) * 16;
#pragma unroll
          for (int i = 0; i < kPickUnroll; ++i) {
            // cache policy 2 = non-temporal: every expert-output row is read exactly once
            const auto q = __builtin_amdgcn_raw_buffer_load_b128(rs[i], ofs, 0, 2);
            v[jj][i] = make_uint4(q[0], q[1], q[2], q[3]);
          }
        }
#pragma unroll
        for (int jj = 0; jj < kPair; ++jj) {
          if (j0 + jj >= CPT) break;
#pragma unroll
          for (int i = 0; i < kPickUnroll; ++i) {
            float f[8];
            unpack8(v[jj][i], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[j0 + jj][e] += wk[i] * f[e];
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < CPT; ++j) st_nt(&dst[threadIdx.x + j * blockDim.x], pack8(acc[j]));
  } else {
    for (int32_t c = threadIdx.x; c < cpr; c += blockDim.x) {
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int k = 0; k < K; ++k) {
        int64_t r;
        float w;
        if (!pick(k, &r, &w)) continue;
        float f[8];
        unpack8(Y[r * cpr + c], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += w * f[e];
      }
      dst[c] = pack8(acc);
    }
  }
}

// EXPERT_MAJOR combine: out[t] = bf16(sum_k w[t,k] * Y[row(slot_of[t,k])]), k ascending, fp32.
// Y row of slot s = el*cap + j is offsets_packed[el] + j when packed, else s.
// Launched with at most 256 threads (row_shape).  Bounding the workgroup lets the compiler keep
// the 7- and 8-piece forms in registers: under its default bound of 1024 threads it caps them at
// 128 VGPRs and spills 24-28 bytes per lane.  Measured: decode combine_em<7> 15.6 -> 14.5 us
// (same 4 waves per SIMD, no spill); prefill finalize_rows<7> 515 -> 505 us (130 VGPRs, 3 waves
// per SIMD, no spill).
template <int CPT>
__global__ __launch_bounds__(256) void k_combine_em(const int32_t* __restrict__ slot_of, const float* __restrict__ w, int32_t N, int32_t K,
                             int32_t cpr, int64_t cap, const int32_t* __restrict__ offsets_packed,
                             const int32_t* __restrict__ active, int32_t T, const uint4* __restrict__ Y,
                             uint4* __restrict__ out) {
  for (int32_t t = blockIdx.x; t < N; t += gridDim.x) {
    const int32_t* so = slot_of + (int64_t)t * K;
    const float* wt = w + (int64_t)t * K;
    const bool skip = active && active[t / T] == 0;  // inactive source rank: zero output
    auto pick = [&](int k, int64_t* r, float* wk) {
      const int32_t s = so[k];
      if (skip || s < 0) return false;
      *r = offsets_packed ? (int64_t)offsets_packed[s / cap] + s % cap : (int64_t)s;
      *wk = wt[k];
      return true;
    };
    weighted_row<CPT>(K, pick, Y, cpr, out + (int64_t)t * cpr);
  }
}

// RANK_MAJOR / FLAT: value of a received row = sum_k wmask[row,k] * y(pick k), fp32, k ascending.
// Token-major mode writes out[t] for every token (0 without a local pick); row mode writes z[row].
template <int CPT>
__global__ __launch_bounds__(256) void k_finalize_rows(const int32_t* __restrict__ row_of_token, const int32_t* __restrict__ pick_slot,
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
    auto pick = [&](int k, int64_t* r, float* wk) {
      const int32_t p = ps[k];
      if (p < 0) return false;
      *r = y ? (int64_t)p : (int64_t)row;  // identity expert: y(pick) is the received row
      *wk = wm[k];
      return true;
    };
    weighted_row<CPT>(K, pick, y ? y : recv_x, cpr, dst + (token_major ? (int64_t)t : (int64_t)row) * cpr);
  }
}

// RANK_MAJOR / FLAT combine: out[t] = z[row_of_token[t]] (0 without a local pick).
__global__ void k_combine_rows(const int32_t* __restrict__ row_of_token, int32_t N, int32_t cpr,
                               const int32_t* __restrict__ active, int32_t T, const uint4* __restrict__ z,
                               uint4* __restrict__ out) {
  for (int32_t t = blockIdx.x; t < N; t += gridDim.x) {
    const int32_t row = (active && active[t / T] == 0) ? -1 : row_of_token[t];
    for (int32_t c = threadIdx.x; c < cpr; c += blockDim.x)
      out[(int64_t)t * cpr + c] = row >= 0 ? z[(int64_t)row * cpr + c] : make_uint4(0, 0, 0, 0);
  }
}

__global__ void k_zero(uint4* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

// Threads per workgroup and pieces per thread for a row of cpr pieces: 128 threads with a
// compile-time piece count when cpr = CPT * 128 (CPT in 1, 2, 4, 7, 8); otherwise a generic
// loop with up to 256 threads.
struct RowShape {
  int threads, cpt;
};
RowShape row_shape(int32_t cpr) {
  if (cpr % 128 == 0) {
    const int c = cpr / 128;
    if (c == 1 || c == 2 || c == 4 || c == 7 || c == 8) return {128, c};
  }
  if (cpr % 256 == 0) return {256, 0};
  if (cpr % 128 == 0) return {128, 0};
  return {64, 0};
}

#define MOE_DISPATCH_CPT(cpt, KERNEL, ...)                                       \
  switch (cpt) {                                                                 \
    case 1: hipLaunchKernelGGL(KERNEL<1>, __VA_ARGS__); break;                   \
    case 2: hipLaunchKernelGGL(KERNEL<2>, __VA_ARGS__); break;                   \
    case 4: hipLaunchKernelGGL(KERNEL<4>, __VA_ARGS__); break;                   \
    case 7: hipLaunchKernelGGL(KERNEL<7>, __VA_ARGS__); break;                   \
    case 8: hipLaunchKernelGGL(KERNEL<8>, __VA_ARGS__); break;                   \
    default: hipLaunchKernelGGL(KERNEL<0>, __VA_ARGS__); break;                  \
  }

}  // namespace

hipError_t launch_permute(const Geom& g, const void* x, const int32_t* slot_of, const int32_t* row_of_token,
                          void* recv_x, hipStream_t stream, const LayoutRangeArgs& lr) {
  const int32_t cpr = g.H / 8;
  if (g.N == 0) return hipSuccess;
  const RowShape rs = row_shape(cpr);
  if (g.layout == 0) {
    MOE_DISPATCH_CPT(rs.cpt, k_permute_em, dim3(grid_for(g.N)), dim3(rs.threads), 0, stream, (const uint4*)x, slot_of,
                     g.N, g.K, cpr, (uint4*)recv_x, lr);
  } else {
    MOE_DISPATCH_CPT(rs.cpt, k_permute_rows, dim3(grid_for(g.N)), dim3(rs.threads), 0, stream, (const uint4*)x,
                     row_of_token, g.N, cpr, (uint4*)recv_x);
  }
  return hipGetLastError();
}

hipError_t launch_copy_slots(const Geom& g, const int32_t* slot_of, const void* recv_x, void* expert_out,
                             hipStream_t stream) {
  const int32_t cpr = g.H / 8;
  if (g.N == 0) return hipSuccess;
  hipLaunchKernelGGL(k_copy_slots, dim3(grid_for(g.N)), dim3(row_shape(cpr).threads), 0, stream, slot_of, g.N, g.K,
                     cpr, (const uint4*)recv_x, (uint4*)expert_out);
  return hipGetLastError();
}

hipError_t launch_combine_em(const Geom& g, const int32_t* slot_of, const float* topk_weights,
                             const int32_t* offsets_packed, const void* Y, void* out, hipStream_t stream) {
  const int32_t cpr = g.H / 8;
  if (g.N == 0) return hipSuccess;
  const RowShape rs = row_shape(cpr);
  MOE_DISPATCH_CPT(rs.cpt, k_combine_em, dim3(grid_for(g.N)), dim3(rs.threads), 0, stream, slot_of, topk_weights, g.N,
                   g.K, cpr, g.cap, offsets_packed, g.active, g.T, (const uint4*)Y, (uint4*)out);
  return hipGetLastError();
}

hipError_t launch_finalize_rows(const Geom& g, const int32_t* row_of_token, const int32_t* pick_slot,
                                const float* topk_wmask, const void* y_packed, const void* recv_x, void* dst,
                                bool out_token_major, hipStream_t stream) {
  const int32_t cpr = g.H / 8;
  if (g.N == 0) return hipSuccess;
  const RowShape rs = row_shape(cpr);
  MOE_DISPATCH_CPT(rs.cpt, k_finalize_rows, dim3(grid_for(g.N)), dim3(rs.threads), 0, stream, row_of_token,
                   pick_slot, topk_wmask, g.N, g.K, cpr, (const uint4*)y_packed, (const uint4*)recv_x, (uint4*)dst,
                   out_token_major ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_combine_rows(const Geom& g, const int32_t* row_of_token, const void* z, void* out,
                               hipStream_t stream) {
  const int32_t cpr = g.H / 8;
  if (g.N == 0) return hipSuccess;
  hipLaunchKernelGGL(k_combine_rows, dim3(grid_for(g.N)), dim3(row_shape(cpr).threads), 0, stream, row_of_token, g.N,
                     cpr, g.active, g.T, (const uint4*)z, (uint4*)out);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, int64_t n, hipStream_t stream) {
  const int64_t n16 = n / 16;
  if (n16 <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero, dim3(grid_for((n16 + 255) / 256 < 4096 ? (n16 + 255) / 256 : 4096)), dim3(256), 0, stream,
                     (uint4*)p, n16);
  return hipGetLastError();
}

}  // namespace moe
