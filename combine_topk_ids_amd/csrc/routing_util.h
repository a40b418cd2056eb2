// Device helpers shared by the routing kernels (routing.hip) and the one-launch low-latency
// dispatch (dispatch_ll.hip): wave ballots that find equal expert ids, dispatch's view of the global
// expert ids, block-wide scans, and the GEMM tile table written from the final counts.
#pragma once

#include "common.h"

namespace moe {

__device__ __forceinline__ uint64_t lanes_below(int lane) { return (1ull << lane) - 1ull; }

// Lanes whose expert id equals this lane's (meaningful only for el >= 0).
__device__ __forceinline__ uint64_t match_mask(int el, int nbits) {
  uint64_t m = __ballot(el >= 0);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (el >> b) & 1;
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

// Global expert ids of dispatch: local iff in [o, o+L); ids outside [-1, E) are errors.
struct GlobalIds {
  const int64_t* ids;
  int64_t o;
  int32_t L, E;
  const int32_t* active;  // source-rank mask or nullptr
  int32_t T, K;
  __device__ __forceinline__ int local(int64_t q, int* err) const {
    // a pick of a token from an inactive source rank is not received (nor checked)
    if (active && active[(int32_t)q / K / T] == 0) return -1;
    const int64_t id = ids[q];
    if (id < -1 || id >= E) *err = 1;
    return (id >= o && id < o + L) ? (int)(id - o) : -1;
  }
};

// Exclusive scan of one value per thread over the block (blockDim.x == 1024); *total = block sum.
static __device__ int32_t block_exclusive_scan(int32_t v, int32_t* total) {
  __shared__ int32_t wsum[1024 / kWave];
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  int32_t x = v;
  for (int d = 1; d < kWave; d <<= 1) {
    const int32_t y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  if (lane == kWave - 1) wsum[w] = x;
  __syncthreads();
  if (w == 0) {
    int32_t s = lane < nw ? wsum[lane] : 0;
    for (int d = 1; d < kWave; d <<= 1) {
      const int32_t y = __shfl_up(s, d, kWave);
      if (lane >= d) s += y;
    }
    if (lane < nw) wsum[lane] = s;  // inclusive wave totals
  }
  __syncthreads();
  const int32_t before = w > 0 ? wsum[w - 1] : 0;
  *total = wsum[nw - 1];
  __syncthreads();
  return before + x - v;
}

// Exclusive scan of in[0..n) into out[0..n) with one 1024-thread block; returns the sum.
static __device__ int32_t block_scan_array(const int32_t* in, int32_t* out, int32_t n) {
  int32_t carry = 0;
  for (int32_t base = 0; base < n; base += blockDim.x) {
    const int32_t i = base + threadIdx.x;
    const int32_t v = i < n ? in[i] : 0;
    int32_t total;
    const int32_t ex = block_exclusive_scan(v, &total);
    if (i < n) out[i] = carry + ex;
    carry += total;
  }
  return carry;
}

// Workgroup 0 of a fused routing kernel, counts final in s_tot: the GEMM tile table (each expert's
// ceil(min(count, clamp) / bm) tiles, placed by an exclusive scan over the experts; s_tb [L + 1]).
static __device__ void write_tiles(const TileArgs& ta, int32_t L, const int32_t* s_tot, int32_t* s_tb) {
  for (int32_t i = threadIdx.x; i < ta.nzero; i += blockDim.x) ta.zero[i] = 0;
  for (int el = threadIdx.x; el < L; el += blockDim.x)
    s_tb[el] = (int32_t)((min((int64_t)s_tot[el], ta.clamp) + ta.bm - 1) / ta.bm);
  __syncthreads();
  const int32_t nt = block_scan_array(s_tb, s_tb, L);  // in place: each thread rewrites what it read
  if (threadIdx.x == 0) *ta.num_tiles = nt;
  __syncthreads();
  for (int el = threadIdx.x; el < L; el += blockDim.x) {
    const int32_t first = s_tb[el], n = (el + 1 < L ? s_tb[el + 1] : nt) - first;
    for (int32_t j = 0; j < n; ++j) ta.tiles[first + j] = make_int2(el, j * ta.bm);
  }
}

}  // namespace moe
