// Router upstream of dispatch: for each token, the top_k experts by score and softmax weights
// over the selected scores (Mooncake PG/EP guide quick start: topk_idx is the top_k of per-token
// expert scores, topk_weights a softmax; FlashInfer "MoE-EP implementation & usage", section 4,
// step 2).  Equal scores are ordered by the lower expert id, so the result is unique.
//
// One wave per token.  Each (score, id) becomes a 64-bit key whose unsigned order is the
// selection order (higher score first, then lower id); lane l holds the keys of experts
// l, l+64, l+128, ... (coalesced loads), sorted descending in registers.  top_k rounds of a
// wave-wide maximum over the lanes' heads pick the winners in order; the winning lane drops
// its head.  Lane k keeps the k-th winner, then the wave computes the softmax.
#include "common.h"

namespace moe {
namespace {

constexpr int kRouterThreads = 256;

// Unsigned order of the high word = numeric order of the score (negative scores: every bit
// flipped; non-negative: sign bit set); -0.0 is first made +0.0 so that it ties with +0.0.
// The low word ~id puts the lower id first among equal scores.  Key 0 is below every score.
__device__ __forceinline__ uint64_t make_key(float s, int32_t id) {
  s = s + 0.0f;  // -0.0 + 0.0 = +0.0 in round-to-nearest
  uint32_t b = __float_as_uint(s);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)b << 32) | (uint64_t)(~(uint32_t)id);
}
__device__ __forceinline__ float key_score(uint64_t k) {
  uint32_t b = (uint32_t)(k >> 32);
  b = (b & 0x80000000u) ? (b & 0x7fffffffu) : ~b;
  return __uint_as_float(b);
}
__device__ __forceinline__ int32_t key_id(uint64_t k) { return (int32_t)(~(uint32_t)k); }

template <int EPT>
__global__ __launch_bounds__(kRouterThreads) void k_router_topk(const float* __restrict__ scores, int32_t N,
                                                                int32_t E, int32_t K, int64_t* __restrict__ ids,
                                                                float* __restrict__ weights) {
  const int lane = threadIdx.x % kWave;
  const int32_t nwaves = gridDim.x * (kRouterThreads / kWave);
  for (int32_t t = blockIdx.x * (kRouterThreads / kWave) + threadIdx.x / kWave; t < N; t += nwaves) {
    const float* s = scores + (int64_t)t * E;
    uint64_t key[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int32_t j = i * kWave + lane;
      key[i] = j < E ? make_key(s[j], j) : 0ull;
    }
    // odd-even transposition sort, descending (EPT passes sort EPT keys)
#pragma unroll
    for (int pass = 0; pass < EPT; ++pass)
#pragma unroll
      for (int b = pass & 1; b + 1 < EPT; b += 2)
        if (key[b] < key[b + 1]) {
          const uint64_t x = key[b];
          key[b] = key[b + 1];
          key[b + 1] = x;
        }
    uint64_t mine = 0;
    for (int k = 0; k < K; ++k) {
      uint64_t best = key[0];
#pragma unroll
      for (int off = kWave / 2; off >= 1; off >>= 1) {
        const uint64_t o = __shfl_xor(best, off, kWave);
        best = o > best ? o : best;
      }
      if (key[0] == best) {  // keys are distinct (distinct ids): exactly one lane
#pragma unroll
        for (int i = 0; i + 1 < EPT; ++i) key[i] = key[i + 1];
        key[EPT - 1] = 0ull;
      }
      if (lane == k) mine = best;
    }
    // softmax over the K winners, relative to the largest; one lane's sum is broadcast so every
    // weight is divided by the same value
    const float sk = key_score(mine);
    const float s0 = __shfl(sk, 0, kWave);
    const float e = lane < K ? expf(sk - s0) : 0.0f;
    float sum = e;
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, kWave);
    sum = __shfl(sum, 0, kWave);
    if (lane < K) {
      ids[(int64_t)t * K + lane] = key_id(mine);
      weights[(int64_t)t * K + lane] = e / sum;
    }
  }
}

}  // namespace

hipError_t launch_router_topk(const float* scores, int32_t N, int32_t E, int32_t K, int64_t* ids, float* weights,
                              hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const int ept = (E + kWave - 1) / kWave;
  const int waves_per_block = kRouterThreads / kWave;
  const int64_t want = ((int64_t)N + waves_per_block - 1) / waves_per_block;
  const int blocks = (int)(want < 8192 ? want : 8192);
  const dim3 grid(blocks), block(kRouterThreads);
  if (ept <= 1)
    hipLaunchKernelGGL(k_router_topk<1>, grid, block, 0, stream, scores, N, E, K, ids, weights);
  else if (ept <= 2)
    hipLaunchKernelGGL(k_router_topk<2>, grid, block, 0, stream, scores, N, E, K, ids, weights);
  else if (ept <= 4)
    hipLaunchKernelGGL(k_router_topk<4>, grid, block, 0, stream, scores, N, E, K, ids, weights);
  else if (ept <= 8)
    hipLaunchKernelGGL(k_router_topk<8>, grid, block, 0, stream, scores, N, E, K, ids, weights);
  else
    hipLaunchKernelGGL(k_router_topk<16>, grid, block, 0, stream, scores, N, E, K, ids, weights);
  return hipGetLastError();
}

}  // namespace moe
