// Work distribution of the persistent 256x256 grouped-GEMM kernels (gemm.hip, gemm_fp8.hip).
#pragma once

#include "common.h"

namespace moe {

// Items (expert row tile x column tile, in the grouped order of the tile table) are dealt in
// rounds: round r gives XCD x the `per` consecutive items (r * kGemmTickets + x) * per + [0, per)
// (workgroup b runs on XCD b mod kGemmTickets), whose A and B panels that XCD's L2 shares.  Round 0
// is static: workgroup j of XCD x takes item x * per + j.  After that a workgroup takes XCD x's next
// ticket from its counter as soon as it finishes an item, so XCDs that run faster do more items;
// once XCD x has no items left, its workgroups take what remains of the other XCDs' items in turn.
// Only thread 0 of a workgroup calls issue() / resolve(); the item is broadcast through LDS.
struct WorkTickets {
  int32_t* counters;  // kGemmTickets counters, zero at launch
  int64_t total;      // items
  int32_t per;        // workgroups per XCD
  int32_t xcd;
  int32_t victim;     // offset of the XCD whose items this workgroup takes (kGemmTickets: none left)

  __device__ int64_t item_of(int x, int64_t n) const {
    const int64_t it = ((n / per) * kGemmTickets + x) * per + n % per;
    return it < total ? it : -1;
  }
  __device__ int64_t first(int jx) const { return item_of(xcd, jx); }
  // Takes a ticket of the current XCD; its value is needed only by resolve(), so the atomic's latency
  // can overlap other work.  Returns 0 (unused) once every XCD is exhausted.
  __device__ int32_t issue() const {
    if (victim >= kGemmTickets) return 0;
    return __hip_atomic_fetch_add(&counters[(xcd + victim) % kGemmTickets], 1, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
  }
  // The item of ticket tk from issue(), or the next XCD's next item when that XCD is exhausted, or
  // -1 when every XCD is.  At most kGemmTickets further atomics.
  __device__ int64_t resolve(int32_t tk) {
    while (victim < kGemmTickets) {
      const int64_t it = item_of((xcd + victim) % kGemmTickets, (int64_t)per + tk);
      if (it >= 0) return it;
      if (++victim == kGemmTickets) break;
      tk = issue();
    }
    return -1;
  }
};

// A wave-uniform copy of a value that is the same in every lane.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

}  // namespace moe
