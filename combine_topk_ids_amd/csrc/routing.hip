// Routing kernels: the front half of dispatch and the compute-side bridge.
//
// What is computed (FlashInfer "MoE-EP implementation & usage", section 3
// "Algorithm / layout contracts"; Mooncake PG/EP guide, "Buffer.dispatch"):
// for every local expert the number of picks it receives and, for every pick,
// its slot.  Slots of one expert follow (source rank, token, k) order; token
// t = r*T + i, so that is the flat pick index q = t*K + k, ascending.  The
// result is therefore a stable counting sort of the picks by local expert.
//
// How: picks are cut into chunks of kChunkTokens tokens (one workgroup each)
// and each chunk into wave segments of 64 consecutive picks.  In a segment,
// lanes holding the same expert find each other with ballots over the bits of
// the expert id (one ballot per bit), so a pick's rank among equal picks of
// the segment is popcount(match & lanes-below) and the segment's count per
// expert is popcount(match), added by the lowest matching lane into a
// per-wave LDS counter.  Pass 1 writes per-chunk histograms; pass 2 (one
// workgroup) scans them per expert across chunks and exclusively across
// experts; pass 3 recomputes the per-wave counts, turns them into per-wave
// bases and hands out slots.  When the histograms are small (chunks x local
// experts up to kFusedScanMax) pass 2 is folded into pass 3: each workgroup
// sums the histograms of the chunks before its own (and of all chunks, for the
// totals), and workgroup 0 writes the totals, their scan and the status word,
// which saves a launch on the latency-bound small layers.  Every count is an
// ordered sum of ballot popcounts: no atomics, so the permutation is
// deterministic.

#include "common.h"
#include "routing_util.h"

namespace moe {
namespace {

// Local ids of received routing (-1 = masked); anything outside [-1, L) is an error.
struct LocalIds {
  const int32_t* ids;
  int32_t L;
  __device__ __forceinline__ int local(int64_t q, int* err) const {
    const int32_t id = ids[q];
    if (id < -1 || id >= L) *err = 1;
    return (id >= 0 && id < L) ? id : -1;
  }
};

struct ChunkRange {
  int64_t q0, q1;  // this wave's picks [q0, q1)
  int32_t r0, r1;  // the chunk's rows [r0, r1)
};

__device__ __forceinline__ ChunkRange chunk_range(int32_t nrows, int32_t K) {
  ChunkRange cr;
  cr.r0 = blockIdx.x * kChunkTokens;
  cr.r1 = min(cr.r0 + kChunkTokens, nrows);
  const int64_t cq0 = (int64_t)cr.r0 * K, cq1 = (int64_t)max(cr.r1, cr.r0) * K;
  const int64_t seg = kRouteWaves * (int64_t)kWave;
  const int64_t per_wave = ((cq1 - cq0 + seg - 1) / seg) * kWave;
  const int w = threadIdx.x / kWave;
  cr.q0 = cq0 + w * per_wave;
  cr.q1 = min(cr.q0 + per_wave, cq1);
  if (cr.q0 > cr.q1) cr.q0 = cr.q1;
  return cr;
}

__device__ __forceinline__ int32_t rows_now(int32_t nrows_max, const int32_t* nrows_dev) {
  return nrows_dev ? min(max(*nrows_dev, 0), nrows_max) : nrows_max;
}

// Walk this wave's picks; per segment add the per-expert counts into cnt (this wave's row).
template <class Src>
__device__ __forceinline__ void wave_count(const Src& src, const ChunkRange& cr, int nbits, int32_t* cnt,
                                           int* err) {
  const int lane = threadIdx.x % kWave;
  for (int64_t base = cr.q0; base < cr.q1; base += kWave) {
    const int64_t q = base + lane;
    const int el = (q < cr.q1) ? src.local(q, err) : -1;
    const uint64_t m = match_mask(el, nbits);
    if (el >= 0 && (m & lanes_below(lane)) == 0) cnt[el] += __popcll(m);
  }
}

// Pass 1: per-chunk histogram of local picks (+ per-chunk count of rows with a local pick).
template <class Src>
__global__ __launch_bounds__(kRouteThreads) void k_route_count(Src src, int32_t nrows_max, const int32_t* nrows_dev,
                                                               int32_t K, int32_t L, int32_t nbits,
                                                               int32_t* chunk_hist, int32_t* chunk_tok,
                                                               int32_t* chunk_err) {
  __shared__ int32_t cnt[kRouteWaves][kMaxLocalExperts];
  __shared__ int32_t s_err, s_tok;
  const int w = threadIdx.x / kWave;
  for (int i = threadIdx.x; i < kRouteWaves * L; i += blockDim.x) cnt[i / L][i % L] = 0;
  if (threadIdx.x == 0) s_err = 0, s_tok = 0;
  __syncthreads();
  const int32_t nrows = rows_now(nrows_max, nrows_dev);
  const ChunkRange cr = chunk_range(nrows, K);
  int err = 0;
  wave_count(src, cr, nbits, cnt[w], &err);
  // rows of the chunk that hold at least one local pick (one row per thread)
  int has = 0;
  const int32_t row = cr.r0 + (int32_t)threadIdx.x;
  if (row < cr.r1) {
    for (int k = 0; k < K; ++k) has |= src.local((int64_t)row * K + k, &err) >= 0;
  }
  const uint64_t hb = __ballot(has);
  if (err) atomicOr(&s_err, 1);
  if (threadIdx.x % kWave == 0 && hb) atomicAdd(&s_tok, (int)__popcll(hb));  // integer sum: order-free
  __syncthreads();
  for (int el = threadIdx.x; el < L; el += blockDim.x) {
    int32_t s = 0;
    for (int v = 0; v < kRouteWaves; ++v) s += cnt[v][el];
    chunk_hist[(int64_t)blockIdx.x * L + el] = s;
  }
  if (threadIdx.x == 0) {
    if (chunk_tok) chunk_tok[blockIdx.x] = s_tok;
    chunk_err[blockIdx.x] = s_err;
  }
}

// Pass 2 (one 1024-thread block): per-expert exclusive scan across chunks (thread el walks the
// chunks of expert el in order; a chunk's L histogram entries are contiguous, so each step's loads
// are coalesced across the experts, and the loads of kScanBatch chunks are issued together),
// exclusive scan across experts, row compaction bases, status.
constexpr int kScanBatch = 8;
__global__ __launch_bounds__(1024) void k_route_scan(const int32_t* chunk_hist, const int32_t* chunk_tok,
                                                     const int32_t* chunk_err, int32_t nchunks, int32_t L,
                                                     int64_t cap, int32_t* chunk_base, int32_t* counts,
                                                     int32_t* offsets, int32_t* chunk_tokbase, int32_t* num_rows,
                                                     int32_t* status, int status_overwrite) {
  __shared__ int32_t s_err;
  if (threadIdx.x == 0) s_err = 0;
  __syncthreads();
  int err = 0;
  for (int el = threadIdx.x; el < L; el += blockDim.x) {
    int32_t carry = 0;
    int32_t c0 = 0;
    for (; c0 + kScanBatch <= nchunks; c0 += kScanBatch) {
      int32_t v[kScanBatch];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) v[j] = chunk_hist[(int64_t)(c0 + j) * L + el];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) {
        chunk_base[(int64_t)(c0 + j) * L + el] = carry;
        carry += v[j];
      }
    }
    for (; c0 < nchunks; ++c0) {
      const int32_t v = chunk_hist[(int64_t)c0 * L + el];
      chunk_base[(int64_t)c0 * L + el] = carry;
      carry += v;
    }
    counts[el] = carry;
    if (cap > 0 && carry > cap) err |= kStatusCapacity;
  }
  for (int32_t c = threadIdx.x; c < nchunks; c += blockDim.x)
    if (chunk_err[c]) err |= kStatusBadExpertId;
  if (err) atomicOr(&s_err, err);
  __threadfence_block();
  __syncthreads();
  const int32_t total = block_scan_array(counts, offsets, L);
  if (threadIdx.x == 0) offsets[L] = total;
  if (chunk_tok) {
    const int32_t nr = block_scan_array(chunk_tok, chunk_tokbase, nchunks);
    if (threadIdx.x == 0 && num_rows) *num_rows = nr;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (status_overwrite) *status = s_err;
    else if (s_err) atomicOr(status, s_err);
  }
}

// Pass 2 folded into the consumer (see the header).  Every workgroup: s_base[el] = picks of expert
// el in the chunks before this one, s_tot[el] = in all chunks, s_off = exclusive scan of s_tot (s_off[L]
// = total).  Workgroup 0 also writes counts, offsets and the status word (overwrite: a fresh
// dispatch; otherwise OR-ed in).
constexpr int64_t kFusedScanMax = 1 << 15;
struct ScanArgs {
  const int32_t* chunk_hist;  // [nchunks * L]
  const int32_t* chunk_err;   // [nchunks]
  int32_t nchunks;
  int64_t cap;                // EXPERT_MAJOR capacity check (0: none)
  int32_t* counts;
  int32_t* offsets;           // [L + 1]
  int32_t* status;
  int status_overwrite;
  TileArgs tiles;             // optional: the GEMM tile table, written by workgroup 0
};

__device__ void fused_scan(const ScanArgs& sa, int32_t L, int32_t* s_base, int32_t* s_tot, int32_t* s_off,
                           int32_t* s_tb) {
  __shared__ int32_t s_err;
  if (threadIdx.x == 0) s_err = 0;
  const int32_t c = blockIdx.x;
  for (int el = threadIdx.x; el < L; el += blockDim.x) s_base[el] = s_tot[el] = 0;
  __syncthreads();
  // G groups of threads split the chunks (G = 1 once L fills the workgroup); their integer partial
  // sums meet in LDS, exact in any order
  const int32_t G = L < (int32_t)blockDim.x ? (int32_t)blockDim.x / L : 1;
  const int32_t grp = (int32_t)threadIdx.x / (G > 1 ? L : (int32_t)blockDim.x);
  if (grp < G) {
    for (int el = G > 1 ? (int32_t)threadIdx.x % L : (int32_t)threadIdx.x; el < L; el += blockDim.x) {
      int32_t b = 0, t = 0;
#pragma unroll 8
      for (int32_t cc = grp; cc < sa.nchunks; cc += G) {
        const int32_t v = sa.chunk_hist[(int64_t)cc * L + el];
        b += cc < c ? v : 0;
        t += v;
      }
      if (G > 1) {
        atomicAdd(&s_base[el], b);
        atomicAdd(&s_tot[el], t);
      } else {
        s_base[el] = b;
        s_tot[el] = t;
      }
    }
  }
  __syncthreads();
  const int32_t total = block_scan_array(s_tot, s_off, L);
  if (threadIdx.x == 0) s_off[L] = total;
  __syncthreads();
  if (blockIdx.x == 0) {
    int err = 0;
    for (int el = threadIdx.x; el < L; el += blockDim.x) {
      sa.counts[el] = s_tot[el];
      sa.offsets[el] = s_off[el];
      if (sa.cap > 0 && s_tot[el] > sa.cap) err |= kStatusCapacity;
    }
    if (threadIdx.x == 0) sa.offsets[L] = total;
    for (int32_t cc = threadIdx.x; cc < sa.nchunks; cc += blockDim.x)
      if (sa.chunk_err[cc]) err |= kStatusBadExpertId;
    if (err) atomicOr(&s_err, err);
    __syncthreads();
    if (threadIdx.x == 0) {
      if (sa.status_overwrite) *sa.status = s_err;
      else if (s_err) atomicOr(sa.status, s_err);
    }
    if (sa.tiles.tiles) write_tiles(sa.tiles, L, s_tot, s_tb);
  }
}

// Pass 3: hand out slots.  Sink::emit(q, el, slot) is called for every pick of the chunk
// (el = -1 for picks that are not local).
// kFused: pass 2 folded in (fused_scan); chunk_base is then unused.
template <class Src, class Sink, bool kFused>
__global__ __launch_bounds__(kRouteThreads) void k_route_assign(Src src, Sink sink, int32_t nrows_max,
                                                                const int32_t* nrows_dev, int32_t K, int32_t L,
                                                                int32_t nbits, const int32_t* chunk_base,
                                                                ScanArgs sa) {
  __shared__ int32_t run[kRouteWaves][kMaxLocalExperts];
  __shared__ int32_t s_base[kFused ? kMaxLocalExperts : 1], s_tot[kFused ? kMaxLocalExperts : 1];
  __shared__ int32_t s_off[kFused ? kMaxLocalExperts + 1 : 1];
  __shared__ int32_t s_tb[kFused ? kMaxLocalExperts + 1 : 1];
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  if constexpr (kFused) {
    fused_scan(sa, L, s_base, s_tot, s_off, s_tb);
    if constexpr (Sink::kUsesOffsets) sink.offsets = s_off;
  }
  for (int i = threadIdx.x; i < kRouteWaves * L; i += blockDim.x) run[i / L][i % L] = 0;
  __syncthreads();
  const int32_t nrows = rows_now(nrows_max, nrows_dev);
  const ChunkRange cr = chunk_range(nrows, K);
  int err = 0;
  wave_count(src, cr, nbits, run[w], &err);
  __syncthreads();
  // per-wave bases: chunk base of the expert plus the counts of the waves before
  for (int el = threadIdx.x; el < L; el += blockDim.x) {
    int32_t acc = kFused ? s_base[el] : chunk_base[(int64_t)blockIdx.x * L + el];
    for (int v = 0; v < kRouteWaves; ++v) {
      const int32_t c = run[v][el];
      run[v][el] = acc;
      acc += c;
    }
  }
  __syncthreads();
  int32_t* my = run[w];
  for (int64_t base = cr.q0; base < cr.q1; base += kWave) {
    const int64_t q = base + lane;
    const int el = (q < cr.q1) ? src.local(q, &err) : -1;
    const uint64_t m = match_mask(el, nbits);
    int32_t slot = -1;
    if (el >= 0) slot = my[el] + (int32_t)__popcll(m & lanes_below(lane));
    // the wave's LDS accesses complete in program order: every lane read my[el] above
    if (el >= 0 && (m & lanes_below(lane)) == 0) my[el] += __popcll(m);
    if (q < cr.q1) sink.emit(q, el, slot);
  }
}

// EXPERT_MAJOR dispatch sink: slot_of and src_info.
struct EmSink {
  static constexpr bool kUsesOffsets = false;
  int32_t* slot_of;
  int32_t* src_info;
  int64_t cap;
  int32_t K;
  __device__ __forceinline__ void emit(int64_t q, int el, int32_t slot) const {
    if (el >= 0 && slot < cap) {
      const int64_t s = el * cap + slot;
      slot_of[q] = (int32_t)s;
      src_info[s] = (int32_t)(q / K);
    } else {
      slot_of[q] = -1;  // not local, or over capacity (latched in the status word)
    }
  }
};

// Bridge sink: expert-sorted pick order, local -> global ids, masked weights; for the combine fused
// into the down GEMM also each pick's weight and source token in expert-sorted order.
struct BridgeSink {
  static constexpr bool kUsesOffsets = true;
  const int32_t* offsets;  // expert offsets (in LDS when pass 2 is folded in)
  const float* w;
  int32_t* perm;
  int32_t* pick_slot;
  int32_t* gid;
  float* wmask;
  int32_t o;
  BridgeCombine bc;
  int32_t K;
  __device__ __forceinline__ void emit(int64_t q, int el, int32_t slot) const {
    if (el >= 0) {
      const int32_t pos = offsets[el] + slot;
      perm[pos] = (int32_t)q;
      pick_slot[q] = pos;
      gid[q] = el + o;
      wmask[q] = w[q];
      if (bc.pick_w) {
        const int32_t row = (int32_t)(q / K);
        bc.pick_w[pos] = w[q];
        bc.pick_tok[pos] = bc.src_idx ? bc.src_idx[row] : row;
      }
    } else {
      pick_slot[q] = -1;
      gid[q] = -1;
      wmask[q] = 0.0f;
    }
  }
};

// EXPERT_MAJOR layout ranges: (first slot, count) per (local expert, source rank), by binary
// search over the expert's ascending src_info.
__global__ void k_layout_range(const int32_t* counts, const int32_t* src_info, int32_t L, int32_t W, int32_t T,
                               int64_t cap, int32_t* layout_range) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)L * W) return;
  const int32_t el = (int32_t)(i / W), r = (int32_t)(i % W);
  const int32_t n = (int32_t)min((int64_t)counts[el], cap);
  const int32_t* s = src_info + el * cap;
  auto lower_bound = [&](int32_t key) {
    int32_t lo = 0, hi = n;
    while (lo < hi) {
      const int32_t mid = (lo + hi) >> 1;
      if (s[mid] < key) lo = mid + 1;
      else hi = mid;
    }
    return lo;
  };
  const int32_t b = lower_bound(r * T), e = lower_bound((r + 1) * T);
  layout_range[i * 2 + 0] = b;
  layout_range[i * 2 + 1] = e - b;
}

// RANK_MAJOR / FLAT dispatch: the received routing rows.  One thread per source row.
// kFused: pass 2 folded in (fused_scan, and the row base of this chunk summed from chunk_tok);
// chunk_tokbase is then unused.
template <bool kFused>
__global__ __launch_bounds__(kRouteThreads) void k_route_rows(GlobalIds src, const float* topk_weights,
                                                              int32_t nrows, int32_t N, int32_t K, int flat,
                                                              const int32_t* chunk_tokbase, int32_t* recv_topk_idx,
                                                              float* recv_topk_weights, int32_t* row_of_token,
                                                              int32_t* recv_src_idx, ScanArgs sa,
                                                              const int32_t* chunk_tok, int32_t* num_rows) {
  __shared__ int32_t wtot[kRouteWaves];
  __shared__ int32_t s_base[kFused ? kMaxLocalExperts : 1], s_tot[kFused ? kMaxLocalExperts : 1];
  __shared__ int32_t s_off[kFused ? kMaxLocalExperts + 1 : 1];
  __shared__ int32_t s_tokbase;
  if constexpr (kFused) {
    fused_scan(sa, src.L, s_base, s_tot, s_off, nullptr);  // sa carries no tile table here
    // rows before this chunk (and, for workgroup 0, all rows) from the per-chunk row counts
    if (threadIdx.x < kWave) {
      int32_t before = 0, all = 0;
      for (int32_t cc = threadIdx.x; cc < sa.nchunks; cc += kWave) {
        const int32_t v = chunk_tok[cc];
        before += cc < (int32_t)blockIdx.x ? v : 0;
        all += v;
      }
      for (int d = kWave / 2; d >= 1; d >>= 1) {
        before += __shfl_xor(before, d, kWave);
        all += __shfl_xor(all, d, kWave);
      }
      if (threadIdx.x == 0) {
        s_tokbase = before;
        if (blockIdx.x == 0 && num_rows) *num_rows = all;
      }
    }
    __syncthreads();
  }
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int32_t t = blockIdx.x * kChunkTokens + threadIdx.x;
  int err = 0, has = 0;
  if (t < N)
    for (int k = 0; k < K; ++k) has |= src.local((int64_t)t * K + k, &err) >= 0;
  const uint64_t hb = __ballot(has);
  if (lane == 0) wtot[w] = (int32_t)__popcll(hb);
  __syncthreads();
  int32_t row = t;
  if (flat) {
    int32_t before = kFused ? s_tokbase : chunk_tokbase[blockIdx.x];
    for (int v = 0; v < w; ++v) before += wtot[v];
    row = before + (int32_t)__popcll(hb & lanes_below(lane));
  }
  if (t < N) row_of_token[t] = has ? row : -1;
  if (has) {
    if (flat) recv_src_idx[row] = t;
    for (int k = 0; k < K; ++k) {
      const int64_t q = (int64_t)t * K + k;
      recv_topk_idx[(int64_t)row * K + k] = src.local(q, &err);
      recv_topk_weights[(int64_t)row * K + k] = topk_weights[q];
    }
  } else if (!flat && t < nrows) {
    for (int k = 0; k < K; ++k) {
      recv_topk_idx[(int64_t)t * K + k] = -1;
      recv_topk_weights[(int64_t)t * K + k] = 0.0f;
    }
  }
}

__global__ void k_tile_table(int32_t L, const int32_t* counts, int64_t clamp, int32_t bm, int2* tiles,
                             int32_t* num_tiles, int32_t* zero, int32_t nzero) {
  __shared__ int32_t base[kMaxLocalExperts + 1];
  for (int32_t i = threadIdx.x; i < nzero; i += blockDim.x) zero[i] = 0;
  if (threadIdx.x == 0) {
    int32_t s = 0;
    for (int el = 0; el < L; ++el) {
      base[el] = s;
      const int64_t c = min((int64_t)counts[el], clamp);
      s += (int32_t)((c + bm - 1) / bm);
    }
    base[L] = s;
    *num_tiles = s;
  }
  __syncthreads();
  for (int el = 0; el < L; ++el) {
    const int32_t nt = base[el + 1] - base[el];
    for (int j = threadIdx.x; j < nt; j += blockDim.x) tiles[base[el] + j] = make_int2(el, j * bm);
  }
}

bool fused_scan_fits(const RouteBufs& rb, int32_t L) {
  return rb.nchunks > 0 && (int64_t)rb.nchunks * L <= kFusedScanMax;
}

int bits_for(int32_t L) {
  int b = 0;
  while ((1 << b) < L) ++b;
  return b;
}

}  // namespace

hipError_t launch_route_expert_major(const Geom& g, const int64_t* topk_ids, RouteBufs rb, int32_t* recv_count,
                                     int32_t* expert_offsets, int32_t* slot_of, int32_t* src_info,
                                     int32_t* layout_range, int32_t* status, hipStream_t stream,
                                     const TileArgs& ta, bool* built) {
  GlobalIds src{topk_ids, (int64_t)g.rank * g.L, g.L, g.E, g.active, g.T, g.K};
  const int nbits = bits_for(g.L);
  if (rb.nchunks > 0) {
    hipLaunchKernelGGL(k_route_count<GlobalIds>, dim3(rb.nchunks), dim3(kRouteThreads), 0, stream, src, g.N,
                       (const int32_t*)nullptr, g.K, g.L, nbits, rb.chunk_hist, (int32_t*)nullptr, rb.chunk_err);
  }
  ScanArgs sa{rb.chunk_hist, rb.chunk_err, rb.nchunks, g.cap, recv_count, expert_offsets, status, 1};
  EmSink sink{slot_of, src_info, g.cap, g.K};
  if (built) *built = false;
  if (fused_scan_fits(rb, g.L)) {
    sa.tiles = ta;
    if (built) *built = ta.tiles != nullptr;
    hipLaunchKernelGGL((k_route_assign<GlobalIds, EmSink, true>), dim3(rb.nchunks), dim3(kRouteThreads), 0, stream,
                       src, sink, g.N, (const int32_t*)nullptr, g.K, g.L, nbits, rb.chunk_base, sa);
  } else {
    hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(1024), 0, stream, rb.chunk_hist, (const int32_t*)nullptr,
                       rb.chunk_err, rb.nchunks, g.L, g.cap, rb.chunk_base, recv_count, expert_offsets,
                       (int32_t*)nullptr, (int32_t*)nullptr, status, 1);
    if (rb.nchunks > 0)
      hipLaunchKernelGGL((k_route_assign<GlobalIds, EmSink, false>), dim3(rb.nchunks), dim3(kRouteThreads), 0,
                         stream, src, sink, g.N, (const int32_t*)nullptr, g.K, g.L, nbits, rb.chunk_base, sa);
  }
  // the layout ranges are computed by the EXPERT_MAJOR permute (layout_ranges), which does not run
  // without tokens
  if (g.N == 0) {
    const int64_t n = (int64_t)g.L * g.W;
    hipLaunchKernelGGL(k_layout_range, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, recv_count, src_info,
                       g.L, g.W, g.T, g.cap, layout_range);
  }
  return hipGetLastError();
}

hipError_t launch_route_rows(const Geom& g, const int64_t* topk_ids, const float* topk_weights, RouteBufs rb,
                             int32_t* recv_count, int32_t* expert_offsets, int32_t* recv_topk_idx,
                             float* recv_topk_weights, int32_t* row_of_token, int32_t* recv_src_idx,
                             int32_t* num_recv, int32_t* status, hipStream_t stream) {
  GlobalIds src{topk_ids, (int64_t)g.rank * g.L, g.L, g.E, g.active, g.T, g.K};
  const int nbits = bits_for(g.L);
  const int flat = g.layout == 2;
  // chunks cover the receive rows: RM W*T rows (tokens >= N have no picks), FLAT N tokens
  if (rb.nchunks > 0) {
    hipLaunchKernelGGL(k_route_count<GlobalIds>, dim3(rb.nchunks), dim3(kRouteThreads), 0, stream, src, g.N,
                       (const int32_t*)nullptr, g.K, g.L, nbits, rb.chunk_hist, rb.chunk_tok, rb.chunk_err);
  }
  const int32_t nrows = flat ? g.N : g.rows;
  const int32_t nblk = (nrows + kChunkTokens - 1) / kChunkTokens;
  const ScanArgs sa{rb.chunk_hist, rb.chunk_err, rb.nchunks, 0, recv_count, expert_offsets, status, 1};
  int32_t* const nrecv = flat ? num_recv : (int32_t*)nullptr;
  // the fused rows kernel takes its chunk totals from the count pass, whose chunks are its blocks
  if (fused_scan_fits(rb, g.L) && nblk == rb.nchunks) {
    hipLaunchKernelGGL(k_route_rows<true>, dim3(nblk), dim3(kRouteThreads), 0, stream, src, topk_weights, nrows, g.N,
                       g.K, flat, rb.chunk_tokbase, recv_topk_idx, recv_topk_weights, row_of_token, recv_src_idx, sa,
                       (const int32_t*)rb.chunk_tok, nrecv);
  } else {
    hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(1024), 0, stream, rb.chunk_hist, rb.chunk_tok, rb.chunk_err,
                       rb.nchunks, g.L, (int64_t)0, rb.chunk_base, recv_count, expert_offsets, rb.chunk_tokbase,
                       nrecv, status, 1);
    if (nblk > 0)
      hipLaunchKernelGGL(k_route_rows<false>, dim3(nblk), dim3(kRouteThreads), 0, stream, src, topk_weights, nrows,
                         g.N, g.K, flat, rb.chunk_tokbase, recv_topk_idx, recv_topk_weights, row_of_token,
                         recv_src_idx, sa, (const int32_t*)nullptr, (int32_t*)nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_bridge(const Geom& g, const int32_t* recv_topk_idx, const float* recv_topk_weights,
                         const int32_t* num_rows_dev, RouteBufs rb, int32_t* pick_count, int32_t* pick_offsets,
                         int32_t* perm, int32_t* pick_slot, int32_t* topk_gid, float* topk_wmask, int32_t* status,
                         hipStream_t stream, const TileArgs& ta, bool* built, const BridgeCombine& bc) {
  LocalIds src{recv_topk_idx, g.L};
  const int nbits = bits_for(g.L);
  const int32_t nrows = g.rows;
  if (rb.nchunks > 0) {
    hipLaunchKernelGGL(k_route_count<LocalIds>, dim3(rb.nchunks), dim3(kRouteThreads), 0, stream, src, nrows,
                       num_rows_dev, g.K, g.L, nbits, rb.chunk_hist, (int32_t*)nullptr, rb.chunk_err);
  }
  ScanArgs sa{rb.chunk_hist, rb.chunk_err, rb.nchunks, 0, pick_count, pick_offsets, status, 0};
  BridgeSink sink{pick_offsets, recv_topk_weights, perm, pick_slot, topk_gid, topk_wmask, g.rank * g.L, bc, g.K};
  if (built) *built = false;
  if (fused_scan_fits(rb, g.L)) {
    sa.tiles = ta;
    if (built) *built = ta.tiles != nullptr;
    hipLaunchKernelGGL((k_route_assign<LocalIds, BridgeSink, true>), dim3(rb.nchunks), dim3(kRouteThreads), 0,
                       stream, src, sink, nrows, num_rows_dev, g.K, g.L, nbits, rb.chunk_base, sa);
  } else {
    hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(1024), 0, stream, rb.chunk_hist, (const int32_t*)nullptr,
                       rb.chunk_err, rb.nchunks, g.L, (int64_t)0, rb.chunk_base, pick_count, pick_offsets,
                       (int32_t*)nullptr, (int32_t*)nullptr, status, 0);
    if (rb.nchunks > 0)
      hipLaunchKernelGGL((k_route_assign<LocalIds, BridgeSink, false>), dim3(rb.nchunks), dim3(kRouteThreads), 0,
                         stream, src, sink, nrows, num_rows_dev, g.K, g.L, nbits, rb.chunk_base, sa);
  }
  return hipGetLastError();
}

hipError_t launch_tile_table(int32_t L, const int32_t* counts, int64_t count_clamp, int32_t bm, int2* tiles,
                             int32_t* num_tiles, hipStream_t stream, int32_t* zero, int32_t nzero) {
  hipLaunchKernelGGL(k_tile_table, dim3(1), dim3(256), 0, stream, L, counts, count_clamp, bm, tiles, num_tiles, zero,
                     nzero);
  return hipGetLastError();
}

int32_t max_tiles(int64_t max_rows, int32_t L, int32_t bm) { return (int32_t)((max_rows + bm - 1) / bm + L); }

}  // namespace moe
