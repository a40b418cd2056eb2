// Low-latency dispatch in one launch, for layers of up to kLLMaxPicks picks.
//
// What is computed: the same outputs as the multi-launch dispatch (routing.hip + movement.hip),
// bit for bit (FlashInfer "MoE-EP implementation & usage", section 3 "Algorithm / layout
// contracts"; Mooncake PG/EP guide, "Buffer.dispatch"): per local expert the received picks and
// their exclusive offsets; per pick its slot in (source rank, token, k) order, i.e. ascending flat
// pick index q = t*K + k within each expert; the EXPERT_MAJOR slot map, source info and
// per-(expert, source rank) layout ranges, or the RANK_MAJOR / FLAT received routing rows; and the
// received rows themselves.  In the fused layer forward it also writes the RANK_MAJOR / FLAT
// compute-side bridge (same page, section 2 "_inner_compute" and section 3: local -> global ids,
// picks masked to weight 0, expert-sorted pick order).  That order is this same counting sort:
// received rows keep the token order, so (expert, row, k) order is (expert, token, k) order.
//
// How.  One launch of 1024-thread workgroups.  Every workgroup loads all topk_ids at once (thread
// i holds picks i, i + 1024, ...) and computes the whole stable counting sort in LDS.  Picks fall
// into segments of 64 (one wave's share of a round); in each segment, ballots over the expert-id
// bits give every pick its rank among the equal experts of the segment and the segment's count per
// expert; a scan per expert over the segments gives each segment's base, so a pick's slot is its
// segment's base plus its rank.  Every workgroup does the same integer arithmetic and gets the same
// result, so none waits for another, and no atomic decides any order.  The sort takes four block
// barriers; after the last, each workgroup writes its share of the metadata (the segments dealt to
// it, tokens of a grid stride, and per-expert arrays, tile table and layout ranges on the first
// workgroups, each by one wave or thread-per-expert without further barriers) and copies its share
// of the rows: the received rows cut into 16-byte pieces, consecutive threads on consecutive pieces,
// four pieces per thread in flight.  Latency, not bytes, bounds a layer this small: the multi-launch
// path waits on a global load per loop iteration in three kernels.

#include <algorithm>

#include "common.h"
#include "routing_util.h"

namespace moe {
namespace {

constexpr int kLLThreads = 1024;
constexpr int kLLWaves = kLLThreads / kWave;
constexpr int kLLMaxPicks = 16384;                       // N * K
constexpr int kLLMaxRounds = kLLMaxPicks / kLLThreads;   // picks per thread
constexpr int kLLMaxTokens = 16384;                      // N (row and token numbers fit 16 bits)
constexpr int kLLMaxCnt = 4096;                          // segments (N*K / 64) * L counters
constexpr int kLLMaxRanges = 2048;                       // EXPERT_MAJOR L * W layout ranges
constexpr int kLLMaxExperts = 256;
constexpr uint16_t kNoRow = 0xFFFF;
constexpr int kUnits = 4;                                // row pieces in flight per thread

typedef unsigned int u4v_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  const u4v_t v = __builtin_nontemporal_load((const u4v_t*)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

struct LLOut {
  int32_t* counts;
  int32_t* offsets;
  int32_t* status;
  TileArgs tiles;            // tiles == nullptr: no tile table
  // EXPERT_MAJOR
  int32_t* slot_of;
  int32_t* src_info;
  int32_t* layout_range;
  // RANK_MAJOR / FLAT
  const float* w;
  int32_t* recv_topk_idx;
  float* recv_topk_weights;
  int32_t* row_of_token;
  int32_t* recv_src_idx;     // FLAT
  int32_t* num_recv;         // FLAT
  int32_t nrows;             // RANK_MAJOR: W*T receive rows
  // bridge (perm == nullptr: not written)
  int32_t* pick_count;
  int32_t* pick_offsets;
  int32_t* perm;
  int32_t* pick_slot;
  int32_t* gid;
  float* wmask;
  float* pick_w;             // fused combine (nullptr: not written)
  int32_t* pick_tok;
};

template <int kLayout>
__global__ __launch_bounds__(kLLThreads) void k_dispatch_ll(GlobalIds src, int32_t N, int32_t K, int32_t L,
                                                            uint32_t mK, uint32_t mT, int32_t W, int32_t T, int64_t cap,
                                                            const uint4* __restrict__ x, int32_t cpr,
                                                            uint4* __restrict__ recv, LLOut o) {
  __shared__ int32_t s_cnt[kLLMaxCnt];          // per (expert, 64-pick segment): count, then base
  __shared__ int16_t s_el[kLLMaxPicks];         // local expert of pick q, -1 if not local
  __shared__ uint8_t s_rank[kLLMaxPicks];       // rank of pick q among its segment's picks of its expert
  __shared__ uint16_t s_row[kLLMaxTokens];      // token t: 1 if it has a local pick; then its compacted row
  // compacted row -> token; before the rows are compacted, the per-(wave, expert) lane masks of the
  // ranking (kLLWaves * kLLMaxExperts 64-bit words: the same 32 KB)
  __shared__ union {
    uint16_t list[kLLMaxTokens];
    uint64_t masks[kLLWaves * kLLMaxExperts];
  } s_u;
  uint16_t* const s_list = s_u.list;
  uint64_t* const s_mask = s_u.masks + (threadIdx.x / kWave) * kLLMaxExperts;
  __shared__ int32_t s_rcnt[kLLMaxRanges];      // EXPERT_MAJOR: picks per (expert, source rank)
  __shared__ int32_t s_tot[kLLMaxExperts], s_off[kLLMaxExperts + 1];
  __shared__ int32_t s_wtot[kLLWaves];
  __shared__ int32_t s_err;

  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  const int32_t NK = N * K;
  const int32_t J = (NK + kLLThreads - 1) / kLLThreads;  // rounds of 1024 picks
  const int32_t S = J * kLLWaves;                         // segments of 64 picks: segment of q = q / 64
  for (int32_t i = tid; i < S * L; i += kLLThreads) s_cnt[i] = 0;
  for (int32_t i = tid; i < N; i += kLLThreads) s_row[i] = 0;
  if constexpr (kLayout == 0)
    for (int32_t i = tid; i < L * W; i += kLLThreads) s_rcnt[i] = 0;
  if (tid == 0) s_err = 0;
  // All picks loaded into LDS, every load issued before any is used.  Every workgroup reads the same
  // ids at the same time, so each starts at a different round and 64-pick offset: in lockstep they
  // would all queue on the same L2 channel.
  const int32_t b = blockIdx.x;
  {
    const int32_t jr = J > 0 ? b % J : 0, sr = ((b / max(J, 1)) % kLLWaves) * kWave;
    int el[kLLMaxRounds];
    int32_t qs[kLLMaxRounds];
    int err = 0;
#pragma unroll
    for (int jj = 0; jj < kLLMaxRounds; ++jj) {
      int32_t j = jj + jr;
      j = j >= J ? j - J : j;
      const int32_t q = j * kLLThreads + ((tid + sr) & (kLLThreads - 1));
      qs[jj] = q;
      el[jj] = (jj < J && q < NK) ? src.local(q, &err) : -1;
    }
#pragma unroll
    for (int jj = 0; jj < kLLMaxRounds; ++jj)
      if (jj < J && qs[jj] < NK) s_el[qs[jj]] = (int16_t)el[jj];
    if (err) atomicOr(&s_err, kStatusBadExpertId);
  }
  __syncthreads();
  // Each segment's per-expert counts, and each pick's rank among the equal experts of its segment
  // (pick q = j * 1024 + tid: segment q / 64 is round j's share of wave w).  The lanes of a wave
  // holding expert e find each other through a 64-bit word per (wave, expert) into which each ORs its
  // lane bit (an OR is order-free); the wave's LDS operations complete in program order, so the
  // word is whole when read back.
#pragma unroll
  for (int j = 0; j < kLLMaxRounds; ++j) {
    if (j < J) {
      const int32_t q = j * kLLThreads + tid;
      const int e = q < NK ? s_el[q] : -1;
      for (int32_t i = lane; i < L; i += kWave) s_mask[i] = 0;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (e >= 0) atomicOr((unsigned long long*)&s_mask[e], 1ull << lane);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const uint64_t m = e >= 0 ? s_mask[e] : 0ull;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const uint64_t below = m & lanes_below(lane);
      if (e >= 0) {
        const uint32_t t = mK ? __umulhi((uint32_t)q, mK) : (uint32_t)q;  // q / K
        if (below == 0) s_cnt[e * S + q / kWave] = __popcll(m);
        s_row[t] = 1;
        if constexpr (kLayout == 0) atomicAdd(&s_rcnt[e * W + (mT ? __umulhi(t, mT) : t)], 1);  // t / T; order-free
      }
      if (q < NK) s_rank[q] = (uint8_t)__popcll(below);
    }
  }
  __syncthreads();
  // Per expert, the exclusive scan of its counts over the segments: P threads per expert (P a power
  // of two, P * L <= 1024), each summing a run of consecutive segments, meet in a shuffle scan.
  // Counters are expert-major (s_cnt[e * S + segment]), so a wave's reads are nearly consecutive.
  int P = kWave;
  while (P * L > kLLThreads) P >>= 1;
  {
    const int32_t e = tid / P, part = tid % P;
    const int32_t c = (S + P - 1) / P;
    const int32_t s0 = min(part * c, S), s1 = min(s0 + c, S);
    int32_t sum = 0;
    if (e < L)
      for (int32_t sg = s0; sg < s1; ++sg) sum += s_cnt[e * S + sg];
    int32_t inc = sum;
    for (int d = 1; d < P; d <<= 1) {
      const int32_t y = __shfl_up(inc, d, P);
      if (part >= d) inc += y;
    }
    if (e < L) {
      int32_t run = inc - sum;
      for (int32_t sg = s0; sg < s1; ++sg) {
        const int32_t cv = s_cnt[e * S + sg];
        s_cnt[e * S + sg] = run;
        run += cv;
      }
      if (part == P - 1) s_tot[e] = inc;
    }
  }
  // tokens with a local pick: this thread's TPT consecutive tokens, scanned across the wave
  const int32_t TPT = (N + kLLThreads - 1) / kLLThreads;
  const int32_t t0 = min(tid * TPT, N), t1 = min(t0 + TPT, N);
  int32_t mine = 0;
  for (int32_t t = t0; t < t1; ++t) mine += s_row[t];
  int32_t tinc = mine;
  for (int d = 1; d < kWave; d <<= 1) {
    const int32_t y = __shfl_up(tinc, d, kWave);
    if (lane >= d) tinc += y;
  }
  if (lane == kWave - 1) s_wtot[w] = tinc;
  __syncthreads();
  // expert offsets (wave 0: a shuffle scan of the totals, 64 experts per step; capacity check)
  if (w == 0) {
    int32_t carry = 0;
    bool over = false;
    for (int32_t base = 0; base < L; base += kWave) {
      const int32_t e = base + lane;
      const int32_t v = e < L ? s_tot[e] : 0;
      over |= v > cap;
      int32_t inc = v;
      for (int d = 1; d < kWave; d <<= 1) {
        const int32_t y = __shfl_up(inc, d, kWave);
        if (lane >= d) inc += y;
      }
      if (e < L) s_off[e] = carry + inc - v;
      carry += __shfl(inc, kWave - 1, kWave);
    }
    if (lane == 0) s_off[L] = carry;
    if (kLayout == 0 && __ballot(over) != 0 && lane == 0) atomicOr(&s_err, kStatusCapacity);
  }
  // compacted rows: tokens with a pick in earlier waves, then in earlier lanes
  int32_t R = 0, before = 0;
  for (int v = 0; v < kLLWaves; ++v) {
    const int32_t c = s_wtot[v];
    before += v < w ? c : 0;
    R += c;
  }
  {
    int32_t r = before + tinc - mine;
    for (int32_t t = t0; t < t1; ++t) {
      if (s_row[t]) {
        s_list[r] = (uint16_t)t;
        s_row[t] = (uint16_t)r++;
      } else {
        s_row[t] = kNoRow;
      }
    }
  }
  __syncthreads();

  // ---- from here on every workgroup only reads its LDS: no more barriers
  const int32_t G = gridDim.x;
  auto slot_of_pick = [&](int32_t q, int e) { return s_cnt[e * S + q / kWave] + (int32_t)s_rank[q]; };
  // metadata of the segments dealt to this workgroup
#pragma unroll
  for (int j = 0; j < kLLMaxRounds; ++j) {
    if (j >= J || (j * kLLWaves + w) % G != b) continue;
    const int32_t q = j * kLLThreads + tid;
    if (q >= NK) continue;
    const int e = s_el[q];
    const int32_t t = q / K, k = q % K;
    if constexpr (kLayout == 0) {
      int32_t code = -1;
      if (e >= 0) {
        const int32_t sl = slot_of_pick(q, e);
        if (sl < cap) {  // over capacity: dropped (latched from the counts)
          code = (int32_t)(e * cap + sl);
          o.src_info[code] = t;
        }
      }
      o.slot_of[q] = code;
    } else {
      const int32_t row = s_row[t] == kNoRow ? -1 : (kLayout == 1 ? t : (int32_t)s_row[t]);
      if (row >= 0) {
        const int64_t rq = (int64_t)row * K + k;
        const float wq = o.w[q];
        o.recv_topk_idx[rq] = e;
        o.recv_topk_weights[rq] = wq;
        if (o.perm) {
          if (e >= 0) {
            const int32_t pos = s_off[e] + slot_of_pick(q, e);
            o.perm[pos] = (int32_t)rq;
            o.pick_slot[rq] = pos;
            o.gid[rq] = (int32_t)(e + src.o);
            o.wmask[rq] = wq;
            if (o.pick_w) {
              o.pick_w[pos] = wq;
              o.pick_tok[pos] = t;
            }
          } else {
            o.pick_slot[rq] = -1;
            o.gid[rq] = -1;
            o.wmask[rq] = 0.0f;
          }
        }
      } else if (kLayout == 1) {  // RANK_MAJOR row of a token without a local pick
        o.recv_topk_idx[q] = -1;
        o.recv_topk_weights[q] = 0.0f;
        if (o.perm) {
          o.pick_slot[q] = -1;
          o.gid[q] = -1;
          o.wmask[q] = 0.0f;
        }
      }
    }
  }
  if constexpr (kLayout == 1) {  // RANK_MAJOR rows of absent tokens (N <= q / K < W*T)
    const int64_t nq = (int64_t)o.nrows * K;
    for (int64_t q = NK + (int64_t)b * kLLThreads + tid; q < nq; q += (int64_t)G * kLLThreads) {
      o.recv_topk_idx[q] = -1;
      o.recv_topk_weights[q] = 0.0f;
      if (o.perm) {
        o.pick_slot[q] = -1;
        o.gid[q] = -1;
        o.wmask[q] = 0.0f;
      }
    }
  }
  if constexpr (kLayout != 0) {  // per token
    for (int32_t t = b * kLLThreads + tid; t < N; t += G * kLLThreads) {
      const bool has = s_row[t] != kNoRow;
      o.row_of_token[t] = has ? (kLayout == 1 ? t : (int32_t)s_row[t]) : -1;
      if (kLayout == 2 && has) o.recv_src_idx[s_row[t]] = t;
    }
  }
  // per-expert outputs, spread over the first workgroups
  if (b == 0) {
    for (int32_t e = tid; e < L; e += kLLThreads) {
      o.counts[e] = s_tot[e];
      o.offsets[e] = s_off[e];
      if (o.perm) {
        o.pick_count[e] = s_tot[e];
        o.pick_offsets[e] = s_off[e];
      }
    }
    if (tid == 0) {
      o.offsets[L] = s_off[L];
      if (o.perm) o.pick_offsets[L] = s_off[L];
      if (kLayout == 2) *o.num_recv = R;
      *o.status = s_err;
    }
  }
  if (o.tiles.tiles && b == 1 % G && w == 0) {
    // the GEMM tile table: each expert's ceil(min(count, clamp) / bm) tiles, placed by a shuffle scan
    for (int32_t i = lane; i < o.tiles.nzero; i += kWave) o.tiles.zero[i] = 0;
    int32_t carry = 0;
    for (int32_t base = 0; base < L; base += kWave) {
      const int32_t e = base + lane;
      const int32_t n = e < L ? (int32_t)((min((int64_t)s_tot[e], o.tiles.clamp) + o.tiles.bm - 1) / o.tiles.bm) : 0;
      int32_t inc = n;
      for (int d = 1; d < kWave; d <<= 1) {
        const int32_t y = __shfl_up(inc, d, kWave);
        if (lane >= d) inc += y;
      }
      for (int32_t jt = 0; jt < n; ++jt) o.tiles.tiles[carry + inc - n + jt] = make_int2(e, jt * o.tiles.bm);
      carry += __shfl(inc, kWave - 1, kWave);
    }
    if (lane == 0) *o.tiles.num_tiles = carry;
  }
  if constexpr (kLayout == 0) {
    if (b == 2 % G) {
      // layout ranges: the expert's slots run through the source ranks in order, so each range starts
      // where the ranks before it end; picks over capacity were dropped from the end
      for (int32_t e = tid; e < L; e += kLLThreads) {
        int64_t first = 0;
        for (int32_t rr = 0; rr < W; ++rr) {
          const int64_t end = min(first + s_rcnt[e * W + rr], cap);
          o.layout_range[((int64_t)e * W + rr) * 2 + 0] = (int32_t)min(first, cap);
          o.layout_range[((int64_t)e * W + rr) * 2 + 1] = (int32_t)(end - min(first, cap));
          first += s_rcnt[e * W + rr];
        }
      }
    }
  }

  // ---- the received rows: compacted row i of token t = s_list[i], cut into cpr 16-byte pieces
  const int64_t units = (int64_t)R * cpr;
  const int64_t stride = (int64_t)G * kLLThreads;
  for (int64_t u0 = (int64_t)b * kLLThreads + tid; u0 < units; u0 += stride * kUnits) {
    uint4 v[kUnits];
    int32_t ti[kUnits], ri[kUnits], ci[kUnits];
#pragma unroll
    for (int m = 0; m < kUnits; ++m) {
      const int64_t u = u0 + m * stride;
      ri[m] = -1;
      if (u < units) {
        ri[m] = (int32_t)(u / cpr);
        ci[m] = (int32_t)(u % cpr);
        ti[m] = s_list[ri[m]];
        v[m] = ld_nt(&x[(int64_t)ti[m] * cpr + ci[m]]);
      }
    }
#pragma unroll
    for (int m = 0; m < kUnits; ++m) {
      if (ri[m] < 0) continue;
      if constexpr (kLayout == 0) {
        for (int k = 0; k < K; ++k) {
          const int32_t q = ti[m] * K + k;
          const int e = s_el[q];
          if (e >= 0) {
            const int32_t sl = slot_of_pick(q, e);
            if (sl < cap) recv[((int64_t)e * cap + sl) * cpr + ci[m]] = v[m];
          }
        }
      } else {
        const int64_t row = kLayout == 1 ? ti[m] : ri[m];
        recv[row * cpr + ci[m]] = v[m];
      }
    }
  }
}

int g_ll_cus[64];
int ll_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (g_ll_cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_ll_cus[dev] = n;
  }
  return g_ll_cus[dev];
}

}  // namespace

bool dispatch_ll_fits(const Geom& g) {
  const int64_t nk = (int64_t)g.N * g.K;
  const int64_t rounds = (nk + kLLThreads - 1) / kLLThreads;
  if (g.N < 1 || g.N > kLLMaxTokens || nk > kLLMaxPicks || g.L > kLLMaxExperts || g.T >= (1 << 18)) return false;
  if (rounds * kLLWaves * g.L > kLLMaxCnt) return false;
  if (g.layout == 0 && (int64_t)g.L * g.W > kLLMaxRanges) return false;
  return true;
}

hipError_t launch_dispatch_ll(const Geom& g, const int64_t* topk_ids, const float* topk_weights, const void* x,
                              void* recv_x, int32_t* recv_count, int32_t* expert_offsets, int32_t* status,
                              const TileArgs& ta, const LLDispatchOut& d, hipStream_t stream) {
  GlobalIds src{topk_ids, (int64_t)g.rank * g.L, g.L, g.E, g.active, g.T, g.K};
  LLOut o{};
  o.counts = recv_count;
  o.offsets = expert_offsets;
  o.status = status;
  o.tiles = ta;
  o.slot_of = d.slot_of;
  o.src_info = d.src_info;
  o.layout_range = d.layout_range;
  o.w = topk_weights;
  o.recv_topk_idx = d.recv_topk_idx;
  o.recv_topk_weights = d.recv_topk_weights;
  o.row_of_token = d.row_of_token;
  o.recv_src_idx = d.recv_src_idx;
  o.num_recv = d.num_recv;
  o.nrows = g.rows;
  o.pick_count = d.pick_count;
  o.pick_offsets = d.pick_offsets;
  o.perm = d.perm;
  o.pick_slot = d.pick_slot;
  o.gid = d.gid;
  o.wmask = d.wmask;
  o.pick_w = d.pick_w;
  o.pick_tok = d.pick_tok;
  const int32_t cpr = g.H / 8;
  // workgroups: about two row pieces per thread over the largest possible receive set, at most one
  // per CU (each holds the whole routing in LDS)
  const int64_t units = (int64_t)g.N * cpr;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(ll_cus(), (units + 2 * kLLThreads - 1) / (2 * kLLThreads)));
  // floor(n / d) = umulhi(n, ceil(2^32 / d)) exactly when n * d < 2^32 (here n < 16384 picks or
  // tokens, d = K <= 64 or T < 2^18); d = 1 (no 32-bit constant) is passed as 0
  const uint32_t mK = g.K == 1 ? 0u : (uint32_t)((((uint64_t)1 << 32) + g.K - 1) / g.K);
  const uint32_t mT = g.T == 1 ? 0u : (uint32_t)((((uint64_t)1 << 32) + g.T - 1) / g.T);
  switch (g.layout) {
    case 0:
      hipLaunchKernelGGL(k_dispatch_ll<0>, dim3(grid), dim3(kLLThreads), 0, stream, src, g.N, g.K, g.L, mK, mT, g.W, g.T,
                         g.cap, (const uint4*)x, cpr, (uint4*)recv_x, o);
      break;
    case 1:
      hipLaunchKernelGGL(k_dispatch_ll<1>, dim3(grid), dim3(kLLThreads), 0, stream, src, g.N, g.K, g.L, mK, mT, g.W, g.T,
                         g.cap, (const uint4*)x, cpr, (uint4*)recv_x, o);
      break;
    default:
      hipLaunchKernelGGL(k_dispatch_ll<2>, dim3(grid), dim3(kLLThreads), 0, stream, src, g.N, g.K, g.L, mK, mT, g.W, g.T,
                         g.cap, (const uint4*)x, cpr, (uint4*)recv_x, o);
      break;
  }
  return hipGetLastError();
}

}  // namespace moe
