// Shared device helpers and the launch interface between the C ABI (api.hip)
// and the kernel files.  gfx950 only: wave64, bf16 MFMA, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// Routing works on chunks of kChunkTokens consecutive source tokens (or
// received rows), one workgroup of kRouteThreads per chunk.
constexpr int kChunkTokens = 256;
constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kMaxLocalExperts = 1024;
constexpr int kMaxTopK = 64;

// Device status bits (folded into moe_ep_status_t by the host).
constexpr int kStatusBadExpertId = 1;
constexpr int kStatusCapacity = 2;

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (lo in the low half), round to nearest even, one v_cvt_pk_bf16_f32; a NaN
// stays a NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.0f) & 0xFFFFu; }

// SiLU(g) * u = g / (1 + e^-g) * u on the hardware exp2 and reciprocal (each about 1 ulp).
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g)) * u;
}

// Unpack 8 bf16 held in a uint4 into fp32.
__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xFFFF0000u);
  f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xFFFF0000u);
  f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xFFFF0000u);
  f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xFFFF0000u);
}

__device__ __forceinline__ uint4 pack8(const float* f) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

// Geometry shared by all kernels of one call (plain values, passed by value).
struct Geom {
  int32_t E, L, rank, T, N, H, I, K, layout, W;
  int64_t cap;      // EM slots per local expert = W*T
  int32_t rows;     // receive rows: RM W*T, FLAT N (upper bound), EM unused
  // Source-rank health mask (device int32 [W], nullptr = all active): token t of source rank
  // t / T is skipped when its entry is 0 (Mooncake PG/EP guide, "Buffer.dispatch" and
  // "Buffer.combine", active_ranks).
  const int32_t* active;
};

// EXPERT_MAJOR layout ranges: (first slot, count) of each (local expert, source rank), by binary search
// over the expert's ascending src_info.  The EXPERT_MAJOR permute kernels compute them as a side task
// (grid-stride over the L x W entries) once routing is complete; out == nullptr: none.
struct LayoutRangeArgs {
  const int32_t* counts = nullptr;
  const int32_t* src_info = nullptr;
  int32_t L = 0, W = 0, T = 0;
  int64_t cap = 0;
  int32_t* out = nullptr;
};
__device__ __forceinline__ void layout_ranges(const LayoutRangeArgs& a) {
  if (!a.out) return;
  const int64_t n = (int64_t)a.L * a.W;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int32_t el = (int32_t)(i / a.W), r = (int32_t)(i % a.W);
    const int32_t cnt = (int32_t)min((int64_t)a.counts[el], a.cap);
    const int32_t* s = a.src_info + el * a.cap;
    auto lower_bound = [&](int32_t key) {
      int32_t lo = 0, hi = cnt;
      while (lo < hi) {
        const int32_t mid = (lo + hi) >> 1;
        if (s[mid] < key) lo = mid + 1;
        else hi = mid;
      }
      return lo;
    };
    const int32_t b = lower_bound(r * a.T), e = lower_bound((r + 1) * a.T);
    a.out[i * 2 + 0] = b;
    a.out[i * 2 + 1] = e - b;
  }
}


// Routing scratch + outputs (device pointers into the workspace).
struct RouteBufs {
  int32_t* chunk_hist;     // [nchunks * L]
  int32_t* chunk_base;     // [nchunks * L]
  int32_t* chunk_tok;      // [nchunks]
  int32_t* chunk_tokbase;  // [nchunks]
  int32_t* chunk_err;      // [nchunks]
  int32_t nchunks;
};

// ---- launchers (each enqueues on `stream`, returns the hipError_t of the launch)

// Dispatch routing, EXPERT_MAJOR: slots in (source rank, token, k) order.
// Optional extra output of the routing that ends in per-expert counts: the grouped GEMMs' tile
// table (entries (expert, first row) of bm rows each over min(count, clamp) rows, and their number),
// written by the fused routing kernel once the counts are known instead of by a kernel of its own.
// tiles == nullptr: none.  The launchers set *built when they wrote it.
struct TileArgs {
  int2* tiles = nullptr;
  int32_t* num_tiles = nullptr;
  int32_t bm = 0;
  int64_t clamp = 0;
  // counters the GEMMs need at zero (split-K arrival counts), cleared along with the table
  int32_t* zero = nullptr;
  int32_t nzero = 0;
};

hipError_t launch_route_expert_major(const Geom& g, const int64_t* topk_ids, RouteBufs rb, int32_t* recv_count,
                                     int32_t* expert_offsets, int32_t* slot_of, int32_t* src_info,
                                     int32_t* layout_range, int32_t* status, hipStream_t stream,
                                     const TileArgs& ta = TileArgs{}, bool* built = nullptr);

// Dispatch routing, RANK_MAJOR / FLAT: received routing rows.
hipError_t launch_route_rows(const Geom& g, const int64_t* topk_ids, const float* topk_weights, RouteBufs rb,
                             int32_t* recv_count, int32_t* expert_offsets, int32_t* recv_topk_idx,
                             float* recv_topk_weights, int32_t* row_of_token, int32_t* recv_src_idx,
                             int32_t* num_recv, int32_t* status, hipStream_t stream);

// Extra bridge outputs for the combine fused into the down GEMM: per pick in expert-sorted order, its
// weight and its source token (RANK_MAJOR: the receive row; FLAT: src_idx[row]).  pick_w == nullptr:
// not written.
struct BridgeCombine {
  float* pick_w = nullptr;
  int32_t* pick_tok = nullptr;
  const int32_t* src_idx = nullptr;  // FLAT recv_src_idx; nullptr for RANK_MAJOR
};

// Compute-side bridge over received routing: local -> global ids, masked weights, expert-sorted picks.
hipError_t launch_bridge(const Geom& g, const int32_t* recv_topk_idx, const float* recv_topk_weights,
                         const int32_t* num_rows_dev, RouteBufs rb, int32_t* pick_count, int32_t* pick_offsets,
                         int32_t* perm, int32_t* pick_slot, int32_t* topk_gid, float* topk_wmask,
                         int32_t* status, hipStream_t stream, const TileArgs& ta = TileArgs{},
                         bool* built = nullptr, const BridgeCombine& bc = BridgeCombine{});

// One-launch dispatch for small layers (dispatch_ll.hip): routing, received routing / slot maps,
// optionally the RANK_MAJOR / FLAT bridge (perm != nullptr) and the GEMM tile table (ta.tiles !=
// nullptr), and the row copies; the same results as the multi-launch path.  Arrays of other layouts
// stay nullptr.
struct LLDispatchOut {
  int32_t* slot_of = nullptr;
  int32_t* src_info = nullptr;
  int32_t* layout_range = nullptr;
  int32_t* recv_topk_idx = nullptr;
  float* recv_topk_weights = nullptr;
  int32_t* row_of_token = nullptr;
  int32_t* recv_src_idx = nullptr;
  int32_t* num_recv = nullptr;
  int32_t* pick_count = nullptr;
  int32_t* pick_offsets = nullptr;
  int32_t* perm = nullptr;
  int32_t* pick_slot = nullptr;
  int32_t* gid = nullptr;
  float* wmask = nullptr;
  float* pick_w = nullptr;      // with the bridge: the fused combine's per-pick weight and token
  int32_t* pick_tok = nullptr;
};
bool dispatch_ll_fits(const Geom& g);
hipError_t launch_dispatch_ll(const Geom& g, const int64_t* topk_ids, const float* topk_weights, const void* x,
                              void* recv_x, int32_t* recv_count, int32_t* expert_offsets, int32_t* status,
                              const TileArgs& ta, const LLDispatchOut& d, hipStream_t stream);

// Permute source rows into the receive buffer.
// FP8 rows (E4M3 codes, one power-of-two scale byte per 128 values, scale rows padded to 4 bytes).
int32_t fp8_scale_stride(int32_t cols);
hipError_t launch_quantize_rows_fp8(const void* x, int64_t rows, int32_t cols, void* codes, void* scales,
                                    hipStream_t stream);
// FP8 dispatch: the permute with each source row quantised once on the way (codes [rows, H] and
// scales [rows, fp8_scale_stride(H)] in the receive layout's rows).
hipError_t launch_permute_fp8(const Geom& g, const void* x, const int32_t* slot_of, const int32_t* row_of_token,
                              void* codes, void* scales, hipStream_t stream,
                              const LayoutRangeArgs& lr = LayoutRangeArgs{});

// Router: per token the top K of scores [N, E] (ties to the lower id) and softmax weights over them.
hipError_t launch_router_topk(const float* scores, int32_t N, int32_t E, int32_t K, int64_t* ids, float* weights,
                              hipStream_t stream);

hipError_t launch_permute(const Geom& g, const void* x, const int32_t* slot_of, const int32_t* row_of_token,
                          void* recv_x, hipStream_t stream, const LayoutRangeArgs& lr = LayoutRangeArgs{});

// Grouped GEMM tile table: for each expert, ceil(count/bm) tiles of (expert, first row); also zeroes
// zero[0 .. nzero).
hipError_t launch_tile_table(int32_t L, const int32_t* counts, int64_t count_clamp, int32_t bm, int2* tiles,
                             int32_t* num_tiles, hipStream_t stream, int32_t* zero = nullptr, int32_t nzero = 0);
int32_t max_tiles(int64_t max_rows, int32_t L, int32_t bm);

// A-row source of the grouped GEMM for one call.
struct GemmRows {
  const bf16_t* a;          // EM: recv_x; RM/FLAT: recv_x (gathered via perm)
  const int32_t* perm;      // NULL for EM
  int32_t K;                // top_k (perm / K = receive row)
  int64_t slab;             // EM: rows per expert slab (cap); 0 for gathered
};

// Row-tile height of the grouped GEMMs for this geometry (64 or 256); the tile table is built
// with it.  kGemmMinBM sizes the tile table buffer.
int32_t gemm_row_tile(const Geom& g);
// Split-K of the 256-row GEMMs (when too few items would fill the grid) and the split tail of the
// narrow 64-row gate_up GEMM: whether this geometry may use either, and the workspace it then needs
// (fp32 partials, and arrival and ticket counters that are zero before the GEMMs).
struct SplitBufs {
  float* partial = nullptr;
  int32_t* cnt = nullptr;
  int32_t* tickets = nullptr;  // kGemmTickets counters of the 256-row kernels' dynamic rounds
};
bool gemm_split_possible(const Geom& g);
size_t gemm_split_partial_bytes(const Geom& g);
int32_t gemm_split_counters(const Geom& g);
// The GEMMs' counters that must be zero before they run: kGemmTickets ticket counters, then (when the
// geometry may split) the split counters; the tile-table writers clear them.
constexpr int32_t kGemmTickets = 16;
int32_t gemm_zero_words(const Geom& g);
// Whether the gate_up GEMM runs the narrow 64 x 128 tiles for this geometry.
bool gemm_narrow(const Geom& g);
// Whether every operand byte offset of both grouped GEMMs fits 32 bits (the 256-row kernel
// addresses its operands with 32-bit offsets from the operand base).
bool gemm_offsets_fit_32(const Geom& g);
constexpr int kGemmMinBM = 64;

// gate_up GEMM + SwiGLU: h[off[e] + m, :] = SiLU(A W1g^T) * (A W1u^T), bf16.  Expert e has
// min(counts[e], count_clamp) rows; tiles/num_tiles is the device tile table built with row tile bm.
hipError_t launch_gemm_gate_up(const Geom& g, GemmRows rows, const int32_t* counts, const int32_t* offsets,
                               int64_t count_clamp, const bf16_t* w_gate_up, bf16_t* h, const int2* tiles,
                               const int32_t* num_tiles, int32_t bm, hipStream_t stream,
                               const SplitBufs& split = SplitBufs{});

// The combine fused into the down GEMM (RANK_MAJOR / FLAT): out[pick_tok[p]] += pick_w[p] * y(p) for every
// pick p in packed order, bf16 atomics into a zeroed token-major output; out == nullptr: not fused.
struct DownCombine {
  bf16_t* out = nullptr;
  const float* pick_w = nullptr;
  const int32_t* pick_tok = nullptr;
};

// down GEMM: y rows = h rows W2^T; output row = out_slab ? e*out_slab + m : off[e] + m (or, with comb.out,
// the fused combine instead of y).
hipError_t launch_gemm_down(const Geom& g, const int32_t* counts, const int32_t* offsets, int64_t count_clamp,
                            const bf16_t* h, const bf16_t* w_down, bf16_t* y, int64_t out_slab, const int2* tiles,
                            const int32_t* num_tiles, int32_t bm, hipStream_t stream,
                            const DownCombine& comb = DownCombine{}, const SplitBufs& split = SplitBufs{});

// Zero n bytes (a multiple of 16, 16-byte aligned) with a fill kernel (graph-capturable, unlike a memset node).
hipError_t launch_zero(void* p, int64_t n, hipStream_t stream);

// EM identity expert: expert_out[slot] = recv_x[slot] for every used slot.
hipError_t launch_copy_slots(const Geom& g, const int32_t* slot_of, const void* recv_x, void* expert_out,
                             hipStream_t stream);

// Combine, EXPERT_MAJOR: out[t] = sum_k w[t,k] * Y[row(slot_of[t,k])].
// Y row of slot s = el*cap + j is: packed ? offsets[el] + j : s.
hipError_t launch_combine_em(const Geom& g, const int32_t* slot_of, const float* topk_weights,
                             const int32_t* offsets_packed, const void* Y, void* out, hipStream_t stream);

// RM / FLAT finalize: z[row] = sum_k wmask[row,k] * Y(pick); Y(pick) = y[pick_slot] or (identity) recv_x[row].
// If out_token_major, writes out[t] for every token t (0 when row_of_token[t] < 0) instead of z rows.
hipError_t launch_finalize_rows(const Geom& g, const int32_t* row_of_token, const int32_t* pick_slot,
                                const float* topk_wmask, const void* y_packed, const void* recv_x, void* dst,
                                bool out_token_major, hipStream_t stream);

// RM / FLAT combine: out[t] = z[row_of_token[t]] or 0.
hipError_t launch_combine_rows(const Geom& g, const int32_t* row_of_token, const void* z, void* out,
                               hipStream_t stream);

// FP8 gate_up GEMM (256x256 tiles; the tile table must be built with bm = 256): A = received FP8
// rows (codes + scales, gathered like the bf16 rows), W1 FP8 [L, 2I, H] + scales [L * 2I, stride].
hipError_t launch_gemm_gate_up_fp8(const Geom& g, GemmRows rows, const uint8_t* a_codes, const uint8_t* a_scales,
                                   const int32_t* counts, const int32_t* offsets, int64_t count_clamp,
                                   const uint8_t* w_codes, const uint8_t* w_scales, bf16_t* h, const int2* tiles,
                                   const int32_t* num_tiles, hipStream_t stream, int32_t* tickets = nullptr);

}  // namespace moe
