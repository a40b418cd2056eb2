// The C ABI of include/moe_ep.h: argument checks, workspace carving, the
// per-workspace dispatch epoch, and the order in which each entry point
// enqueues the kernels on the caller's stream.  No entry point allocates
// device memory or synchronises, except moe_ep_query_status.
//
// Stage order (FlashInfer "MoE-EP implementation & usage", section 2 "Call
// stack"): dispatch = routing + permute; expert compute = (RANK_MAJOR / FLAT:
// the bridge) + gate_up GEMM with SwiGLU + down GEMM (+ RANK_MAJOR / FLAT:
// weighting of the picks per received row); combine.

#include <cstdlib>
#include <cstring>
#include <mutex>
#include <unordered_map>

#include "../../include/moe_ep.h"
#include "common.h"
#include "gemm_stream.h"

namespace moe {
namespace {

constexpr size_t kAlign = 256;

struct Layout {
  size_t status, recv_count, expert_offsets;
  size_t chunk_hist, chunk_base, chunk_tok, chunk_tokbase, chunk_err;
  size_t slot_of, src_info, layout_range;
  size_t recv_topk_idx, recv_topk_weights, row_of_token, recv_src_idx, num_recv;
  size_t pick_count, pick_offsets, perm, pick_slot, topk_gid, topk_wmask, pick_w, pick_tok;
  size_t tiles, num_tiles, recv_x, h, y, split_partial, split_cnt, gemm_zero;
  size_t total;
  int32_t nchunks_dispatch, nchunks_bridge, max_tiles;
  int64_t pmax;
};

constexpr size_t kAbsent = ~(size_t)0;

Geom geom_of(const moe_ep_params_t& p, const int32_t* active_ranks = nullptr) {
  Geom g;
  g.active = active_ranks;
  g.E = p.num_experts;
  g.L = p.num_local_experts;
  g.rank = p.rank;
  g.T = p.max_tokens_per_rank;
  g.N = p.num_tokens;
  g.H = p.hidden;
  g.I = p.intermediate;
  g.K = p.top_k;
  g.layout = p.layout;
  g.W = p.num_experts / p.num_local_experts;
  g.cap = (int64_t)g.W * g.T;
  g.rows = p.layout == MOE_EP_RANK_MAJOR ? (int32_t)(g.W * g.T) : (p.layout == MOE_EP_FLAT ? g.N : 0);
  return g;
}

moe_ep_status_t check_params(const moe_ep_params_t* p) {
  if (!p) return MOE_EP_EINVAL;
  if (p->num_experts < 1 || p->num_local_experts < 1) return MOE_EP_EINVAL;
  if (p->num_experts % p->num_local_experts != 0) return MOE_EP_EINVAL;
  const int64_t W = p->num_experts / p->num_local_experts;
  if (p->rank < 0 || p->rank >= W) return MOE_EP_EINVAL;
  if (p->max_tokens_per_rank < 1 || p->num_tokens < 0) return MOE_EP_EINVAL;
  if ((int64_t)p->num_tokens > W * p->max_tokens_per_rank) return MOE_EP_EINVAL;
  if (p->hidden < 128 || p->hidden % 128 != 0) return MOE_EP_EINVAL;
  if (p->top_k < 1 || p->intermediate < 0) return MOE_EP_EINVAL;
  if (p->layout < MOE_EP_EXPERT_MAJOR || p->layout > MOE_EP_FLAT) return MOE_EP_EINVAL;
  // limits of this build
  if (p->num_local_experts > kMaxLocalExperts || p->top_k > kMaxTopK) return MOE_EP_EUNSUPPORTED;
  if (p->intermediate % 64 != 0 || p->hidden > 65536) return MOE_EP_EUNSUPPORTED;
  const int64_t cap = W * p->max_tokens_per_rank;
  const int64_t lim = (int64_t)1 << 31;
  if (cap * p->num_local_experts >= lim) return MOE_EP_EUNSUPPORTED;
  if ((int64_t)p->num_tokens * p->top_k >= lim || cap * p->top_k >= lim) return MOE_EP_EUNSUPPORTED;
  return MOE_EP_OK;
}

Layout layout_of(const moe_ep_params_t& p) {
  const Geom g = geom_of(p);
  Layout l;
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t o = at;
    at += (bytes + kAlign - 1) / kAlign * kAlign;
    return o;
  };
  const size_t L = (size_t)g.L, K = (size_t)g.K, N = (size_t)g.N, H = (size_t)g.H, I = (size_t)g.I;
  l.nchunks_dispatch = (g.N + kChunkTokens - 1) / kChunkTokens;
  l.nchunks_bridge = (g.rows + kChunkTokens - 1) / kChunkTokens;
  const size_t nch = (size_t)std::max(l.nchunks_dispatch, l.nchunks_bridge);
  // local picks <= N*K; EXPERT_MAJOR offsets count every pick, including those over capacity
  l.pmax = (int64_t)N * (int64_t)K;
  l.max_tiles = max_tiles(l.pmax, g.L, kGemmMinBM);

  l.status = take(64);
  l.recv_count = take(4 * L);
  l.expert_offsets = take(4 * (L + 1));
  l.chunk_hist = take(4 * nch * L);
  l.chunk_base = take(4 * nch * L);
  l.chunk_tok = take(4 * nch);
  l.chunk_tokbase = take(4 * nch);
  l.chunk_err = take(4 * nch);
  l.slot_of = l.src_info = l.layout_range = kAbsent;
  l.recv_topk_idx = l.recv_topk_weights = l.row_of_token = l.recv_src_idx = l.num_recv = kAbsent;
  l.pick_count = l.pick_offsets = l.perm = l.pick_slot = l.topk_gid = l.topk_wmask = l.pick_w = l.pick_tok = kAbsent;
  const size_t rows = (size_t)g.rows;
  if (p.layout == MOE_EP_EXPERT_MAJOR) {
    l.slot_of = take(4 * N * K);
    l.src_info = take(4 * L * (size_t)g.cap);
    l.layout_range = take(8 * L * (size_t)g.W);
  } else {
    l.recv_topk_idx = take(4 * rows * K);
    l.recv_topk_weights = take(4 * rows * K);
    l.row_of_token = take(4 * N);
    if (p.layout == MOE_EP_FLAT) {
      l.recv_src_idx = take(4 * N);
      l.num_recv = take(4);
    }
    l.pick_count = take(4 * L);
    l.pick_offsets = take(4 * (L + 1));
    l.perm = take(4 * rows * K);
    l.pick_slot = take(4 * rows * K);
    l.topk_gid = take(4 * rows * K);
    l.topk_wmask = take(4 * rows * K);
    // the combine fused into the down GEMM: weight and source token of each pick, expert-sorted
    l.pick_w = take(4 * (size_t)l.pmax);
    l.pick_tok = take(4 * (size_t)l.pmax);
  }
  l.tiles = take(8 * (size_t)l.max_tiles);
  l.num_tiles = take(4);
  // the GEMMs' counters that start at zero (cleared with the tile table): the 256-row kernels' ticket
  // counters, then the split counters
  l.split_partial = l.split_cnt = kAbsent;
  l.gemm_zero = take(4 * (size_t)gemm_zero_words(g));
  if (gemm_split_possible(g)) {
    l.split_partial = take(gemm_split_partial_bytes(g));
    l.split_cnt = l.gemm_zero + 4 * (size_t)kGemmTickets;
  }
  size_t recv_rows = p.layout == MOE_EP_EXPERT_MAJOR ? L * (size_t)g.cap : rows;
  // bf16 rows, or (FP8 dispatch) the codes and, 256-byte aligned after them, the scales: with an
  // odd number of rows of H = 128 the alignment pad leaves the scales no room in 2*H bytes per row
  const size_t fp8_bytes = (recv_rows * H + kAlign - 1) / kAlign * kAlign + recv_rows * (size_t)fp8_scale_stride(g.H);
  l.recv_x = take(std::max(2 * recv_rows * H, fp8_bytes));
  l.h = l.y = kAbsent;
  if (g.I > 0) {
    l.h = take(2 * (size_t)l.pmax * I);
    l.y = take(2 * (size_t)l.pmax * H);
  }
  l.total = at;
  return l;
}

template <class T>
T* at(void* ws, size_t off) {
  return off == kAbsent ? nullptr : (T*)((char*)ws + off);
}

// The last dispatch's serial number per workspace, for the most recently dispatched
// kMaxWorkspaces workspaces of the process (serial numbers are process-wide, so the entry with the
// smallest one is the least recently dispatched; it is dropped when a new workspace would exceed
// the bound, and its handles are then rejected as stale).
constexpr size_t kMaxWorkspaces = 1024;
std::mutex g_epoch_mu;
std::unordered_map<const void*, uint64_t> g_epoch;
uint64_t g_serial = 0;

uint64_t next_epoch(const void* ws) {
  std::lock_guard<std::mutex> lk(g_epoch_mu);
  if (g_epoch.size() >= kMaxWorkspaces && g_epoch.find(ws) == g_epoch.end()) {
    auto oldest = g_epoch.begin();
    for (auto it = g_epoch.begin(); it != g_epoch.end(); ++it)
      if (it->second < oldest->second) oldest = it;
    g_epoch.erase(oldest);
  }
  return g_epoch[ws] = ++g_serial;
}

bool is_current(const moe_ep_handle_t* h) {
  std::lock_guard<std::mutex> lk(g_epoch_mu);
  auto it = g_epoch.find(h->workspace);
  return it != g_epoch.end() && it->second == h->epoch;
}

RouteBufs route_bufs(void* ws, const Layout& l, int32_t nchunks) {
  RouteBufs rb;
  rb.chunk_hist = at<int32_t>(ws, l.chunk_hist);
  rb.chunk_base = at<int32_t>(ws, l.chunk_base);
  rb.chunk_tok = at<int32_t>(ws, l.chunk_tok);
  rb.chunk_tokbase = at<int32_t>(ws, l.chunk_tokbase);
  rb.chunk_err = at<int32_t>(ws, l.chunk_err);
  rb.nchunks = nchunks;
  return rb;
}

void fill_handle(const moe_ep_params_t& p, void* ws, const Layout& l, moe_ep_handle_t* h) {
  std::memset(h, 0, sizeof(*h));
  h->workspace = ws;
  h->params = p;
  h->recv_x = at<void>(ws, l.recv_x);
  h->recv_count = at<int32_t>(ws, l.recv_count);
  h->expert_offsets = at<int32_t>(ws, l.expert_offsets);
  h->slot_of = at<int32_t>(ws, l.slot_of);
  h->src_info = at<int32_t>(ws, l.src_info);
  h->layout_range = at<int32_t>(ws, l.layout_range);
  h->recv_topk_idx = at<int32_t>(ws, l.recv_topk_idx);
  h->recv_topk_weights = at<float>(ws, l.recv_topk_weights);
  h->row_of_token = at<int32_t>(ws, l.row_of_token);
  h->recv_src_idx = at<int32_t>(ws, l.recv_src_idx);
  h->num_recv = at<int32_t>(ws, l.num_recv);
  h->pick_count = at<int32_t>(ws, l.pick_count);
  h->pick_offsets = at<int32_t>(ws, l.pick_offsets);
  h->perm = at<int32_t>(ws, l.perm);
  h->pick_slot = at<int32_t>(ws, l.pick_slot);
  h->topk_gid = at<int32_t>(ws, l.topk_gid);
  h->topk_wmask = at<float>(ws, l.topk_wmask);
  h->status = at<int32_t>(ws, l.status);
  h->internal = at<void>(ws, l.tiles);
}

moe_ep_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_EP_OK : MOE_EP_EHIP; }

// Rows of the receive buffer (EM: L*W*T slots; RM: W*T; FLAT: N).
int64_t recv_rows(const Geom& g) { return g.layout == MOE_EP_EXPERT_MAJOR ? (int64_t)g.L * g.cap : (int64_t)g.rows; }

// FP8 dispatch writes the receive buffer as codes [rows, H] followed (256-byte aligned) by scales
// [rows, fp8_scale_stride(H)]; layout_of sizes the buffer for both.
uint8_t* fp8_scales_of(const Geom& g, void* recv_x) {
  const size_t codes = (size_t)recv_rows(g) * g.H;
  return (uint8_t*)recv_x + (codes + kAlign - 1) / kAlign * kAlign;
}

// Whether the one-launch dispatch serves small layers (a test knob turns it off: the environment
// variable MOE_EP_MULTI_LAUNCH_DISPATCH set to 1 selects the multi-launch path everywhere).
bool use_dispatch_ll(const Geom& g) {
  const char* v = std::getenv("MOE_EP_MULTI_LAUNCH_DISPATCH");
  return !(v && v[0] == '1') && dispatch_ll_fits(g);
}

// Dispatch.  ta: the GEMM tile table for the fused routing to write (EXPERT_MAJOR always; RANK_MAJOR /
// FLAT only when the bridge is fused in).  bridge: non-null in the fused forward for RANK_MAJOR /
// FLAT, which lets the one-launch dispatch write the bridge too; *bridged tells whether it did.
moe_ep_status_t dispatch_impl(const moe_ep_params_t& p, const void* x, const int64_t* ids, const float* w,
                              const int32_t* active_ranks, void* ws, moe_ep_handle_t* h, hipStream_t s,
                              bool fp8 = false, const TileArgs& ta = TileArgs{}, bool* tiles_built = nullptr,
                              bool* bridged = nullptr, const BridgeCombine& bc = BridgeCombine{}) {
  const Geom g = geom_of(p, active_ranks);
  const Layout l = layout_of(p);
  fill_handle(p, ws, l, h);
  h->epoch = next_epoch(ws);
  if (tiles_built) *tiles_built = false;
  if (bridged) *bridged = false;
  hipError_t e;
  if (!fp8 && use_dispatch_ll(g)) {
    const bool em = p.layout == MOE_EP_EXPERT_MAJOR;
    const bool with_bridge = !em && bridged != nullptr;
    LLDispatchOut d;
    d.slot_of = h->slot_of;
    d.src_info = h->src_info;
    d.layout_range = h->layout_range;
    d.recv_topk_idx = h->recv_topk_idx;
    d.recv_topk_weights = h->recv_topk_weights;
    d.row_of_token = h->row_of_token;
    d.recv_src_idx = h->recv_src_idx;
    d.num_recv = h->num_recv;
    if (with_bridge) {
      d.pick_count = h->pick_count;
      d.pick_offsets = h->pick_offsets;
      d.perm = h->perm;
      d.pick_slot = h->pick_slot;
      d.gid = h->topk_gid;
      d.wmask = h->topk_wmask;
      d.pick_w = bc.pick_w;
      d.pick_tok = bc.pick_tok;
    }
    const TileArgs t = (em || with_bridge) ? ta : TileArgs{};
    e = launch_dispatch_ll(g, ids, w, x, h->recv_x, h->recv_count, h->expert_offsets, h->status, t, d, s);
    if (e != hipSuccess) return MOE_EP_EHIP;
    if (tiles_built) *tiles_built = t.tiles != nullptr;
    if (bridged) *bridged = with_bridge;
    return MOE_EP_OK;
  }
  if (p.layout == MOE_EP_EXPERT_MAJOR) {
    e = launch_route_expert_major(g, ids, route_bufs(ws, l, l.nchunks_dispatch), h->recv_count, h->expert_offsets,
                                  h->slot_of, h->src_info, h->layout_range, h->status, s, ta, tiles_built);
  } else {
    e = launch_route_rows(g, ids, w, route_bufs(ws, l, l.nchunks_dispatch), h->recv_count, h->expert_offsets,
                          h->recv_topk_idx, h->recv_topk_weights, h->row_of_token, h->recv_src_idx, h->num_recv,
                          h->status, s);
  }
  if (e != hipSuccess) return MOE_EP_EHIP;
  LayoutRangeArgs lr;  // EXPERT_MAJOR: computed by the permute kernel
  if (p.layout == MOE_EP_EXPERT_MAJOR) {
    lr.counts = h->recv_count;
    lr.src_info = h->src_info;
    lr.L = g.L;
    lr.W = g.W;
    lr.T = g.T;
    lr.cap = g.cap;
    lr.out = h->layout_range;
  }
  if (fp8)
    return hip_status(
        launch_permute_fp8(g, x, h->slot_of, h->row_of_token, h->recv_x, fp8_scales_of(g, h->recv_x), s, lr));
  return hip_status(launch_permute(g, x, h->slot_of, h->row_of_token, h->recv_x, s, lr));
}

// Grouped GEMMs for the handle's rows.  EM: rows are the slab slots (count clamp cap), output to
// out_em (slab layout) when non-NULL, else packed into the workspace y.  RM/FLAT: the bridge's
// expert-sorted picks, output packed into the workspace y.
// Records events[i] on the stream if the caller asked for it (stage timing).
struct Marks {
  void* const* ev;
  hipStream_t s;
  hipError_t mark(int i) const { return (ev && ev[i]) ? hipEventRecord((hipEvent_t)ev[i], s) : hipSuccess; }
};

// The tile table of the grouped GEMMs: bm-row tiles over each expert's rows (EXPERT_MAJOR: clamped
// at the slot capacity).  The fused routing kernels can write it along with the counts.
TileArgs tile_args(const moe_ep_params_t& p, void* ws, const Layout& l, int32_t bm) {
  TileArgs ta;
  ta.tiles = at<int2>(ws, l.tiles);
  ta.num_tiles = at<int32_t>(ws, l.num_tiles);
  ta.bm = bm;
  ta.clamp = p.layout == MOE_EP_EXPERT_MAJOR ? geom_of(p).cap : ((int64_t)1 << 40);
  ta.zero = at<int32_t>(ws, l.gemm_zero);
  ta.nzero = gemm_zero_words(geom_of(p));
  return ta;
}

// tiles_built: the routing already wrote the tile table for gemm_row_tile's tile height
moe_ep_status_t gemms(const moe_ep_params_t& p, const moe_ep_handle_t* h, const Layout& l, const void* w1,
                      const void* w2, void* out_em, hipStream_t s, const Marks& mk = Marks{nullptr, nullptr},
                      bool tiles_built = false, const DownCombine& comb = DownCombine{}) {
  const Geom g = geom_of(p);
  void* ws = h->workspace;
  int2* tiles = at<int2>(ws, l.tiles);
  int32_t* num_tiles = at<int32_t>(ws, l.num_tiles);
  bf16_t* hbuf = at<bf16_t>(ws, l.h);
  bf16_t* ybuf = at<bf16_t>(ws, l.y);
  const bool em = p.layout == MOE_EP_EXPERT_MAJOR;
  const int32_t* counts = em ? h->recv_count : h->pick_count;
  const int32_t* offsets = em ? h->expert_offsets : h->pick_offsets;
  const int64_t clamp = em ? g.cap : ((int64_t)1 << 40);
  const int32_t bm = gemm_row_tile(g);
  SplitBufs split;
  split.tickets = at<int32_t>(ws, l.gemm_zero);
  if (l.split_partial != kAbsent) {
    split.partial = at<float>(ws, l.split_partial);
    split.cnt = at<int32_t>(ws, l.split_cnt);
  }
  hipError_t e = tiles_built ? hipSuccess
                             : launch_tile_table(g.L, counts, clamp, bm, tiles, num_tiles, s, split.tickets,
                                                 gemm_zero_words(g));
  if (e != hipSuccess || mk.mark(2) != hipSuccess) return MOE_EP_EHIP;
  GemmRows rows;
  rows.a = (const bf16_t*)h->recv_x;
  rows.perm = em ? nullptr : h->perm;
  rows.K = g.K;
  rows.slab = em ? g.cap : 0;
  e = launch_gemm_gate_up(g, rows, counts, offsets, clamp, (const bf16_t*)w1, hbuf, tiles, num_tiles, bm, s, split);
  if (e != hipSuccess || mk.mark(3) != hipSuccess) return MOE_EP_EHIP;
  bf16_t* y = out_em ? (bf16_t*)out_em : ybuf;
  if (bm == kGemmMinBM && gemm_stream_fits(g.I) && !comb.out) {
    // 64-row tiles (few rows per expert): the weight-streaming down GEMM where I fits its stages
    StreamArgs sa;
    sa.a = hbuf;
    sa.counts = counts;
    sa.offsets = offsets;
    sa.clamp = clamp;
    sa.w = (const bf16_t*)w2;
    sa.out = y;
    sa.out_slab = out_em ? g.cap : 0;
    sa.tiles = tiles;
    sa.num_tiles = num_tiles;
    sa.Kd = g.I;
    sa.H = g.H;
    e = launch_gemm_stream_down(sa, s);
  } else {
    e = launch_gemm_down(g, counts, offsets, clamp, hbuf, (const bf16_t*)w2, y, out_em ? g.cap : 0, tiles, num_tiles,
                         bm, s, comb, split);
  }
  if (e != hipSuccess || mk.mark(4) != hipSuccess) return MOE_EP_EHIP;
  return MOE_EP_OK;
}

moe_ep_status_t check_handle(const moe_ep_params_t* p, const moe_ep_handle_t* h) {
  moe_ep_status_t st = check_params(p);
  if (st != MOE_EP_OK) return st;
  if (!h || !h->workspace) return MOE_EP_EINVAL;
  if (std::memcmp(&h->params, p, sizeof(*p)) != 0) return MOE_EP_EINVAL;
  if (!is_current(h)) return MOE_EP_ESTALE_HANDLE;
  return MOE_EP_OK;
}

moe_ep_status_t check_weights(const moe_ep_params_t& p, const void* w1, const void* w2) {
  if ((w1 == nullptr) != (w2 == nullptr)) return MOE_EP_EINVAL;
  if (w1 && p.intermediate == 0) return MOE_EP_EINVAL;
  return MOE_EP_OK;
}

// The workspace of moe_ep_layer_forward_noalloc, for callers that cannot allocate: a file-scope
// device array of kNoallocWorkspaceBytes, one copy on each GPU the library's code runs on, held
// until the process ends.  Its name is a host-side stand-in in host code; the device address of the
// current GPU's copy comes from hipGetSymbolAddress, looked up once per device (with that device
// current) and kept per device.
constexpr size_t kNoallocWorkspaceBytes = MOE_EP_NOALLOC_WORKSPACE_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoallocWorkspaceBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

moe_ep_status_t check_workspace(const moe_ep_params_t& p, const void* ws, size_t bytes) {
  if (!ws) return MOE_EP_EINVAL;
  if (((uintptr_t)ws) % kAlign != 0) return MOE_EP_EWORKSPACE;
  if (bytes < layout_of(p).total) return MOE_EP_EWORKSPACE;
  return MOE_EP_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_ep_workspace_size(const moe_ep_params_t* params) {
  if (check_params(params) != MOE_EP_OK) return 0;
  return layout_of(*params).total;
}

moe_ep_status_t moe_ep_dispatch(const moe_ep_params_t* params, const void* hidden_states, const int64_t* topk_ids,
                                const float* topk_weights, const int32_t* active_ranks, void* workspace,
                                size_t workspace_bytes, moe_ep_handle_t* handle, void* stream) {
  moe_ep_status_t st = check_params(params);
  if (st != MOE_EP_OK) return st;
  if (!handle || (params->num_tokens > 0 && (!hidden_states || !topk_ids))) return MOE_EP_EINVAL;
  if (params->layout != MOE_EP_EXPERT_MAJOR && params->num_tokens > 0 && !topk_weights) return MOE_EP_EINVAL;
  st = check_workspace(*params, workspace, workspace_bytes);
  if (st != MOE_EP_OK) return st;
  return dispatch_impl(*params, hidden_states, topk_ids, topk_weights, active_ranks, workspace, handle,
                       (hipStream_t)stream);
}

moe_ep_status_t moe_ep_expert_compute(const moe_ep_params_t* params, const moe_ep_handle_t* handle,
                                      const void* w_gate_up, const void* w_down, void* expert_out, void* stream) {
  moe_ep_status_t st = check_handle(params, handle);
  if (st != MOE_EP_OK) return st;
  const moe_ep_params_t& p = *params;
  if ((st = check_weights(p, w_gate_up, w_down)) != MOE_EP_OK) return st;
  const Geom g = geom_of(p);
  // expert_out has the receive layout's rows (FLAT: num_tokens, possibly 0)
  if (!expert_out && (p.layout != MOE_EP_FLAT || g.N > 0)) return MOE_EP_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  const Layout l = layout_of(p);
  const bool identity = w_gate_up == nullptr;
  if (p.layout == MOE_EP_EXPERT_MAJOR) {
    if (identity) return hip_status(launch_copy_slots(g, handle->slot_of, handle->recv_x, expert_out, s));
    return gemms(p, handle, l, w_gate_up, w_down, expert_out, s);
  }
  void* ws = handle->workspace;
  bool built = false;
  hipError_t e = launch_bridge(g, handle->recv_topk_idx, handle->recv_topk_weights,
                               p.layout == MOE_EP_FLAT ? handle->num_recv : nullptr,
                               route_bufs(ws, l, l.nchunks_bridge), handle->pick_count, handle->pick_offsets,
                               handle->perm, handle->pick_slot, handle->topk_gid, handle->topk_wmask, handle->status,
                               s, identity ? TileArgs{} : tile_args(p, ws, l, gemm_row_tile(g)), &built);
  if (e != hipSuccess) return MOE_EP_EHIP;
  if (!identity && (st = gemms(p, handle, l, w_gate_up, w_down, nullptr, s, Marks{nullptr, nullptr}, built)) !=
                       MOE_EP_OK)
    return st;
  return hip_status(launch_finalize_rows(g, handle->row_of_token, handle->pick_slot, handle->topk_wmask,
                                         identity ? nullptr : at<void>(ws, l.y), handle->recv_x, expert_out, false,
                                         s));
}

moe_ep_status_t moe_ep_combine(const moe_ep_params_t* params, const moe_ep_handle_t* handle, const void* expert_out,
                               const float* topk_weights, const int32_t* active_ranks, void* out, void* stream) {
  moe_ep_status_t st = check_handle(params, handle);
  if (st != MOE_EP_OK) return st;
  const moe_ep_params_t& p = *params;
  const Geom g = geom_of(p, active_ranks);
  if (!expert_out && (p.layout != MOE_EP_FLAT || g.N > 0)) return MOE_EP_EINVAL;
  if (p.num_tokens > 0 && !out) return MOE_EP_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  if (p.layout == MOE_EP_EXPERT_MAJOR) {
    if (p.num_tokens > 0 && !topk_weights) return MOE_EP_EINVAL;
    return hip_status(launch_combine_em(g, handle->slot_of, topk_weights, nullptr, expert_out, out, s));
  }
  return hip_status(launch_combine_rows(g, handle->row_of_token, expert_out, out, s));
}

}  // extern "C"

namespace moe {
namespace {

// The fused layer forward.  fused_combine (RANK_MAJOR / FLAT with an expert GEMM): the down GEMM adds
// each pick's weighted output straight into the zeroed token-major output (no y, no finalize).
moe_ep_status_t layer_forward(const moe_ep_params_t* params, const void* hidden_states, const int64_t* topk_ids,
                              const float* topk_weights, const int32_t* active_ranks, const void* w_gate_up,
                              const void* w_down, void* out, void* workspace, size_t workspace_bytes,
                              void* const* events, void* stream, bool fused_combine) {
  moe_ep_status_t st = check_params(params);
  if (st != MOE_EP_OK) return st;
  const moe_ep_params_t& p = *params;
  if (p.num_tokens > 0 && (!hidden_states || !topk_ids || !topk_weights || !out)) return MOE_EP_EINVAL;
  if ((st = check_weights(p, w_gate_up, w_down)) != MOE_EP_OK) return st;
  if ((st = check_workspace(p, workspace, workspace_bytes)) != MOE_EP_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const Marks mk{events, s};
  if (mk.mark(0) != hipSuccess) return MOE_EP_EHIP;
  moe_ep_handle_t h;
  const Geom g = geom_of(p);
  const Layout l = layout_of(p);
  const bool identity = w_gate_up == nullptr;
  const bool em = p.layout == MOE_EP_EXPERT_MAJOR;
  if (fused_combine && (em || identity)) return MOE_EP_EUNSUPPORTED;
  BridgeCombine bc;
  DownCombine dc;
  if (fused_combine) {
    bc.pick_w = at<float>(workspace, l.pick_w);
    bc.pick_tok = at<int32_t>(workspace, l.pick_tok);
    dc.out = (bf16_t*)out;
    dc.pick_w = bc.pick_w;
    dc.pick_tok = bc.pick_tok;
  }
  // the fused routing writes the GEMM tile table along with the counts (EM: dispatch; RM/FLAT: the
  // bridge)
  const TileArgs ta = identity ? TileArgs{} : tile_args(p, workspace, l, gemm_row_tile(g));
  bool built = false, bridged = false;
  if ((st = dispatch_impl(p, hidden_states, topk_ids, topk_weights, active_ranks, workspace, &h, s, false, ta, &built,
                          em ? nullptr : &bridged, bc)) != MOE_EP_OK)
    return st;
  if (mk.mark(1) != hipSuccess) return MOE_EP_EHIP;
  // dispatch gave tokens of inactive source ranks no local pick, so the combines below write
  // zeros for them whatever the mask
  auto marks_234 = [&]() {
    return (mk.mark(2) == hipSuccess && mk.mark(3) == hipSuccess && mk.mark(4) == hipSuccess) ? MOE_EP_OK
                                                                                               : MOE_EP_EHIP;
  };
  if (p.layout == MOE_EP_EXPERT_MAJOR) {
    const void* Y = h.recv_x;
    const int32_t* packed = nullptr;
    if (identity) {
      st = marks_234();
    } else {
      st = gemms(p, &h, l, w_gate_up, w_down, nullptr, s, mk, built);
      Y = at<void>(workspace, l.y);
      packed = h.expert_offsets;
    }
    if (st != MOE_EP_OK) return st;
    if (launch_combine_em(g, h.slot_of, topk_weights, packed, Y, out, s) != hipSuccess) return MOE_EP_EHIP;
    return hip_status(mk.mark(5));
  }
  // the bridge, unless the one-launch dispatch wrote it
  if (fused_combine) bc.src_idx = p.layout == MOE_EP_FLAT ? h.recv_src_idx : nullptr;
  if (!bridged &&
      launch_bridge(g, h.recv_topk_idx, h.recv_topk_weights, p.layout == MOE_EP_FLAT ? h.num_recv : nullptr,
                    route_bufs(workspace, l, l.nchunks_bridge), h.pick_count, h.pick_offsets, h.perm, h.pick_slot,
                    h.topk_gid, h.topk_wmask, h.status, s, ta, &built, bc) != hipSuccess)
    return MOE_EP_EHIP;
  // fused combine: the output starts at zero (tokens without a local pick keep it) and the down GEMM
  // adds every pick into it
  if (fused_combine && launch_zero(out, (int64_t)p.num_tokens * p.hidden * 2, s) != hipSuccess) return MOE_EP_EHIP;
  st = identity ? marks_234() : gemms(p, &h, l, w_gate_up, w_down, nullptr, s, mk, built, dc);
  if (st != MOE_EP_OK) return st;
  if (fused_combine) return hip_status(mk.mark(5));
  if (launch_finalize_rows(g, h.row_of_token, h.pick_slot, h.topk_wmask, identity ? nullptr : at<void>(workspace, l.y),
                           h.recv_x, out, true, s) != hipSuccess)
    return MOE_EP_EHIP;
  return hip_status(mk.mark(5));
}

}  // namespace
}  // namespace moe

extern "C" {

moe_ep_status_t moe_ep_layer_forward_timed(const moe_ep_params_t* params, const void* hidden_states,
                                           const int64_t* topk_ids, const float* topk_weights,
                                           const int32_t* active_ranks, const void* w_gate_up, const void* w_down,
                                           void* out, void* workspace, size_t workspace_bytes,
                                           void* const* events, void* stream) {
  return layer_forward(params, hidden_states, topk_ids, topk_weights, active_ranks, w_gate_up, w_down, out, workspace,
                       workspace_bytes, events, stream, false);
}

moe_ep_status_t moe_ep_layer_forward_fused_combine(const moe_ep_params_t* params, const void* hidden_states,
                                                   const int64_t* topk_ids, const float* topk_weights,
                                                   const int32_t* active_ranks, const void* w_gate_up,
                                                   const void* w_down, void* out, void* workspace,
                                                   size_t workspace_bytes, void* const* events, void* stream) {
  return layer_forward(params, hidden_states, topk_ids, topk_weights, active_ranks, w_gate_up, w_down, out, workspace,
                       workspace_bytes, events, stream, true);
}

moe_ep_status_t moe_ep_layer_forward_fp8(const moe_ep_params_t* params, const void* hidden_states,
                                         const int64_t* topk_ids, const float* topk_weights,
                                         const int32_t* active_ranks, const void* w_gate_up_fp8,
                                         const void* w_gate_up_scales, const void* w_down, void* out,
                                         void* workspace, size_t workspace_bytes, void* const* events,
                                         void* stream) {
  moe_ep_status_t st = check_params(params);
  if (st != MOE_EP_OK) return st;
  const moe_ep_params_t& p = *params;
  if (p.num_tokens > 0 && (!hidden_states || !topk_ids || !topk_weights || !out)) return MOE_EP_EINVAL;
  if (p.intermediate == 0 || !w_gate_up_fp8 || !w_gate_up_scales || !w_down) return MOE_EP_EINVAL;
  if ((st = check_workspace(p, workspace, workspace_bytes)) != MOE_EP_OK) return st;
  const Geom g = geom_of(p);
  // the FP8 gate_up GEMM and the 256-row bf16 down GEMM address operand rows with 32-bit byte offsets
  if ((int64_t)recv_rows(g) * g.H >= ((int64_t)1 << 32) || (int64_t)g.L * 2 * g.I * g.H >= ((int64_t)1 << 32) ||
      !gemm_offsets_fit_32(g))
    return MOE_EP_EUNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  const Marks mk{events, s};
  if (mk.mark(0) != hipSuccess) return MOE_EP_EHIP;
  moe_ep_handle_t h;
  const Layout l = layout_of(p);
  const bool em = p.layout == MOE_EP_EXPERT_MAJOR;
  constexpr int32_t bm = 256;  // the FP8 kernel's tile
  const TileArgs ta = tile_args(p, workspace, l, bm);
  bool built = false;
  if ((st = dispatch_impl(p, hidden_states, topk_ids, topk_weights, active_ranks, workspace, &h, s, true,
                          em ? ta : TileArgs{}, &built)) != MOE_EP_OK)
    return st;
  if (mk.mark(1) != hipSuccess) return MOE_EP_EHIP;
  if (!em && launch_bridge(g, h.recv_topk_idx, h.recv_topk_weights, p.layout == MOE_EP_FLAT ? h.num_recv : nullptr,
                           route_bufs(workspace, l, l.nchunks_bridge), h.pick_count, h.pick_offsets, h.perm,
                           h.pick_slot, h.topk_gid, h.topk_wmask, h.status, s, ta, &built) != hipSuccess)
    return MOE_EP_EHIP;
  int2* tiles = at<int2>(workspace, l.tiles);
  int32_t* num_tiles = at<int32_t>(workspace, l.num_tiles);
  bf16_t* hbuf = at<bf16_t>(workspace, l.h);
  bf16_t* ybuf = at<bf16_t>(workspace, l.y);
  const int32_t* counts = em ? h.recv_count : h.pick_count;
  const int32_t* offsets = em ? h.expert_offsets : h.pick_offsets;
  const int64_t clamp = em ? g.cap : ((int64_t)1 << 40);
  SplitBufs split;
  split.tickets = at<int32_t>(workspace, l.gemm_zero);
  if (l.split_partial != kAbsent) {
    split.partial = at<float>(workspace, l.split_partial);
    split.cnt = at<int32_t>(workspace, l.split_cnt);
  }
  if ((!built && launch_tile_table(g.L, counts, clamp, bm, tiles, num_tiles, s, split.tickets,
                                   gemm_zero_words(g)) != hipSuccess) ||
      mk.mark(2) != hipSuccess)
    return MOE_EP_EHIP;
  GemmRows rows;
  rows.a = nullptr;
  rows.perm = em ? nullptr : h.perm;
  rows.K = g.K;
  rows.slab = em ? g.cap : 0;
  if (launch_gemm_gate_up_fp8(g, rows, (const uint8_t*)h.recv_x, fp8_scales_of(g, h.recv_x), counts, offsets, clamp,
                              (const uint8_t*)w_gate_up_fp8, (const uint8_t*)w_gate_up_scales, hbuf, tiles, num_tiles,
                              s, split.tickets) != hipSuccess ||
      mk.mark(3) != hipSuccess)
    return MOE_EP_EHIP;
  if (launch_gemm_down(g, counts, offsets, clamp, hbuf, (const bf16_t*)w_down, ybuf, 0, tiles, num_tiles, bm, s,
                       DownCombine{}, split) !=
          hipSuccess ||
      mk.mark(4) != hipSuccess)
    return MOE_EP_EHIP;
  hipError_t e;
  if (em) e = launch_combine_em(g, h.slot_of, topk_weights, h.expert_offsets, ybuf, out, s);
  else e = launch_finalize_rows(g, h.row_of_token, h.pick_slot, h.topk_wmask, ybuf, nullptr, out, true, s);
  if (e != hipSuccess) return MOE_EP_EHIP;
  return hip_status(mk.mark(5));
}

moe_ep_status_t moe_ep_layer_forward(const moe_ep_params_t* params, const void* hidden_states,
                                     const int64_t* topk_ids, const float* topk_weights,
                                     const int32_t* active_ranks, const void* w_gate_up, const void* w_down,
                                     void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return moe_ep_layer_forward_timed(params, hidden_states, topk_ids, topk_weights, active_ranks, w_gate_up, w_down,
                                    out, workspace, workspace_bytes, nullptr, stream);
}

moe_ep_status_t moe_ep_layer_forward_noalloc(const moe_ep_params_t* params, const void* hidden_states,
                                             const int64_t* topk_ids, const float* topk_weights,
                                             const int32_t* active_ranks, const void* w_gate_up,
                                             const void* w_down, void* out, void* stream) {
  moe_ep_status_t st = check_params(params);
  if (st != MOE_EP_OK) return st;
  if (layout_of(*params).total > kNoallocWorkspaceBytes) return MOE_EP_EWORKSPACE;
  void* ws = scratch_on_current_device();
  if (!ws) return MOE_EP_EHIP;
  // Nothing in the workspace has to start at zero for the fused forward: the routing overwrites
  // the status word, counts, offsets and the tile table, dispatch writes every receive row a pick
  // reads, the GEMMs write h and y for every pick, and no kernel reads an EXPERT_MAJOR slot past
  // its expert's count.  So the previous call's contents need no clearing.
  return moe_ep_layer_forward_timed(params, hidden_states, topk_ids, topk_weights, active_ranks, w_gate_up, w_down,
                                    out, ws, kNoallocWorkspaceBytes, nullptr, stream);
}

moe_ep_status_t moe_ep_router_topk(const float* scores, int32_t num_tokens, int32_t num_experts, int32_t top_k,
                                   int64_t* topk_ids, float* topk_weights, void* stream) {
  if (num_tokens < 0 || num_experts < 1 || top_k < 1 || top_k > num_experts) return MOE_EP_EINVAL;
  if (num_tokens > 0 && (!scores || !topk_ids || !topk_weights)) return MOE_EP_EINVAL;
  if (num_experts > 1024 || top_k > 64) return MOE_EP_EUNSUPPORTED;
  if ((int64_t)num_tokens * num_experts >= ((int64_t)1 << 31)) return MOE_EP_EUNSUPPORTED;
  return hip_status(launch_router_topk(scores, num_tokens, num_experts, top_k, topk_ids, topk_weights,
                                       (hipStream_t)stream));
}

int32_t moe_ep_fp8_scale_stride(int32_t cols) {
  return (cols > 0 && cols % 128 == 0) ? fp8_scale_stride(cols) : 0;
}

moe_ep_status_t moe_ep_quantize_fp8(const void* x, int64_t rows, int32_t cols, void* codes, void* scales,
                                    void* stream) {
  if (rows < 0 || cols <= 0 || cols % 128 != 0) return MOE_EP_EINVAL;
  if (rows > 0 && (!x || !codes || !scales)) return MOE_EP_EINVAL;
  return hip_status(launch_quantize_rows_fp8(x, rows, cols, codes, scales, (hipStream_t)stream));
}

moe_ep_status_t moe_ep_query_status(const moe_ep_handle_t* handle, void* stream) {
  if (!handle || !handle->status) return MOE_EP_EINVAL;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return MOE_EP_EHIP;
  int32_t v = 0;
  if (hipMemcpy(&v, handle->status, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return MOE_EP_EHIP;
  if (v & kStatusBadExpertId) return MOE_EP_EEXPERT_ID;
  if (v & kStatusCapacity) return MOE_EP_ECAPACITY;
  return MOE_EP_OK;
}

const char* moe_ep_strerror(moe_ep_status_t s) {
  switch (s) {
    case MOE_EP_OK: return "ok";
    case MOE_EP_EINVAL: return "invalid argument (null pointer or geometry rule)";
    case MOE_EP_EUNSUPPORTED: return "outside the limits of this build";
    case MOE_EP_EWORKSPACE:
      return "workspace too small or not 256-byte aligned (no-allocation forward: layer over its static workspace)";
    case MOE_EP_EEXPERT_ID: return "a topk id outside [-1, num_experts)";
    case MOE_EP_ECAPACITY: return "an EXPERT_MAJOR expert received more picks than its capacity";
    case MOE_EP_ESTALE_HANDLE: return "handle older than the last dispatch on its workspace";
    case MOE_EP_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

}  // extern "C"
