/*
 * moe_ep.h — C ABI of the MoE expert-parallel layer on one MI355X (gfx950).
 *
 * One GPU's share of an expert-parallel MoE layer: dispatch (route token rows
 * by topk_ids into a receive layout), a per-expert grouped SwiGLU GEMM, and a
 * topk_weights-weighted combine back to token-major [num_tokens, hidden] bf16.
 *
 * Sources, cited by page title and section:
 *  [FI-1] FlashInfer "MoE-EP implementation & usage", section 1 "Public API":
 *         MoEEpTensors(hidden_states, topk_ids, topk_weights), FleetParams
 *         (num_experts, max_tokens_per_rank, token_hidden_size, ..., layout),
 *         BootstrapConfig(world_size, rank, stream, ...), EpLayout
 *         {EXPERT_MAJOR, RANK_MAJOR, FLAT}; a missing backend raises a
 *         "not built" error.
 *  [FI-2] same page, section 2 "Call stack": forward = create handle from
 *         topk_ids and topk_weights on the user stream, dispatch, the
 *         EP->compute bridge, the per-expert grouped GEMM (no routing inside
 *         it), reshape for combine, combine; the result is [num_tokens,
 *         hidden] bf16; every stage runs on the user stream.
 *  [FI-3] same page, section 3 "Algorithm / layout contracts": the receive
 *         buffer of each layout, what compute does with it, how combine
 *         reduces; received topk_idx are LOCAL ids (-1 = non-local), int32;
 *         the bridge converts local -> global ids and masks non-local picks
 *         to weight 0.
 *  [FI-4] same page, section 4 "Usage walkthrough": expert weights
 *         w1 [E, 2I, H] and w2 [E, H, I]; this rank's slice is experts
 *         [offset, offset + num_local_experts).
 *  [MC-H] Mooncake PG/EP guide, "Buffer.get_ep_buffer_size_hint": the
 *         workspace is sized for the peak dispatch of one step.
 *  [MC-D] Mooncake PG/EP guide, "Buffer.dispatch": topk_idx int64
 *         [num_tokens, top_k] with -1 for masked picks; ids in
 *         [0, num_experts); num_experts divisible by the number of ranks;
 *         hidden divisible by 128; the receive buffer is local-expert-major
 *         [num_local_experts, num_ranks * max_tokens_per_rank, hidden] with a
 *         received count per local expert, per-slot source info and
 *         per-(expert, rank) layout ranges, kept in the handle.
 *  [MC-C] Mooncake PG/EP guide, "Buffer.combine" and "get_next_combine_buffer":
 *         combine takes the expert output in the dispatch layout plus
 *         topk_idx / topk_weights and the matching handle; a handle must not
 *         be reused across unrelated dispatch/combine pairs.
 *  [MC-A] Mooncake PG/EP guide, "Buffer.dispatch" / "Buffer.combine"
 *         (active_ranks) and the troubleshooting notes: an int32 [num_ranks]
 *         EP-level rank-health tensor passed to both; an inactive source
 *         rank is skipped (its slot stays, it is not renumbered).  Timeout
 *         detection (timeout_us >= 0), which may clear entries, is not part
 *         of this library: the mask is only read.
 *  [MC-F] Mooncake PG/EP guide, "Buffer.dispatch" (use_fp8: the receive
 *         buffer holds FP8 data plus scales; hidden divisible by 128).
 *  [MC-R] Mooncake PG/EP guide, quick start, and FlashInfer "MoE-EP
 *         implementation & usage" section 4 step 2: topk_idx is the top_k of
 *         per-token expert scores, topk_weights a softmax.
 *
 * Conventions for every entry point
 *  - Pointers named "device" are HIP device pointers; the library never
 *    allocates, frees or copies them to the host.  The caller owns them.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every kernel is
 *    enqueued asynchronously on it; no entry point synchronises the host,
 *    except moe_ep_query_status.
 *  - Host-detectable errors (null pointers, geometry rules, a small
 *    workspace, a stale handle) return at once and enqueue nothing.
 *    Data-dependent errors (an expert id outside [-1, num_experts), an
 *    EXPERT_MAJOR expert over capacity) are latched in a device status word
 *    of the workspace and read by moe_ep_query_status; the kernels skip the
 *    offending picks and never write out of bounds.
 *  - bf16 means IEEE bfloat16 bit patterns (uint16); conversions from fp32
 *    round to nearest even.
 */
#ifndef MOE_EP_H
#define MOE_EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Receive layouts [FI-1], [FI-3]. */
typedef enum {
  MOE_EP_EXPERT_MAJOR = 0, /* recv [L, W*T, H]: rows pre-assigned to local experts */
  MOE_EP_RANK_MAJOR = 1,   /* recv [W, T, H]: row (r, i) = token i of source rank r */
  MOE_EP_FLAT = 2          /* recv [num_recv, H]: token-major, tokens with >= 1 local pick */
} moe_ep_layout_t;

typedef enum {
  MOE_EP_OK = 0,
  MOE_EP_EINVAL = 1,        /* null pointer or a geometry rule broken (see moe_ep_params_t) */
  MOE_EP_EUNSUPPORTED = 2,  /* a valid request outside this build's limits ("not built" [FI-1]) */
  MOE_EP_EWORKSPACE = 3,    /* workspace smaller than moe_ep_workspace_size or not 256-byte aligned */
  MOE_EP_EEXPERT_ID = 4,    /* device: a topk id outside [-1, num_experts) [MC-D] */
  MOE_EP_ECAPACITY = 5,     /* device: an EXPERT_MAJOR expert got more than W*T picks (repeated ids) */
  MOE_EP_ESTALE_HANDLE = 6, /* handle older than the last dispatch on its workspace [MC-C] */
  MOE_EP_EHIP = 7           /* a HIP runtime call failed */
} moe_ep_status_t;

/*
 * Layer geometry [FI-1], [MC-D].  World W = num_experts / num_local_experts;
 * this GPU owns global experts [rank*L, rank*L + L).  Source token t
 * (0 <= t < num_tokens) is token t % T of source rank t / T, T =
 * max_tokens_per_rank; its pick k is local iff its expert is owned here.
 * Rules (MOE_EP_EINVAL otherwise): num_experts % num_local_experts == 0,
 * 0 <= rank < W, 0 <= num_tokens <= W*T, hidden % 128 == 0, top_k >= 1,
 * intermediate >= 0, layout one of moe_ep_layout_t.
 * Limits of this build (MOE_EP_EUNSUPPORTED otherwise): num_local_experts
 * <= 1024, top_k <= 64, intermediate % 64 == 0, hidden <= 65536,
 * W*T*num_local_experts and num_tokens*top_k below 2^31.
 * intermediate == 0 selects the identity expert (y = received row).
 */
typedef struct {
  int32_t num_experts;         /* E, global experts */
  int32_t num_local_experts;   /* L */
  int32_t rank;                /* this GPU's EP rank (BootstrapConfig.rank) */
  int32_t max_tokens_per_rank; /* T */
  int32_t num_tokens;          /* N, rows of hidden_states */
  int32_t hidden;              /* H */
  int32_t intermediate;        /* I; 0 = identity expert */
  int32_t top_k;               /* K */
  int32_t layout;              /* moe_ep_layout_t */
} moe_ep_params_t;

/*
 * Dispatch metadata (the analogue of Mooncake's handle tuple and FlashInfer's
 * DispatchOutput).  Filled by moe_ep_dispatch; every pointer is a device
 * pointer into the caller's workspace and lives as long as the workspace.
 * Integer arrays are int32, weights fp32, rows bf16.  Arrays of other layouts
 * are NULL.
 */
typedef struct {
  uint64_t epoch;             /* dispatch serial number (process-wide); a handle is current while it
                                 holds its workspace's last dispatch, and that record is kept for the
                                 1024 most recently dispatched workspaces of the process (a handle of
                                 an older one is rejected as stale) */
  void* workspace;            /* the workspace it points into */
  moe_ep_params_t params;
  void* recv_x;               /* bf16: EM [L, W*T, H]; RM [W*T, H]; FLAT [N, H] (first num_recv rows) */
  int32_t* recv_count;        /* [L] local picks received per local expert */
  int32_t* expert_offsets;    /* [L+1] exclusive prefix sum of recv_count */
  /* EXPERT_MAJOR (cap = W*T slots per expert, slot order (source rank, token, k)) */
  int32_t* slot_of;           /* [N*K] el*cap + slot of pick (t,k); -1 if not local */
  int32_t* src_info;          /* [L*cap] source token of each used slot (unused slots untouched) */
  int32_t* layout_range;      /* [L*W*2] (first slot, count) per (local expert, source rank) */
  /* RANK_MAJOR (rows W*T, row of token t is t) / FLAT (rows compacted in token order) */
  int32_t* recv_topk_idx;     /* [rows*K] local expert id, -1 = non-local or masked */
  float* recv_topk_weights;   /* [rows*K] topk_weights of the row's token as sent; 0 on RM rows without local picks */
  int32_t* row_of_token;      /* [N] receive row of token t; -1 if it has no local pick */
  int32_t* recv_src_idx;      /* FLAT [N] source token of received row j < num_recv */
  int32_t* num_recv;          /* FLAT [1] number of received rows */
  /* compute-side bridge over the received routing (RM / FLAT), filled by moe_ep_expert_compute */
  int32_t* pick_count;        /* [L] */
  int32_t* pick_offsets;      /* [L+1] */
  int32_t* perm;              /* [P] row*K + k of each local pick in (expert, row, k) order */
  int32_t* pick_slot;         /* [rows*K] index of pick (row, k) in perm; -1 if masked */
  int32_t* topk_gid;          /* [rows*K] global expert id = local id + rank*L; -1 if masked */
  float* topk_wmask;          /* [rows*K] routing weight; 0 if masked */
  int32_t* status;            /* device status word (see moe_ep_query_status) */
  void* internal;             /* library scratch inside the workspace */
} moe_ep_handle_t;

/* Bytes of workspace the entry points need for `params` (peak dispatch [MC-H]); 0 if params are invalid.
 * EXPERT_MAJOR's receive buffer alone is L*W*T*H*2 bytes. */
size_t moe_ep_workspace_size(const moe_ep_params_t* params);

/*
 * Dispatch [FI-2], [FI-3], [MC-D].  Routes the rows of hidden_states (device
 * bf16 [N, H]) by topk_ids (device int64 [N, K]) into the receive layout in
 * the workspace and fills *handle.  topk_weights (device fp32 [N, K]) is
 * carried into the received routing for RM / FLAT; EM ignores it (combine
 * weights on receive).  For EXPERT_MAJOR, slots >= recv_count[el] of the
 * receive buffer are not written: a caller that wants them zero clears the
 * workspace once after allocating it.
 * active_ranks [MC-A]: device int32 [W] or NULL (every rank active).  Every
 * token t of a source rank r = t / T with active_ranks[r] == 0 is skipped:
 * none of its picks is local, its ids are not checked, it gets no slot and no
 * receive row.  Any nonzero entry means active.
 */
moe_ep_status_t moe_ep_dispatch(const moe_ep_params_t* params, const void* hidden_states,
                                const int64_t* topk_ids, const float* topk_weights, const int32_t* active_ranks,
                                void* workspace, size_t workspace_bytes, moe_ep_handle_t* handle, void* stream);

/*
 * Expert compute [FI-2], [FI-3], [FI-4]: the per-expert grouped SwiGLU GEMM
 * y = W2_e (SiLU(W1_e[0:I] x) * W1_e[I:2I] x), bf16 MFMA with fp32
 * accumulation, h and y rounded to bf16.  w_gate_up: device bf16 [L, 2I, H]
 * (gate rows [0, I), up rows [I, 2I)); w_down: device bf16 [L, H, I]; both
 * NULL selects the identity expert.
 *  EXPERT_MAJOR: top_k = 1 per received row; writes expert_out [L, W*T, H]
 *    bf16 in the receive layout (slots below recv_count).
 *  RANK_MAJOR / FLAT: runs the bridge (local -> global ids, masked weights,
 *    expert-sorted pick order) over the received routing, then real top_k:
 *    expert_out row j = sum_k masked weight * y(pick), rows as in recv_x
 *    (rows without a local pick are not written).
 */
moe_ep_status_t moe_ep_expert_compute(const moe_ep_params_t* params, const moe_ep_handle_t* handle,
                                      const void* w_gate_up, const void* w_down, void* expert_out,
                                      void* stream);

/*
 * Combine [FI-3], [MC-C] into out (device bf16 [N, H]).
 *  EXPERT_MAJOR: out[t] = sum over local picks k (ascending) of
 *    topk_weights[t,k] * expert_out[slot_of[t,k]], fp32 accumulation;
 *    topk_weights (device fp32 [N, K]) is required.
 *  RANK_MAJOR / FLAT: weights were applied in compute; out[t] =
 *    expert_out[row_of_token[t]] (the unweighted sum over this GPU's single
 *    contribution); topk_weights is ignored and may be NULL.
 * Tokens with no local pick get 0, and so does every token of a source rank
 * whose active_ranks entry is 0 (device int32 [W], or NULL = every rank
 * active [MC-A]; normally the mask given to the matching dispatch).
 */
moe_ep_status_t moe_ep_combine(const moe_ep_params_t* params, const moe_ep_handle_t* handle,
                               const void* expert_out, const float* topk_weights, const int32_t* active_ranks,
                               void* out, void* stream);

/*
 * The fused layer forward [FI-2]: dispatch, expert compute and combine in
 * one call, with RM / FLAT's weighting fused into the combine (no expert_out
 * round trip).  Same arguments and rules as the three stages; out is device
 * bf16 [N, H].
 */
moe_ep_status_t moe_ep_layer_forward(const moe_ep_params_t* params, const void* hidden_states,
                                     const int64_t* topk_ids, const float* topk_weights,
                                     const int32_t* active_ranks, const void* w_gate_up, const void* w_down,
                                     void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The fused layer forward with stage timing (the analogue of FlashInfer's
 * enable_timing, section 2 "Call stack": events bracket dispatch, compute and
 * combine on the user stream).  events[0..5] are hipEvent_t handles (an entry
 * may be NULL; events itself may be NULL) recorded on `stream` at: 0 start,
 * 1 after dispatch (routing + permute), 2 before the gate_up GEMM (after the
 * RM / FLAT bridge and the tile table), 3 after the gate_up GEMM, 4 after the
 * down GEMM, 5 after combine.  For the identity expert 2, 3 and 4 coincide.
 * Results are those of moe_ep_layer_forward.
 */
moe_ep_status_t moe_ep_layer_forward_timed(const moe_ep_params_t* params, const void* hidden_states,
                                           const int64_t* topk_ids, const float* topk_weights,
                                           const int32_t* active_ranks, const void* w_gate_up, const void* w_down,
                                           void* out, void* workspace, size_t workspace_bytes,
                                           void* const* events, void* stream);

/*
 * The fused layer forward with the combine fused into the down GEMM (zero-copy combine: Mooncake PG/EP
 * guide, "Buffer.get_next_combine_buffer" and combine with zero_copy, where the expert computation
 * writes straight into what combine reads; here that is the token-major output itself).
 * RANK_MAJOR / FLAT: the down GEMM's epilogue multiplies each pick's output row by its masked routing
 * weight and adds it into out[token] with packed-bf16 global atomics, after out is zeroed; neither the
 * expert outputs nor a separate combine pass go through memory.  The additions of a token's picks
 * arrive in no fixed order and each sum is rounded to bf16, so the result differs from
 * moe_ep_layer_forward by rounding, and between runs in the last bits, within the layer's float
 * tolerance.  Same arguments as moe_ep_layer_forward_timed (events 4 and 5 both mark the end of the
 * down GEMM, which is also the combine).  MOE_EP_EUNSUPPORTED: EXPERT_MAJOR layout, identity expert.
 */
moe_ep_status_t moe_ep_layer_forward_fused_combine(const moe_ep_params_t* params, const void* hidden_states,
                                                   const int64_t* topk_ids, const float* topk_weights,
                                                   const int32_t* active_ranks, const void* w_gate_up,
                                                   const void* w_down, void* out, void* workspace,
                                                   size_t workspace_bytes, void* const* events, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): moe_ep_layer_forward without a workspace argument.  Its
 * workspace is a static device buffer of MOE_EP_NOALLOC_WORKSPACE_BYTES inside the library, one copy
 * per GPU (each GPU this entry point runs on holds its copy until the process ends); a call uses the
 * copy of the current device, so `stream` must belong to that device.  The call allocates nothing.
 * MOE_EP_EWORKSPACE (nothing enqueued): moe_ep_workspace_size(params) is larger than the buffer;
 * for example a 2048-token RANK_MAJOR layer with H = 4096, I = 1408, top-6 needs 145 MiB and fits,
 * a 1024-token EXPERT_MAJOR decode with 32 local experts and H = 7168 needs 592 MiB and does not.
 * Every call on a GPU shares that GPU's buffer, which keeps the last call's contents (no call needs
 * any of it cleared first): calls on one stream run one after another, but calls that overlap on
 * one GPU (other streams, other host threads) race and corrupt each other's results.  Data errors
 * are skipped as in moe_ep_layer_forward, which returns no handle to query either.
 */
#define MOE_EP_NOALLOC_WORKSPACE_BYTES ((size_t)256 << 20)
moe_ep_status_t moe_ep_layer_forward_noalloc(const moe_ep_params_t* params, const void* hidden_states,
                                             const int64_t* topk_ids, const float* topk_weights,
                                             const int32_t* active_ranks, const void* w_gate_up,
                                             const void* w_down, void* out, void* stream);

/*
 * Router, upstream of dispatch [MC-R]: for each token t of scores (device fp32
 * [num_tokens, num_experts], row-major, no NaN), topk_ids[t] (device int64
 * [num_tokens, top_k]) = the top_k experts with the largest scores, largest
 * first, equal scores ordered by the lower expert id (-0.0 equals +0.0);
 * topk_weights[t] (device fp32 [num_tokens, top_k]) = softmax over those
 * top_k scores, exp(s_k - s_0) / sum_j exp(s_j - s_0), fp32.
 * MOE_EP_EINVAL: num_tokens < 0, num_experts < 1, top_k < 1, top_k >
 * num_experts, or a NULL pointer with num_tokens > 0.  MOE_EP_EUNSUPPORTED:
 * num_experts > 1024 or top_k > 64.  The outputs feed moe_ep_dispatch /
 * moe_ep_layer_forward directly.
 */
moe_ep_status_t moe_ep_router_topk(const float* scores, int32_t num_tokens, int32_t num_experts, int32_t top_k,
                                   int64_t* topk_ids, float* topk_weights, void* stream);

/*
 * FP8 rows [MC-F].  A bf16 row is cut into blocks of 128 values; a block with
 * largest magnitude a gets the scale 2^k, k the smallest integer with
 * a <= 448 * 2^k (k = 0 for an all-zero block; clamped to [-127, 127]); each
 * value v is stored as the OCP FP8 E4M3 code of v * 2^-k, round to nearest
 * even (never saturates), and the block's scale as the byte k + 127.  The
 * value a code stands for is e4m3(code) * 2^k.  A row's scale bytes are padded
 * with zeros to moe_ep_fp8_scale_stride(cols) bytes.
 *
 * moe_ep_quantize_fp8: x device bf16 [rows, cols] -> codes device uint8
 * [rows, cols] and scales device uint8 [rows, moe_ep_fp8_scale_stride(cols)]
 * (used for the FP8 expert weights, and the same format the FP8 dispatch
 * writes).  MOE_EP_EINVAL: rows < 0, cols <= 0, cols % 128 != 0, or a NULL
 * pointer with rows > 0.  moe_ep_fp8_scale_stride returns 0 for invalid cols.
 */
int32_t moe_ep_fp8_scale_stride(int32_t cols);
moe_ep_status_t moe_ep_quantize_fp8(const void* x, int64_t rows, int32_t cols, void* codes, void* scales,
                                    void* stream);

/*
 * The fused layer forward with FP8 dispatch and an FP8 gate_up GEMM [MC-F],
 * [FI-2]: dispatch quantises each received row into the FP8 row format above
 * (in the workspace's receive buffer), the gate_up GEMM multiplies those rows
 * by W1 in the same format on the block-scaled MFMA (fp32 accumulation,
 * SwiGLU, h in bf16), and the down GEMM and combine run as in
 * moe_ep_layer_forward.  Equivalently: the layer forward on the dequantised
 * hidden_states and W1.
 *   w_gate_up_fp8: device uint8 [L, 2I, H] codes; w_gate_up_scales: device
 *   uint8 [L*2I, moe_ep_fp8_scale_stride(H)] (both from moe_ep_quantize_fp8 of
 *   the bf16 W1 viewed as [L*2I, H]); w_down: device bf16 [L, H, I].
 * events: as moe_ep_layer_forward_timed (NULL for none).  Same workspace as
 * the bf16 forward.  MOE_EP_EINVAL: intermediate == 0 or a NULL weight;
 * MOE_EP_EUNSUPPORTED: receive rows x H, L x 2I x H, 2 x N x top_k x I or 2 x L x H x I of 2^32 bytes or
 * more (the FP8 gate_up GEMM and the down GEMM address operands with 32-bit byte offsets).
 */
moe_ep_status_t moe_ep_layer_forward_fp8(const moe_ep_params_t* params, const void* hidden_states,
                                         const int64_t* topk_ids, const float* topk_weights,
                                         const int32_t* active_ranks, const void* w_gate_up_fp8,
                                         const void* w_gate_up_scales, const void* w_down, void* out,
                                         void* workspace, size_t workspace_bytes, void* const* events,
                                         void* stream);

/* Synchronises `stream` and returns the first data error latched since the handle's dispatch
 * (MOE_EP_EEXPERT_ID, then MOE_EP_ECAPACITY), or MOE_EP_OK. */
moe_ep_status_t moe_ep_query_status(const moe_ep_handle_t* handle, void* stream);

/* Static English text of a status code. */
const char* moe_ep_strerror(moe_ep_status_t status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_EP_H */
