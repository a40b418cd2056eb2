/*
 * CPU oracle of the MoE expert-parallel layer, one GPU's share.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, single-threaded
 * definition that the GPU library is checked against.  Only the tests, the
 * smoke check and the benchmark's CPU-baseline leg may call it; the product
 * path never does.  It shares no code with the GPU library.
 *
 * What it computes (FlashInfer "MoE-EP implementation & usage", section 3
 * "Algorithm / layout contracts" and section 4 "Usage walkthrough"; Mooncake
 * PG/EP guide, "Buffer.dispatch" and "Buffer.combine"):
 *
 *   out[t] = sum over local picks k of token t, k ascending, of
 *            topk_weights[t,k] * W2_e( SiLU(W1g_e x_t) * (W1u_e x_t) ),
 *   e = topk_ids[t,k] - rank*L,
 *
 * plus the integer products of dispatch (per-expert counts, offsets, slots,
 * the received routing) and of the compute-side bridge (local -> global ids,
 * masked weights, expert-sorted pick order).
 *
 * Precision: bf16 inputs are widened exactly to fp32; every sum is fp32 in
 * the order documented at each function; nothing is rounded to bf16.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_EXPERT_MAJOR = 0, ORC_RANK_MAJOR = 1, ORC_FLAT = 2 };
enum { ORC_OK = 0, ORC_EINVAL = 1, ORC_EEXPERT_ID = 2, ORC_ECAPACITY = 3 };

typedef struct {
  int32_t num_experts;         /* E, global experts */
  int32_t num_local_experts;   /* L; world W = E / L; this GPU owns experts [rank*L, rank*L + L) */
  int32_t rank;
  int32_t max_tokens_per_rank; /* T; source token t belongs to source rank t / T */
  int32_t num_tokens;          /* N <= W * T source tokens presented to this GPU */
  int32_t hidden;              /* H */
  int32_t intermediate;        /* I (0: identity expert) */
  int32_t top_k;               /* K */
  int32_t layout;              /* ORC_EXPERT_MAJOR / ORC_RANK_MAJOR / ORC_FLAT */
  /* [W] source-rank health mask (Mooncake PG/EP guide, "Buffer.dispatch" and "Buffer.combine":
   * the EP-level active_ranks tensor, timeout detection off).  Entry r == 0: every token of
   * source rank r is skipped -- its picks are not received (not even checked) and its output
   * is zero.  NULL: every rank is active. */
  const int32_t* active_ranks;
} orc_params_t;

/* Integer outputs of dispatch.  Pointers of the other layouts may be NULL. */
typedef struct {
  int32_t* recv_count;        /* [L] local picks per local expert */
  int32_t* expert_offsets;    /* [L+1] exclusive prefix sum of recv_count */
  /* EXPERT_MAJOR, cap = W*T slots per local expert */
  int32_t* slot_of;           /* [N*K] el*cap + slot, -1 for picks that are not local */
  int32_t* src_info;          /* [L*cap] source token of each slot, -1 for unused slots */
  int32_t* layout_range;      /* [L*W*2] (first slot, number of slots) per (expert, source rank) */
  /* RANK_MAJOR: rows = W*T, row of token t is t.  FLAT: rows = N, compacted. */
  int32_t* recv_topk_idx;     /* [rows*K] local expert id, -1 for non-local / masked picks */
  float*   recv_topk_weights; /* [rows*K] routing weights as sent (unmasked), 0 on rows with no local pick */
  int32_t* row_of_token;      /* [N] receive row of token t, -1 if it has no local pick */
  int32_t* recv_src_idx;      /* FLAT [N] source token of each received row */
  int32_t* num_recv;          /* FLAT [1] received rows */
} orc_route_t;

/* Outputs of the compute-side bridge over the received routing (RANK_MAJOR / FLAT). */
typedef struct {
  int32_t* pick_count;        /* [L] */
  int32_t* pick_offsets;      /* [L+1] */
  int32_t* perm;              /* [P] row*K + k of each pick, in (expert, row, k) order */
  int32_t* pick_slot;         /* [rows*K] position of pick (row,k) in perm, -1 if masked */
  int32_t* topk_gid;          /* [rows*K] global expert id (local + rank*L), -1 if masked */
  float*   topk_wmask;        /* [rows*K] weight, 0 if masked */
} orc_bridge_t;

/* Number of receive rows of the layout (EM: L*W*T slots; RM: W*T; FLAT: N). */
int64_t orc_recv_rows(const orc_params_t* p);

int orc_check_params(const orc_params_t* p);

/* Dispatch routing (integers only). Returns ORC_OK / ORC_EINVAL / ORC_EEXPERT_ID / ORC_ECAPACITY. */
int orc_route(const orc_params_t* p, const int64_t* topk_ids, const float* topk_weights, const orc_route_t* out);

/* Bridge over `rows` received rows of recv_topk_idx / recv_topk_weights. */
int orc_bridge(const orc_params_t* p, int32_t rows, const int32_t* recv_topk_idx,
               const float* recv_topk_weights, const orc_bridge_t* out);

/* y[H] = W2 (SiLU(W1[0:I] x) * W1[I:2I] x) for one bf16 row x; w_gate_up [2I,H], w_down [H,I]
 * of one expert.  Identity (y = x) when w_gate_up == NULL.  a_scratch holds I floats. */
void orc_expert_ffn(int32_t H, int32_t I, const uint16_t* x, const uint16_t* w_gate_up,
                    const uint16_t* w_down, float* y, float* a_scratch);

/* out[j] (fp32 [ntok, H]) = the layer output of source token tokens[j]. */
int orc_forward_tokens(const orc_params_t* p, const uint16_t* hidden_states, const int64_t* topk_ids,
                       const float* topk_weights, const uint16_t* w_gate_up, const uint16_t* w_down,
                       int32_t ntok, const int32_t* tokens, float* out);

/* RANK_MAJOR / FLAT expert stage: z[j] = sum_k masked weight * y(pick) for received rows rows[j]
 * (recv_x [rows, H] bf16, recv routing [rows, K]). */
int orc_recv_rows_z(const orc_params_t* p, const uint16_t* recv_x, const int32_t* recv_topk_idx,
                    const float* recv_topk_weights, const uint16_t* w_gate_up, const uint16_t* w_down,
                    int32_t nrows, const int32_t* rows, float* z);

/* FP8 dispatch format (Mooncake PG/EP guide, "Buffer.dispatch": use_fp8 returns FP8 data plus
 * scales; hidden must be a multiple of 128).  Reading: each row is cut into blocks of 128
 * values; a block with largest magnitude a gets the scale 2^k, k the smallest integer with
 * a <= 448 * 2^k (k = 0 when a = 0; k clamped to [-127, 127]); every value v of the block is
 * stored as the OCP FP8 E4M3 code of v * 2^-k rounded to nearest even (|v * 2^-k| <= 448, so it
 * never saturates).  The scale is kept as the byte k + 127 (E8M0).  Dequantised values
 * e4m3(code) * 2^k are exact in bf16 and fp32 for the ranges used here.
 * orc_e4m3_encode / orc_e4m3_decode: one value.  orc_quantize_rows_fp8: rows [n, cols] of bf16
 * (cols % 128 == 0) -> codes [n, cols] and scale bytes [n, cols / 128]. */
uint8_t orc_e4m3_encode(float v);
float orc_e4m3_decode(uint8_t code);
int orc_quantize_rows_fp8(int64_t n, int32_t cols, const uint16_t* x, uint8_t* codes, uint8_t* scales);

/* Router upstream of dispatch (Mooncake PG/EP guide quick start: topk_idx = the top_k of
 * per-token expert scores, topk_weights a softmax; FlashInfer "MoE-EP implementation & usage"
 * section 4, step 2).  For each token t of scores [N, E] (fp32, no NaN): topk_ids[t] = the K
 * experts with the largest scores, largest first, equal scores ordered by the lower expert id;
 * topk_weights[t,k] = exp(s_k - s_0) / sum_j exp(s_j - s_0) over the K selected scores,
 * evaluated in double and rounded to float.  Returns ORC_EINVAL for K < 1, K > E or a NaN. */
int orc_router_topk(int32_t N, int32_t E, int32_t K, const float* scores, int64_t* topk_ids, float* topk_weights);

#ifdef __cplusplus
}
#endif
#endif
