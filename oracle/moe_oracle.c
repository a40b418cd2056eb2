/*
 * CPU oracle of the MoE expert-parallel layer, one GPU's share.
 *
 * TEST INFRASTRUCTURE ONLY: called by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path.  Plain
 * single-threaded C written from the definitions; it shares nothing with the
 * GPU library.  Build with -ffp-contract=off so that every fp32 operation is
 * rounded where it is written.
 *
 * Sources (cited by page title and section):
 *  [FI-3] FlashInfer "MoE-EP implementation & usage", section 3 "Algorithm /
 *         layout contracts": the three receive layouts, what compute does
 *         with each, how combine reduces; received topk_idx are LOCAL expert
 *         indices with -1 for non-local picks; the bridge converts local ->
 *         global ids and masks non-local picks to weight 0.
 *  [FI-4] same page, section 4 "Usage walkthrough": w1 [E, 2I, H] and
 *         w2 [E, H, I] per expert; this rank's slice is experts
 *         [offset, offset + num_local_experts); the reference is a dense MoE
 *         where a token's output is the weighted sum over its top-k experts.
 *  [FI-5] same page, section 5 "Correctness status": the two multi-rank bug
 *         classes (local vs global ids; received ids are local).
 *  [MC-D] Mooncake PG/EP guide, "Buffer.dispatch": topk_idx [num_tokens,
 *         top_k] int64 with -1 for masked picks; expert ids must lie in
 *         [0, num_experts); num_experts divisible by the number of ranks;
 *         hidden divisible by 128; the receive buffer is local-expert-major
 *         [num_local_experts, num_ranks * max_tokens_per_rank, hidden] with a
 *         per-expert received count, per-slot source info and per-(expert,
 *         rank) layout ranges.
 *  [MC-C] Mooncake PG/EP guide, "Buffer.combine" and the EP data-flow
 *         paragraph: expert outputs are sent back weighted by the routing
 *         weights and reduced into the original token owner.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

int64_t orc_recv_rows(const orc_params_t* p) {
  const int64_t W = p->num_experts / p->num_local_experts;
  if (p->layout == ORC_EXPERT_MAJOR) return (int64_t)p->num_local_experts * W * p->max_tokens_per_rank;
  if (p->layout == ORC_RANK_MAJOR) return W * p->max_tokens_per_rank;
  return p->num_tokens;
}

/* Geometry rules of [MC-D] and [FI-3]. */
int orc_check_params(const orc_params_t* p) {
  if (!p) return ORC_EINVAL;
  if (p->num_experts < 1 || p->num_local_experts < 1) return ORC_EINVAL;
  if (p->num_experts % p->num_local_experts != 0) return ORC_EINVAL;
  const int32_t W = p->num_experts / p->num_local_experts;
  if (p->rank < 0 || p->rank >= W) return ORC_EINVAL;
  if (p->max_tokens_per_rank < 1 || p->num_tokens < 0) return ORC_EINVAL;
  if ((int64_t)p->num_tokens > (int64_t)W * p->max_tokens_per_rank) return ORC_EINVAL;
  if (p->hidden < 128 || p->hidden % 128 != 0) return ORC_EINVAL;
  if (p->intermediate < 0 || p->top_k < 1) return ORC_EINVAL;
  if (p->layout < ORC_EXPERT_MAJOR || p->layout > ORC_FLAT) return ORC_EINVAL;
  return ORC_OK;
}

/* Pick (t,k) is local iff its global id lies in this GPU's expert range. */
static int local_id(const orc_params_t* p, int64_t id) {
  const int64_t o = (int64_t)p->rank * p->num_local_experts;
  return (id >= o && id < o + p->num_local_experts) ? (int)(id - o) : -1;
}

/* Token t comes from source rank t / T; a rank whose active_ranks entry is 0 is skipped. */
static int source_active(const orc_params_t* p, int32_t t) {
  return p->active_ranks == NULL || p->active_ranks[t / p->max_tokens_per_rank] != 0;
}

/* Local id of pick (t,k), -1 if the pick is not local or its source rank is inactive. */
static int pick_local(const orc_params_t* p, const int64_t* topk_ids, int32_t t, int32_t k) {
  return source_active(p, t) ? local_id(p, topk_ids[(int64_t)t * p->top_k + k]) : -1;
}

/*
 * Dispatch routing.  Slots of a local expert are handed out in (source rank,
 * token, k) order; since token t = r*T + i, that is t ascending then k
 * ascending.  The loops below walk experts in the outer loop and the picks in
 * that order inside, so the n-th pick met for expert el gets slot n.
 */
int orc_route(const orc_params_t* p, const int64_t* topk_ids, const float* topk_weights, const orc_route_t* o) {
  int rc = orc_check_params(p);
  if (rc != ORC_OK) return rc;
  const int32_t E = p->num_experts, L = p->num_local_experts, K = p->top_k, N = p->num_tokens;
  const int32_t T = p->max_tokens_per_rank, W = E / L;
  const int64_t cap = (int64_t)W * T;

  /* ids of active source ranks must be -1 (masked) or a valid global expert [MC-D] */
  for (int32_t t = 0; t < N; ++t)
    for (int32_t k = 0; k < K; ++k)
      if (source_active(p, t) && (topk_ids[(int64_t)t * K + k] < -1 || topk_ids[(int64_t)t * K + k] >= E))
        return ORC_EEXPERT_ID;

  if (p->layout == ORC_EXPERT_MAJOR) {
    for (int64_t q = 0; q < (int64_t)N * K; ++q) o->slot_of[q] = -1;
    for (int64_t s = 0; s < (int64_t)L * cap; ++s) o->src_info[s] = -1;
  }

  for (int32_t el = 0; el < L; ++el) {
    int64_t n = 0;
    for (int32_t t = 0; t < N; ++t) {
      for (int32_t k = 0; k < K; ++k) {
        if (pick_local(p, topk_ids, t, k) != el) continue;
        if (p->layout == ORC_EXPERT_MAJOR) {
          if (n >= cap) return ORC_ECAPACITY; /* only possible with repeated ids in a token */
          o->slot_of[(int64_t)t * K + k] = (int32_t)(el * cap + n);
          o->src_info[el * cap + n] = t;
        }
        ++n;
      }
    }
    o->recv_count[el] = (int32_t)n;
  }
  o->expert_offsets[0] = 0;
  for (int32_t el = 0; el < L; ++el) o->expert_offsets[el + 1] = o->expert_offsets[el] + o->recv_count[el];

  if (p->layout == ORC_EXPERT_MAJOR) {
    /* layout_range[el][r] = (first slot holding a token of source rank r, slots from rank r) */
    for (int32_t el = 0; el < L; ++el) {
      int32_t first = 0;
      for (int32_t r = 0; r < W; ++r) {
        int32_t cnt = 0;
        for (int32_t s = 0; s < o->recv_count[el]; ++s)
          if (o->src_info[el * cap + s] / T == r) ++cnt;
        o->layout_range[((int64_t)el * W + r) * 2 + 0] = first;
        o->layout_range[((int64_t)el * W + r) * 2 + 1] = cnt;
        first += cnt;
      }
    }
    return ORC_OK;
  }

  /* RANK_MAJOR: row (r, i) = token t = r*T + i, all W*T rows exist.
   * FLAT: tokens with at least one local pick, compacted in token order. */
  const int64_t rows = orc_recv_rows(p);
  for (int64_t q = 0; q < rows * K; ++q) {
    o->recv_topk_idx[q] = -1;
    o->recv_topk_weights[q] = 0.0f;
  }
  int32_t j = 0;
  for (int32_t t = 0; t < N; ++t) {
    int has_local = 0;
    for (int32_t k = 0; k < K; ++k) has_local |= pick_local(p, topk_ids, t, k) >= 0;
    if (!has_local) {
      o->row_of_token[t] = -1;
      continue;
    }
    const int32_t row = (p->layout == ORC_RANK_MAJOR) ? t : j;
    o->row_of_token[t] = row;
    if (p->layout == ORC_FLAT) o->recv_src_idx[j] = t;
    ++j;
    for (int32_t k = 0; k < K; ++k) {
      o->recv_topk_idx[(int64_t)row * K + k] = pick_local(p, topk_ids, t, k);
      o->recv_topk_weights[(int64_t)row * K + k] = topk_weights[(int64_t)t * K + k];
    }
  }
  if (p->layout == ORC_FLAT) o->num_recv[0] = j;
  return ORC_OK;
}

/*
 * Compute-side bridge [FI-3], [FI-5]: over the received routing, picks with
 * a local id l >= 0 get the global id l + rank*L and keep their weight;
 * masked picks (-1) get id -1 and weight 0.  The picks are ordered by
 * (expert, row, k) for the per-expert grouped GEMM.
 */
int orc_bridge(const orc_params_t* p, int32_t rows, const int32_t* idx, const float* w, const orc_bridge_t* o) {
  int rc = orc_check_params(p);
  if (rc != ORC_OK) return rc;
  const int32_t L = p->num_local_experts, K = p->top_k, off = p->rank * L;
  for (int64_t q = 0; q < (int64_t)rows * K; ++q) {
    if (idx[q] < -1 || idx[q] >= L) return ORC_EEXPERT_ID;
    o->pick_slot[q] = -1;
    o->topk_gid[q] = idx[q] >= 0 ? idx[q] + off : -1;
    o->topk_wmask[q] = idx[q] >= 0 ? w[q] : 0.0f;
  }
  int32_t pos = 0;
  o->pick_offsets[0] = 0;
  for (int32_t el = 0; el < L; ++el) {
    for (int32_t row = 0; row < rows; ++row)
      for (int32_t k = 0; k < K; ++k)
        if (idx[(int64_t)row * K + k] == el) {
          o->perm[pos] = row * K + k;
          o->pick_slot[(int64_t)row * K + k] = pos;
          ++pos;
        }
    o->pick_offsets[el + 1] = pos;
    o->pick_count[el] = pos - o->pick_offsets[el];
  }
  return ORC_OK;
}

/*
 * fp32 dot product of a[0..n) with bf16 w[0..n): 16 partial sums, partial j
 * taking the terms i = j, j+16, j+32, ... in order, then s0 + s1 + ... + s15
 * left to right.
 */
static float dot_f32_bf16(const float* a, const uint16_t* w, int32_t n) {
  float s[16] = {0};
  int32_t i = 0;
  for (; i + 16 <= n; i += 16)
    for (int32_t j = 0; j < 16; ++j) s[j] += a[i + j] * bf16_to_f32(w[i + j]);
  for (int32_t j = 0; i + j < n; ++j) s[j] += a[i + j] * bf16_to_f32(w[i + j]);
  float total = 0.0f;
  for (int32_t j = 0; j < 16; ++j) total += s[j];
  return total;
}

/* SiLU(g) = g * sigmoid(g) = g / (1 + exp(-g)) */
static float silu(float g) { return g / (1.0f + expf(-g)); }

/*
 * One expert on one row [FI-4]: gate = rows [0, I) of w_gate_up, up = rows
 * [I, 2I); a_n = SiLU(gate_n . x) * (up_n . x); y_m = down_m . a.
 */
void orc_expert_ffn(int32_t H, int32_t I, const uint16_t* x, const uint16_t* w_gate_up, const uint16_t* w_down,
                    float* y, float* a) {
  float* xf = (float*)malloc(sizeof(float) * (size_t)H);
  for (int32_t h = 0; h < H; ++h) xf[h] = bf16_to_f32(x[h]);
  if (!w_gate_up) { /* identity expert */
    memcpy(y, xf, sizeof(float) * (size_t)H);
    free(xf);
    return;
  }
  for (int32_t n = 0; n < I; ++n) {
    const float g = dot_f32_bf16(xf, w_gate_up + (int64_t)n * H, H);
    const float u = dot_f32_bf16(xf, w_gate_up + (int64_t)(I + n) * H, H);
    a[n] = silu(g) * u;
  }
  for (int32_t m = 0; m < H; ++m) y[m] = dot_f32_bf16(a, w_down + (int64_t)m * I, I);
  free(xf);
}

static const uint16_t* expert_w1(const orc_params_t* p, const uint16_t* w_gate_up, int el) {
  return w_gate_up ? w_gate_up + (int64_t)el * 2 * p->intermediate * p->hidden : NULL;
}
static const uint16_t* expert_w2(const orc_params_t* p, const uint16_t* w_down, int el) {
  return w_down ? w_down + (int64_t)el * p->hidden * p->intermediate : NULL;
}

/* Layer output of listed source tokens [FI-4], [MC-C]: weighted sum over local picks, k ascending. */
int orc_forward_tokens(const orc_params_t* p, const uint16_t* x, const int64_t* topk_ids, const float* topk_weights,
                       const uint16_t* w_gate_up, const uint16_t* w_down, int32_t ntok, const int32_t* tokens,
                       float* out) {
  int rc = orc_check_params(p);
  if (rc != ORC_OK) return rc;
  const int32_t H = p->hidden, I = p->intermediate, K = p->top_k;
  float* y = (float*)malloc(sizeof(float) * (size_t)H);
  float* a = (float*)malloc(sizeof(float) * (size_t)(I > 0 ? I : 1));
  for (int32_t j = 0; j < ntok; ++j) {
    const int32_t t = tokens[j];
    float* o = out + (int64_t)j * H;
    for (int32_t h = 0; h < H; ++h) o[h] = 0.0f;
    if (t < 0 || t >= p->num_tokens) {
      rc = ORC_EINVAL;
      break;
    }
    if (!source_active(p, t)) continue; /* skipped source rank: zero output */
    for (int32_t k = 0; k < K; ++k) {
      const int64_t id = topk_ids[(int64_t)t * K + k];
      if (id < -1 || id >= p->num_experts) {
        rc = ORC_EEXPERT_ID;
        break;
      }
      const int el = local_id(p, id);
      if (el < 0) continue;
      orc_expert_ffn(H, I, x + (int64_t)t * H, expert_w1(p, w_gate_up, el), expert_w2(p, w_down, el), y, a);
      const float wk = topk_weights[(int64_t)t * K + k];
      for (int32_t h = 0; h < H; ++h) o[h] += wk * y[h];
    }
    if (rc != ORC_OK) break;
  }
  free(y);
  free(a);
  return rc;
}

/* RANK_MAJOR / FLAT expert stage [FI-3]: real top_k over the received routing, masked picks weigh 0. */
int orc_recv_rows_z(const orc_params_t* p, const uint16_t* recv_x, const int32_t* idx, const float* w,
                    const uint16_t* w_gate_up, const uint16_t* w_down, int32_t nrows, const int32_t* rows,
                    float* z) {
  int rc = orc_check_params(p);
  if (rc != ORC_OK) return rc;
  const int32_t H = p->hidden, I = p->intermediate, K = p->top_k, L = p->num_local_experts;
  float* y = (float*)malloc(sizeof(float) * (size_t)H);
  float* a = (float*)malloc(sizeof(float) * (size_t)(I > 0 ? I : 1));
  for (int32_t j = 0; j < nrows; ++j) {
    const int64_t row = rows[j];
    float* o = z + (int64_t)j * H;
    for (int32_t h = 0; h < H; ++h) o[h] = 0.0f;
    for (int32_t k = 0; k < K; ++k) {
      const int32_t el = idx[row * K + k];
      if (el < -1 || el >= L) {
        rc = ORC_EEXPERT_ID;
        break;
      }
      if (el < 0) continue; /* masked pick: weight 0 */
      orc_expert_ffn(H, I, recv_x + row * H, expert_w1(p, w_gate_up, el), expert_w2(p, w_down, el), y, a);
      const float wk = w[row * K + k];
      for (int32_t h = 0; h < H; ++h) o[h] += wk * y[h];
    }
    if (rc != ORC_OK) break;
  }
  free(y);
  free(a);
  return rc;
}

/* Router: repeated selection of the best remaining expert, "best" meaning the larger score or,
 * for equal scores, the lower id; then the softmax of the selected scores in double. */
int orc_router_topk(int32_t N, int32_t E, int32_t K, const float* scores, int64_t* topk_ids, float* topk_weights) {
  if (N < 0 || E < 1 || K < 1 || K > E) return ORC_EINVAL;
  for (int64_t q = 0; q < (int64_t)N * E; ++q)
    if (scores[q] != scores[q]) return ORC_EINVAL;
  char* taken = (char*)malloc((size_t)E);
  double* e = (double*)malloc(sizeof(double) * (size_t)K);
  for (int32_t t = 0; t < N; ++t) {
    const float* s = scores + (int64_t)t * E;
    for (int32_t j = 0; j < E; ++j) taken[j] = 0;
    for (int32_t k = 0; k < K; ++k) {
      int32_t best = -1;
      for (int32_t j = 0; j < E; ++j) {
        if (taken[j]) continue;
        if (best < 0 || s[j] > s[best]) best = j; /* ascending j: an equal score keeps the lower id */
      }
      taken[best] = 1;
      topk_ids[(int64_t)t * K + k] = best;
    }
    const double m = s[topk_ids[(int64_t)t * K]];
    double den = 0.0;
    for (int32_t k = 0; k < K; ++k) {
      e[k] = exp((double)s[topk_ids[(int64_t)t * K + k]] - m);
      den += e[k];
    }
    for (int32_t k = 0; k < K; ++k) topk_weights[(int64_t)t * K + k] = (float)(e[k] / den);
  }
  free(taken);
  free(e);
  return ORC_OK;
}

/* OCP FP8 E4M3 ("fn" variant): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent
 * field 0 holds the subnormals m * 2^-9; the largest finite value is 1.75 * 2^8 = 448; code
 * S.1111.111 is NaN and there is no infinity.  Encoding rounds to nearest, ties to even. */
static double round_half_even(double v) {
  const double f = floor(v), d = v - f;
  if (d > 0.5) return f + 1.0;
  if (d < 0.5) return f;
  return fmod(f, 2.0) == 0.0 ? f : f + 1.0;
}

uint8_t orc_e4m3_encode(float v) {
  const uint8_t sign = signbit(v) ? 0x80 : 0x00;
  const double a = fabs((double)v);
  if (a < ldexp(1.0, -6)) {                 /* subnormal range: steps of 2^-9 */
    const int m = (int)round_half_even(a / ldexp(1.0, -9));
    return (uint8_t)(sign | m);             /* m == 8 is the smallest normal, code 0x08 */
  }
  int e;
  frexp(a, &e);                             /* a = f * 2^e, f in [0.5, 1) */
  e -= 1;                                   /* a in [2^e, 2^(e+1)) */
  int m = (int)round_half_even((a / ldexp(1.0, e) - 1.0) * 8.0);
  if (m == 8) {
    m = 0;
    e += 1;
  }
  return (uint8_t)(sign | ((e + 7) << 3) | m);
}

float orc_e4m3_decode(uint8_t code) {
  const int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  const double mag = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return (float)(s ? -mag : mag);
}

static float bf16_to_float(uint16_t b) {
  union {
    uint32_t u;
    float f;
  } c;
  c.u = (uint32_t)b << 16;
  return c.f;
}

/* smallest k with a <= 448 * 2^k, by direct comparison with the exact value 448 * 2^k */
static int block_scale_exp(double a) {
  if (a == 0.0) return 0;
  int k = -127;
  while (k < 127 && a > ldexp(448.0, k)) ++k;
  return k;
}

int orc_quantize_rows_fp8(int64_t n, int32_t cols, const uint16_t* x, uint8_t* codes, uint8_t* scales) {
  if (n < 0 || cols <= 0 || cols % 128 != 0) return ORC_EINVAL;
  for (int64_t r = 0; r < n; ++r) {
    for (int32_t b = 0; b < cols / 128; ++b) {
      const uint16_t* blk = x + r * cols + (int64_t)b * 128;
      double amax = 0.0;
      for (int i = 0; i < 128; ++i) amax = fmax(amax, fabs((double)bf16_to_float(blk[i])));
      const int k = block_scale_exp(amax);
      scales[r * (cols / 128) + b] = (uint8_t)(k + 127);
      for (int i = 0; i < 128; ++i)
        codes[r * cols + (int64_t)b * 128 + i] = orc_e4m3_encode((float)ldexp((double)bf16_to_float(blk[i]), -k));
    }
  }
  return ORC_OK;
}
