/*
 * Seeded synthetic inputs for the MoE expert-parallel layer (dispatch ->
 * grouped SwiGLU GEMM -> combine).  This file draws random numbers and
 * nothing else: it holds none of the layer's arithmetic.  Both the CPU
 * oracle and the GPU library are fed from the arrays it writes.
 *
 * Generator: counter-based SplitMix64.  SplitMix64 (Steele, Lea & Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014) advances a
 * 64-bit state by the golden-ratio increment 0x9E3779B97F4A7C15 and passes
 * it through the mix13 finaliser.  Using the state after (c+1) increments
 * directly as the counter c makes every element independently addressable,
 * so any slice (one GPU's expert weights, one source rank's tokens) can be
 * generated without generating the rest.
 *
 * Workload recipe (FlashInfer "MoE-EP implementation & usage", section 4
 * "Usage walkthrough", steps 1-2; Mooncake EP quick-start on the Mooncake
 * PG/EP guide): weights from seed 2024 with std 1/sqrt(fan_in), each source
 * rank r's tokens and routing from seed 1000+r, topk_ids = top-k of random
 * scores, topk_weights = softmax of N(0,1) logits over the picks.
 */
#include <stdint.h>
#include <math.h>
#include <string.h>
#include <stdlib.h>

#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Stream key for (seed, tag): distinct tensors of one seed never share a stream. */
uint64_t synth_key(uint64_t seed, uint64_t tag) {
  return mix64(mix64(seed + GOLDEN_GAMMA) ^ (tag * 0xD1B54A32D192ED03ULL));
}

/* c-th output of the stream (c >= 0). */
static inline uint64_t draw(uint64_t key, uint64_t c) { return mix64(key + (c + 1) * GOLDEN_GAMMA); }

/* Uniform on [0, 1) with 53 random bits. */
static inline double unif01(uint64_t key, uint64_t c) { return (double)(draw(key, c) >> 11) * 0x1.0p-53; }
/* Uniform on (0, 1): never 0, never 1. */
static inline double unif_open(uint64_t key, uint64_t c) {
  return ((double)(draw(key, c) >> 11) + 0.5) * 0x1.0p-53;
}

/* Standard normal for element i: Box-Muller on draws 2i and 2i+1 (cosine branch). */
static inline double normal01(uint64_t key, uint64_t i) {
  double u1 = unif01(key, 2 * i), u2 = unif01(key, 2 * i + 1);
  return sqrt(-2.0 * log(1.0 - u1)) * cos(6.283185307179586476925 * u2);
}

/* float -> bf16 bit pattern, round to nearest even (NaN kept quiet). */
static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* out[j] = bf16(std * N(0,1) element (start + j)) of stream (seed, tag). */
void synth_normal_bf16(uint64_t seed, uint64_t tag, uint64_t start, int64_t count, double std_dev,
                       uint16_t* out) {
  const uint64_t key = synth_key(seed, tag);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < count; ++j) out[j] = f32_to_bf16_rne((float)(std_dev * normal01(key, start + (uint64_t)j)));
}

/* out[j] = fp32(std * N(0,1) element (start + j)). */
void synth_normal_f32(uint64_t seed, uint64_t tag, uint64_t start, int64_t count, double std_dev, float* out) {
  const uint64_t key = synth_key(seed, tag);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < count; ++j) out[j] = (float)(std_dev * normal01(key, start + (uint64_t)j));
}

/* Raw 64-bit draws c = start .. start+count-1 of the stream with the given key:
 * the outputs of a SplitMix64 generator whose state starts at `key`. */
void synth_raw_key(uint64_t key, uint64_t start, int64_t count, uint64_t* out) {
  for (int64_t j = 0; j < count; ++j) out[j] = draw(key, start + (uint64_t)j);
}

/* Raw 64-bit draws of stream (seed, tag). */
void synth_raw(uint64_t seed, uint64_t tag, uint64_t start, int64_t count, uint64_t* out) {
  synth_raw_key(synth_key(seed, tag), start, count, out);
}

enum { TAG_X = 1, TAG_SCORE = 2, TAG_LOGIT = 3, TAG_W_GATE_UP = 4, TAG_W_DOWN = 5 };

/*
 * Source tokens: token t = r*T + i belongs to source rank r = t / T and is
 * row i of that rank; its hidden state is N(0,1) from seed (seed_base + r).
 */
void synth_tokens_bf16(uint64_t seed_base, int32_t T, int32_t N, int32_t H, uint16_t* x) {
#pragma omp parallel for schedule(static)
  for (int32_t t = 0; t < N; ++t) {
    const uint64_t key = synth_key(seed_base + (uint64_t)(t / T), TAG_X);
    const uint64_t i = (uint64_t)(t % T);
    for (int32_t h = 0; h < H; ++h) x[(int64_t)t * H + h] = f32_to_bf16_rne((float)normal01(key, i * H + h));
  }
}

/*
 * Routing of the source tokens.  For token i of source rank r (seed
 * seed_base + r), expert e gets the score
 *     uniform routing (zipf_s == 0):  s_e = U_e
 *     Zipf(zipf_s) popularity:         s_e = log p_e + Gumbel_e,  p_e ~ (e+1)^-zipf_s
 * and topk_ids holds the K experts of largest score in descending score order
 * (equal scores: lower expert id first).  Top-K of Gumbel-perturbed log
 * probabilities is a draw of K distinct experts without replacement with
 * probabilities p (Gumbel-top-k); with uniform scores it is the top-k of iid
 * scores of the pages' quick-start.  topk_weights = softmax over the K picks of
 * N(0,1) logits drawn from the same seed, independent of the scores.
 */
void synth_routing(uint64_t seed_base, int32_t T, int32_t N, int32_t E, int32_t K, double zipf_s,
                   int64_t* topk_ids, float* topk_weights) {
  double* logp = (double*)malloc(sizeof(double) * (size_t)E);
  for (int32_t e = 0; e < E; ++e) logp[e] = zipf_s > 0 ? -zipf_s * log((double)(e + 1)) : 0.0;
#pragma omp parallel
  {
    double* score = (double*)malloc(sizeof(double) * (size_t)E);
    int32_t* pick = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
#pragma omp for schedule(static)
    for (int32_t t = 0; t < N; ++t) {
      const uint64_t r = (uint64_t)(t / T), i = (uint64_t)(t % T);
      const uint64_t ks = synth_key(seed_base + r, TAG_SCORE), kl = synth_key(seed_base + r, TAG_LOGIT);
      for (int32_t e = 0; e < E; ++e) {
        const uint64_t c = i * (uint64_t)E + (uint64_t)e;
        score[e] = zipf_s > 0 ? logp[e] - log(-log(unif_open(ks, c))) : unif01(ks, c);
      }
      /* K rounds of arg-max over the experts not picked yet. */
      for (int32_t k = 0; k < K; ++k) {
        int32_t best = -1;
        for (int32_t e = 0; e < E; ++e) {
          int taken = 0;
          for (int32_t q = 0; q < k; ++q) taken |= (pick[q] == e);
          if (taken) continue;
          if (best < 0 || score[e] > score[best]) best = e;
        }
        pick[k] = best;
        topk_ids[(int64_t)t * K + k] = best;
      }
      /* softmax of K N(0,1) logits, in double, stored as fp32 */
      double lg[64], mx = -INFINITY, den = 0.0;
      for (int32_t k = 0; k < K; ++k) {
        lg[k] = normal01(kl, i * (uint64_t)K + (uint64_t)k);
        if (lg[k] > mx) mx = lg[k];
      }
      for (int32_t k = 0; k < K; ++k) den += exp(lg[k] - mx);
      for (int32_t k = 0; k < K; ++k) topk_weights[(int64_t)t * K + k] = (float)(exp(lg[k] - mx) / den);
    }
    free(score);
    free(pick);
  }
  free(logp);
}
