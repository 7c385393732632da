/*
 * Seeded synthetic inputs for MoE token dispatch and combine.
 *
 * This file is shared input plumbing: the oracle and the GPU library both
 * consume what it produces, and it contains none of the dispatch or combine
 * arithmetic (no counting, scanning, packing, permuting or weighted sums).
 *
 * Every value is a pure function of (seed, stream, index), built from the
 * splitmix64 finaliser (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014), so results do not depend on thread count
 * or on the order in which values are produced.
 *
 *   h(seed, stream, i) = sm64( sm64( sm64(seed) ^ stream * 0xD1B54A32D192ED03 ) ^ i )
 *   U(i)  = ((h >> 11) + 1) * 2^-53                  uniform on (0, 1]
 *   N(i)  = sqrt(-2 ln U(2i)) * cos(2 pi U(2i+1))    Box-Muller, in double
 *
 * Streams: 0 = hidden states, 1 = router logits, 2 = expert outputs,
 *          3 = permutations (expert popularity order, forced-token choice).
 *
 * Router (input generation, not part of dispatch or combine): per token the
 * logit of expert e is float(N(t*E + e)) + bias[e] (+ force offset); the k
 * largest are taken with ties broken by the lower expert id, in that order;
 * the weights are the softmax over the k chosen logits, computed in double and
 * rounded to float, which equals renormalising the full softmax over the k.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static inline uint64_t sm64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

static inline uint64_t ctr_hash(uint64_t seed, uint64_t stream, uint64_t idx) {
  return sm64(sm64(sm64(seed) ^ (stream * 0xD1B54A32D192ED03ull)) ^ idx);
}

static inline double unit_open0(uint64_t h) {
  return (double)((h >> 11) + 1) * 0x1.0p-53;
}

static inline double normal_at(uint64_t seed, uint64_t stream, uint64_t i) {
  const double u1 = unit_open0(ctr_hash(seed, stream, 2 * i));
  const double u2 = unit_open0(ctr_hash(seed, stream, 2 * i + 1));
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

/* float -> bfloat16 bit pattern, round to nearest even (inputs here are finite). */
static inline uint16_t gen_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

uint64_t synth_hash(uint64_t seed, uint64_t stream, uint64_t idx) {
  return ctr_hash(seed, stream, idx);
}

double synth_normal(uint64_t seed, uint64_t stream, uint64_t idx) {
  return normal_at(seed, stream, idx);
}

/* out[i] = bf16(float(N(base + i))) for i in [0, n). */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t base, int64_t n,
                       uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = gen_bf16((float)normal_at(seed, stream, base + (uint64_t)i));
}

/* out[i] = float(N(base + i)). */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t base, int64_t n,
                      float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = (float)normal_at(seed, stream, base + (uint64_t)i);
}

/* Fisher-Yates shuffle of 0..n-1; step i swaps i with h(seed, stream, salt+i) mod (i+1). */
void synth_permutation(uint64_t seed, uint64_t stream, uint64_t salt, int32_t n,
                       int32_t* perm) {
  for (int32_t i = 0; i < n; ++i) perm[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    const uint64_t j = ctr_hash(seed, stream, salt + (uint64_t)i) % (uint64_t)(i + 1);
    const int32_t tmp = perm[i];
    perm[i] = perm[j];
    perm[j] = tmp;
  }
}

/*
 * Router: ids[T,k] int32, weights[T,k] float.
 * bias: E floats added to every token's logits, or NULL.
 * force: T bytes or NULL; where force[t] != 0, experts e >= force_below get
 *        force_offset added to their logit (force_offset < 0 pushes the picks
 *        onto experts [0, force_below)).
 */
void synth_router(uint64_t seed, int32_t T, int32_t E, int32_t k, const float* bias,
                  const uint8_t* force, int32_t force_below, float force_offset,
                  int32_t* ids, float* weights) {
#pragma omp parallel
  {
    float* logit = (float*)malloc(sizeof(float) * (size_t)E);
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
    double* lsel = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
#pragma omp for schedule(static)
    for (int32_t t = 0; t < T; ++t) {
      for (int32_t e = 0; e < E; ++e) {
        float l = (float)normal_at(seed, 1, (uint64_t)t * (uint64_t)E + (uint64_t)e);
        if (bias) l += bias[e];
        if (force && force[t] && e >= force_below) l += force_offset;
        logit[e] = l;
        taken[e] = 0;
      }
      for (int32_t j = 0; j < k; ++j) {
        int32_t best = -1;
        for (int32_t e = 0; e < E; ++e) {
          if (taken[e]) continue;
          if (best < 0 || logit[e] > logit[best]) best = e; /* '>' keeps the lower id on ties */
        }
        taken[best] = 1;
        ids[(int64_t)t * k + j] = best;
        lsel[j] = (double)logit[best];
      }
      double z = 0.0;
      for (int32_t j = 0; j < k; ++j) z += exp(lsel[j] - lsel[0]);
      for (int32_t j = 0; j < k; ++j)
        weights[(int64_t)t * k + j] = (float)(exp(lsel[j] - lsel[0]) / z);
    }
    free(logit);
    free(taken);
    free(lsel);
  }
}

/*
 * Synthetic expert outputs in (token, slot) order: y[t][j][h] = bf16(N(idx)) with
 * idx = (t*E + e)*H + h and e = ids[t][j], so a value depends on the token, the
 * expert and the column only. Slots with e outside [0, E) are zero-filled.
 */
void synth_expert_out_slots(uint64_t seed, int32_t T, int32_t E, int32_t k, int32_t H,
                            const int32_t* ids, uint16_t* y) {
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < (int64_t)T * k; ++p) {
    const int64_t t = p / k;
    const int32_t e = ids[p];
    uint16_t* row = y + p * (int64_t)H;
    if (e < 0 || e >= E) {
      memset(row, 0, sizeof(uint16_t) * (size_t)H);
      continue;
    }
    const uint64_t base = ((uint64_t)t * (uint64_t)E + (uint64_t)e) * (uint64_t)H;
    for (int32_t h = 0; h < H; ++h) row[h] = gen_bf16((float)normal_at(seed, 2, base + h));
  }
}
