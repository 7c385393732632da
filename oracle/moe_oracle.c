/*
 * CPU oracle for MoE token dispatch and combine. TEST INFRASTRUCTURE ONLY:
 * see moe_oracle.h for who may call it, the pages it follows and the shapes.
 * Plain loops in token order, single-threaded, no blocking or reordering.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static int id_is_expert(int32_t e, int32_t E) { return e >= 0 && e < E; }

/* Widen a bf16 bit pattern to float: the 16 bits are the top half of a float. */
static float widen_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Round a float to bf16, to nearest, ties to even; NaN stays NaN (quiet bit set). */
static uint16_t narrow_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  const uint32_t lower = u & 0xFFFFu;
  uint32_t upper = u >> 16;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
  return (uint16_t)upper;
}

int oracle_layout(int32_t T, int32_t E, int32_t R, int32_t k, int32_t align, int32_t block,
                  const int32_t* topk_ids, int32_t* rank_counts, int32_t* rank_offsets,
                  int32_t* expert_counts, int32_t* expert_offsets, int32_t* token_rank_slot,
                  int32_t* pair_row) {
  const int32_t m = E / R; /* experts per rank; expert e is on rank e / m */
  int err = 0;
  unsigned char* on_rank = (unsigned char*)malloc((size_t)R);
  int32_t* next_rank = (int32_t*)malloc(sizeof(int32_t) * (size_t)R);
  int32_t* next_expert = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);

  /* Counts: a token adds one row to every distinct rank among its experts,
   * and one pair to the expert of every valid slot. */
  for (int32_t r = 0; r < R; ++r) rank_counts[r] = 0;
  for (int32_t e = 0; e < E; ++e) expert_counts[e] = 0;
  for (int32_t t = 0; t < T; ++t) {
    memset(on_rank, 0, (size_t)R);
    for (int32_t j = 0; j < k; ++j) {
      const int32_t e = topk_ids[(int64_t)t * k + j];
      if (!id_is_expert(e, E)) {
        if (e != -1) err |= ORACLE_ERR_BAD_ID;
        continue;
      }
      expert_counts[e] += 1;
      on_rank[e / m] = 1;
    }
    for (int32_t r = 0; r < R; ++r) rank_counts[r] += on_rank[r];
  }

  /* Exclusive prefix sums: where each rank's segment and each expert's run begins. */
  rank_offsets[0] = 0;
  for (int32_t r = 0; r < R; ++r) rank_offsets[r + 1] = rank_offsets[r] + rank_counts[r];
  expert_offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) {
    if (block > 0) {
      /* masked: a fixed block of rows per expert */
      expert_offsets[e + 1] = (e + 1) * block;
    } else {
      /* contiguous: the expert's run, padded up to a multiple of align rows */
      const int32_t run = (expert_counts[e] + align - 1) / align * align;
      expert_offsets[e + 1] = expert_offsets[e] + run;
    }
  }

  /* Positions: walk the tokens in order and hand out the next free row of the
   * segment (rank) or run (expert), so rows ascend with the token index. */
  for (int32_t r = 0; r < R; ++r) next_rank[r] = rank_offsets[r];
  for (int32_t e = 0; e < E; ++e) next_expert[e] = expert_offsets[e];
  for (int32_t t = 0; t < T; ++t) {
    memset(on_rank, 0, (size_t)R);
    for (int32_t j = 0; j < k; ++j) {
      const int32_t e = topk_ids[(int64_t)t * k + j];
      if (!id_is_expert(e, E)) {
        pair_row[(int64_t)t * k + j] = -1;
        continue;
      }
      const int32_t row = next_expert[e]++;
      if (block > 0 && row >= (e + 1) * block) {
        /* masked: the expert's block is full; the pair is dropped */
        pair_row[(int64_t)t * k + j] = -1;
        err |= ORACLE_ERR_EXPERT_CAP;
      } else {
        pair_row[(int64_t)t * k + j] = row;
      }
      on_rank[e / m] = 1;
    }
    for (int32_t r = 0; r < R; ++r)
      token_rank_slot[(int64_t)t * R + r] = on_rank[r] ? next_rank[r]++ : -1;
  }

  free(on_rank);
  free(next_rank);
  free(next_expert);
  return err;
}

int oracle_pack(int32_t T, int32_t H, int32_t R, const uint16_t* hidden,
                const int32_t* token_rank_slot, uint16_t* rank_buf, int32_t* rank_src_token,
                int64_t cap_rank) {
  int err = 0;
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t r = 0; r < R; ++r) {
      const int64_t row = token_rank_slot[(int64_t)t * R + r];
      if (row < 0) continue;
      if (row >= cap_rank) {
        err |= ORACLE_ERR_RANK_CAP;
        continue;
      }
      memcpy(rank_buf + row * H, hidden + (int64_t)t * H, sizeof(uint16_t) * (size_t)H);
      rank_src_token[row] = t;
    }
  }
  return err;
}

int oracle_permute(int32_t T, int32_t H, int32_t E, int32_t R, int32_t k, int32_t block,
                   const uint16_t* rank_buf, const int32_t* rank_src_token,
                   const int32_t* rank_offsets, const int32_t* topk_ids,
                   const int32_t* pair_row, const int32_t* expert_counts,
                   const int32_t* expert_offsets, int64_t cap_rank, uint16_t* expert_buf,
                   int32_t* expert_src_pair, int64_t cap_expert) {
  (void)T;
  const int32_t m = E / R;
  int err = 0;
  int64_t rows = rank_offsets[R];
  if (rows > cap_rank) rows = cap_rank;
  int32_t r = 0;
  for (int64_t i = 0; i < rows; ++i) {
    while (i >= rank_offsets[r + 1]) ++r; /* the segment that holds row i */
    const int32_t t = rank_src_token[i];
    for (int32_t j = 0; j < k; ++j) {
      const int32_t e = topk_ids[(int64_t)t * k + j];
      if (!id_is_expert(e, E) || e / m != r) continue;
      const int64_t dst = pair_row[(int64_t)t * k + j];
      if (dst < 0 || dst >= cap_expert) { /* dropped by the layout (full block) or past the cap */
        err |= ORACLE_ERR_EXPERT_CAP;
        continue;
      }
      memcpy(expert_buf + dst * H, rank_buf + i * H, sizeof(uint16_t) * (size_t)H);
      expert_src_pair[dst] = t * k + j;
    }
  }
  /* Rows of an expert's run or block that no pair fills (padding) are marked
   * -1 in expert_src_pair; their row data is left as it was. */
  for (int32_t e = 0; e < E; ++e) {
    int64_t used = expert_counts[e];
    if (block > 0 && used > block) used = block;
    const int64_t end = block > 0 ? (int64_t)(e + 1) * block : expert_offsets[e + 1];
    for (int64_t row = expert_offsets[e] + used; row < end && row < cap_expert; ++row)
      expert_src_pair[row] = -1;
  }
  return err;
}

int oracle_combine(int32_t T, int32_t H, int32_t k, const uint16_t* expert_out,
                   const int32_t* pair_row, const float* topk_weights, int64_t cap_expert,
                   uint16_t* out, float* out_f32) {
  int err = 0;
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t h = 0; h < H; ++h) {
      float acc = 0.0f;
      for (int32_t j = 0; j < k; ++j) {
        const int64_t row = pair_row[(int64_t)t * k + j];
        if (row < 0) continue;
        if (row >= cap_expert) {
          err |= ORACLE_ERR_EXPERT_CAP;
          continue;
        }
        acc = fmaf(topk_weights[(int64_t)t * k + j], widen_bf16(expert_out[row * H + h]), acc);
      }
      out[(int64_t)t * H + h] = narrow_bf16_rne(acc);
      if (out_f32) out_f32[(int64_t)t * H + h] = acc;
    }
  }
  return err;
}

int oracle_combine_f64(int32_t T, int32_t H, int32_t k, const uint16_t* expert_out,
                       const int32_t* pair_row, const float* topk_weights, int64_t cap_expert,
                       double* out_f64) {
  int err = 0;
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t h = 0; h < H; ++h) {
      double acc = 0.0;
      for (int32_t j = 0; j < k; ++j) {
        const int64_t row = pair_row[(int64_t)t * k + j];
        if (row < 0) continue;
        if (row >= cap_expert) {
          err |= ORACLE_ERR_EXPERT_CAP;
          continue;
        }
        acc += (double)topk_weights[(int64_t)t * k + j] * (double)widen_bf16(expert_out[row * H + h]);
      }
      out_f64[(int64_t)t * H + h] = acc;
    }
  }
  return err;
}

int oracle_combine_rank_partial(int32_t T, int32_t H, int32_t E, int32_t R, int32_t k,
                                const uint16_t* expert_out, int64_t cap_expert,
                                const int32_t* rank_src_token, const int32_t* rank_offsets,
                                const int32_t* topk_ids, const int32_t* pair_row,
                                const float* topk_weights, int64_t cap_rank, uint16_t* partial,
                                float* partial_f32) {
  (void)T;
  const int32_t m = E / R;
  int err = 0;
  for (int32_t r = 0; r < R; ++r) {
    /* the rows of rank r's segment that fit in the buffer */
    int64_t lo = rank_offsets[r], hi = rank_offsets[r + 1];
    if (hi > cap_rank) hi = cap_rank;
    for (int64_t i = lo; i < hi; ++i) {
      const int32_t t = rank_src_token[i];
      for (int32_t h = 0; h < H; ++h) {
        float acc = 0.0f;
        for (int32_t j = 0; j < k; ++j) {
          const int32_t e = topk_ids[(int64_t)t * k + j];
          if (!id_is_expert(e, E) || e / m != r) continue; /* not an expert of rank r */
          const int64_t row = pair_row[(int64_t)t * k + j];
          if (row < 0) continue;
          if (row >= cap_expert) {
            err |= ORACLE_ERR_EXPERT_CAP;
            continue;
          }
          acc = fmaf(topk_weights[(int64_t)t * k + j], widen_bf16(expert_out[row * H + h]), acc);
        }
        partial[i * H + h] = narrow_bf16_rne(acc);
        if (partial_f32) partial_f32[i * H + h] = acc;
      }
    }
  }
  return err;
}

int oracle_combine_ranks(int32_t T, int32_t H, int32_t R, const uint16_t* partial,
                         int64_t cap_rank, const int32_t* token_rank_slot, uint16_t* out,
                         float* out_f32) {
  int err = 0;
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t h = 0; h < H; ++h) {
      float acc = 0.0f;
      for (int32_t r = 0; r < R; ++r) {
        const int64_t s = token_rank_slot[(int64_t)t * R + r];
        if (s < 0) continue; /* no copy of t on rank r */
        if (s >= cap_rank) {
          err |= ORACLE_ERR_RANK_CAP;
          continue;
        }
        acc = acc + widen_bf16(partial[s * H + h]);
      }
      out[(int64_t)t * H + h] = narrow_bf16_rne(acc);
      if (out_f32) out_f32[(int64_t)t * H + h] = acc;
    }
  }
  return err;
}

/* The value of a finite OCP FP8 E4M3 code (sign ignored): exponent bias 7,
 * three mantissa bits, subnormals at exponent field 0. */
static double e4m3_magnitude(int code) {
  const int ef = (code >> 3) & 0xF, mf = code & 7;
  if (ef == 0) return ldexp((double)mf, -9); /* mf/8 * 2^-6 */
  return ldexp(1.0 + mf / 8.0, ef - 7);
}

void oracle_quantize_mxfp8(int64_t rows, int32_t H, const uint16_t* x, uint8_t* q,
                           uint8_t* scale) {
  const int32_t nblk = H / 32;
  for (int64_t r = 0; r < rows; ++r) {
    for (int32_t b = 0; b < nblk; ++b) {
      const uint16_t* v = x + r * H + (int64_t)b * 32;
      uint8_t* out = q + r * H + (int64_t)b * 32;
      double amax = 0.0;
      int special = 0;
      for (int i = 0; i < 32; ++i) {
        const double a = fabs((double)widen_bf16(v[i]));
        if (!isfinite(a)) special = 1;
        else if (a > amax) amax = a;
      }
      if (special) {
        scale[r * nblk + b] = 0xFF;
        for (int i = 0; i < 32; ++i) out[i] = (uint8_t)(((v[i] >> 15) << 7) | 0x7F);
        continue;
      }
      int e = -127;
      if (amax > 0.0) {
        int ex;
        frexp(amax, &ex); /* amax = m * 2^ex with m in [0.5, 1): floor(log2(amax)) = ex - 1 */
        e = ex - 1 - 8;
        if (e < -127) e = -127;
        if (e > 127) e = 127;
      }
      scale[r * nblk + b] = (uint8_t)(e + 127);
      for (int i = 0; i < 32; ++i) {
        const double val = (double)widen_bf16(v[i]);
        const double mag = fabs(ldexp(val, -e)); /* exact: a power-of-two scaling */
        /* nearest of the 127 finite non-negative codes; on a tie, the even code */
        int best = 0;
        double best_d = fabs(mag - e4m3_magnitude(0));
        for (int c = 1; c <= 0x7E; ++c) {
          const double d = fabs(mag - e4m3_magnitude(c));
          if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_d = d;
          }
        }
        out[i] = (uint8_t)(((v[i] >> 15) << 7) | best);
      }
    }
  }
}

/* The value of a non-negative OCP FP4 E2M1 code: exponent bias 1, one
 * mantissa bit, a subnormal at exponent field 0. */
static double e2m1_magnitude(int code) {
  const int ef = (code >> 1) & 3, mf = code & 1;
  if (ef == 0) return 0.5 * mf;
  return ldexp(1.0 + mf / 2.0, ef - 1);
}

void oracle_quantize_mxfp4(int64_t rows, int32_t H, const uint16_t* x, uint8_t* q,
                           uint8_t* scale) {
  const int32_t nblk = H / 32;
  for (int64_t r = 0; r < rows; ++r) {
    for (int32_t b = 0; b < nblk; ++b) {
      const uint16_t* v = x + r * H + (int64_t)b * 32;
      uint8_t* out = q + r * (H / 2) + (int64_t)b * 16;
      double amax = 0.0;
      int special = 0;
      for (int i = 0; i < 32; ++i) {
        const double a = fabs((double)widen_bf16(v[i]));
        if (!isfinite(a)) special = 1;
        else if (a > amax) amax = a;
      }
      int e = -127;
      if (!special && amax > 0.0) {
        int ex;
        frexp(amax, &ex); /* floor(log2(amax)) = ex - 1 */
        e = ex - 1 - 2;
        if (e < -127) e = -127;
        if (e > 127) e = 127;
      }
      scale[r * nblk + b] = special ? 0xFF : (uint8_t)(e + 127);
      for (int i = 0; i < 32; ++i) {
        int code;
        if (special) {
          code = 7;
        } else {
          const double mag = fabs(ldexp((double)widen_bf16(v[i]), -e));
          /* nearest of the 8 non-negative codes; on a tie, the even code */
          int best = 0;
          double best_d = fabs(mag - e2m1_magnitude(0));
          for (int c = 1; c < 8; ++c) {
            const double d = fabs(mag - e2m1_magnitude(c));
            if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
              best = c;
              best_d = d;
            }
          }
          code = best;
        }
        code |= (v[i] >> 15) << 3;
        if (i % 2 == 0)
          out[i / 2] = (uint8_t)code;
        else
          out[i / 2] = (uint8_t)(out[i / 2] | (code << 4));
      }
    }
  }
}

/* The nearest of the finite non-negative codes 0..last of a format (magnitude
 * given by mag_of) to the non-negative value x; on a tie, the even code. At or
 * past the largest magnitude that is the last code (saturation), decided
 * before any distance is taken: far past it the distances to the two largest
 * codes round to the same double. */
static int nearest_code(double x, int last, double (*mag_of)(int)) {
  if (x >= mag_of(last)) return last;
  int best = 0;
  for (int c = 1; c <= last; ++c) {
    const double dc = fabs(x - mag_of(c)), db = fabs(x - mag_of(best));
    if (dc < db || (dc == db && c % 2 == 0)) best = c;
  }
  return best;
}

void oracle_quantize_nvfp4(int64_t rows, int32_t H, const uint16_t* x, uint8_t* q,
                           uint8_t* scale) {
  const int32_t nblk = H / 16;
  for (int64_t r = 0; r < rows; ++r) {
    for (int32_t b = 0; b < nblk; ++b) {
      const uint16_t* v = x + r * H + (int64_t)b * 16;
      uint8_t* out = q + r * (H / 2) + (int64_t)b * 8;
      double amax = 0.0;
      int nonfinite = 0;
      for (int i = 0; i < 16; ++i) {
        const double a = fabs((double)widen_bf16(v[i]));
        if (!isfinite(a)) nonfinite = 1;
        else if (a > amax) amax = a;
      }
      /* the block scale: the E4M3 code nearest to amax / 6 */
      const int sc = nonfinite ? 0x7F : nearest_code(amax / 6.0, 0x7E, e4m3_magnitude);
      const double s = nonfinite ? 0.0 : e4m3_magnitude(sc);
      scale[r * nblk + b] = (uint8_t)sc;
      for (int i = 0; i < 16; ++i) {
        int code = 0;
        if (nonfinite)
          code = 7;
        else if (s > 0.0)
          code = nearest_code(fabs((double)widen_bf16(v[i])) / s, 7, e2m1_magnitude);
        code |= (int)(v[i] >> 15) << 3; /* the sign */
        if ((i & 1) == 0)
          out[i >> 1] = (uint8_t)code;
        else
          out[i >> 1] |= (uint8_t)(code << 4);
      }
    }
  }
}
