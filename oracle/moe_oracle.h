/*
 * CPU oracle for MoE token dispatch and combine (one GPU's share of an
 * expert-parallel layer, the R destination ranks being logical buffers).
 *
 * TEST INFRASTRUCTURE ONLY. This is the plain, slow, single-threaded
 * definition that the GPU library is checked against. Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load or call it;
 * the product path never does. It shares no code with the GPU library.
 *
 * Source pages (cited by title and section):
 *  [A2A]  "A2A backends" page, vincentzed.com/writing/a2a-backends
 *  [GPUs] "How GPUs Talk to Each Other During LLM Inference", how-gpus-talk.vercel.app
 *  [EP]   "Beyond One GPU: Tensor, Pipeline and Expert Parallelism, and Split
 *         Prefill and Decode", ishwarj.com
 *
 * Shapes: T tokens, H hidden (bf16 elements), E experts, R ranks, k slots per
 * token. Expert e lives on rank e / (E/R) (contiguous placement: [A2A] sec 1.1
 * gives 48 of 384 experts per GPU, sec 2.1 gives each GPU the id range
 * [first_local, first_local + num_local); [EP] places experts in order, E/G per GPU).
 *
 * Id convention: -1 means "no expert in this slot" and is skipped silently
 * ([A2A] sec 2.1 marks non-local experts with -1; sec 6.3 marks empty slots
 * with an invalid id). Any other id outside [0, E) is skipped and reported
 * with ORACLE_ERR_BAD_ID.
 *
 * Parity status: every function below is pinned by the CPU tests (stable-sort
 * and brute-force equivalence, closed-form copy count, prose examples,
 * identity and one-hot combine, exact-rational error bound, hand-derived
 * rounding and addition-order cases, exact integer sums for the two-stage
 * combine); none is unpinned.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_ERR_BAD_ID 1        /* an id outside [-1, E) was skipped */
#define ORACLE_ERR_RANK_CAP 2      /* a rank-buffer row at or past cap_rank was dropped */
#define ORACLE_ERR_EXPERT_CAP 4    /* an expert row at or past cap_expert was dropped/ignored */

/*
 * Layout ([A2A] sec 3.2 first step; sec 5.1). Counts rows per destination rank
 * (one per token per distinct rank holding one of its experts, [A2A] sec 1.1
 * Figure 1 and sec 1.3 third answer) and pairs per expert, takes exclusive
 * prefix sums, and numbers every (token, rank) copy and every (token, slot)
 * pair in ascending token order inside its segment.
 * The expert-grouped rows come in one of three shapes ([A2A] sec 2.2,
 * Figure 4): contiguous (align = 1, block = 0); contiguous with every expert's
 * run padded to a multiple of `align` rows (the DeepGEMM contiguous kernel
 * wants 128); masked (block > 0): a fixed block of `block` rows per expert,
 * expert e's rows starting at e * block, pairs past a full block dropped
 * (pair_row -1, ORACLE_ERR_EXPERT_CAP) while expert_counts keeps the full
 * count ([A2A] sec 4.1 and 4.2: a region per expert of a fixed cap, the count
 * per expert in a small tensor).
 *   rank_counts[R], rank_offsets[R+1], expert_counts[E], expert_offsets[E+1]
 *   token_rank_slot[T*R]: row of token t in rank r's segment, or -1
 *   pair_row[T*k]: row of pair (t, j) in the expert-grouped buffer, or -1
 * Returns the OR of ORACLE_ERR_* bits.
 */
int oracle_layout(int32_t T, int32_t E, int32_t R, int32_t k, int32_t align, int32_t block,
                  const int32_t* topk_ids, int32_t* rank_counts, int32_t* rank_offsets,
                  int32_t* expert_counts, int32_t* expert_offsets, int32_t* token_rank_slot,
                  int32_t* pair_row);

/*
 * Pack ([A2A] sec 1.3 third answer, sec 3.2 first step): copy token t's hidden
 * row once into every rank segment row token_rank_slot[t*R + r] >= 0, and
 * record the source token of that row. Rows at or past cap_rank are dropped.
 */
int oracle_pack(int32_t T, int32_t H, int32_t R, const uint16_t* hidden,
                const int32_t* token_rank_slot, uint16_t* rank_buf, int32_t* rank_src_token,
                int64_t cap_rank);

/*
 * Permute by expert, on the receiving side ([A2A] sec 3.3 regroup; sec 5.1
 * copy epilogue with do_expand): every rank-buffer row i below
 * min(rank_offsets[R], cap_rank), sitting in the segment of rank r and holding
 * token t = rank_src_token[i], is copied once for each slot j of t whose expert
 * lives on r, to row pair_row[t*k + j]; expert_src_pair of that row is t*k + j.
 * Padding rows (rows of an expert's padded run or block that no pair fills)
 * get expert_src_pair -1; their row data is left as it was.
 */
int oracle_permute(int32_t T, int32_t H, int32_t E, int32_t R, int32_t k, int32_t block,
                   const uint16_t* rank_buf, const int32_t* rank_src_token,
                   const int32_t* rank_offsets, const int32_t* topk_ids,
                   const int32_t* pair_row, const int32_t* expert_counts,
                   const int32_t* expert_offsets, int64_t cap_rank, uint16_t* expert_buf,
                   int32_t* expert_src_pair, int64_t cap_expert);

/*
 * Combine ([A2A] sec 1.1: the MoE output is the sum of the chosen experts'
 * outputs, each multiplied by its weight; sec 7.1: the sum is taken in 32-bit
 * floats; [GPUs] sec 3.3: a fixed addition order gives identical results).
 * acc = +0.0f; for j = 0..k-1 with pair_row[t*k+j] valid:
 *   acc = fmaf(w[t*k+j], float(expert_out[row][h]), acc)
 * out[t][h] = bf16 round-to-nearest-even of acc; out_f32 (if not NULL) = acc.
 */
int oracle_combine(int32_t T, int32_t H, int32_t k, const uint16_t* expert_out,
                   const int32_t* pair_row, const float* topk_weights, int64_t cap_expert,
                   uint16_t* out, float* out_f32);

/* The same weighted sum in double precision (each product of a float weight and
 * a bf16 value is exact in double), used as the reference value of the fp32
 * tolerance check. */
int oracle_combine_f64(int32_t T, int32_t H, int32_t k, const uint16_t* expert_out,
                       const int32_t* pair_row, const float* topk_weights, int64_t cap_expert,
                       double* out_f64);

/*
 * Two-stage combine, first stage ([A2A] sec 7.1: a token's weighted sum splits
 * into a sum over the experts that sit on one GPU and a sum over the GPUs;
 * with the layout by expert the expert's GPU does the first stage, so one row
 * per GPU travels back, and what travels back is 16-bit). For every
 * rank-buffer row i below min(rank_offsets[R], cap_rank), in the segment of
 * rank r and holding token t = rank_src_token[i]:
 *   acc = +0.0f; for j = 0..k-1 whose expert lives on r and whose pair_row is valid:
 *     acc = fmaf(w[t*k+j], float(expert_out[pair_row[t*k+j]][h]), acc)
 *   partial[i][h] = bf16 round-to-nearest-even of acc; partial_f32 (if not NULL) = acc.
 * A pair row at or past cap_expert is skipped and reported (ORACLE_ERR_EXPERT_CAP).
 */
int oracle_combine_rank_partial(int32_t T, int32_t H, int32_t E, int32_t R, int32_t k,
                                const uint16_t* expert_out, int64_t cap_expert,
                                const int32_t* rank_src_token, const int32_t* rank_offsets,
                                const int32_t* topk_ids, const int32_t* pair_row,
                                const float* topk_weights, int64_t cap_rank, uint16_t* partial,
                                float* partial_f32);

/*
 * Two-stage combine, second stage at the token's home ([A2A] sec 7.1: the home
 * GPU adds up the rows it receives, in 32-bit floats), ranks in ascending order:
 *   acc = +0.0f; for r = 0..R-1 with s = token_rank_slot[t*R+r] a row in [0, cap_rank):
 *     acc = acc + float(partial[s][h])
 *   out[t][h] = bf16 round-to-nearest-even of acc; out_f32 (if not NULL) = acc.
 * A slot at or past cap_rank is skipped and reported (ORACLE_ERR_RANK_CAP).
 */
int oracle_combine_ranks(int32_t T, int32_t H, int32_t R, const uint16_t* partial,
                         int64_t cap_rank, const int32_t* token_rank_slot, uint16_t* out,
                         float* out_f32);

/*
 * Quantised wire format for dispatch ([A2A] sec 7.2: a token can be sent as
 * 8-bit values with a one-byte scale factor for every 32 values, 5,280 bytes
 * for a 5,120-wide row instead of 10,240). The byte-per-32 scale is read as
 * the OCP Microscaling (MX) format MXFP8: per block of 32 consecutive values
 * of a row, with amax the largest magnitude in the block,
 *   e     = floor(log2(amax)) - 8  (8 = exponent of the largest e4m3 normal, 448),
 *           clamped to [-127, 127]; amax = 0 gives -127;
 *   scale = e + 127 as one byte (E8M0, the value 2^e); 0xFF if the block holds
 *           a NaN or an infinity;
 *   q_i   = the OCP FP8 E4M3 value nearest to v_i / 2^e (ties to the even
 *           mantissa; magnitudes past 448 saturate to 448; the sign is kept, so
 *           a negative value that rounds to zero gives 0x80); in a NaN/Inf block
 *           every q_i is the e4m3 NaN 0x7F with the value's sign.
 * Rows of x are H bf16 values; q gets H bytes and scale H/32 bytes per row.
 */
void oracle_quantize_mxfp8(int64_t rows, int32_t H, const uint16_t* x, uint8_t* q,
                           uint8_t* scale);

/*
 * The 4-bit variant of the quantised wire format ([A2A] sec 7.2 lists a 4-bit
 * row beside the 8-bit one). Read as OCP MX MXFP4, the 4-bit MX format: per
 * block of 32 consecutive values,
 *   e     = floor(log2(amax)) - 2  (2 = exponent of the largest e2m1 value, 6),
 *           clamped to [-127, 127]; amax = 0 gives -127;
 *   scale = e + 127 as one byte (E8M0); 0xFF if the block holds a NaN or an
 *           infinity;
 *   q_i   = the OCP FP4 E2M1 value nearest to v_i / 2^e (values 0, 0.5, 1,
 *           1.5, 2, 3, 4, 6; ties to the even code, magnitudes past 6 saturate
 *           to 6, sign kept); in a NaN/Inf block every q_i is the largest
 *           magnitude (code 7) with the value's sign.
 * Two codes per byte, the even-indexed value in the low nibble. Rows of x are
 * H bf16 values; q gets H/2 bytes and scale H/32 bytes per row.
 */
void oracle_quantize_mxfp4(int64_t rows, int32_t H, const uint16_t* x, uint8_t* q,
                           uint8_t* scale);

/*
 * The pages' own 4-bit row ([A2A] sec 7.2: NVFP4, 2,880 bytes for a 5,120-wide
 * row, a one-byte scale for every 16 values): per block of 16 consecutive
 * values,
 *   s     = the OCP FP8 E4M3 value nearest to amax / 6 (6 = the largest e2m1
 *           value; ties to the even code, past 448 saturating to 448, small
 *           enough quotients giving 0); the scale byte is its code; 0x7F (the
 *           E4M3 NaN) if the block holds a NaN or an infinity;
 *   q_i   = the OCP FP4 E2M1 value nearest to |v_i| / s (ties to the even code,
 *           past 6 saturating to 6) with the sign of v_i; 0 with the sign when
 *           s = 0; in a NaN/Inf block the largest magnitude (code 7) with the
 *           value's sign.
 * No second, per-tensor scale (the row size the pages give has no room for
 * one): s scales the values themselves. Two codes per byte, the even-indexed
 * value in the low nibble. Rows of x are H bf16 values; q gets H/2 bytes and
 * scale H/16 bytes per row.
 */
void oracle_quantize_nvfp4(int64_t rows, int32_t H, const uint16_t* x, uint8_t* q,
                           uint8_t* scale);

#ifdef __cplusplus
}
#endif
#endif
