/*
 * moe_dispatch.h — C ABI of libmoe_dispatch.so: MoE token dispatch and combine
 * for one GPU's share of an expert-parallel layer, on AMD Instinct MI355X
 * (gfx950). The R destination ranks are logical segments of one buffer in the
 * GPU's own HBM.
 *
 * Pages cited (title, section):
 *  [A2A]  "A2A backends" page, vincentzed.com/writing/a2a-backends
 *  [GPUs] "How GPUs Talk to Each Other During LLM Inference"
 *  [EP]   "Beyond One GPU: Tensor, Pipeline and Expert Parallelism, and Split
 *         Prefill and Decode"
 *
 * Common conventions
 *  - Every pointer argument except `shape` is a DEVICE pointer (hipMalloc'd or
 *    a torch CUDA tensor). The caller owns every buffer, the layout's small
 *    workspace included; the library allocates nothing, keeps no state between
 *    calls and is re-entrant for calls that do not share output buffers or
 *    workspaces.
 *  - All calls are asynchronous on `stream` (a hipStream_t passed as void*;
 *    NULL = the null stream), never synchronise with the host and launch a
 *    fixed number of kernels whose grids depend only on the shape and caps, so
 *    they can be recorded in a HIP graph ([A2A] sec 1.4: fixed shapes, no CPU
 *    wait for counts; sec 4.2 and 6.2: counts stay on the GPU).
 *  - Return value: MOE_OK, or a negative moe_status_t for errors the host can
 *    see (bad shape, NULL or misaligned pointer, launch failure). On an
 *    argument error no kernel is launched.
 *  - Data-dependent errors are OR-ed by the kernels into `*err_word` (a device
 *    int32 the caller zeroes and reads when it chooses; may be NULL to ignore):
 *    MOE_ERRBIT_BAD_ID, MOE_ERRBIT_RANK_CAP, MOE_ERRBIT_EXPERT_CAP. Offending
 *    rows are dropped, never written out of bounds ([A2A] sec 4.3: a batch
 *    larger than the cap fails).
 *  - Types: expert ids int32; weights float32; hidden states and expert
 *    outputs bf16 (passed as uint16_t bit patterns), row-major, row stride H.
 *  - Ids: -1 means "no expert in this slot" and is skipped ([A2A] sec 2.1,
 *    sec 6.3); any other id outside [0, E) is skipped and flagged. Duplicate
 *    ids of one token each form their own (token, slot) pair and share the
 *    token's single copy on that rank.
 *  - Placement: expert e lives on rank e / (E/R) ([A2A] sec 1.1, 48 of 384
 *    experts per GPU; sec 2.1, the local id range [first_local,
 *    first_local + num_local); [EP] experts placed in order, E/G per GPU).
 *  - Sizes: C = number of (token, rank) copies = rank_offsets[R];
 *    P = rows of the expert-grouped buffer in use = expert_offsets[E] (the
 *    valid (token, slot) pairs, plus padding when align > 1; E*block when
 *    block > 0). Buffers sized for the worst case, cap_rank = T*min(k,R) rows
 *    and cap_expert = T*k + E*(align-1) rows (E*block when block > 0), can
 *    never overflow ([A2A] sec 5.1: worst-case output plus an offsets list).
 *  - Limits: 0 <= T, T*k < 2^30, T*R < 2^31; 1 <= R <= 64; E % R == 0;
 *    1 <= E <= 1024; 1 <= k <= 16; H > 0 and H % 8 == 0; 1 <= align <= 65536;
 *    block >= 0, and align = 1 when block > 0; T*k + E*(align-1) < 2^31 and
 *    T*k + E*block < 2^31; row buffers and topk_ids 16-byte aligned.
 */
#ifndef MOE_DISPATCH_H
#define MOE_DISPATCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_DISPATCH_ABI_VERSION 9

/*
 * The expert-grouped buffer comes in one of three shapes ([A2A] sec 2.2,
 * Figure 4; sec 4.1-4.2):
 *  - contiguous (align = 1, block = 0): expert e's rows are
 *    [expert_offsets[e], expert_offsets[e] + expert_counts[e]);
 *  - contiguous, padded (align > 1, block = 0): every expert's run is padded
 *    up to a multiple of `align` rows (a contiguous grouped GEMM such as
 *    DeepGEMM's wants 128); the padding rows are marked -1 in expert_src_pair;
 *  - masked (block > 0, align = 1): expert e owns the fixed block of rows
 *    [e*block, (e+1)*block) whatever the batch (a masked kernel reads
 *    expert_counts to know how many rows of each block to use); pairs that
 *    find their expert's block full are dropped (pair_row -1,
 *    MOE_ERRBIT_EXPERT_CAP) while expert_counts keeps counting them.
 */
typedef struct moe_shape {
  int32_t T;     /* tokens on this GPU */
  int32_t H;     /* hidden size, bf16 elements per row */
  int32_t E;     /* experts */
  int32_t R;     /* ranks (logical destination GPUs) */
  int32_t k;     /* expert slots per token (top-k) */
  int32_t align; /* expert runs padded to a multiple of align rows (1: no padding) */
  int32_t block; /* 0: contiguous runs; > 0: fixed blocks of `block` rows per expert */
} moe_shape_t;

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_ARG = -1,       /* bad shape, NULL or misaligned pointer */
  MOE_ERR_HIP = -2        /* a kernel launch failed (hipGetLastError) */
} moe_status_t;

#define MOE_ERRBIT_BAD_ID 1         /* an id outside [-1, E) was skipped */
#define MOE_ERRBIT_RANK_CAP 2       /* a copy at or past cap_rank was dropped */
#define MOE_ERRBIT_EXPERT_CAP 4     /* a pair row at or past cap_expert was dropped or ignored */

/* ABI version of the loaded library (MOE_DISPATCH_ABI_VERSION at build time). */
int moe_abi_version(void);

/* Static text for a moe_status_t value. */
const char* moe_status_string(int status);

/*
 * Dispatch, step 1: layout ([A2A] sec 3.2 first step: per token, the set of
 * ranks holding at least one of its experts, and how many rows each rank gets;
 * sec 5.1: counts and offsets stay on the GPU, an offsets list says where each
 * expert's rows begin; sec 1.3: one copy per distinct rank).
 *   topk_ids         [T*k]   in:  router expert ids, row-major [T, k]
 *   rank_counts      [R]     out: copies per rank, #{t : rank r holds an expert of t}
 *   rank_offsets     [R+1]   out: exclusive prefix sum of rank_counts (rank_offsets[R] = C)
 *   expert_counts    [E]     out: valid pairs per expert
 *   expert_offsets   [E+1]   out: first row of each expert's run: the exclusive prefix sum
 *                                 of the run lengths (expert_counts, rounded up to a
 *                                 multiple of align), or e*block (expert_offsets[E] = P)
 *   token_rank_slot  [T*R]   out: row of token t's copy in rank r's segment, or -1;
 *                                 rows of a segment ascend with t
 *   pair_row         [T*k]   out: row of pair (t, j) in the expert-grouped buffer, or -1;
 *                                 rows of an expert's run ascend with (t, j)
 *   workspace        [workspace_bytes] scratch: device memory of at least
 *                    moe_layout_workspace_bytes(shape) bytes, 16-byte aligned (owned by
 *                    the caller; no clearing needed: every call overwrites what it
 *                    reads), or NULL
 *   err_word: device int32 or NULL (MOE_ERRBIT_BAD_ID; MOE_ERRBIT_EXPERT_CAP when a
 *             pair finds its fixed block full)
 * The tokens are cut into at most 64 tiles of a multiple of 256 tokens. With a
 * workspace, more than one tile and more than 49,152 (token, slot) pairs, two
 * kernel launches: per-tile counts into the workspace, then one workgroup per
 * tile scans them and ranks its tile. Otherwise one launch in which every
 * workgroup counts all tokens itself (cheaper for small T, slower for large). Either way the result is a
 * pure function of topk_ids: no order depends on timing. Calls that run at
 * the same time must not share a workspace. A workspace smaller than needed
 * is an argument error.
 */
int moe_dispatch_layout(const moe_shape_t* shape, const int32_t* topk_ids, int32_t* rank_counts,
                        int32_t* rank_offsets, int32_t* expert_counts, int32_t* expert_offsets,
                        int32_t* token_rank_slot, int32_t* pair_row, void* workspace,
                        size_t workspace_bytes, int32_t* err_word, void* stream);

/* Bytes of layout workspace for this shape: 4 * (tiles rounded up to a
 * multiple of 4) * (E + R) when there is more than one tile (at most
 * 64 * 1088 * 4 = 278,528), else 0. 0 for an invalid shape. */
size_t moe_layout_workspace_bytes(const moe_shape_t* shape);

/* Size of the library's static layout workspace (one per GPU): 64 tiles of
 * (1024 + 64) int32 tile counts, the most any accepted shape needs. */
#define MOE_LAYOUT_STATIC_WORKSPACE_BYTES 278528

/*
 * Dispatch, step 1, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It is moe_dispatch_layout with its workspace taken from a static device
 * array inside the library instead of the caller's, and otherwise the same:
 * the same arguments minus the workspace, the same kernels (one or two
 * launches, chosen by size as with a workspace) and the same results.
 *  - The array is MOE_LAYOUT_STATIC_WORKSPACE_BYTES per GPU, enough for every
 *    shape the library accepts; a shape needing more is an argument error.
 *  - The array of the current device is used (the stream's device must be
 *    current). Its address is looked up on the first call on each device; the
 *    array lives until the process ends.
 *  - Every call on one GPU shares that GPU's array: calls that run at the same
 *    time on one GPU (for instance on two streams) race and must not overlap.
 *    Nothing in it needs clearing: a call writes every entry it reads.
 *  - No memory is allocated (no hipMalloc, no allocating library call).
 * Returns MOE_ERR_HIP if the array's address cannot be obtained.
 */
int moe_dispatch_layout_noalloc(const moe_shape_t* shape, const int32_t* topk_ids,
                                int32_t* rank_counts, int32_t* rank_offsets,
                                int32_t* expert_counts, int32_t* expert_offsets,
                                int32_t* token_rank_slot, int32_t* pair_row, int32_t* err_word,
                                void* stream);

/*
 * Dispatch, step 2: pack ([A2A] sec 1.3 third answer and sec 3.2: a token is
 * sent once to each rank in its set, however many of its experts live there).
 * Reads each hidden row once and writes it to every row token_rank_slot[t*R+r]
 * >= 0 of the rank-major buffer; rank_src_token[row] = t.
 *   hidden          [T*H]          in:  bf16
 *   token_rank_slot [T*R]          in:  from moe_dispatch_layout
 *   rank_buf        [cap_rank*H]   out: bf16 rows, segment r = rows
 *                                       [rank_offsets[r], rank_offsets[r+1])
 *   rank_src_token  [cap_rank]     out: source token of each written row
 *   cap_rank: rows available; copies at or past it are dropped (MOE_ERRBIT_RANK_CAP)
 * Rows past C are left untouched.
 */
int moe_dispatch_pack(const moe_shape_t* shape, const uint16_t* hidden,
                      const int32_t* token_rank_slot, uint16_t* rank_buf, int32_t* rank_src_token,
                      int64_t cap_rank, int32_t* err_word, void* stream);

/*
 * Dispatch, step 3: permute by expert on the receiving side ([A2A] sec 3.3:
 * each arrived row is copied once for each of its experts on this rank, into
 * one run of rows per expert; sec 5.1: the copy epilogue with do_expand, one
 * row per (token, local expert), grouped by expert).
 * Every rank-buffer row i < min(rank_offsets[R], cap_rank), in the segment of
 * rank r and holding token t = rank_src_token[i], is read once and written to
 * pair_row[t*k+j] for every slot j of t whose expert lives on rank r;
 * expert_src_pair[that row] = t*k + j. With a padded or blocked layout
 * (align > 1 or block > 0), the rows of each run or block that no pair fills
 * get expert_src_pair -1 (their row data is not written).
 *   rank_buf [cap_rank*H], rank_src_token [cap_rank], rank_offsets [R+1],
 *   topk_ids [T*k], pair_row [T*k]                      in
 *   expert_counts [E], expert_offsets [E+1]             in: from moe_dispatch_layout; read
 *                                                       only when align > 1 or block > 0
 *                                                       (may be NULL otherwise)
 *   expert_buf [cap_expert*H], expert_src_pair [cap_expert]   out
 *   cap_rank: rows of rank_buf; cap_expert: rows of expert_buf (rows at or past
 *   it are dropped, MOE_ERRBIT_EXPERT_CAP; so is a pair the layout dropped).
 *   Rows past P are left untouched.
 */
int moe_permute_by_expert(const moe_shape_t* shape, const uint16_t* rank_buf,
                          const int32_t* rank_src_token, const int32_t* rank_offsets,
                          const int32_t* topk_ids, const int32_t* pair_row,
                          const int32_t* expert_counts, const int32_t* expert_offsets,
                          int64_t cap_rank, uint16_t* expert_buf, int32_t* expert_src_pair,
                          int64_t cap_expert, int32_t* err_word, void* stream);

/*
 * The whole dispatch in one call: moe_dispatch_layout, moe_dispatch_pack and
 * moe_permute_by_expert on the same arguments, with the same results bit for
 * bit and the same error bits. For a decode-sized batch (any align or block)
 * the three run as one kernel launch: up to 256 tokens when k is 1, 2, 4, 6
 * or 8, up to 64 for any other k. There the time is in launches and in each
 * kernel waiting for the one before ([A2A] sec 8.1: a call that does nothing
 * already costs about 10 microseconds; [GPUs] sec 7: DeepEP kept separate
 * low-latency kernels for decoding). In that launch every wave works out the rows of its
 * own token from the ids alone, as a low-latency sender places its rows
 * without asking anyone ([A2A] sec 4.1), so nothing waits for the counts.
 * Otherwise the layout runs as moe_dispatch_layout, then one kernel packs and
 * permutes: each hidden row is read once and written to every copy and to
 * every pair row the permute would write, so the packed rows are not read
 * back (on one GPU nothing lies between the two, [A2A] sec 5.1 do_expand).
 *   Arguments: those of the three calls (hidden, topk_ids, the layout's
 *   outputs, rank_buf / rank_src_token / cap_rank, expert_buf /
 *   expert_src_pair / cap_expert, the layout workspace), with the same
 *   sizes, alignment and NULL rules; all are checked before anything is
 *   launched, and an argument error launches nothing. The one-launch form
 *   needs no workspace. rank_buf holds every copy as after
 *   moe_dispatch_pack (both forms here store the bf16 rows non-temporally,
 *   since nothing reads them back in this call). With padded or blocked
 *   runs the padding rows of expert_src_pair are marked -1 as by the permute.
 */
int moe_dispatch(const moe_shape_t* shape, const uint16_t* hidden, const int32_t* topk_ids,
                 int32_t* rank_counts, int32_t* rank_offsets, int32_t* expert_counts,
                 int32_t* expert_offsets, int32_t* token_rank_slot, int32_t* pair_row,
                 uint16_t* rank_buf, int32_t* rank_src_token, int64_t cap_rank,
                 uint16_t* expert_buf, int32_t* expert_src_pair, int64_t cap_expert,
                 void* workspace, size_t workspace_bytes, int32_t* err_word, void* stream);

/* Wire formats of moe_dispatch_quantised. */
#define MOE_WIRE_MXFP8 1 /* moe_dispatch_pack_mxfp8 / moe_permute_by_expert_mxfp8 */
#define MOE_WIRE_MXFP4 2 /* moe_dispatch_pack_mxfp4 / moe_permute_by_expert_mxfp4 */
#define MOE_WIRE_NVFP4 3 /* moe_dispatch_pack_nvfp4 / moe_permute_by_expert_nvfp4 */

/*
 * The whole quantised dispatch in one call: moe_dispatch_layout, then the
 * quantise-and-pack and the permute of the chosen wire format ([A2A] sec 7.2),
 * on the same arguments, with the same results bit for bit and the same error
 * bits; one kernel launch for a decode-sized batch exactly as moe_dispatch
 * (the wave quantises its part of the row once and writes the codes and
 * scales to every copy and every pair), otherwise the layout and one kernel
 * that quantises each part of a row once and writes its codes and scales to
 * every copy and every pair row, the code rows not read back.
 *   format: MOE_WIRE_MXFP8, MOE_WIRE_MXFP4 or MOE_WIRE_NVFP4 (anything else
 *   is an argument error).
 *   The other arguments: those of the three calls, with their sizes,
 *   alignment and NULL rules (H a multiple of 512); all are checked before
 *   anything is launched.
 */
int moe_dispatch_quantised(const moe_shape_t* shape, int format, const uint16_t* hidden,
                           const int32_t* topk_ids, int32_t* rank_counts, int32_t* rank_offsets,
                           int32_t* expert_counts, int32_t* expert_offsets,
                           int32_t* token_rank_slot, int32_t* pair_row, uint8_t* rank_q,
                           uint8_t* rank_scale, int32_t* rank_src_token, int64_t cap_rank,
                           uint8_t* expert_q, uint8_t* expert_scale, int32_t* expert_src_pair,
                           int64_t cap_expert, void* workspace, size_t workspace_bytes,
                           int32_t* err_word, void* stream);

/*
 * Quantised dispatch, step 2: fused quantise-and-pack to MXFP8 ([A2A] sec 7.2:
 * a token can travel as 8-bit values with a one-byte scale for every 32
 * values, 5,280 bytes for a 5,120-wide row instead of 10,240; the expert kernel
 * takes that format as input). Each hidden row is read once and quantised once;
 * its codes and scales are written to every row token_rank_slot[t*R+r] >= 0.
 * The one-byte scale is read as OCP MX: per block of 32 consecutive values,
 * scale byte = e + 127 with e = floor(log2(max |v|)) - 8 clamped to [-127, 127]
 * (0xFF if the block holds a NaN or an infinity), and each code is the OCP FP8
 * E4M3 value nearest to v / 2^e (ties to the even mantissa, magnitudes past 448
 * saturate to 448, sign kept; NaN codes in a NaN/Inf block).
 *   hidden [T*H] in: bf16; token_rank_slot [T*R] in
 *   rank_q [cap_rank*H] out: e4m3 codes; rank_scale [cap_rank*H/32] out: E8M0 scales
 *   rank_src_token [cap_rank] out; cap_rank as for moe_dispatch_pack
 * Requires H % 512 == 0 (whole 16-byte groups of scales); rank_q and
 * rank_scale 16-byte aligned.
 */
int moe_dispatch_pack_mxfp8(const moe_shape_t* shape, const uint16_t* hidden,
                            const int32_t* token_rank_slot, uint8_t* rank_q,
                            uint8_t* rank_scale, int32_t* rank_src_token, int64_t cap_rank,
                            int32_t* err_word, void* stream);

/*
 * Quantised dispatch, step 3: moe_permute_by_expert for MXFP8 rows. Each
 * rank-buffer row's H codes and H/32 scales move together to the rows
 * pair_row[t*k+j] of its token's experts on that rank, exactly as bf16 rows do
 * (same grouping, padding marks and error handling).
 *   rank_q [cap_rank*H], rank_scale [cap_rank*H/32] in
 *   expert_q [cap_expert*H], expert_scale [cap_expert*H/32] out
 *   other arguments as for moe_permute_by_expert. Requires H % 512 == 0.
 */
int moe_permute_by_expert_mxfp8(const moe_shape_t* shape, const uint8_t* rank_q,
                                const uint8_t* rank_scale, const int32_t* rank_src_token,
                                const int32_t* rank_offsets, const int32_t* topk_ids,
                                const int32_t* pair_row, const int32_t* expert_counts,
                                const int32_t* expert_offsets, int64_t cap_rank,
                                uint8_t* expert_q, uint8_t* expert_scale,
                                int32_t* expert_src_pair, int64_t cap_expert, int32_t* err_word,
                                void* stream);

/*
 * The 4-bit variant of the quantised dispatch ([A2A] sec 7.2 lists a 4-bit row
 * beside the 8-bit one): MXFP4, OCP FP4 E2M1 codes (0, 0.5, 1, 1.5, 2, 3, 4, 6
 * and their negatives) with one E8M0 scale byte per 32 values, e =
 * floor(log2(max |v|)) - 2 clamped to [-127, 127] (0xFF for a block holding a
 * NaN or an infinity, whose codes are then the largest magnitude with the
 * value's sign); codes nearest to v / 2^e, ties to the even code, saturating at
 * 6. Two codes per byte, the even-indexed value in the low nibble.
 *   rank_q [cap_rank*H/2] out: codes; rank_scale [cap_rank*H/32] out: scales
 *   other arguments and requirements as for moe_dispatch_pack_mxfp8.
 */
int moe_dispatch_pack_mxfp4(const moe_shape_t* shape, const uint16_t* hidden,
                            const int32_t* token_rank_slot, uint8_t* rank_q,
                            uint8_t* rank_scale, int32_t* rank_src_token, int64_t cap_rank,
                            int32_t* err_word, void* stream);

/*
 * moe_permute_by_expert for MXFP4 rows: each row's H/2 code bytes and H/32
 * scales move together, as in moe_permute_by_expert_mxfp8.
 *   rank_q [cap_rank*H/2], rank_scale [cap_rank*H/32] in
 *   expert_q [cap_expert*H/2], expert_scale [cap_expert*H/32] out
 */
int moe_permute_by_expert_mxfp4(const moe_shape_t* shape, const uint8_t* rank_q,
                                const uint8_t* rank_scale, const int32_t* rank_src_token,
                                const int32_t* rank_offsets, const int32_t* topk_ids,
                                const int32_t* pair_row, const int32_t* expert_counts,
                                const int32_t* expert_offsets, int64_t cap_rank,
                                uint8_t* expert_q, uint8_t* expert_scale,
                                int32_t* expert_src_pair, int64_t cap_expert, int32_t* err_word,
                                void* stream);

/*
 * The pages' own 4-bit row ([A2A] sec 7.2: 2,880 bytes for a 5,120-wide row,
 * "NVFP4", with a one-byte scale for every 16 values): per block of 16
 * consecutive values the scale byte is the OCP FP8 E4M3 code of s, the E4M3
 * value nearest to max|v| / 6 (ties to the even code, saturating at 448, 0 for
 * small enough blocks; 0x7F, the E4M3 NaN, if the block holds a NaN or an
 * infinity), and each code is the OCP FP4 E2M1 value nearest to |v| / s (ties
 * to the even code, saturating at 6) with the sign of v: 0 with the sign when
 * s = 0, the largest magnitude with the sign in a NaN/Inf block. No second,
 * per-tensor scale: s scales the values themselves. Two codes per byte, the
 * even-indexed value in the low nibble.
 *   rank_q [cap_rank*H/2] out: codes; rank_scale [cap_rank*H/16] out: scales
 *   other arguments and requirements as for moe_dispatch_pack_mxfp8.
 */
int moe_dispatch_pack_nvfp4(const moe_shape_t* shape, const uint16_t* hidden,
                            const int32_t* token_rank_slot, uint8_t* rank_q,
                            uint8_t* rank_scale, int32_t* rank_src_token, int64_t cap_rank,
                            int32_t* err_word, void* stream);

/*
 * moe_permute_by_expert for the 16-value-block 4-bit rows of
 * moe_dispatch_pack_nvfp4: each row's H/2 code bytes and H/16 scales move
 * together, as in moe_permute_by_expert_mxfp8.
 *   rank_q [cap_rank*H/2], rank_scale [cap_rank*H/16] in
 *   expert_q [cap_expert*H/2], expert_scale [cap_expert*H/16] out
 */
int moe_permute_by_expert_nvfp4(const moe_shape_t* shape, const uint8_t* rank_q,
                                const uint8_t* rank_scale, const int32_t* rank_src_token,
                                const int32_t* rank_offsets, const int32_t* topk_ids,
                                const int32_t* pair_row, const int32_t* expert_counts,
                                const int32_t* expert_offsets, int64_t cap_rank,
                                uint8_t* expert_q, uint8_t* expert_scale,
                                int32_t* expert_src_pair, int64_t cap_expert, int32_t* err_word,
                                void* stream);

/*
 * Combine ([A2A] sec 1.1: the MoE output of a token is the sum of its chosen
 * experts' outputs, each multiplied by its weight; sec 7.1: the sum is taken
 * in 32-bit floats; [GPUs] sec 3.3: a fixed addition order makes the result
 * reproducible).
 *   out[t][h] = bf16_rne(acc), acc = +0.0f then, for j = 0..k-1 in order with
 *   row = pair_row[t*k+j] >= 0: acc = fmaf(topk_weights[t*k+j],
 *   float(expert_out[row][h]), acc). Rows at or past cap_expert are skipped
 *   and flagged (MOE_ERRBIT_EXPERT_CAP).
 *   expert_out [cap_expert*H] in: bf16 expert outputs in the expert-grouped order
 *   pair_row [T*k], topk_weights [T*k] in
 *   out [T*H] out: bf16; out_f32 [T*H] out: the float32 sums, or NULL
 */
int moe_combine(const moe_shape_t* shape, const uint16_t* expert_out, const int32_t* pair_row,
                const float* topk_weights, int64_t cap_expert, uint16_t* out, float* out_f32,
                int32_t* err_word, void* stream);

/*
 * Two-stage combine, first stage: per-rank pre-add ([A2A] sec 7.1: a token's
 * weighted sum splits into a sum over the experts that sit on one GPU and a
 * sum over the GPUs; with the layout by expert the first stage runs on the
 * expert's GPU, so one row per GPU travels back instead of one per expert, and
 * what travels back is 16-bit).
 * For every rank-buffer row i < min(rank_offsets[R], cap_rank), in the segment
 * of rank r and holding token t = rank_src_token[i]:
 *   acc = +0.0f, then for j = 0..k-1 in order whose expert lives on rank r and
 *   whose row = pair_row[t*k+j] is in [0, cap_expert):
 *   acc = fmaf(topk_weights[t*k+j], float(expert_out[row][h]), acc);
 *   partial[i][h] = bf16_rne(acc); partial_f32[i][h] = acc.
 *   expert_out [cap_expert*H], rank_src_token [cap_rank], rank_offsets [R+1],
 *   topk_ids [T*k], pair_row [T*k], topk_weights [T*k]       in
 *   partial [cap_rank*H] out: bf16; partial_f32 [cap_rank*H] out: float32, or NULL
 *   Pair rows at or past cap_expert are skipped and flagged (MOE_ERRBIT_EXPERT_CAP).
 *   Rows past C are left untouched.
 */
int moe_combine_rank_partial(const moe_shape_t* shape, const uint16_t* expert_out,
                             const int32_t* rank_src_token, const int32_t* rank_offsets,
                             const int32_t* topk_ids, const int32_t* pair_row,
                             const float* topk_weights, int64_t cap_expert, int64_t cap_rank,
                             uint16_t* partial, float* partial_f32, int32_t* err_word,
                             void* stream);

/*
 * Two-stage combine, second stage at the token's home ([A2A] sec 7.1: the home
 * GPU adds up the one row per GPU that it receives, in 32-bit floats).
 *   out[t][h] = bf16_rne(acc), acc = +0.0f then, for r = 0..R-1 in order with
 *   s = token_rank_slot[t*R+r] in [0, cap_rank): acc = acc + float(partial[s][h]).
 *   partial [cap_rank*H] in: bf16 rows from moe_combine_rank_partial
 *   token_rank_slot [T*R] in: from moe_dispatch_layout
 *   out [T*H] out: bf16; out_f32 [T*H] out: the float32 sums, or NULL
 *   Slots at or past cap_rank are skipped and flagged (MOE_ERRBIT_RANK_CAP).
 * The result differs from moe_combine's by the bf16 rounding of each partial
 * row (relative 2^-8 of that row at most) and the changed addition order.
 */
int moe_combine_ranks(const moe_shape_t* shape, const uint16_t* partial,
                      const int32_t* token_rank_slot, int64_t cap_rank, uint16_t* out,
                      float* out_f32, int32_t* err_word, void* stream);

/*
 * Testing hook (not for production callers; it changes a process-wide setting
 * of this library and returns the previous value): which form of the layout
 * runs when a workspace is given: -1 (default) by size as described at
 * moe_dispatch_layout, 0 every workgroup counts all ids, 1 two launches.
 */
int moe_testing_set_layout_form(int form);

/*
 * Testing hook (not for production callers; process-wide; returns the
 * previous value): how the layout finds the pairs of one expert among the 64
 * pairs a wave ranks at once: 1 (default) through per-wave LDS tables where
 * they fit (8 KiB plus E bytes beside the layout's other LDS, within 64 KiB),
 * else with one wave ballot per bit of the expert id; 0 always with ballots.
 * Both give the same results.
 */
int moe_testing_set_layout_match(int match);

/*
 * Testing hook (not for production callers; process-wide; returns the
 * previous value): 1 (default) moe_dispatch and moe_dispatch_quantised run
 * as described there (one launch, or the layout and one pack-and-permute
 * kernel); 0 they always make the three calls. Both give the same results.
 */
int moe_testing_set_dispatch_fused(int fused);

/*
 * Measurement hook (not for production callers; process-wide, not
 * thread-safe): the next kernel this library launches, on any stream, has the
 * runtime record start_event as it begins and stop_event as it ends, so that
 * hipEventElapsedTime(start_event, stop_event) is that kernel's own duration.
 * The events are the caller's (hipEvent_t as void*, created with timing
 * enabled) and are used once; NULL, NULL disarms. Returns MOE_ERR_ARG if only
 * one of them is NULL. A call that launches two kernels (the two-launch
 * layout) times its first.
 */
int moe_testing_time_next_launch(void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif
#endif
