// MoE token dispatch and combine for one GPU's share of an expert-parallel
// layer: HIP kernels for CDNA4 (gfx950, wave64) behind the C ABI declared in
// include/moe_dispatch.h.
//
// Pages cited (title, section):
//  [A2A]  "A2A backends" page, vincentzed.com/writing/a2a-backends
//  [GPUs] "How GPUs Talk to Each Other During LLM Inference"
//
// Kernels
//  layout_tiles  one launch. Every workgroup histograms all tokens (LDS
//                atomics per expert, wavefront ballots per rank; for one
//                tile the ranking waves' own counts), scans the totals into
//                expert and rank offsets, then ranks its own tile of tokens
//                (an LDS match of equal experts) and writes absolute rows
//                ([A2A] sec 3.2 step 1: per-token rank set and per-rank
//                counts; sec 5.1: offsets stay on the GPU, no CPU wait)
//  pack_rows     one wave per token: read the row once, write one copy per
//                distinct rank ([A2A] sec 1.3 third answer); pack_rows_small
//                the same with one wave per 1 KiB of the row, for small
//                batches and for copies larger than the Infinity Cache
//  permute_rows  one wave per rank-buffer row: read once, write once per
//                local expert ([A2A] sec 3.3, sec 5.1 do_expand)
//  combine_rows  one wave per (token, column slice): k row gathers, fp32 FMA
//                in slot order, bf16 round-to-nearest-even ([A2A] sec 1.1,
//                7.1; [GPUs] sec 3.3 fixed addition order)
//  rank_partial_rows / rank_sum_rows  the two-stage combine of [A2A] sec 7.1:
//                one bf16 partial row per (token, rank) copy, then the sum of
//                a token's partial rows at home in rank order
//  dispatch_small  layout, pack and permute of a batch of at most 256 tokens
//                in one launch (moe_dispatch): every wave finds its own
//                token's rows from the ids ([A2A] sec 4.1, sec 8.1)
//  pack_expand_rows  pack and permute in one kernel for moe_dispatch past
//                dispatch_small's sizes, after the layout: one wave per
//                (token, 1 KiB of the row) reads it once and writes it to
//                every copy and every pair row, so the packed rows are not
//                read back (ordinary loads, streamed stores: by measurement)
//  pack_rows_mx  fused quantise-and-pack to the [A2A] sec 7.2 wire formats:
//                MXFP8, MXFP4, and the 4-bit row with an E4M3 scale per 16
//                values; permute_rows moves their codes and scales
// Rows move 16 bytes per lane (global_load/store_dwordx4), 1 KiB per wave
// instruction. Cache policy per stream, chosen by measurement of the whole
// layout -> pack -> permute -> combine sequence: the packed rows are written
// with ordinary stores, so the permute finds them in the 256 MB Infinity
// Cache; the hidden rows are read with ordinary loads (which keeps that
// hand-off working whatever large writes other kernels made before); every
// other row stream (packed rows on their second read, expert rows, combine
// outputs, the rows of the one-call dispatch) is non-temporal so it does not
// evict them.
// Nothing here is a dense contraction, so no MFMA.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "moe_dispatch.h"

// The layout workspace of moe_dispatch_layout_noalloc: a static device array
// (each GPU the library runs on holds its own copy until the process ends).
// Host code never passes `scratch` itself (its host name is only a stand-in);
// it passes the device address hipGetSymbolAddress returns for the current
// device.
static __device__ __align__(256) int32_t scratch[MOE_LAYOUT_STATIC_WORKSPACE_BYTES / 4];

namespace {

typedef uint32_t vec4 __attribute__((ext_vector_type(4)));  // 8 bf16

constexpr int kWave = 64;
constexpr int kBlock = 256;                 // row movers: 4 waves per workgroup
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kMaxTiles = 64;               // layout workgroups per call
constexpr int kMaxExperts = 1024;
constexpr int kMaxRanks = 64;
constexpr int kMaxK = 16;
constexpr int kMaxVec = 16;                 // vec4 per lane held in registers per pass
constexpr int kMaxAlign = 1 << 16;          // largest run padding
constexpr int kMxRowQuantum = 512;          // quantised rows: H a multiple of 512 (whole vec4 of scales)

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanes_below() {
  return (uint64_t(1) << lane_id()) - 1;  // lane 63: 2^63 - 1
}

// The wave's index in its workgroup, through a scalar register: the compiler
// does not know that threadIdx.x / 64 is the same in every lane of a wave,
// and would otherwise keep the row or token a wave works on, and every row
// number, mask and branch derived from it, per lane.
__device__ __forceinline__ int wave_in_block() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

__device__ __forceinline__ int read_lane(int v, int lane) {
  return __builtin_amdgcn_readlane(v, lane);
}

__device__ __forceinline__ void flag_error(int32_t* err_word, int bit) {
  if (err_word) atomicOr(err_word, bit);
}

// Row loads and stores with a cache policy: non-temporal (streaming) or
// ordinary (allocating in L2 and the Infinity Cache).
template <bool kStream>
__device__ __forceinline__ vec4 load_row(const vec4* p) {
  if (kStream) return __builtin_nontemporal_load(p);
  return *p;
}

template <bool kStream>
__device__ __forceinline__ void store_row(vec4* p, vec4 v) {
  if (kStream)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

// ---------------------------------------------------------------------------
// Layout

constexpr int kLayoutWaves = 16;                 // 1024 threads per workgroup
constexpr int kLayoutThreads = kLayoutWaves * kWave;
constexpr int kOwnTokens = 256;                  // tokens ranked per sub-tile
constexpr int kOwnWaves = 8;                     // waves 0..7 rank ...
constexpr int kTokW = kOwnTokens / kOwnWaves;    // ... 32 tokens each
constexpr int kBatchVecs = 8;                    // 16-byte id loads per lane per batch
constexpr size_t kLayoutLdsLimit = 64 * 1024 - 256;  // dynamic LDS without a launch attribute

// Which form of the layout runs when a workspace is given: -1 by size (the
// default), 0 every workgroup counts all ids, 1 two launches through tile
// counts. Changed only by the testing hook.
int g_layout_form = -1;
// 0: the layout matches equal experts with ballots even where the LDS tables
// fit. Changed only by the testing hook.
int g_layout_match = 1;
// 0: moe_dispatch always makes the three calls, also where one launch would
// do. Changed only by the testing hook.
int g_dispatch_fused = 1;

// Events armed by moe_testing_time_next_launch for the next kernel launch.
hipEvent_t g_time_start = nullptr;
hipEvent_t g_time_stop = nullptr;

// Every kernel launch of the library: a plain launch, or, once after
// moe_testing_time_next_launch, a launch that has the runtime record the armed
// events as the kernel begins and ends (so the pair brackets that kernel
// alone, without the gap a separately recorded event leaves before it).
#define MOE_LAUNCH(kernel, grid, block, shmem, stream, ...)                               \
  do {                                                                                    \
    if (g_time_start) {                                                                   \
      const hipEvent_t start_ = g_time_start, stop_ = g_time_stop;                        \
      g_time_start = g_time_stop = nullptr;                                               \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, start_, stop_, 0,         \
                            __VA_ARGS__);                                                 \
    } else {                                                                              \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                \
    }                                                                                     \
  } while (0)

struct LayoutGeom {
  int T, E, R, k, m;    // m = experts per rank
  int align, block;     // expert runs padded to multiples of align; or fixed blocks (block > 0)
  int ncols;            // E expert columns followed by R rank columns
  int tile_tokens;      // tokens ranked per workgroup (multiple of kOwnTokens)
  int ntiles;
  int tiles_pad;        // ntiles rounded up to a multiple of 4 (tile-count column stride)
  int lds_match;        // 1: equal experts of a chunk are matched through LDS tables
  int e_pad;            // E rounded up to a multiple of 4 (byte-table stride)
  float inv_m;          // 1/m rounded to float
};

// rank(e) = e / m, as floor(fl(e * c + c/2)) with c = fl(1/m) and one fused
// multiply-add: the result lies within 2^-13 of (e + 1/2)/m for e < 2^10 and
// m <= 2^10, which is at least 1/(2m) >= 2^-11 away from the integers around
// it, so the truncation is exact. (Full-rate instructions, unlike the
// quarter-rate 32-bit integer multiply-high.)
__device__ __forceinline__ int rank_of(int e, float inv_m) {
  return int(__builtin_fmaf(float(e), inv_m, 0.5f * inv_m));
}

// Inclusive prefix sum across a wave with DPP row shifts and broadcasts.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Rank sets of a token as bit masks. kRB is a compile-time bound on R (8, 32
// or 64): one 32-bit word up to 32 ranks, two above; with kRB = 8 the loops
// over ranks are unrolled.
template <int kRB>
struct RankSet {
  static constexpr int NW = kRB > 32 ? 2 : 1;  // 32-bit words
  uint32_t w[NW];
  __device__ __forceinline__ RankSet() {
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] = 0;
  }
  // Adds rank r (< kRB) when `on`.
  __device__ __forceinline__ void add(int r, bool on) {
    const uint32_t bit = uint32_t(on) << (r & 31);
    if (NW == 1) {
      w[0] |= bit;
    } else {
      w[0] |= r < 32 ? bit : 0u;
      w[NW - 1] |= r >= 32 ? bit : 0u;
    }
  }
  __device__ __forceinline__ bool has(int r) const {
    return (((NW == 1 || r < 32) ? w[0] : w[NW - 1]) >> (r & 31)) & 1;
  }
};

// Copies per rank over the wave's 64 tokens (one rank set of at most 8 ranks
// per lane), in lane r: one ballot per rank.
__device__ __forceinline__ int wave_rank_counts8(uint32_t mask) {
  int mine = 0;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int c = __popcll(__ballot((mask >> r) & 1));
    mine = lane_id() == r ? c : mine;
  }
  return mine;
}

// Adds one to counts[r] for every rank r in the lane's rank set (LDS
// atomics). Used for more than 8 ranks, where a ballot per rank and a
// per-lane pick of the counts gave wrong copies per rank on MI355X in one
// form of the layout (64-bit rank sets, k = 4, the tile ranked before the
// counting pass) for reasons not found in the generated code; a later form
// with 64-bit masks and these atomics failed the same way after an unrelated
// change, so rank sets are kept in 32-bit words throughout.
template <int kRB>
__device__ __forceinline__ void count_rank_set(int32_t* counts, RankSet<kRB> set) {
#pragma unroll
  for (int i = 0; i < RankSet<kRB>::NW; ++i) {
    uint32_t m = set.w[i];
    while (m) {
      const int r = __ffs(m) - 1;
      m &= m - 1;
      atomicAdd(&counts[32 * i + r], 1);
    }
  }
}

// Sum over the ranking waves of their counts in column c (0 without them).
__device__ __forceinline__ int own_sum(const int32_t* s_own, int ncols, int c) {
  if (!s_own) return 0;
  int v[kOwnWaves];  // all reads first: one LDS round trip
#pragma unroll
  for (int w = 0; w < kOwnWaves; ++w) v[w] = s_own[w * ncols + c];
  int sum = 0;
#pragma unroll
  for (int w = 0; w < kOwnWaves; ++w) sum += v[w];
  return sum;
}

// Column totals, exclusive scans and the tile's first rows, in one pass: for
// every column c, count = s_tot[c] + s_pre[c] (tokens from the tile on, and
// before it) + the ranking waves' counts s_own[w][c] when given (then the
// tile's tokens were not counted into s_tot), offset = exclusive prefix of the run lengths (experts in id
// order over waves 0..7, ranks in rank order in wave 8), and s_pre[c] becomes
// offset + (count before the tile), the tile's first row in that column. An
// expert's run length is its count, rounded up to a multiple of `align`, or
// the fixed `block` when block > 0. The workgroup that is `writer` also
// stores the counts and offsets.
__device__ void scan_columns(int32_t* s_pre, const int32_t* s_tot, const int32_t* s_own,
                             int ncols, int E, int R, int align, int block,
                             int32_t* s_tmp /* [16] */, bool writer,
                             int32_t* expert_counts, int32_t* expert_offsets,
                             int32_t* rank_counts, int32_t* rank_offsets) {
  const int tid = threadIdx.x;
  const int wave = wave_in_block();
  const int lane = lane_id();
  constexpr int kScanThreads = 8 * kWave;
  constexpr int kPer = (kMaxExperts + kScanThreads - 1) / kScanThreads;
  const int per = (E + kScanThreads - 1) / kScanThreads;  // <= kPer
  int lo = 0, sum = 0, x = 0;
  int run_len[kPer];  // rows of the expert's run: its count, padded, or the fixed block
  if (wave < 8) {
    lo = min(E, tid * per);
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int i = lo + q;
      const int cnt = (q < per && i < E) ? s_tot[i] + s_pre[i] + own_sum(s_own, ncols, i) : 0;
      if (writer && q < per && i < E) expert_counts[i] = cnt;
      run_len[q] = block > 0 ? ((q < per && i < E) ? block : 0)
                             : (align == 1 ? cnt : (cnt + align - 1) / align * align);
      sum += run_len[q];
    }
    x = wave_inclusive_scan(sum);
    if (lane == kWave - 1) s_tmp[wave] = x;
  } else if (wave == 8) {
    const int v = lane < R ? s_tot[E + lane] + s_pre[E + lane] + own_sum(s_own, ncols, E + lane) : 0;
    const int inc = wave_inclusive_scan(v);
    if (lane < R) {
      s_pre[E + lane] += inc - v;
      if (writer) {
        rank_counts[lane] = v;
        rank_offsets[lane] = inc - v;
      }
    }
    if (writer && lane == kWave - 1) rank_offsets[R] = inc;
  }
  __syncthreads();
  if (wave < 8) {
    int run = x - sum, total = 0;
    for (int w = 0; w < 8; ++w) {
      const int t = s_tmp[w];
      run += w < wave ? t : 0;
      total += t;
    }
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int i = lo + q;
      if (q < per && i < E) {
        s_pre[i] += run;
        if (writer) expert_offsets[i] = run;
        run += run_len[q];
      }
    }
    if (writer && tid == 0) expert_offsets[E] = total;
  }
  __syncthreads();
}

// Whole tokens per lane for the counting pass: each lane takes TPL tokens
// (K * TPL ids, a multiple of 4, so 16-byte aligned loads) per pass and NQ
// passes per batch (at most kBatchVecs loads per lane). A wave's tokens are
// 64 * TPL consecutive ones, at most 256, so they never straddle a tile start
// (a multiple of 256). K = 0 (k known only at run time): one token per lane,
// its ids loaded one by one.
template <int K>
struct IdLanes {
  static constexpr int TPL = K == 0 ? 1 : (K % 4 == 0 ? 1 : (K % 2 == 0 ? 2 : 4));
  static constexpr int VPL = K == 0 ? 0 : K * TPL / 4;  // 16-byte loads per lane per pass
  static constexpr int NQ = K == 0 ? 1 : (kBatchVecs / VPL > 0 ? kBatchVecs / VPL : 1);
  static constexpr int NW = K == 0 ? kMaxK : NQ * VPL * 4;  // ids held per lane
  static constexpr int BATCH = kLayoutThreads * TPL * NQ;  // tokens per batch
};

// Ids of this lane's tokens of the batch starting at token b0 (-1 past T):
// pass q, token u of the lane holds w[q * VPL * 4 + u * K + j].
template <int K>
__device__ __forceinline__ void load_tokens(const int32_t* __restrict__ ids, int T, int k, int b0,
                                            int32_t (&w)[IdLanes<K>::NW]) {
  using L = IdLanes<K>;
  const int64_t n_ids = (int64_t)T * k;
  if (K > 0) {
#pragma unroll
    for (int q = 0; q < L::NQ; ++q) {
      const int64_t f0 = (b0 + int64_t(q * kLayoutThreads + threadIdx.x) * L::TPL) * K;
#pragma unroll
      for (int i = 0; i < L::VPL; ++i) {
        const int64_t f = f0 + 4 * i;
        int32_t* d = w + (q * L::VPL + i) * 4;
        if (f + 4 <= n_ids) {
          const vec4 v = *reinterpret_cast<const vec4*>(ids + f);
#pragma unroll
          for (int x = 0; x < 4; ++x) d[x] = int32_t(v[x]);
        } else {
#pragma unroll
          for (int x = 0; x < 4; ++x) d[x] = f + x < n_ids ? ids[f + x] : -1;
        }
      }
    }
  } else {
    const int t = b0 + int(threadIdx.x);
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) w[j] = (j < k && t < T) ? ids[(int64_t)t * k + j] : -1;
  }
}

// Tile counts for the two-launch layout: one workgroup of 256 threads per
// tile of g.tile_tokens tokens writes hist[c * g.tiles_pad + tile], the tile's
// pairs per expert (c < E) and copies per rank (c = E + r). Column-major, so
// that the ranking kernel reads a column's counts as whole 16-byte groups
// (tiles_pad = ntiles rounded up to 4; the padding entries are never used).
// Every entry a later read uses is written, so the workspace needs no
// clearing between calls.
constexpr int kCountThreads = 256;
constexpr int64_t kTwoLaunchMinIds = 49152;  // ids above which the two-launch layout is used

template <int K, int kRB>
__global__ __launch_bounds__(kCountThreads) void layout_count(LayoutGeom g,
                                                              const int32_t* __restrict__ ids,
                                                              int32_t* __restrict__ hist) {
  constexpr int KR = K > 0 ? K : kMaxK;
  const int k = K > 0 ? K : g.k;
  __shared__ int32_t s_h[kMaxExperts + kMaxRanks + 1];  // + a slot for invalid ids
  const int tid = threadIdx.x;
  const int lane = lane_id();
  for (int c = tid; c <= g.ncols; c += kCountThreads) s_h[c] = 0;
  __syncthreads();
  const int tile_lo = blockIdx.x * g.tile_tokens;
  const int tile_hi = min(g.T, tile_lo + g.tile_tokens);
  int rc = 0;  // lane r: this wave's copies on rank r
  for (int t0 = tile_lo; t0 < tile_hi; t0 += kCountThreads) {
    const int t = t0 + tid;
    const bool in = t < tile_hi;
    int ev[KR];
#pragma unroll
    for (int j = 0; j < KR; ++j)
      if (j < k) ev[j] = in ? ids[(int64_t)t * k + j] : -1;
    RankSet<kRB> set;
#pragma unroll
    for (int j = 0; j < KR; ++j) {
      if (j < k) {
        const bool valid = uint32_t(ev[j]) < uint32_t(g.E);
        atomicAdd(&s_h[valid ? ev[j] : g.ncols], 1);
        set.add(rank_of(valid ? ev[j] : 0, g.inv_m), valid);
      }
    }
    if (kRB == 8)
      rc += wave_rank_counts8(set.w[0]);
    else
      count_rank_set(s_h + g.E, set);
  }
  if (kRB == 8 && lane < g.R && rc) atomicAdd(&s_h[g.E + lane], rc);
  __syncthreads();
  for (int c = tid; c < g.ncols; c += kCountThreads)
    hist[(int64_t)c * g.tiles_pad + blockIdx.x] = s_h[c];
}

// One workgroup of 1024 threads per tile of g.tile_tokens tokens; K = k known
// at compile time (0: any k up to kMaxK, read at run time). With kFromHist the
// counts before and from the tile come from the tile counts in `hist`
// (written by layout_count); otherwise every workgroup counts all tokens
// itself. Writes:
//   pair_row[t][j]        = expert_offsets[e] + #{pairs of e before (t, j)}
//                           (-1 when that is past the end of a fixed block)
//   token_rank_slot[t][r] = rank_offsets[r] + #{tokens before t with a copy on r}
// Workgroup 0 also writes the counts and offsets.
template <int K, int kRB, bool kFromHist>
__global__ __launch_bounds__(kLayoutThreads) void layout_tiles(
    LayoutGeom g, const int32_t* __restrict__ ids, const int32_t* __restrict__ hist,
    int32_t* __restrict__ rank_counts,
    int32_t* __restrict__ rank_offsets, int32_t* __restrict__ expert_counts,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ token_rank_slot,
    int32_t* __restrict__ pair_row, int32_t* err_word) {
  constexpr int KR = K > 0 ? K : kMaxK;
  const int k = K > 0 ? K : g.k;
  extern __shared__ __align__(16) int32_t smem[];
  // With lds_match: per ranking wave a table of 64 lane masks (first, so
  // 8-byte aligned) and a byte per expert (last).
  uint64_t* s_peer = reinterpret_cast<uint64_t*>(smem);  // [kOwnWaves][64]
  int32_t* s_pack = smem + (g.lds_match ? kOwnWaves * kWave * 2 : 0);  // [kOwnTokens * k] own ids
  int32_t* s_cnt = s_pack + kOwnTokens * k;       // [kOwnWaves][ncols] per-wave counts
  int32_t* s_pre = s_cnt + kOwnWaves * g.ncols;   // [ncols + 1] before the tile -> running base
  int32_t* s_tot = s_pre + g.ncols + 1;           // [ncols + 1] other tokens -> totals -> offsets
  uint8_t* s_rep = reinterpret_cast<uint8_t*>(s_tot + g.ncols + 1);  // [kOwnWaves][e_pad]
  // (the extra slot of each takes the counts of invalid ids, so counting needs no branch)
  __shared__ int32_t s_tmp[kLayoutWaves];

  const int tid = threadIdx.x;
  const int wave = wave_in_block();
  const int lane = lane_id();
  const int tile_lo = blockIdx.x * g.tile_tokens;
  const int tile_hi = min(g.T, tile_lo + g.tile_tokens);
  // A tile of one sub-tile (every tile when T <= kMaxTiles * kOwnTokens) is
  // ranked before the counts are known: its ranking waves take their ids
  // straight from memory and work out the ranks inside the tile while the
  // counting runs; only the final rows wait for the scan. Larger tiles rank
  // their sub-tiles one after the other, after the scan, through s_pack.
  const bool early = g.tile_tokens == kOwnTokens;

  // 4. (Ranking, used by both orders.) Wave w < kOwnWaves owns tokens
  //    [32w, 32w+32) of a sub-tile, i.e. the contiguous pairs [32wk, 32(w+1)k),
  //    and walks them 64 at a time in order (chunks). Lanes holding the same
  //    expert find each other (the match); the lowest of them adds the
  //    group's size to the wave's running count for that expert with an LDS
  //    atomic that returns the old count. A wave's atomics complete in issue
  //    order, so the counts are exact without waiting between chunks; the
  //    waves' counts are then chained in wave order per column.
  const int ebits = 32 - __clz(g.E > 1 ? g.E - 1 : 1);
  constexpr int KC = (kTokW * KR + kWave - 1) / kWave;  // chunks of 64 pairs per wave (bound)
  const int nch = (kTokW * k + kWave - 1) / kWave;
  bool bad_id = false;
  bool full_block = false;  // a pair found its expert's fixed block full
  const bool ranker = wave < kOwnWaves;
  int32_t* cnt_w = s_cnt + (ranker ? wave : 0) * g.ncols;
  const int ti = wave * kTokW + lane;  // this lane's token in the sub-tile (lanes < kTokW)
  int ex[KC], rk[KC];  // per chunk: this lane's expert (or -1) and its rank in the wave
  int own[KR];         // ids of token ti, for its rank set
  RankSet<kRB> mask;   // rank set of token ti (lanes < kTokW)

  // Ranks inside the sub-tile from ex[] and own[]: rk[] relative to the
  // wave's running counts, which it advances (cnt_w), and the wave's copies
  // per rank (cnt_w[E + r]).
  auto rank_in_wave = [&]() {
    int lead[KC], grp[KC];
    uint64_t peers[KC];  // lanes of the chunk holding the same expert
#pragma unroll
    for (int ch = 0; ch < KC; ++ch) {
      if (ch < nch) {
        const bool valid = uint32_t(ex[ch]) < uint32_t(g.E);
        bad_id |= (ex[ch] != -1) && !valid;
        ex[ch] = valid ? ex[ch] : -1;
        peers[ch] = __ballot(valid);
      }
    }
    if (g.lds_match) {
      // Through the wave's own LDS tables, one chunk after the other: each
      // lane writes its lane number at its expert's byte and reads it back,
      // which gives every lane of a group the same member of it (whichever
      // write landed last); each lane then sets its bit in that member's
      // mask and reads the mask. The wave's LDS operations take effect in
      // issue order; atomic loads and stores keep the compiler from
      // forwarding a lane's own write to its read.
      uint8_t* rep_w = s_rep + wave * g.e_pad;
      uint64_t* peer_w = s_peer + wave * kWave;
#pragma unroll
      for (int ch = 0; ch < KC; ++ch) {
        if (ch < nch) {
          const bool on = ex[ch] >= 0;
          int rep = lane;
          uint64_t pm = 0;
          if (on) {
            __hip_atomic_store(rep_w + ex[ch], uint8_t(lane), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WAVEFRONT);
            rep = __hip_atomic_load(rep_w + ex[ch], __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_WAVEFRONT);
            __hip_atomic_store(peer_w + rep, uint64_t(0), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WAVEFRONT);
            __hip_atomic_fetch_or(peer_w + rep, uint64_t(1) << lane, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_WAVEFRONT);
            pm = __hip_atomic_load(peer_w + rep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
          }
          peers[ch] = pm;
        }
      }
    } else {
      // One ballot per id bit, all chunks side by side (independent chains).
      for (int b = 0; b < ebits; ++b) {
#pragma unroll
        for (int ch = 0; ch < KC; ++ch) {
          if (ch < nch) {
            const bool bit = (ex[ch] >> b) & 1;
            const uint64_t ones = __ballot(ex[ch] >= 0 && bit);
            peers[ch] &= bit ? ones : ~ones;
          }
        }
      }
    }
#pragma unroll
    for (int ch = 0; ch < KC; ++ch) {
      if (ch < nch) {
        rk[ch] = __popcll(peers[ch] & lanes_below());
        lead[ch] = ex[ch] >= 0 ? __ffsll((unsigned long long)peers[ch]) - 1 : lane;
        grp[ch] = __popcll(peers[ch]);
      }
    }
    int cnt_old[KC];
#pragma unroll
    for (int ch = 0; ch < KC; ++ch) {
      if (ch < nch) {
        cnt_old[ch] = 0;
        if (ex[ch] >= 0 && rk[ch] == 0) cnt_old[ch] = atomicAdd(&cnt_w[ex[ch]], grp[ch]);
      }
    }
#pragma unroll
    for (int ch = 0; ch < KC; ++ch)
      if (ch < nch) rk[ch] += __shfl(cnt_old[ch], lead[ch], kWave);
    mask = RankSet<kRB>();
#pragma unroll
    for (int j = 0; j < KR; ++j)
      if (j < k) mask.add(rank_of(own[j] >= 0 && own[j] < g.E ? own[j] : 0, g.inv_m),
                          own[j] >= 0 && own[j] < g.E);
    if (kRB == 8) {
      const int copies = wave_rank_counts8(mask.w[0]);  // lane r: tokens with a copy on r
      if (lane < g.R) cnt_w[g.E + lane] = copies;
    } else {
      count_rank_set(cnt_w + g.E, mask);  // the wave's rank columns start at zero
    }
  };

  // Per column: each ranking wave's first row, then advance the running base
  // (between barriers).
  auto chain_columns = [&]() {
    for (int c = tid; c < g.ncols; c += kLayoutThreads) {
      int v[kOwnWaves];  // all reads first: one LDS round trip, not one per wave
#pragma unroll
      for (int w = 0; w < kOwnWaves; ++w) v[w] = s_cnt[w * g.ncols + c];
      int run = s_pre[c];
#pragma unroll
      for (int w = 0; w < kOwnWaves; ++w) {
        s_cnt[w * g.ncols + c] = run;
        run += v[w];
      }
      s_pre[c] = run;
    }
  };

  // The rows of the sub-tile starting at token t0 (nt tokens), from the
  // chained bases (ranking waves).
  auto write_rows = [&](int t0, int nt) {
    const int npairs = nt * k;
    const bool tok_lane = lane < kTokW && ti < nt;
#pragma unroll
    for (int ch = 0; ch < KC; ++ch) {
      if (ch < nch) {
        const int pl = wave * kTokW * k + ch * kWave + lane;
        if (ch * kWave + lane < kTokW * k && pl < npairs) {
          int row = ex[ch] >= 0 ? cnt_w[ex[ch]] + rk[ch] : -1;
          if (g.block > 0 && row >= (ex[ch] + 1) * g.block) {
            row = -1;
            full_block = true;
          }
          pair_row[(int64_t)t0 * k + pl] = row;
        }
      }
    }
    auto write_slot = [&](int r) {
      const bool has = mask.has(r);
      const uint64_t on = __ballot(has);
      if (tok_lane)
        token_rank_slot[(int64_t)(t0 + ti) * g.R + r] =
            has ? cnt_w[g.E + r] + __popcll(on & lanes_below()) : -1;
    };
    if (kRB == 8) {
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (r < g.R) write_slot(r);
    } else {
      for (int r = 0; r < g.R; ++r) write_slot(r);
    }
  };

  // Early order: the ranking waves request their ids before anything else
  // (pairs past the tile's last token read as -1).
  if (early && ranker) {
    const int64_t pair0 = (int64_t)tile_lo * k;
    const int npairs = max(0, tile_hi - tile_lo) * k;
#pragma unroll
    for (int ch = 0; ch < KC; ++ch) {
      if (ch < nch) {
        const int f = wave * kTokW * k + ch * kWave + lane;
        const bool mine = ch * kWave + lane < kTokW * k && f < npairs;
        ex[ch] = mine ? ids[pair0 + f] : -1;
      }
    }
    const bool tok_lane = lane < kTokW && tile_lo + ti < tile_hi;
#pragma unroll
    for (int j = 0; j < KR; ++j)
      if (j < k) own[j] = tok_lane ? ids[(int64_t)(tile_lo + ti) * k + j] : -1;
  }

  // One tile (T <= 256, one launch): the ranking waves' own counts are the
  // totals, so there is no counting pass; the scan adds them up.
  const bool own_counts = !kFromHist && g.ntiles == 1;

  // The first batch of ids for the counting pass is requested before the
  // LDS is cleared.
  int32_t nxt[IdLanes<K>::NW];
  if (!kFromHist && !own_counts) load_tokens<K>(ids, g.T, k, 0, nxt);

  for (int c = tid; c < g.ncols; c += kLayoutThreads) {
    s_pre[c] = 0;
    s_tot[c] = 0;
  }
  // The per-wave running counts of the first sub-tile start at zero (cleared
  // here, while the ids load, rather than after the scan).
  for (int c = tid; c < kOwnWaves * g.ncols; c += kLayoutThreads) s_cnt[c] = 0;

  if (kFromHist) {
    // 1'. Counts before the tile and from it on, per column, from the tile
    //     counts: a column's tiles_pad entries are contiguous, all of its
    //     16-byte groups are requested at once.
    constexpr int kMaxGroups = kMaxTiles / 4;
    const int groups = g.tiles_pad / 4;
    const int me = int(blockIdx.x);
    for (int c = tid; c < g.ncols; c += kLayoutThreads) {
      const vec4* col = reinterpret_cast<const vec4*>(hist + (int64_t)c * g.tiles_pad);
      vec4 v[kMaxGroups];
#pragma unroll
      for (int q = 0; q < kMaxGroups; ++q)
        if (q < groups) v[q] = col[q];
      int before = 0, total = 0;
#pragma unroll
      for (int q = 0; q < kMaxGroups; ++q) {
        if (q < groups) {
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int j = 4 * q + x;
            const int cnt = j < g.ntiles ? int(v[q][x]) : 0;
            before += j < me ? cnt : 0;
            total += cnt;
          }
        }
      }
      s_pre[c] = before;
      s_tot[c] = total - before;
    }
    __syncthreads();  // s_pre / s_tot final, s_cnt zeroed
    if (early && ranker) rank_in_wave();  // before the scan, which needs no s_cnt
  } else {
    // 1. Histogram of every token, straight from registers: a batch of
    //    whole tokens per lane is loaded (16 bytes per load, coalesced) while
    //    the previous one is counted. Experts: one LDS atomic per pair. Ranks:
    //    one ballot per rank per 64 tokens (a wave's tokens sit on one side of
    //    the tile start). The ranking waves of the early order rank their
    //    pairs first, so that their LDS work overlaps the others' counting.
    using L = IdLanes<K>;
    int rc_pre = 0, rc_tot = 0;  // lane r: this wave's copies on rank r, before / from the tile
    __syncthreads();  // s_pre / s_tot / s_cnt zeroed
    if (early && ranker) rank_in_wave();
    for (int b0 = 0; !own_counts && b0 < g.T; b0 += L::BATCH) {
      int32_t cur[L::NW];
#pragma unroll
      for (int x = 0; x < L::NW; ++x) cur[x] = nxt[x];
      if (b0 + L::BATCH < g.T) load_tokens<K>(ids, g.T, k, b0 + L::BATCH, nxt);
#pragma unroll
      for (int q = 0; q < L::NQ; ++q) {
        const int tw = b0 + (q * kLayoutThreads + wave * kWave) * L::TPL;  // the wave's first
        if (tw >= g.T) continue;  // a wave past the last token counts nothing
        const bool before = tw < tile_lo;
        int32_t* cnt = before ? s_pre : s_tot;
        int c = 0;
#pragma unroll
        for (int u = 0; u < L::TPL; ++u) {
          const int32_t* ev = cur + q * L::VPL * 4 + u * K;
          RankSet<kRB> tset;
#pragma unroll
          for (int j = 0; j < KR; ++j) {
            if (j < k) {
              const bool valid = uint32_t(ev[j]) < uint32_t(g.E);
              atomicAdd(&cnt[valid ? ev[j] : g.ncols], 1);
              tset.add(rank_of(valid ? ev[j] : 0, g.inv_m), valid);
            }
          }
          if (kRB == 8)
            c += wave_rank_counts8(tset.w[0]);
          else
            count_rank_set(cnt + g.E, tset);  // at most k atomics per token
        }
        (before ? rc_pre : rc_tot) += c;
      }
    }
    if (lane < g.R) {  // lane r holds this wave's copies on rank r
      if (rc_pre) atomicAdd(&s_pre[g.E + lane], rc_pre);
      if (rc_tot) atomicAdd(&s_tot[g.E + lane], rc_tot);
    }
    __syncthreads();
  }

  // 2.-3. Counts, exclusive scans (experts in id order, ranks in rank order)
  //    and the absolute first row of this tile in every column (in s_pre).
  scan_columns(s_pre, s_tot, own_counts ? s_cnt : nullptr, g.ncols, g.E, g.R, g.align, g.block,
               s_tmp, blockIdx.x == 0, expert_counts, expert_offsets, rank_counts, rank_offsets);

  if (early) {
    chain_columns();
    __syncthreads();
    if (ranker) write_rows(tile_lo, max(0, tile_hi - tile_lo));
  } else {
    // Sub-tiles one after the other, their ids staged in LDS.
    for (int t0 = tile_lo; t0 < tile_hi; t0 += kOwnTokens) {
      const int nt = min(kOwnTokens, tile_hi - t0);
      const int npairs = nt * k;
      __syncthreads();  // s_pack and s_cnt free; s_pre final
      for (int f = tid; f < kOwnTokens * k; f += kLayoutThreads) {
        const int64_t gf = (int64_t)t0 * k + f;
        s_pack[f] = f < npairs ? ids[gf] : -1;
      }
      if (t0 > tile_lo)  // the first sub-tile's counts were cleared at the start
        for (int c = tid; c < kOwnWaves * g.ncols; c += kLayoutThreads) s_cnt[c] = 0;
      __syncthreads();
      if (ranker) {
        const bool tok_lane = lane < kTokW && ti < nt;
#pragma unroll
        for (int ch = 0; ch < KC; ++ch) {
          if (ch < nch) {
            const bool mine = ch * kWave + lane < kTokW * k;  // past it: the next wave's pairs
            ex[ch] = mine ? s_pack[wave * kTokW * k + ch * kWave + lane] : -1;
          }
        }
#pragma unroll
        for (int j = 0; j < KR; ++j)
          if (j < k) own[j] = tok_lane ? s_pack[ti * k + j] : -1;
        rank_in_wave();
      }
      __syncthreads();
      chain_columns();
      __syncthreads();
      if (ranker) write_rows(t0, nt);
    }
  }
  if (__ballot(bad_id) && lane == 0) flag_error(err_word, MOE_ERRBIT_BAD_ID);
  if (__ballot(full_block) && lane == 0) flag_error(err_word, MOE_ERRBIT_EXPERT_CAP);
}

constexpr size_t layout_lds_bytes(int k, int ncols) {
  return sizeof(int32_t) * (size_t(kOwnTokens) * k + size_t(kOwnWaves + 2) * ncols + 2);
}

// LDS of the layout with the match tables (a lane mask per lane and a byte
// per expert, per ranking wave); they are used when this fits.
constexpr size_t layout_match_lds_bytes(int k, int E, int R) {
  return layout_lds_bytes(k, E + R) +
         size_t(kOwnWaves) * (sizeof(uint64_t) * kWave + size_t((E + 3) / 4 * 4));
}

size_t layout_launch_lds(const LayoutGeom& g) {
  return g.lds_match ? layout_match_lds_bytes(g.k, g.E, g.R) : layout_lds_bytes(g.k, g.ncols);
}
static_assert(layout_lds_bytes(kMaxK, kMaxExperts + kMaxRanks) <= kLayoutLdsLimit,
              "the layout's LDS fits every shape");

LayoutGeom layout_geometry(const moe_shape_t& sh) {
  LayoutGeom g;
  g.T = sh.T;
  g.E = sh.E;
  g.R = sh.R;
  g.k = sh.k;
  g.m = sh.E / sh.R;
  g.align = sh.align;
  g.block = sh.block;
  g.ncols = sh.E + sh.R;
  g.inv_m = float(1.0 / double(g.m));
  g.e_pad = (sh.E + 3) / 4 * 4;
  g.lds_match = (g_layout_match != 0 && layout_match_lds_bytes(sh.k, sh.E, sh.R) <= kLayoutLdsLimit)
                    ? 1 : 0;
  const int64_t subs = (int64_t(sh.T) + kOwnTokens - 1) / kOwnTokens;
  const int64_t per_tile = std::max<int64_t>(1, (subs + kMaxTiles - 1) / kMaxTiles);
  g.tile_tokens = int(per_tile * kOwnTokens);
  g.ntiles = int(std::max<int64_t>(1, (int64_t(sh.T) + g.tile_tokens - 1) / g.tile_tokens));
  g.tiles_pad = (g.ntiles + 3) / 4 * 4;
  return g;
}

struct LayoutArgs {
  const int32_t* ids;
  int32_t *rc, *ro, *ec, *eo, *trs, *pr, *err;
  int32_t* hist;  // tile counts [ntiles][ncols], or NULL: one launch, every workgroup counts all
};

template <int K, int kRB>
void launch_layout_kw(const LayoutGeom& g, hipStream_t st, const LayoutArgs& a) {
  if (a.hist) {
    MOE_LAUNCH((layout_count<K, kRB>), dim3(g.ntiles), dim3(kCountThreads), 0, st, g,
                       a.ids, a.hist);
    MOE_LAUNCH((layout_tiles<K, kRB, true>), dim3(g.ntiles), dim3(kLayoutThreads),
                       layout_launch_lds(g), st, g, a.ids, a.hist, a.rc, a.ro, a.ec,
                       a.eo, a.trs, a.pr, a.err);
  } else {
    MOE_LAUNCH((layout_tiles<K, kRB, false>), dim3(g.ntiles), dim3(kLayoutThreads),
                       layout_launch_lds(g), st, g, a.ids, a.hist,
                       a.rc, a.ro, a.ec, a.eo, a.trs, a.pr, a.err);
  }
}

template <int K>
void launch_layout_k(const LayoutGeom& g, hipStream_t st, const LayoutArgs& a) {
  if (g.R > 32)
    launch_layout_kw<K, 64>(g, st, a);
  else if (g.R > 8)
    launch_layout_kw<K, 32>(g, st, a);
  else
    launch_layout_kw<K, 8>(g, st, a);
}

void launch_layout(const LayoutGeom& g, hipStream_t st, const LayoutArgs& a) {
  switch (g.k) {
    case 1: launch_layout_k<1>(g, st, a); break;
    case 2: launch_layout_k<2>(g, st, a); break;
    case 3: launch_layout_k<3>(g, st, a); break;
    case 4: launch_layout_k<4>(g, st, a); break;
    case 5: launch_layout_k<5>(g, st, a); break;
    case 6: launch_layout_k<6>(g, st, a); break;
    case 8: launch_layout_k<8>(g, st, a); break;
    default: launch_layout_k<0>(g, st, a);
  }
}

// Tile counts live in the caller's workspace: int32 [E + R][tiles_pad].
size_t layout_workspace_bytes(const LayoutGeom& g) {
  return g.ntiles > 1 ? sizeof(int32_t) * size_t(g.tiles_pad) * size_t(g.ncols) : 0;
}

// ---------------------------------------------------------------------------
// Row movers. A row is `nvec` vec4 (8 bf16 each). A wave moves a row in passes
// of 64*V vec4: lane l holds columns c0 + l, c0 + 64 + l, ..., so each wave
// instruction touches 1 KiB of contiguous bytes, and all V loads of a pass are
// in flight before the first store. Columns past the last full pass (H not a
// multiple of 512*V) go one vec4 per lane at a time.

// The first pass of a row (columns [0, 64*V)) into registers: callers issue
// it right behind the loads of the indices that say where the row goes, so
// that the latencies overlap. The loads are unconditional (a row shorter than
// one pass reads its last column instead, and fan_out_row does not use them),
// which keeps the code straight so that the indices can be waited for alone.
template <int V, bool kStreamLoad>
__device__ __forceinline__ void load_first_pass(const vec4* src, int nvec, vec4 (&first)[V]) {
#pragma unroll
  for (int q = 0; q < V; ++q)
    first[q] = load_row<kStreamLoad>(src + min(q * kWave + lane_id(), nvec - 1));
}

// Copies the row at `src` to every row dst_row(d), d in the lane mask `dests`,
// dst_row(d) = readlane(row_of_lane, d), loading and storing with the given
// cache policies; `first` holds the row's first pass (load_first_pass).
template <int V, bool kStreamLoad, bool kStreamStore>
__device__ __forceinline__ void fan_out_row(const vec4 (&first)[V], const vec4* src,
                                            vec4* dst_base, int row_of_lane, uint64_t dests,
                                            int nvec) {
  const int lane = lane_id();
  int c0 = 0;
  if (kWave * V <= nvec) {
    uint64_t d = dests;
    while (d) {
      const int which = __ffsll((unsigned long long)d) - 1;
      d &= d - 1;
      vec4* dst = dst_base + (int64_t)read_lane(row_of_lane, which) * nvec + lane;
#pragma unroll
      for (int q = 0; q < V; ++q) store_row<kStreamStore>(dst + q * kWave, first[q]);
    }
    c0 = kWave * V;
  }
  for (; c0 + kWave * V <= nvec; c0 += kWave * V) {
    vec4 v[V];
#pragma unroll
    for (int q = 0; q < V; ++q) v[q] = load_row<kStreamLoad>(src + c0 + q * kWave + lane);
    uint64_t d = dests;
    while (d) {
      const int which = __ffsll((unsigned long long)d) - 1;
      d &= d - 1;
      vec4* dst = dst_base + (int64_t)read_lane(row_of_lane, which) * nvec + c0 + lane;
#pragma unroll
      for (int q = 0; q < V; ++q) store_row<kStreamStore>(dst + q * kWave, v[q]);
    }
  }
  for (int c = c0 + lane; c < nvec; c += kWave) {
    const vec4 v = load_row<kStreamLoad>(src + c);
    uint64_t d = dests;
    while (d) {
      const int which = __ffsll((unsigned long long)d) - 1;
      d &= d - 1;
      store_row<kStreamStore>(dst_base + (int64_t)read_lane(row_of_lane, which) * nvec + c, v);
    }
  }
}

template <int V>
__global__ __launch_bounds__(kBlock) void pack_rows(const vec4* hidden,
                                                    const int32_t* __restrict__ token_rank_slot,
                                                    vec4* rank_buf,
                                                    int32_t* __restrict__ rank_src_token, int T,
                                                    int R, int nvec, int64_t cap_rank,
                                                    int32_t* err_word) {
  const int lane = lane_id();
  const int t = blockIdx.x * kWavesPerBlock + wave_in_block();
  if (t >= T) return;
  // The hidden row is read once, its first pass requested right behind the
  // token's slots (loads return in order, so the slots can be used while the
  // row is still arriving); the copies are stored with ordinary stores so
  // that they stay in the Infinity Cache for the permute. The row is read
  // with ordinary loads, not streamed: with streamed loads the permute lost
  // that cache hand-off (86 instead of 66 us at T=4096 H=5120) after any
  // large write by another kernel, until a large read came along, while
  // with ordinary loads the step takes the same time after either.
  const int slot_any = token_rank_slot[(int64_t)t * R + min(lane, R - 1)];
  const int slot = lane < R ? slot_any : -1;
  const vec4* src = hidden + (int64_t)t * nvec;
  vec4 first[V];
  load_first_pass<V, false>(src, nvec, first);
  const bool ok = slot >= 0 && slot < cap_rank;
  if (__ballot(slot >= 0 && !ok) && lane == 0) flag_error(err_word, MOE_ERRBIT_RANK_CAP);
  if (ok) rank_src_token[slot] = t;
  const uint64_t dests = __ballot(ok);
  if (dests) fan_out_row<V, false, false>(first, src, rank_buf, slot, dests, nvec);
}

// The pack for small batches (fewer than kFillTokens tokens, where one wave
// per token cannot fill the GPU) and for copies beyond the Infinity Cache
// (kPackSplitBytes): one wave per (token, group of 64 vec4), one
// vec4 per lane, the group index fastest so that a row's groups run side by
// side. The same copies, order and cache policy as pack_rows.
__global__ __launch_bounds__(kBlock) void pack_rows_small(
    const vec4* hidden, const int32_t* __restrict__ token_rank_slot, vec4* rank_buf,
    int32_t* __restrict__ rank_src_token, int T, int R, int nvec, int groups, int64_t cap_rank,
    int32_t* err_word) {
  const int lane = lane_id();
  const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block();
  const int t = int(gw / groups);
  const int g = int(gw - (int64_t)t * groups);
  if (t >= T) return;
  const int c = g * kWave + lane;
  // the slots and the row's column requested together (clamped, unconditional)
  const int slot_any = token_rank_slot[(int64_t)t * R + min(lane, R - 1)];
  const vec4 v = load_row<false>(hidden + (int64_t)t * nvec + min(c, nvec - 1));
  const int slot = lane < R ? slot_any : -1;
  const bool ok = slot >= 0 && slot < cap_rank;
  if (g == 0) {
    if (__ballot(slot >= 0 && !ok) && lane == 0) flag_error(err_word, MOE_ERRBIT_RANK_CAP);
    if (ok) rank_src_token[slot] = t;
  }
  uint64_t d = __ballot(ok);
  while (d) {
    const int which = __ffsll((unsigned long long)d) - 1;
    d &= d - 1;
    if (c < nvec) store_row<false>(rank_buf + (int64_t)read_lane(slot, which) * nvec + c, v);
  }
}

// Marks the padding rows of expert e (rows of its run or block that no pair
// fills) with expert_src_pair -1. A fixed block is [e*block, (e+1)*block)
// whatever the offsets say; a padded run is [offsets[e], offsets[e+1]). The
// counts and offsets are the caller's arguments, so the rows are clipped to
// [0, cap_expert): a store stays inside the buffer even when they disagree.
__device__ __forceinline__ void mark_padding(int e, const int32_t* expert_counts,
                                             const int32_t* expert_offsets, int block,
                                             int32_t* expert_src_pair, int64_t cap_expert) {
  const int64_t cnt = max(0, expert_counts[e]);  // a negative count fills nothing
  int64_t first, end;
  if (block > 0) {
    first = (int64_t)e * block;
    end = first + block;
  } else {
    first = expert_offsets[e];
    end = expert_offsets[e + 1];
  }
  const int64_t filled = block > 0 ? min(cnt, (int64_t)block) : cnt;
  const int64_t lo = max(first + filled, (int64_t)0);
  const int64_t hi = min(end, cap_expert);
  for (int64_t row = lo + lane_id(); row < hi; row += kWave) expert_src_pair[row] = -1;
}

// ---------------------------------------------------------------------------
// MXFP8 wire format: per block of 32 consecutive values of a row, one E8M0
// scale byte (2^e, e = floor(log2 amax) - 8 clamped to [-127, 127]; 0xFF if the
// block holds a NaN or an infinity) and 32 OCP e4m3 codes of v / 2^e, nearest
// with ties to even, saturating at 448, sign kept.

// e of a block from the largest magnitude's bf16 bits (0 < amax < 0x7F80).
// emax: exponent of the element format's largest value (8 for e4m3's 448, 2
// for e2m1's 6).
__device__ __forceinline__ int mx_block_exponent(uint32_t amax, int emax) {
  if (amax == 0) return -127;
  const int eb = int(amax >> 7);
  // floor(log2): a normal bf16 has it in its exponent field; a subnormal
  // m * 2^-133 has it at the top set bit of m.
  const int lg = eb > 0 ? eb - 127 : -133 + (31 - __clz(int(amax & 0x7F)));
  return min(127, max(-127, lg - emax));
}

typedef short mx_short2 __attribute__((ext_vector_type(2)));
typedef __bf16 mx_bf16x2 __attribute__((ext_vector_type(2)));

// Four bf16 (two words) divided by the block scale and rounded to e4m3 by the
// gfx950 scaled conversion (nearest, ties to even), bytes in element order.
// The conversion turns a magnitude that rounds past 448 into NaN (0x7F with
// the sign); in a block of finite values that can only be such an overflow,
// so those bytes are lowered by one, to +-448: the saturation of the MX rule.
__device__ __forceinline__ uint32_t e4m3x4(uint32_t w0, uint32_t w1, float scale) {
  mx_short2 r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(mx_bf16x2, w0), scale,
                                                false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(mx_bf16x2, w1), scale,
                                                true);
  const uint32_t x = __builtin_bit_cast(uint32_t, r);
  const uint32_t nan_bytes = ((x & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
  return x - (nan_bytes >> 7);
}

// Eight bf16 divided by the block scale and rounded to e2m1 by the gfx950
// scaled conversion, two codes per byte, the even value in the low nibble.
// (It rounds to nearest even and saturates at 6 exactly as the MX rule does:
// e2m1 has no NaN to overflow into.) The instruction is written out, one pair
// into byte 0 of a fresh register, because this compiler mis-models which
// source bits the fp4 conversion builtins read (it narrowed the loads feeding
// them and merged conversions of different words).
__device__ __forceinline__ uint32_t e2m1_pair(uint32_t two_bf16, float scale) {
  uint32_t r;
  asm("v_cvt_scalef32_pk_fp4_bf16 %0, %1, %2" : "=v"(r) : "v"(two_bf16), "v"(scale));
  return r & 0xFFu;
}

__device__ __forceinline__ uint32_t e2m1x8(vec4 v, float scale) {
  return e2m1_pair(v[0], scale) | (e2m1_pair(v[1], scale) << 8) |
         (e2m1_pair(v[2], scale) << 16) | (e2m1_pair(v[3], scale) << 24);
}

// The pages' 4-bit row ([A2A] sec 7.2: a one-byte scale for every 16 values):
// the scale is an OCP E4M3 value s nearest to amax / 6 (6 = e2m1's largest
// value), not a power of two, so the codes are found by exact comparisons
// with the e2m1 midpoints times s (each product has at most 7 significant
// bits, exact in float), not by the hardware's power-of-two scaled conversion.

// E4M3 code of a non-negative float y: nearest, ties to the even code,
// saturating at 448 (0x7E). Below 2^-6 the codes are multiples of 2^-9.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  if (!(y < 448.0f)) return 0x7Eu;
  if (y < 0.015625f) return uint32_t(__builtin_rintf(y * 512.0f));
  const uint32_t u = __float_as_uint(y);
  const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);  // mantissa to 3 bits, ties to even
  return (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t ef = c >> 3, mf = c & 7u;
  return ef == 0 ? float(mf) * 0.001953125f : __uint_as_float(((ef + 120u) << 23) | (mf << 20));
}

// e2m1 code of |x| (bf16 bits in the low 16 bits of w) for scale s > 0: the
// number of midpoints below it, a midpoint counting when |x| passes it or
// meets it from the side of the even code (ties to even).
__device__ __forceinline__ uint32_t e2m1_code_scaled(uint32_t w, const float (&mid)[7]) {
  const float a = __uint_as_float((w & 0x7FFFu) << 16);
  return uint32_t(a > mid[0]) + uint32_t(a >= mid[1]) + uint32_t(a > mid[2]) +
         uint32_t(a >= mid[3]) + uint32_t(a > mid[4]) + uint32_t(a >= mid[5]) +
         uint32_t(a > mid[6]);
}

// Eight bf16 (a vec4) to eight sign-and-magnitude e2m1 nibbles, the
// even-indexed value in the low nibble; s = 0 gives zero codes with signs.
__device__ __forceinline__ uint32_t e2m1x8_e4m3(vec4 v, float s) {
  const float mid[7] = {0.25f * s, 0.75f * s, 1.25f * s, 1.75f * s, 2.5f * s, 3.5f * s, 5.0f * s};
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t w = v[i] >> (16 * h);
      const uint32_t mag = s > 0.0f ? e2m1_code_scaled(w, mid) : 0u;
      out |= (mag | ((w >> 12) & 0x8u)) << (8 * i + 4 * h);
    }
  }
  return out;
}

// Fused quantise-and-pack: one wave per token, the row read once and
// quantised once in registers, then written (codes and scales) to every rank
// in the token's set. Each lane takes NL consecutive vec4 of the row per pass
// and produces NL * kBits bytes of codes (one store); a 32-value block is
// 4/NL lanes (its maximum one or two lane-xors away, or in-lane). Measured:
// MXFP8 is fastest with NL = 2 (16-byte stores), MXFP4 with NL = 1 (fully
// coalesced loads; wider lanes made its loads stride). Passes cover 64 * NL
// vec4; the last one may be partial (H is a multiple of 512, so whole blocks
// and lane groups). A wave takes the NP passes [sl*NP, sl*NP + NP) of its
// token, held in registers at once; with slices = 1 it walks all passes of the
// row NP at a time (NP dividing the pass count). Codes and scales are stored
// with ordinary stores, like the bf16 copies, for the permute to find in cache.
template <int kBits> struct MxLane { static constexpr int NL = 2; };
template <> struct MxLane<4> { static constexpr int NL = 1; };

template <int NP, int kBits, bool kE4M3 = false>
__global__ __launch_bounds__(kBlock) void pack_rows_mx(
    const vec4* hidden, const int32_t* __restrict__ token_rank_slot, uint8_t* rank_q,
    uint8_t* rank_scale, int32_t* __restrict__ rank_src_token, int T, int R, int nvec,
    int slices, int64_t cap_rank, int32_t* err_word) {
  static_assert(!kE4M3 || kBits == 4, "E4M3 scales per 16 values go with 4-bit codes");
  constexpr int NL = MxLane<kBits>::NL;  // vec4 per lane per pass
  constexpr int NB = NL * kBits;      // code bytes per lane per pass
  constexpr int kBlockVecs = kE4M3 ? 2 : 4;  // vec4 per scale block (16 or 32 values)
  constexpr int LPB = kBlockVecs / NL;       // lanes per scale block
  constexpr int kEmax = kBits == 8 ? 8 : 2;
  const int lane = lane_id();
  const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block();
  const int t = int(gw / slices);
  const int sl = int(gw - (int64_t)t * slices);  // this wave's NP passes: [sl*NP, sl*NP + NP)
  if (t >= T) return;
  const int slot = lane < R ? token_rank_slot[(int64_t)t * R + lane] : -1;
  const bool ok = slot >= 0 && slot < cap_rank;
  if (sl == 0) {
    if (__ballot(slot >= 0 && !ok) && lane == 0) flag_error(err_word, MOE_ERRBIT_RANK_CAP);
    if (ok) rank_src_token[slot] = t;
  }
  const uint64_t dests = __ballot(ok);
  if (!dests) return;
  const int64_t qrow = (int64_t)nvec * kBits;  // code bytes per row (H or H/2)
  const int64_t srow = nvec / kBlockVecs;      // scale bytes per row (H / 32 or H / 16)
  const int npass = (nvec + kWave * NL - 1) / (kWave * NL);
  const vec4* src = hidden + (int64_t)t * nvec;
  const int p_end = slices == 1 ? npass : sl * NP + NP;
  for (int p0 = sl * NP; p0 < p_end; p0 += NP) {
    vec4 v[NP][NL];
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int col = (p0 + q) * kWave * NL + NL * lane;
      const bool act = NL == 1 || col < nvec;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        if (act) {
          v[q][i] = load_row<false>(src + col + i);
        } else {
          v[q][i] = vec4{0u, 0u, 0u, 0u};
        }
      }
    }
    vec4 code[NP];
    uint32_t sw[NP];
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      uint32_t amax = 0;
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          amax = max(amax, v[q][i][j] & 0x7FFFu);
          amax = max(amax, (v[q][i][j] >> 16) & 0x7FFFu);
        }
      if (LPB >= 2) amax = max(amax, uint32_t(__shfl_xor(int(amax), 1, kWave)));
      if (LPB >= 4) amax = max(amax, uint32_t(__shfl_xor(int(amax), 2, kWave)));
      uint32_t sb;
      if (amax >= 0x7F80u) {  // NaN or infinity in the block: NaN scale, marked codes
        sb = kE4M3 ? 0x7Fu : 0xFFu;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          uint32_t c[8];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (kBits == 8) {  // e4m3 NaN with the value's sign
              c[2 * j] = ((v[q][i][j] >> 8) & 0x80u) | 0x7Fu;
              c[2 * j + 1] = ((v[q][i][j] >> 24) & 0x80u) | 0x7Fu;
            } else {  // the largest e2m1 code with the value's sign
              c[2 * j] = ((v[q][i][j] >> 12) & 0x8u) | 0x7u;
              c[2 * j + 1] = ((v[q][i][j] >> 28) & 0x8u) | 0x7u;
            }
          }
          if (kBits == 8) {
            code[q][2 * i] = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
            code[q][2 * i + 1] = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
          } else {
            uint32_t w = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) w |= c[j] << (4 * j);
            code[q][i] = w;
          }
        }
      } else if (kE4M3) {
        sb = e4m3_code(__uint_as_float(amax << 16) / 6.0f);
        const float sv = e4m3_value(sb);
#pragma unroll
        for (int i = 0; i < NL; ++i) code[q][i] = e2m1x8_e4m3(v[q][i], sv);
      } else {
        const int e = mx_block_exponent(amax, kEmax);
        const float scale = __uint_as_float(uint32_t(e + 127) << 23);  // E8M0 byte as an exponent
        sb = uint32_t(e + 127);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          if (kBits == 8) {
            code[q][2 * i] = e4m3x4(v[q][i][0], v[q][i][1], scale);
            code[q][2 * i + 1] = e4m3x4(v[q][i][2], v[q][i][3], scale);
          } else {
            code[q][i] = e2m1x8(v[q][i], scale);
          }
        }
      }
      // lanes 4*LPB*w collect the scale bytes of blocks 4w..4w+3 (of this pass)
      sw[q] = sb | (uint32_t(__shfl(int(sb), lane + LPB, kWave)) << 8) |
              (uint32_t(__shfl(int(sb), lane + 2 * LPB, kWave)) << 16) |
              (uint32_t(__shfl(int(sb), lane + 3 * LPB, kWave)) << 24);
    }
    uint64_t d = dests;
    while (d) {
      const int which = __ffsll((unsigned long long)d) - 1;
      d &= d - 1;
      const int64_t row = read_lane(slot, which);
      uint8_t* qdst = rank_q + row * qrow;
      uint8_t* sdst = rank_scale + row * srow;
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        const int col = (p0 + q) * kWave * NL + NL * lane;
        if (NL == 1 || col < nvec) {
          uint8_t* at = qdst + (int64_t)col * kBits;
          if (NB == 16) {
            *reinterpret_cast<vec4*>(at) = code[q];
          } else if (NB == 8) {
            uint2 w;
            w.x = code[q][0];
            w.y = code[q][1];
            *reinterpret_cast<uint2*>(at) = w;
          } else {
            *reinterpret_cast<uint32_t*>(at) = code[q][0];
          }
          if (lane % (4 * LPB) == 0)
            *reinterpret_cast<uint32_t*>(sdst + col / kBlockVecs) = sw[q];
        }
      }
    }
  }
}

// Permute: one wave per rank-buffer row, which it copies to the expert row of
// every pair of its token on its rank. With a padded or blocked layout the
// first pad_waves = E waves mark one expert's padding rows each (first, so
// that their latency hides under the row copies).
// kMx: the rows are quantised codes (MXFP8, MXFP4 or the 16-value 4-bit
// row), and each also has a row of nvec_s vec4 of scales in rank_scale /
// expert_scale that moves with it.
//
// Packed bf16 rows are read non-temporally; packed MX codes and scales with
// ordinary loads. With streamed loads the MX step lost the pack's cache
// hand-off after any large write by another kernel (MXFP8 at T=4096 H=5120:
// 130 instead of 120 us, until a large read came along); with ordinary loads
// it takes 121-122 us after either. (For bf16 rows the pack's ordinary loads
// of the hidden rows already keep the hand-off, and are the faster fix.)
template <int V, bool kMx>
__global__ __launch_bounds__(kBlock) void permute_rows(
    const vec4* rank_buf, const vec4* rank_scale, const int32_t* __restrict__ rank_src_token,
    const int32_t* __restrict__ rank_offsets, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ pair_row, const int32_t* __restrict__ expert_counts,
    const int32_t* __restrict__ expert_offsets, vec4* expert_buf, vec4* expert_scale,
    int32_t* __restrict__ expert_src_pair, int T, int E, int R, int k, int m, int block,
    int nvec, int nvec_s, int pad_waves, int64_t cap_rank, int64_t cap_expert,
    int early_row, int32_t* err_word) {
  constexpr bool kStreamIn = !kMx;
  const int lane = lane_id();
  const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block();
  if (gw < pad_waves) {
    mark_padding(int(gw), expert_counts, expert_offsets, block, expert_src_pair, cap_expert);
    return;
  }
  const int64_t i = gw - pad_waves;
  // Two rounds of loads: the offsets and the row's token, then the token's
  // ids and pair rows with the row itself right behind them. The grid is
  // rounded up to whole workgroups, so i can pass the last row: the token's
  // load is clamped into the buffer and such waves return below. With
  // early_row (small batches, where waiting for each round is most of the
  // time and reading a row for nothing is cheap) the row is requested in the
  // first round, clamped into the buffer, before it is known to be in use.
  const int64_t rows = min((int64_t)rank_offsets[R], cap_rank);
  const int end_any = rank_offsets[min(lane, R - 1) + 1];
  const int64_t ic = min(i, cap_rank - 1);
  const int t = ic >= 0 ? rank_src_token[ic] : -1;
  vec4 first[V];
  if (early_row) load_first_pass<V, kStreamIn>(rank_buf + ic * nvec, nvec, first);
  const int end = lane < R ? end_any : 0x7FFFFFFF;
  if (i >= rows || t < 0 || t >= T) return;
  const int e_any = ids[(int64_t)t * k + min(lane, k - 1)];
  const int pr_any = pair_row[(int64_t)t * k + min(lane, k - 1)];
  const int e = lane < k ? e_any : -1;
  const int pr = lane < k ? pr_any : -1;
  // The packed row is read once and the expert rows are not read again here:
  // both streamed (but MX codes: see above).
  const vec4* src = rank_buf + i * nvec;
  if (!early_row) load_first_pass<V, kStreamIn>(src, nvec, first);
  // MX: a scale row of at most 64 vec4 (H <= 32768) is one partial pass,
  // requested with the code row (clamped lanes; lanes >= nvec_s store nothing)
  const bool short_scales = kMx && nvec_s <= kWave;
  vec4 sv;
  if (short_scales) sv = load_row<kStreamIn>(rank_scale + i * nvec_s + min(lane, nvec_s - 1));
  // segment of row i: number of segment ends at or below i
  const int r = __popcll(__ballot(lane < R && end <= i));
  const bool here = e >= 0 && e < E && e / m == r;
  const int p = here ? pr : -1;
  const bool ok = here && p >= 0 && p < cap_expert;
  if (__ballot(here && !ok) && lane == 0) flag_error(err_word, MOE_ERRBIT_EXPERT_CAP);
  if (ok) expert_src_pair[p] = t * k + lane;
  const uint64_t dests = __ballot(ok);
  if (!dests) return;
  fan_out_row<V, kStreamIn, true>(first, src, expert_buf, p, dests, nvec);
  if (short_scales) {
    uint64_t d = dests;
    while (d) {
      const int which = __ffsll((unsigned long long)d) - 1;
      d &= d - 1;
      if (lane < nvec_s)
        store_row<true>(expert_scale + (int64_t)read_lane(p, which) * nvec_s + lane, sv);
    }
  } else if (kMx) {
    const vec4* ssrc = rank_scale + i * nvec_s;
    vec4 sfirst[1];
    load_first_pass<1, kStreamIn>(ssrc, nvec_s, sfirst);
    fan_out_row<1, kStreamIn, true>(sfirst, ssrc, expert_scale, p, dests, nvec_s);
  }
}

// moe_dispatch past the one-launch form: once the layout is written, pack and
// permute in one kernel. Each wave takes one (token, slice of V*64 vec4 of
// its row), reads that part of the hidden row once and stores it to the
// token's copy on each of its ranks and to the row of each of its pairs, so
// the packed rows are not read back. A pair's row is written when the
// permute would write it: its expert is valid, its rank copy is inside the
// rank buffer (the permute reads only those), and its row is inside the
// expert buffer; the cap errors are flagged as the pack and the permute
// flag them. With padded or blocked runs the first pad_waves = E waves mark
// the padding rows as the permute does.
template <int V, bool kStreamLoad, bool kStreamStore>
__global__ __launch_bounds__(kBlock) void pack_expand_rows(
    const vec4* hidden, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ token_rank_slot, const int32_t* __restrict__ pair_row,
    const int32_t* __restrict__ expert_counts, const int32_t* __restrict__ expert_offsets,
    vec4* rank_buf, int32_t* __restrict__ rank_src_token, vec4* expert_buf,
    int32_t* __restrict__ expert_src_pair, int T, int E, int R, int k, float inv_m, int block,
    int nvec, int slices, int pad_waves, int64_t cap_rank, int64_t cap_expert,
    int32_t* err_word) {
  const int lane = lane_id();
  const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block();
  if (gw < pad_waves) {
    mark_padding(int(gw), expert_counts, expert_offsets, block, expert_src_pair, cap_expert);
    return;
  }
  const int64_t w = gw - pad_waves;
  const int t = int(w / slices);
  const int sl = int(w - (int64_t)t * slices);
  if (t >= T) return;
  const int c0 = sl * (V * kWave);
  // the token's slots, ids and pair rows, its part of the row right behind
  // them (clamped into the row; columns past it are not stored)
  const int slot_any = token_rank_slot[(int64_t)t * R + min(lane, R - 1)];
  const int e_any = ids[(int64_t)t * k + min(lane, k - 1)];
  const int pr_any = pair_row[(int64_t)t * k + min(lane, k - 1)];
  const vec4* src = hidden + (int64_t)t * nvec;
  vec4 v[V];
#pragma unroll
  for (int q = 0; q < V; ++q)
    v[q] = load_row<kStreamLoad>(src + min(c0 + q * kWave + lane, nvec - 1));
  const int slot = lane < R ? slot_any : -1;
  const bool ok_r = slot >= 0 && slot < cap_rank;
  const int e = lane < k ? e_any : -1;
  const bool valid = uint32_t(e) < uint32_t(E);
  const int copy = __shfl(slot, valid ? rank_of(e, inv_m) : 0, kWave);
  const bool here = valid && copy >= 0 && copy < cap_rank;
  const int p = here ? pr_any : -1;
  const bool ok_p = here && p >= 0 && p < cap_expert;
  if (sl == 0) {
    if (__ballot(slot >= 0 && !ok_r) && lane == 0) flag_error(err_word, MOE_ERRBIT_RANK_CAP);
    if (__ballot(here && !ok_p) && lane == 0) flag_error(err_word, MOE_ERRBIT_EXPERT_CAP);
    if (ok_r) rank_src_token[slot] = t;
    if (ok_p) expert_src_pair[p] = t * k + lane;
  }
  uint64_t d = __ballot(ok_r);
  while (d) {
    const int which = __ffsll((unsigned long long)d) - 1;
    d &= d - 1;
    vec4* dst = rank_buf + (int64_t)read_lane(slot, which) * nvec;
#pragma unroll
    for (int q = 0; q < V; ++q) {
      const int c = c0 + q * kWave + lane;
      if (c < nvec) store_row<kStreamStore>(dst + c, v[q]);
    }
  }
  d = __ballot(ok_p);
  while (d) {
    const int which = __ffsll((unsigned long long)d) - 1;
    d &= d - 1;
    vec4* dst = expert_buf + (int64_t)read_lane(p, which) * nvec;
#pragma unroll
    for (int q = 0; q < V; ++q) {
      const int c = c0 + q * kWave + lane;
      if (c < nvec) store_row<kStreamStore>(dst + c, v[q]);
    }
  }
}

// ---------------------------------------------------------------------------
// The whole dispatch of a small batch in one launch (moe_dispatch with at most
// kSmallBatch tokens, 64 for a k read at run time; plain, padded or blocked
// runs):
// layout, pack and permute with no
// kernel boundary between them, for the decode step, whose time is launches
// and the waits between them. Every wave holds all T*k ids, TPL tokens per
// lane (token u = 64q + lane in group q), and works out from them, with wave
// ballots, scalar popcounts and wave sums, what it needs: as a low-latency
// sender decides where each row goes without asking anyone ([A2A] sec 4.1),
// here for the rank segments and the expert runs alike. Workgroup 0 writes the counts and
// offsets; with a blocked layout the next pad_waves = E waves mark one
// expert's padding rows each (its count is a wave sum over the ids); every
// other wave takes one (token, 1 KiB of the row), reads that part of the
// hidden row once and writes it to the token's copy on each of its ranks and
// to the row of each of its pairs (the pair's row is written only if its rank
// copy was, as the three calls do). The results are those of
// moe_dispatch_layout, moe_dispatch_pack and moe_permute_by_expert, bit for
// bit.
constexpr int kSmallBatch = 4 * kWave;

// x rounded up to a multiple of a (a >= 1): a padded run's rows.
__device__ __forceinline__ int round_up(int x, int a) { return (x + a - 1) / a * a; }

// Sum over the wave, in every lane.
__device__ __forceinline__ int wave_sum(int x) {
  return __builtin_amdgcn_readlane(wave_inclusive_scan(x), kWave - 1);
}

// Row formats of the one-launch dispatch: bf16 rows, or a wire format of
// pack_rows_mx (codes in one buffer, scale bytes in another).
enum : int { kWireBf16 = 0, kWireMxfp8 = 1, kWireMxfp4 = 2, kWireNvfp4 = 3 };

// One lane's vec4 (8 consecutive values, column c of the row) in a wire
// format, by the rules of pack_rows_mx: `code` gets its 8 (MXFP8) or 4 code
// bytes; a scale block is 4 lanes (32 values; 2 lanes, 16 values, for the
// 16-value 4-bit row), and the first lane of every four blocks gets their
// four scale bytes in `sw`. All lanes of the wave call it together (lane
// shuffles).
__device__ __forceinline__ void quantise_lane(int fmt, vec4 v, uint2& code, uint32_t& sw) {
  const int lpb = fmt == kWireNvfp4 ? 2 : 4;
  uint32_t amax = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    amax = max(amax, v[j] & 0x7FFFu);
    amax = max(amax, (v[j] >> 16) & 0x7FFFu);
  }
  amax = max(amax, uint32_t(__shfl_xor(int(amax), 1, kWave)));
  if (lpb == 4) amax = max(amax, uint32_t(__shfl_xor(int(amax), 2, kWave)));
  uint32_t sb;
  code = uint2{0u, 0u};
  if (amax >= 0x7F80u) {  // NaN or infinity in the block: NaN scale, marked codes
    sb = fmt == kWireNvfp4 ? 0x7Fu : 0xFFu;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (fmt == kWireMxfp8) {  // e4m3 NaN with the value's sign
        const uint32_t two = (((v[j] >> 8) & 0x80u) | 0x7Fu) | ((((v[j] >> 24) & 0x80u) | 0x7Fu) << 8);
        if (j < 2)
          code.x |= two << (16 * j);
        else
          code.y |= two << (16 * (j - 2));
      } else {  // the largest e2m1 code with the value's sign
        code.x |= ((((v[j] >> 12) & 0x8u) | 0x7u) | ((((v[j] >> 28) & 0x8u) | 0x7u) << 4)) << (8 * j);
      }
    }
  } else if (fmt == kWireNvfp4) {
    sb = e4m3_code(__uint_as_float(amax << 16) / 6.0f);
    code.x = e2m1x8_e4m3(v, e4m3_value(sb));
  } else {
    const int e = mx_block_exponent(amax, fmt == kWireMxfp8 ? 8 : 2);
    const float scale = __uint_as_float(uint32_t(e + 127) << 23);  // E8M0 byte as an exponent
    sb = uint32_t(e + 127);
    if (fmt == kWireMxfp8) {
      code.x = e4m3x4(v[0], v[1], scale);
      code.y = e4m3x4(v[2], v[3], scale);
    } else {
      code.x = e2m1x8(v, scale);
    }
  }
  const int lane = lane_id();
  sw = sb | (uint32_t(__shfl(int(sb), lane + lpb, kWave)) << 8) |
       (uint32_t(__shfl(int(sb), lane + 2 * lpb, kWave)) << 16) |
       (uint32_t(__shfl(int(sb), lane + 3 * lpb, kWave)) << 24);
}

// Stores a wave's part of a row (column c of `nvec`, lane-wise) into row
// `row` of a row buffer in format fmt: the bf16 vec4 v, or its codes and (in
// the first lane of every four scale blocks) the four scale bytes.
__device__ __forceinline__ void store_part(int fmt, void* rows, uint8_t* scales, int64_t row,
                                           int c, int nvec, vec4 v, uint2 code, uint32_t sw) {
  if (fmt == kWireBf16) {
    if (c < nvec) store_row<true>(static_cast<vec4*>(rows) + row * nvec + c, v);
    return;
  }
  // quantised rows: nvec is a multiple of 64, so every lane has a column
  const int lane = lane_id();
  uint8_t* q = static_cast<uint8_t*>(rows);
  if (fmt == kWireMxfp8) {
    *reinterpret_cast<uint2*>(q + row * (int64_t(nvec) * 8) + int64_t(c) * 8) = code;
  } else {
    *reinterpret_cast<uint32_t*>(q + row * (int64_t(nvec) * 4) + int64_t(c) * 4) = code.x;
  }
  const int lpb = fmt == kWireNvfp4 ? 2 : 4;
  if (lane % (4 * lpb) == 0)
    *reinterpret_cast<uint32_t*>(scales + row * (nvec / lpb) + c / lpb) = sw;
}

// pack_expand_rows for the wire formats (moe_dispatch_quantised past the
// one-launch form): one wave per (token, 1 KiB of the row) quantises its part
// once, by the rules of pack_rows_mx, and stores the codes and scales to every
// copy and every pair row, under the same guards and error flags. Rows of a
// multiple of 512 values: every lane has a column.
template <int kFmt>
__global__ __launch_bounds__(kBlock) void pack_expand_q(
    const vec4* hidden, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ token_rank_slot, const int32_t* __restrict__ pair_row,
    const int32_t* __restrict__ expert_counts, const int32_t* __restrict__ expert_offsets,
    uint8_t* rank_q, uint8_t* rank_scale, int32_t* __restrict__ rank_src_token,
    uint8_t* expert_q, uint8_t* expert_scale, int32_t* __restrict__ expert_src_pair, int T,
    int E, int R, int k, float inv_m, int block, int nvec, int groups, int pad_waves,
    int64_t cap_rank, int64_t cap_expert, int32_t* err_word) {
  static_assert(kFmt != kWireBf16, "bf16 rows take pack_expand_rows");
  const int lane = lane_id();
  const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block();
  if (gw < pad_waves) {
    mark_padding(int(gw), expert_counts, expert_offsets, block, expert_src_pair, cap_expert);
    return;
  }
  const int64_t w = gw - pad_waves;
  const int t = int(w / groups);
  const int g = int(w - (int64_t)t * groups);
  if (t >= T) return;
  const int c = g * kWave + lane;
  const int slot_any = token_rank_slot[(int64_t)t * R + min(lane, R - 1)];
  const int e_any = ids[(int64_t)t * k + min(lane, k - 1)];
  const int pr_any = pair_row[(int64_t)t * k + min(lane, k - 1)];
  const vec4 v = load_row<false>(hidden + (int64_t)t * nvec + c);
  const int slot = lane < R ? slot_any : -1;
  const bool ok_r = slot >= 0 && slot < cap_rank;
  const int e = lane < k ? e_any : -1;
  const bool valid = uint32_t(e) < uint32_t(E);
  const int copy = __shfl(slot, valid ? rank_of(e, inv_m) : 0, kWave);
  const bool here = valid && copy >= 0 && copy < cap_rank;
  const int p = here ? pr_any : -1;
  const bool ok_p = here && p >= 0 && p < cap_expert;
  if (g == 0) {
    if (__ballot(slot >= 0 && !ok_r) && lane == 0) flag_error(err_word, MOE_ERRBIT_RANK_CAP);
    if (__ballot(here && !ok_p) && lane == 0) flag_error(err_word, MOE_ERRBIT_EXPERT_CAP);
    if (ok_r) rank_src_token[slot] = t;
    if (ok_p) expert_src_pair[p] = t * k + lane;
  }
  uint2 code;
  uint32_t sw;
  quantise_lane(kFmt, v, code, sw);
  uint64_t d = __ballot(ok_r);
  while (d) {
    const int which = __ffsll((unsigned long long)d) - 1;
    d &= d - 1;
    store_part(kFmt, rank_q, rank_scale, read_lane(slot, which), c, nvec, v, code, sw);
  }
  d = __ballot(ok_p);
  while (d) {
    const int which = __ffsll((unsigned long long)d) - 1;
    d &= d - 1;
    store_part(kFmt, expert_q, expert_scale, read_lane(p, which), c, nvec, v, code, sw);
  }
}

template <int K, int kRB, int TPL, int kFmt>
__global__ __launch_bounds__(kBlock) void dispatch_small(
    const vec4* hidden, const int32_t* __restrict__ ids, int T, int E, int R, int k, int block,
    int align, float inv_m, int nvec, int groups, int pad_waves, int32_t* __restrict__ rank_counts,
    int32_t* __restrict__ rank_offsets, int32_t* __restrict__ expert_counts,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ token_rank_slot,
    int32_t* __restrict__ pair_row, void* rank_buf, uint8_t* rank_scale,
    int32_t* __restrict__ rank_src_token, int64_t cap_rank, void* expert_buf,
    uint8_t* expert_scale, int32_t* __restrict__ expert_src_pair, int64_t cap_expert,
    int32_t* err_word) {
  constexpr int KR = K > 0 ? K : kMaxK;
  // The wire format is a template argument: a runtime one leaves every
  // format's code in the one kernel, and measured 0.4 us slower for bf16
  // rows and 1.1 us slower for quantised ones at 64 tokens.
  constexpr int fmt = kFmt;
  const int kk = K > 0 ? K : k;
  const int lane = lane_id();
  const int wave = wave_in_block();
  const bool counter = blockIdx.x == 0;
  // Padding waves, then movers: a mover's token and 1 KiB group; its part of
  // the hidden row is requested first (clamped into the row), the ids right
  // behind it.
  const int64_t gw = counter ? 0 : (int64_t)(blockIdx.x - 1) * kWavesPerBlock + wave;
  const bool padder = !counter && gw < pad_waves;
  const int64_t gm = padder ? 0 : gw - pad_waves;
  const int t = int(gm / groups);
  const int g = int(gm - (int64_t)t * groups);
  // (with padded runs a wave past the last token still takes part in its
  // workgroup's barriers below, and leaves after them)
  const bool idle = !counter && !padder && t >= T;
  if (idle && align == 1) return;
  const int c = g * kWave + lane;
  vec4 v;
  if (!counter && !padder && !idle)
    v = load_row<true>(hidden + (int64_t)t * nvec + min(c, nvec - 1));
  int32_t idv[TPL][KR];  // group q, lane u: the ids of token 64q + u (-1 past T)
  RankSet<kRB> set[TPL];  // and its ranks
#pragma unroll
  for (int q = 0; q < TPL; ++q) {
    const int u = q * kWave + lane;
#pragma unroll
    for (int j = 0; j < KR; ++j) idv[q][j] = (j < kk && u < T) ? ids[u * kk + j] : -1;
#pragma unroll
    for (int j = 0; j < KR; ++j) {
      if (j < kk) {
        const bool valid = uint32_t(idv[q][j]) < uint32_t(E);
        set[q].add(rank_of(valid ? idv[q][j] : 0, inv_m), valid);
      }
    }
  }

  if (counter) {
    // Counts and offsets. Experts: an LDS histogram of all ids, then the
    // exclusive scan of the run lengths (the counts, or `block` each).
    __shared__ int32_t s_hist[kMaxExperts];
    __shared__ int32_t s_part[kWavesPerBlock];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kBlock) s_hist[e] = 0;
    __syncthreads();
    bool bad = false;
    for (int f = tid; f < T * kk; f += kBlock) {
      const int e = ids[f];
      if (uint32_t(e) < uint32_t(E))
        atomicAdd(&s_hist[e], 1);
      else
        bad |= e != -1;
    }
    if (__ballot(bad) && lane == 0) flag_error(err_word, MOE_ERRBIT_BAD_ID);
    __syncthreads();
    const int per = (E + kBlock - 1) / kBlock;
    const int lo = min(E, tid * per), hi = min(E, lo + per);
    int run = 0;
    for (int e = lo; e < hi; ++e) run += block > 0 ? block : round_up(s_hist[e], align);
    const int inc = wave_inclusive_scan(run);
    if (lane == kWave - 1) s_part[wave] = inc;
    __syncthreads();
    int base = inc - run, total = 0;
    for (int w = 0; w < kWavesPerBlock; ++w) {
      base += w < wave ? s_part[w] : 0;
      total += s_part[w];
    }
    for (int e = lo; e < hi; ++e) {
      expert_counts[e] = s_hist[e];
      expert_offsets[e] = base;
      base += block > 0 ? block : round_up(s_hist[e], align);
    }
    if (tid == 0) expert_offsets[E] = total;
    // Copies per rank (wave 0: one ballot per rank and token group) and
    // their offsets.
    if (wave == 0) {
      int mine = 0;
      for (int r = 0; r < R; ++r) {
        int n = 0;
#pragma unroll
        for (int q = 0; q < TPL; ++q) n += __popcll(__ballot(set[q].has(r)));
        mine = lane == r ? n : mine;
      }
      const int rinc = wave_inclusive_scan(mine);
      if (lane < R) {
        rank_counts[lane] = mine;
        rank_offsets[lane] = rinc - mine;
      }
      if (lane == kWave - 1) rank_offsets[R] = rinc;
    }
    return;
  }

  // Padded runs (align > 1): every workgroup histograms the ids in LDS (each
  // wave a quarter of the slots, from its registers) and scans the padded
  // run lengths into each expert's first row, as the counting workgroup
  // does for the offsets it writes.
  __shared__ int32_t s_cnt[kMaxExperts];
  __shared__ int32_t s_first[kMaxExperts];
  __shared__ int32_t s_wsum[kWavesPerBlock];
  if (align > 1) {
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kBlock) s_cnt[e] = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < TPL; ++q)
#pragma unroll
      for (int j = 0; j < KR; ++j)
        if (j < kk && j % kWavesPerBlock == wave && uint32_t(idv[q][j]) < uint32_t(E))
          atomicAdd(&s_cnt[idv[q][j]], 1);
    __syncthreads();
    const int per = (E + kBlock - 1) / kBlock;
    const int lo = min(E, tid * per), hi = min(E, lo + per);
    int run = 0;
    for (int e = lo; e < hi; ++e) run += round_up(s_cnt[e], align);
    const int inc = wave_inclusive_scan(run);
    if (lane == kWave - 1) s_wsum[wave] = inc;
    __syncthreads();
    int base = inc - run;
    for (int w = 0; w < wave; ++w) base += s_wsum[w];
    for (int e = lo; e < hi; ++e) {
      s_first[e] = base;
      base += round_up(s_cnt[e], align);
    }
    __syncthreads();
    if (idle) return;
  }

  if (padder && align > 1) {
    // Expert e = gw of a padded layout: the rows of its run past its pairs,
    // within the buffer, get expert_src_pair -1.
    const int e = int(gw);
    const int64_t first = s_first[e];
    const int64_t end = min(first + round_up(s_cnt[e], align), cap_expert);
    for (int64_t row = first + s_cnt[e] + lane; row < end; row += kWave)
      expert_src_pair[row] = -1;
    return;
  }
  if (padder) {
    // Expert e = gw of a blocked layout: the rows of its block past its pairs,
    // within the buffer, get expert_src_pair -1.
    const int e = int(gw);
    int n = 0;
#pragma unroll
    for (int q = 0; q < TPL; ++q)
#pragma unroll
      for (int j = 0; j < KR; ++j)
        if (j < kk) n += idv[q][j] == e ? 1 : 0;
    const int filled = min(wave_sum(n), block);
    const int64_t end = min((int64_t)(e + 1) * block, cap_expert);
    for (int64_t row = (int64_t)e * block + filled + lane; row < end; row += kWave)
      expert_src_pair[row] = -1;
    return;
  }

  // A quantised format: the part's codes and scales, once for all its rows.
  uint2 code = uint2{0u, 0u};
  uint32_t sw = 0;
  if (fmt != kWireBf16) quantise_lane(fmt, v, code, sw);

  // The token's copies: ranks in order, its slot on rank r kept in lane r.
  const int qt = t / kWave, lt = t - qt * kWave;  // token t is lane lt of group qt
  const uint64_t below = lt == 0 ? 0ull : (~0ull >> (kWave - lt));  // lanes before lt
  int off = 0, my_slot = -1;
  for (int r = 0; r < R; ++r) {
    int n = 0, before = 0;
    bool mine = false;
#pragma unroll
    for (int q = 0; q < TPL; ++q) {
      const uint64_t b = __ballot(set[q].has(r));
      n += __popcll(b);
      before += q < qt ? __popcll(b) : (q == qt ? __popcll(b & below) : 0);
      mine = q == qt ? ((b >> lt) & 1) != 0 : mine;
    }
    if (mine) {
      const int s = off + before;
      if (lane == r) my_slot = s;
      if (s < cap_rank) store_part(fmt, rank_buf, rank_scale, s, c, nvec, v, code, sw);
    }
    off += n;
  }
  if (g == 0) {
    if (lane < R) token_rank_slot[(int64_t)t * R + lane] = my_slot;
    const bool ok = my_slot >= 0 && my_slot < cap_rank;
    if (__ballot(my_slot >= 0 && !ok) && lane == 0) flag_error(err_word, MOE_ERRBIT_RANK_CAP);
    if (ok) rank_src_token[my_slot] = t;
  }

  // The token's pairs, in slot order: the run's first row (the valid ids
  // below e, or e*block) plus the pairs of e before (t, j), each counted
  // with one ballot per (token group, slot) and a scalar popcount, so the
  // expert and the row stay uniform (scalar registers, scalar branches).
  const uint64_t upto = below | (1ull << lt);  // lanes up to and including lt
  bool full = false;
  int my_row = -1;  // lane j: pair_row of slot j
#pragma unroll
  for (int j = 0; j < KR; ++j) {
    int e = -1;
#pragma unroll
    for (int q = 0; q < TPL; ++q)
      if (q == qt) e = __builtin_amdgcn_readlane(idv[q][j], lt);
    e = __builtin_amdgcn_readfirstlane(e);
    if (j >= kk || uint32_t(e) >= uint32_t(E)) continue;  // (no break: keeps the loop unrolled)
    int n_below = 0, rk = 0;
#pragma unroll
    for (int q = 0; q < TPL; ++q) {
      // (t, j) comes after every pair of earlier tokens and of lanes before
      // lt, and after the pairs of token t itself in slots below j
      const uint64_t before_t = q < qt ? ~0ull : (q == qt ? below : 0ull);
      const uint64_t upto_t = q < qt ? ~0ull : (q == qt ? upto : 0ull);
#pragma unroll
      for (int jj = 0; jj < KR; ++jj) {
        if (jj < kk) {
          const int x = idv[q][jj];
          n_below += __popcll(__ballot(uint32_t(x) < uint32_t(e)));
          rk += __popcll(__ballot(x == e) & (jj < j ? upto_t : before_t));
        }
      }
    }
    int p = (block > 0 ? e * block : align > 1 ? s_first[e] : n_below) + rk;
    if (block > 0 && rk >= block) {
      p = -1;
      full = true;
    }
    if (lane == j) my_row = p;
    const int s = __builtin_amdgcn_readlane(my_slot, rank_of(e, inv_m));  // the copy it comes from
    if (s < cap_rank) {
      if (p >= 0 && p < cap_expert) {
        store_part(fmt, expert_buf, expert_scale, p, c, nvec, v, code, sw);
        if (g == 0 && lane == 0) expert_src_pair[p] = t * kk + j;
      } else if (g == 0 && lane == 0) {
        flag_error(err_word, MOE_ERRBIT_EXPERT_CAP);
      }
    }
  }
  if (g == 0) {
    if (lane < kk) pair_row[(int64_t)t * kk + lane] = my_row;
    if (full && lane == 0) flag_error(err_word, MOE_ERRBIT_EXPERT_CAP);
  }
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;  // NaN stays quiet NaN
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void fma_bf16x8(float (&acc)[8], float w, vec4 y) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] = __builtin_fmaf(w, __uint_as_float(y[i] << 16), acc[2 * i]);
    acc[2 * i + 1] = __builtin_fmaf(w, __uint_as_float(y[i] & 0xFFFF0000u), acc[2 * i + 1]);
  }
}

template <bool kStream>
__device__ __forceinline__ void store_sum(const float (&acc)[8], vec4* out, vec4* out_f32,
                                          int64_t at) {
  vec4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = f32_to_bf16_rne(acc[2 * i]) | (f32_to_bf16_rne(acc[2 * i + 1]) << 16);
  store_row<kStream>(out + at, o);
  if (out_f32) {
    vec4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = __float_as_uint(acc[i]);
      b[i] = __float_as_uint(acc[4 + i]);
    }
    store_row<kStream>(out_f32 + 2 * at, a);
    store_row<kStream>(out_f32 + 2 * at + 1, b);
  }
}

// Weighted sum of rows for one column slice, in a fixed order. Lane j holds
// term j: the row it reads (src_row) and its weight (wt); the terms taken are
// the lanes in `terms`, in ascending lane order, each one fused multiply-add
// into float32 accumulators that start at +0. Columns [cb, cb + 64*V) of the
// sum go to row `orow` of out (bf16, round to nearest even) and of out_f32.
// The next term's rows are loaded while the current one is accumulated.
template <int V, bool kStreamLoad, bool kStreamStore>
__device__ __forceinline__ void weighted_row_sum(const vec4* rows, int src_row, float wt,
                                                 uint64_t terms, vec4* out, vec4* out_f32,
                                                 int64_t orow, int cb, int nvec) {
  const int lane = lane_id();
  if (cb + kWave * V <= nvec) {
    float acc[V][8];
#pragma unroll
    for (int q = 0; q < V; ++q)
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[q][x] = 0.0f;
    uint64_t s = terms;
    if (s) {
      int j = __ffsll((unsigned long long)s) - 1;
      s &= s - 1;
      vec4 y[V];
      const vec4* src = rows + (int64_t)read_lane(src_row, j) * nvec + cb + lane;
#pragma unroll
      for (int q = 0; q < V; ++q) y[q] = load_row<kStreamLoad>(src + q * kWave);
      while (s) {
        const int jn = __ffsll((unsigned long long)s) - 1;
        s &= s - 1;
        vec4 yn[V];
        const vec4* srcn = rows + (int64_t)read_lane(src_row, jn) * nvec + cb + lane;
#pragma unroll
        for (int q = 0; q < V; ++q) yn[q] = load_row<kStreamLoad>(srcn + q * kWave);
        const float w = __int_as_float(read_lane(__float_as_int(wt), j));
#pragma unroll
        for (int q = 0; q < V; ++q) fma_bf16x8(acc[q], w, y[q]);
#pragma unroll
        for (int q = 0; q < V; ++q) y[q] = yn[q];
        j = jn;
      }
      const float w = __int_as_float(read_lane(__float_as_int(wt), j));
#pragma unroll
      for (int q = 0; q < V; ++q) fma_bf16x8(acc[q], w, y[q]);
    }
#pragma unroll
    for (int q = 0; q < V; ++q)
      store_sum<kStreamStore>(acc[q], out, out_f32, orow + cb + q * kWave + lane);
    return;
  }
  // Partial slice at the end of the row: one vec4 per lane at a time.
  for (int c = cb + lane; c < nvec; c += kWave) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    uint64_t s = terms;
    while (s) {
      const int j = __ffsll((unsigned long long)s) - 1;
      s &= s - 1;
      const float w = __int_as_float(read_lane(__float_as_int(wt), j));
      fma_bf16x8(acc, w, load_row<kStreamLoad>(rows + (int64_t)read_lane(src_row, j) * nvec + c));
    }
    store_sum<kStreamStore>(acc, out, out_f32, orow + c);
  }
}

// weighted_row_sum with the rows of up to KB terms requested at once, then
// added in the same order (the same fused multiply-adds, so the same sums):
// for small batches, where a wave's time is its rounds of loads.
template <int V, int KB, bool kStreamLoad, bool kStreamStore>
__device__ __forceinline__ void weighted_row_sum_batched(const vec4* rows, int src_row, float wt,
                                                         uint64_t terms, vec4* out, vec4* out_f32,
                                                         int64_t orow, int cb, int nvec) {
  const int lane = lane_id();
  if (cb + kWave * V > nvec) {
    weighted_row_sum<V, kStreamLoad, kStreamStore>(rows, src_row, wt, terms, out, out_f32, orow,
                                                   cb, nvec);
    return;
  }
  float acc[V][8];
#pragma unroll
  for (int q = 0; q < V; ++q)
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[q][x] = 0.0f;
  uint64_t s = terms;
  while (s) {
    vec4 y[KB][V];
    int js[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      js[b] = -1;
      if (s) {
        const int j = __ffsll((unsigned long long)s) - 1;
        s &= s - 1;
        js[b] = j;
        const vec4* src = rows + (int64_t)read_lane(src_row, j) * nvec + cb + lane;
#pragma unroll
        for (int q = 0; q < V; ++q) y[b][q] = load_row<kStreamLoad>(src + q * kWave);
      }
    }
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      if (js[b] >= 0) {
        const float w = __int_as_float(read_lane(__float_as_int(wt), js[b]));
#pragma unroll
        for (int q = 0; q < V; ++q) fma_bf16x8(acc[q], w, y[b][q]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < V; ++q)
    store_sum<kStreamStore>(acc[q], out, out_f32, orow + cb + q * kWave + lane);
}

// Combine: one wave per (token, column slice of 64*V vec4); term j is slot j.
// The expert rows are read non-temporally: an expert kernel writes them
// between the dispatch and the combine, so nothing of them is left in the
// caches to reuse, and streaming them keeps them from evicting other lines.
// kBatch: all of a token's slots are requested at once (small batches).
template <int V, bool kBatch>
__global__ __launch_bounds__(kBlock) void combine_rows(
    const vec4* expert_out, const int32_t* __restrict__ pair_row,
    const float* __restrict__ weights, vec4* out, vec4* out_f32, int T, int k, int nvec,
    int slices, int64_t cap_expert, int32_t* err_word) {
  const int lane = lane_id();
  const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block();
  const int t = int(gw / slices);
  const int slice = int(gw - (int64_t)t * slices);
  if (t >= T) return;
  const int p = lane < k ? pair_row[(int64_t)t * k + lane] : -1;
  const float wt = lane < k ? weights[(int64_t)t * k + lane] : 0.0f;
  const bool ok = p >= 0 && p < cap_expert;
  if (slice == 0 && __ballot(p >= 0 && !ok) && lane == 0)
    flag_error(err_word, MOE_ERRBIT_EXPERT_CAP);
  if (kBatch)
    weighted_row_sum_batched<V, 8, true, true>(expert_out, p, wt, __ballot(ok), out, out_f32,
                                               (int64_t)t * nvec, slice * kWave * V, nvec);
  else
    weighted_row_sum<V, true, true>(expert_out, p, wt, __ballot(ok), out, out_f32,
                                    (int64_t)t * nvec, slice * kWave * V, nvec);
}

// Two-stage combine, first stage: one wave per (rank-buffer row, column
// slice). Row i of rank r's segment holds token t; its terms are the slots j
// of t whose expert lives on r. The partial rows are stored with ordinary
// stores so that the home sum finds them in the Infinity Cache; the expert
// rows are streamed as in combine_rows.
template <int V>
__global__ __launch_bounds__(kBlock) void rank_partial_rows(
    const vec4* expert_out, const int32_t* __restrict__ rank_src_token,
    const int32_t* __restrict__ rank_offsets, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ pair_row, const float* __restrict__ weights, vec4* partial,
    vec4* partial_f32, int T, int E, int R, int k, int m, int nvec, int slices,
    int64_t cap_rank, int64_t cap_expert, int32_t* err_word) {
  const int lane = lane_id();
  const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block();
  const int64_t i = gw / slices;
  const int slice = int(gw - i * slices);
  // Two rounds of index loads, as in the permute: the offsets and the row's
  // token (clamped into the buffer: the rounded-up grid can pass the last
  // row, and those waves return below), then the token's ids, pair rows and
  // weights (unconditional, clamped lanes).
  const int64_t rows = min((int64_t)rank_offsets[R], cap_rank);
  const int end_any = rank_offsets[min(lane, R - 1) + 1];
  const int64_t ic = min(i, cap_rank - 1);
  const int t = ic >= 0 ? rank_src_token[ic] : -1;
  if (i >= rows || t < 0 || t >= T) return;
  const int64_t at = (int64_t)t * k + min(lane, k - 1);
  const int e_any = ids[at];
  const int p_any = pair_row[at];
  const float w_any = weights[at];
  const int end = lane < R ? end_any : 0x7FFFFFFF;
  const int r = __popcll(__ballot(lane < R && end <= i));
  const int e = lane < k ? e_any : -1;
  const bool here = e >= 0 && e < E && e / m == r;
  const int p = here ? p_any : -1;
  const float wt = here ? w_any : 0.0f;
  const bool ok = p >= 0 && p < cap_expert;
  if (slice == 0 && __ballot(p >= 0 && !ok) && lane == 0)
    flag_error(err_word, MOE_ERRBIT_EXPERT_CAP);
  weighted_row_sum<V, true, false>(expert_out, p, wt, __ballot(ok), partial, partial_f32,
                                          i * nvec, slice * kWave * V, nvec);
}

// Two-stage combine, second stage: one wave per (token, column slice); term r
// is the token's partial row on rank r, weight 1 (a fused multiply-add by 1 is
// the plain float32 addition).
template <int V>
__global__ __launch_bounds__(kBlock) void rank_sum_rows(
    const vec4* partial, const int32_t* __restrict__ token_rank_slot, vec4* out,
    vec4* out_f32, int T, int R, int nvec, int slices, int64_t cap_rank, int32_t* err_word) {
  const int lane = lane_id();
  const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block();
  const int t = int(gw / slices);
  const int slice = int(gw - (int64_t)t * slices);
  if (t >= T) return;
  const int s = lane < R ? token_rank_slot[(int64_t)t * R + lane] : -1;
  const bool ok = s >= 0 && s < cap_rank;
  if (slice == 0 && __ballot(s >= 0 && !ok) && lane == 0)
    flag_error(err_word, MOE_ERRBIT_RANK_CAP);
  weighted_row_sum<V, true, true>(partial, s, 1.0f, __ballot(ok), out, out_f32,
                                  (int64_t)t * nvec, slice * kWave * V, nvec);
}

// ---------------------------------------------------------------------------
// Host side

bool shape_ok(const moe_shape_t* s) {
  if (!s) return false;
  if (s->T < 0 || s->H <= 0 || s->H % 8 != 0) return false;
  if (s->R < 1 || s->R > kMaxRanks || s->E < 1 || s->E > kMaxExperts || s->E % s->R != 0)
    return false;
  if (s->k < 1 || s->k > kMaxK) return false;
  if (s->align < 1 || s->align > kMaxAlign || s->block < 0) return false;
  if (s->block > 0 && s->align != 1) return false;
  if (int64_t(s->E) * s->block + int64_t(s->T) * s->k >= (int64_t(1) << 31)) return false;
  if (int64_t(s->T) * s->k + int64_t(s->E) * (s->align - 1) >= (int64_t(1) << 31)) return false;
  if (int64_t(s->T) * s->k >= (int64_t(1) << 30)) return false;
  if (int64_t(s->T) * s->R >= (int64_t(1) << 31)) return false;
  if (layout_lds_bytes(s->k, s->E + s->R) > kLayoutLdsLimit) return false;
  return true;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int launch_status() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Below this many tokens one wave per token leaves the GPU underfilled (fewer
// than 4 waves per compute unit): the pack, the MX pack and the combine then
// split rows across waves.
constexpr int kFillTokens = 1024;

// T * min(k, R) * H * 2 (the most bytes the pack can copy) above which the
// pack takes one wave per 1 KiB of the row at any batch size: the 256 MiB
// Infinity Cache.
constexpr int64_t kPackSplitBytes = int64_t(256) << 20;

// Register tile V of pack and permute (vec4 per lane per pass): the whole row
// in one pass when it has at most 16 groups of 64 vec4, else a divisor of the
// group count in [8, 16] if there is one (no tail), else 16.
int copy_vec(int nvec) {
  const int groups = nvec / kWave;
  if (groups <= 1) return 1;
  if (groups <= kMaxVec) return groups;
  for (int v = kMaxVec; v >= 8; --v)
    if (groups % v == 0) return v;
  return kMaxVec;
}

// Gathers (combine, partial rows, home sum): one wave per (row, column
// slice), a slice being at most `most` groups of 64 vec4 (each group 8 fp32
// accumulators per lane), as few slices as that allows; more groups per slice
// (up to 8) only if the grid would otherwise pass 2^31 - 1 waves. Measured
// (1, 2, 3, 4, 5 and 10 groups, each step on buffers no earlier step left in
// the caches): the combine with up to 8 (two slices of 5 at H=5120) is as
// fast as any within the prefill step, where the expert rows (240 MiB) fit
// the 256 MiB Infinity Cache; with more expert rows than that one group per
// wave is faster (T=8192 H=6144 k=8: 154 vs 159 us; T=16384 H=7168 k=8: 365
// vs 385 us). Below kFillTokens tokens one group per wave too (decode step
// 23.0 vs 24.9 us). The home sum takes one group per wave, the partial rows
// three (their waves first find their rank and terms).
constexpr int kCombineGroups = 8;
constexpr int64_t kCombineOneGroupBytes = int64_t(256) << 20;  // T*k*H*2 above: one group

int combine_groups(const moe_shape_t* sh) {
  if (sh->T < kFillTokens) return 1;
  const int64_t pair_bytes = int64_t(sh->T) * sh->k * sh->H * 2;
  return pair_bytes > kCombineOneGroupBytes ? 1 : kCombineGroups;
}

constexpr int kPartialGroups = 3;
constexpr int kRankSumGroups = 1;

void combine_tiling(int nvec, int64_t rows, int most, int* v, int* slices) {
  const int groups = std::max(1, (nvec + kWave - 1) / kWave);
  int g = most;
  while (g < 8 && rows * ((groups + g - 1) / g) > int64_t(INT32_MAX)) ++g;
  *slices = (groups + g - 1) / g;
  *v = (groups + *slices - 1) / *slices;
}

int blocks_for(int64_t waves) { return int((waves + kWavesPerBlock - 1) / kWavesPerBlock); }

template <template <int> class K>
struct ByVec {
  template <typename... Args>
  static void run(int v, Args&&... args) {
    switch (v) {
#define MOE_CASE(n) \
  case n:           \
    K<n>::go(args...); break;
      MOE_CASE(1) MOE_CASE(2) MOE_CASE(3) MOE_CASE(4) MOE_CASE(5) MOE_CASE(6) MOE_CASE(7)
      MOE_CASE(8) MOE_CASE(9) MOE_CASE(10) MOE_CASE(11) MOE_CASE(12) MOE_CASE(13)
      MOE_CASE(14) MOE_CASE(15)
#undef MOE_CASE
      default:
        K<kMaxVec>::go(args...);
    }
  }
};

template <int V>
struct PackLaunch {
  static void go(dim3 grid, hipStream_t st, const vec4* hid, const int32_t* slots, vec4* rb,
                 int32_t* src, int T, int R, int nvec, int64_t cap, int32_t* err) {
    MOE_LAUNCH(pack_rows<V>, grid, dim3(kBlock), 0, st, hid, slots, rb, src, T, R, nvec,
                       cap, err);
  }
};

// Pack and permute in one kernel: V vec4 per lane, `slices` waves per token.
// One wave per (token, 1 KiB of the row) with ordinary loads was best or
// within 1% of the best of six forms measured (1 or 2 vec4 per lane or the
// whole row per wave; streamed or ordinary loads and stores) over five
// shapes. The stores are streamed: on one buffer set replayed back to back
// ordinary stores were 1-6% faster, but with three buffer sets in turn (as
// layers and batches follow each other) streamed stores took the prefill
// step (this call and the combine) from 153.9 to 143.2 us, and the ordinary
// ones fell to 197 us when other work ran between the steps; skew the same.
constexpr int kExpandVec = 1;
constexpr bool kExpandStreamLoad = false;
constexpr bool kExpandStreamStore = true;
template <int V>
struct PackExpandLaunch {
  static void go(dim3 grid, hipStream_t st, const vec4* hid, const int32_t* ids,
                 const int32_t* slots, const int32_t* prow, const int32_t* ecnt,
                 const int32_t* eoff, vec4* rb, int32_t* rsrc, vec4* eb, int32_t* esrc, int T,
                 int E, int R, int k, float inv_m, int block, int nvec, int slices,
                 int pad_waves, int64_t cap_rank, int64_t cap_expert, int32_t* err) {
    MOE_LAUNCH((pack_expand_rows<V, kExpandStreamLoad, kExpandStreamStore>), grid, dim3(kBlock),
               0, st, hid, ids, slots, prow, ecnt, eoff, rb, rsrc, eb, esrc, T, E, R, k, inv_m,
               block, nvec, slices, pad_waves, cap_rank, cap_expert, err);
  }
};

template <int V>
struct PermuteLaunch {
  static void go(dim3 grid, hipStream_t st, const vec4* rb, const vec4* rs, const int32_t* src,
                 const int32_t* roff, const int32_t* ids, const int32_t* prow,
                 const int32_t* ecnt, const int32_t* eoff, vec4* eb, vec4* es, int32_t* esrc,
                 int T, int E, int R, int k, int m, int block, int nvec, int nvec_s,
                 int pad_waves, int64_t cap_rank, int64_t cap_expert, int early_row,
                 int32_t* err) {
    if (rs)
      MOE_LAUNCH((permute_rows<V, true>), grid, dim3(kBlock), 0, st, rb, rs, src, roff,
                         ids, prow, ecnt, eoff, eb, es, esrc, T, E, R, k, m, block, nvec, nvec_s,
                         pad_waves, cap_rank, cap_expert, early_row, err);
    else
      MOE_LAUNCH((permute_rows<V, false>), grid, dim3(kBlock), 0, st, rb, rs, src, roff,
                         ids, prow, ecnt, eoff, eb, es, esrc, T, E, R, k, m, block, nvec, nvec_s,
                         pad_waves, cap_rank, cap_expert, early_row, err);
  }
};


template <int V>
struct CombineLaunch {
  static void go(bool batch, dim3 grid, hipStream_t st, const vec4* eo, const int32_t* prow,
                 const float* w, vec4* out, vec4* out32, int T, int k, int nvec, int slices,
                 int64_t cap_expert, int32_t* err) {
    // The batched form holds all k slots' rows at once: small V only (the
    // caller picks it for V <= 2), so it is not built for wider registers.
    if constexpr (V <= 2) {
      if (batch) {
        MOE_LAUNCH((combine_rows<V, true>), grid, dim3(kBlock), 0, st, eo, prow, w, out, out32,
                   T, k, nvec, slices, cap_expert, err);
        return;
      }
    }
    MOE_LAUNCH((combine_rows<V, false>), grid, dim3(kBlock), 0, st, eo, prow, w, out, out32, T,
               k, nvec, slices, cap_expert, err);
  }
};

template <int V>
struct RankPartialLaunch {
  static void go(dim3 grid, hipStream_t st, const vec4* eo, const int32_t* src,
                 const int32_t* roff, const int32_t* ids, const int32_t* prow, const float* w,
                 vec4* part, vec4* part32, int T, int E, int R, int k, int m, int nvec,
                 int slices, int64_t cap_rank, int64_t cap_expert, int32_t* err) {
    MOE_LAUNCH(rank_partial_rows<V>, grid, dim3(kBlock), 0, st, eo, src, roff, ids, prow, w,
               part, part32, T, E, R, k, m, nvec, slices, cap_rank, cap_expert, err);
  }
};

template <int V>
struct RankSumLaunch {
  static void go(dim3 grid, hipStream_t st, const vec4* part, const int32_t* slots, vec4* out,
                 vec4* out32, int T, int R, int nvec, int slices, int64_t cap_rank,
                 int32_t* err) {
    MOE_LAUNCH(rank_sum_rows<V>, grid, dim3(kBlock), 0, st, part, slots, out, out32, T,
                       R, nvec, slices, cap_rank, err);
  }
};

// The permute for bf16 rows (rank_scale == NULL) or quantised rows (codes of
// nvec vec4 plus scales of nvec_s vec4 per row).
int permute_impl(const moe_shape_t& sh, const void* rank_rows, const void* rank_scale,
                 const int32_t* rank_src_token, const int32_t* rank_offsets,
                 const int32_t* topk_ids, const int32_t* pair_row, const int32_t* expert_counts,
                 const int32_t* expert_offsets, int64_t cap_rank, void* expert_rows,
                 void* expert_scale, int32_t* expert_src_pair, int64_t cap_expert,
                 int32_t* err_word, void* stream, int nvec, int nvec_s) {
  if (cap_rank < 0 || cap_expert < 0) return MOE_ERR_ARG;
  if (!rank_offsets) return MOE_ERR_ARG;
  const bool padded = sh.align > 1 || sh.block > 0;
  if (padded && (!expert_counts || !expert_offsets)) return MOE_ERR_ARG;
  const int64_t max_rows = std::min<int64_t>(cap_rank, int64_t(sh.T) * std::min(sh.k, sh.R));
  const int pad_waves = padded && cap_expert > 0 ? sh.E : 0;
  if (max_rows + pad_waves == 0) return MOE_OK;
  // With no rows to move (T = 0) only the padding marks are written: the
  // row buffers and token arrays are not touched and may be NULL.
  if (max_rows > 0 && (!rank_rows || !rank_src_token || !topk_ids || !pair_row ||
                       (cap_expert > 0 && !expert_rows)))
    return MOE_ERR_ARG;
  if (cap_expert > 0 && !expert_src_pair) return MOE_ERR_ARG;
  if (!aligned16(rank_rows) || !aligned16(expert_rows)) return MOE_ERR_ARG;
  ByVec<PermuteLaunch>::run(copy_vec(nvec), dim3(blocks_for(max_rows + pad_waves)),
                            static_cast<hipStream_t>(stream),
                            static_cast<const vec4*>(rank_rows),
                            static_cast<const vec4*>(rank_scale), rank_src_token, rank_offsets,
                            topk_ids, pair_row, expert_counts, expert_offsets,
                            static_cast<vec4*>(expert_rows), static_cast<vec4*>(expert_scale),
                            expert_src_pair, sh.T, sh.E, sh.R, sh.k, sh.E / sh.R, sh.block, nvec,
                            nvec_s, pad_waves, cap_rank, cap_expert,
                            max_rows > 0 && sh.T < kFillTokens ? 1 : 0, err_word);
  return launch_status();
}


// The one-launch dispatch of a small batch: workgroup 0 for the counts, E
// padding waves with a blocked layout, then one wave per (token, 1 KiB of the
// row).
struct DispatchSmallArgs {
  const vec4* hidden;
  const int32_t* ids;
  int32_t *rc, *ro, *ec, *eo, *trs, *pr;
  int fmt;  // kWireBf16, or a wire format (rows of codes, scales beside them)
  void* rank_buf;
  uint8_t* rank_scale;
  int32_t* rank_src;
  int64_t cap_rank;
  void* expert_buf;
  uint8_t* expert_scale;
  int32_t* expert_src;
  int64_t cap_expert;
  int32_t* err;
};

template <int K, int kRB, int TPL, int kFmt>
void launch_dispatch_small_f(const moe_shape_t& sh, hipStream_t st, const DispatchSmallArgs& a,
                             int grid, float inv_m, int nvec, int groups, int pad_waves) {
  MOE_LAUNCH((dispatch_small<K, kRB, TPL, kFmt>), dim3(grid), dim3(kBlock), 0, st, a.hidden,
             a.ids, sh.T, sh.E, sh.R, sh.k, sh.block, sh.align, inv_m, nvec, groups, pad_waves,
             a.rc, a.ro, a.ec, a.eo, a.trs, a.pr, a.rank_buf, a.rank_scale, a.rank_src,
             a.cap_rank, a.expert_buf, a.expert_scale, a.expert_src, a.cap_expert, a.err);
}

template <int K, int kRB, int TPL>
void launch_dispatch_small_t(const moe_shape_t& sh, hipStream_t st, const DispatchSmallArgs& a,
                             int grid, float inv_m, int nvec, int groups, int pad_waves) {
  switch (a.fmt) {
    case kWireMxfp8:
      launch_dispatch_small_f<K, kRB, TPL, kWireMxfp8>(sh, st, a, grid, inv_m, nvec, groups,
                                                       pad_waves);
      break;
    case kWireMxfp4:
      launch_dispatch_small_f<K, kRB, TPL, kWireMxfp4>(sh, st, a, grid, inv_m, nvec, groups,
                                                       pad_waves);
      break;
    case kWireNvfp4:
      launch_dispatch_small_f<K, kRB, TPL, kWireNvfp4>(sh, st, a, grid, inv_m, nvec, groups,
                                                       pad_waves);
      break;
    default:
      launch_dispatch_small_f<K, kRB, TPL, kWireBf16>(sh, st, a, grid, inv_m, nvec, groups,
                                                      pad_waves);
  }
}

template <int K, int kRB>
void launch_dispatch_small_kw(const moe_shape_t& sh, hipStream_t st, const DispatchSmallArgs& a) {
  const int nvec = sh.H / 8;
  const int groups = (nvec + kWave - 1) / kWave;
  const int pad_waves = (sh.block > 0 || sh.align > 1) && a.cap_expert > 0 ? sh.E : 0;
  const int grid = 1 + blocks_for(pad_waves + int64_t(sh.T) * groups);
  const float inv_m = float(1.0 / double(sh.E / sh.R));
  // one token per lane up to 64 tokens, else four (only for a k known at
  // compile time: with k read at run time the four groups' ids do not stay in
  // registers; moe_dispatch makes the three calls then)
  if (K == 0 || sh.T <= kWave)
    launch_dispatch_small_t<K, kRB, 1>(sh, st, a, grid, inv_m, nvec, groups, pad_waves);
  else
    launch_dispatch_small_t<K, kRB, K == 0 ? 1 : 4>(sh, st, a, grid, inv_m, nvec, groups,
                                                    pad_waves);
}

template <int K>
void launch_dispatch_small_k(const moe_shape_t& sh, hipStream_t st, const DispatchSmallArgs& a) {
  if (sh.R > 32)
    launch_dispatch_small_kw<K, 64>(sh, st, a);
  else if (sh.R > 8)
    launch_dispatch_small_kw<K, 32>(sh, st, a);
  else
    launch_dispatch_small_kw<K, 8>(sh, st, a);
}

// Whether moe_dispatch runs as one launch: up to 64 tokens, or up to 256 with
// a k the kernels are compiled for (plain, padded or blocked runs).
bool dispatch_one_launch(const moe_shape_t& sh) {
  const bool compiled_k = sh.k == 1 || sh.k == 2 || sh.k == 4 || sh.k == 6 || sh.k == 8;
  return g_dispatch_fused && (sh.T <= kWave || (sh.T <= kSmallBatch && compiled_k));
}

void launch_dispatch_small(const moe_shape_t& sh, hipStream_t st, const DispatchSmallArgs& a) {
  switch (sh.k) {
    case 1: launch_dispatch_small_k<1>(sh, st, a); break;
    case 2: launch_dispatch_small_k<2>(sh, st, a); break;
    case 4: launch_dispatch_small_k<4>(sh, st, a); break;
    case 6: launch_dispatch_small_k<6>(sh, st, a); break;
    case 8: launch_dispatch_small_k<8>(sh, st, a); break;
    default: launch_dispatch_small_k<0>(sh, st, a);
  }
}

// MX pack: NP passes in registers, the largest divisor of the pass count
// that is at most `most` (so every register batch is whole).
int mx_passes(int npass, int most) {
  for (int v = std::min(npass, most); v > 1; --v)
    if (npass % v == 0) return v;
  return 1;
}

template <int NP>
struct PackMxLaunch {
  static void go(int bits, bool e4m3, dim3 grid, hipStream_t st, const vec4* hid,
                 const int32_t* slots, uint8_t* rq, uint8_t* rs, int32_t* src, int T, int R,
                 int nvec, int slices, int64_t cap, int32_t* err) {
    if (bits == 4 && e4m3) {
      MOE_LAUNCH((pack_rows_mx<NP, 4, true>), grid, dim3(kBlock), 0, st, hid, slots, rq, rs,
                 src, T, R, nvec, slices, cap, err);
    } else if (bits == 4) {
      MOE_LAUNCH((pack_rows_mx<NP, 4>), grid, dim3(kBlock), 0, st, hid, slots, rq, rs,
                         src, T, R, nvec, slices, cap, err);
    } else if constexpr (NP * MxLane<8>::NL <= kMaxVec) {
      MOE_LAUNCH((pack_rows_mx<NP, 8>), grid, dim3(kBlock), 0, st, hid, slots, rq, rs,
                         src, T, R, nvec, slices, cap, err);
    }
  }
};

// bits 8: MXFP8; bits 4: MXFP4, or with e4m3 the 16-value-block 4-bit row.
int pack_mx_impl(int bits, bool e4m3, const moe_shape_t* shape, const uint16_t* hidden,
                 const int32_t* token_rank_slot, uint8_t* rank_q, uint8_t* rank_scale,
                 int32_t* rank_src_token, int64_t cap_rank, int32_t* err_word, void* stream) {
  if (!shape_ok(shape) || shape->H % kMxRowQuantum != 0 || cap_rank < 0) return MOE_ERR_ARG;
  if (shape->T == 0) return MOE_OK;
  if (!hidden || !token_rank_slot || (cap_rank > 0 && (!rank_q || !rank_scale || !rank_src_token)))
    return MOE_ERR_ARG;
  if (!aligned16(hidden) || !aligned16(rank_q) || !aligned16(rank_scale)) return MOE_ERR_ARG;
  const int nvec = shape->H / 8;
  const int nl = bits == 8 ? MxLane<8>::NL : MxLane<4>::NL;
  const int npass = (nvec + kWave * nl - 1) / (kWave * nl);
  // One register pass per wave (a wave per (token, pass)) for MXFP8, and for
  // MXFP4 when there are too few tokens for one wave each to fill the GPU;
  // otherwise the whole row per wave. Measured against the whole row per
  // wave: MXFP8 28.4 vs 29.6 us at prefill, 131 vs 141 at adv, 6.4 vs 8.6 at
  // decode; MXFP4 6.3 vs 8.7 us at decode but 24.7 vs 21.5 at prefill.
  int np = mx_passes(npass, kMaxVec / nl), slices = 1;
  if ((bits == 8 || shape->T < kFillTokens) && int64_t(shape->T) * npass <= INT32_MAX) {
    np = 1;
    slices = npass;
  }
  ByVec<PackMxLaunch>::run(np, bits, e4m3, dim3(blocks_for(int64_t(shape->T) * slices)),
                           static_cast<hipStream_t>(stream),
                           reinterpret_cast<const vec4*>(hidden), token_rank_slot, rank_q,
                           rank_scale, rank_src_token, shape->T, shape->R, nvec, slices,
                           cap_rank, err_word);
  return launch_status();
}

// Device address of `scratch` per device, looked up once per device with that
// device current.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mutex;

int static_workspace(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MOE_OK;
}

static_assert(size_t(kMaxTiles) * (kMaxExperts + kMaxRanks) * 4 ==
                  MOE_LAYOUT_STATIC_WORKSPACE_BYTES,
              "the static workspace holds the largest tile counts");

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_DISPATCH_ABI_VERSION; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument";
    case MOE_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

int moe_testing_set_layout_form(int form) {
  const int old = g_layout_form;
  if (form >= -1 && form <= 1) g_layout_form = form;
  return old;
}

int moe_testing_set_layout_match(int match) {
  const int old = g_layout_match;
  if (match == 0 || match == 1) g_layout_match = match;
  return old;
}

int moe_testing_set_dispatch_fused(int fused) {
  const int old = g_dispatch_fused;
  if (fused == 0 || fused == 1) g_dispatch_fused = fused;
  return old;
}

int moe_testing_time_next_launch(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr)) return MOE_ERR_ARG;
  g_time_start = static_cast<hipEvent_t>(start_event);
  g_time_stop = static_cast<hipEvent_t>(stop_event);
  return MOE_OK;
}

size_t moe_layout_workspace_bytes(const moe_shape_t* shape) {
  if (!shape_ok(shape)) return 0;
  return layout_workspace_bytes(layout_geometry(*shape));
}

int moe_dispatch_layout(const moe_shape_t* shape, const int32_t* topk_ids, int32_t* rank_counts,
                        int32_t* rank_offsets, int32_t* expert_counts, int32_t* expert_offsets,
                        int32_t* token_rank_slot, int32_t* pair_row, void* workspace,
                        size_t workspace_bytes, int32_t* err_word, void* stream) {
  if (!shape_ok(shape)) return MOE_ERR_ARG;
  if (!rank_counts || !rank_offsets || !expert_counts || !expert_offsets) return MOE_ERR_ARG;
  if (shape->T > 0 && (!topk_ids || !token_rank_slot || !pair_row)) return MOE_ERR_ARG;
  if (shape->T > 0 && !aligned16(topk_ids)) return MOE_ERR_ARG;
  const LayoutGeom g = layout_geometry(*shape);
  const size_t need = layout_workspace_bytes(g);
  if (workspace && (workspace_bytes < need || !aligned16(workspace))) return MOE_ERR_ARG;
  // Two launches pay about 3 us more in fixed cost; one launch counts all
  // T*k ids in every workgroup. Measured on MI355X (calls back to back), they
  // break even between 65,536 and 81,920 ids (k = 6 and k = 8) for uniform
  // routing, but with a few hot experts (most lanes of a counting atomic on
  // one address) one launch loses much earlier: 23.5 against 17.6 us at
  // 65,536 ids. The tile counts are used above 49,152 ids.
  const bool big = int64_t(shape->T) * shape->k > kTwoLaunchMinIds;
  const bool two = need > 0 && workspace && (g_layout_form < 0 ? big : g_layout_form == 1);
  LayoutArgs a{topk_ids, rank_counts, rank_offsets, expert_counts, expert_offsets,
               token_rank_slot, pair_row, err_word,
               two ? static_cast<int32_t*>(workspace) : nullptr};
  launch_layout(g, static_cast<hipStream_t>(stream), a);
  return launch_status();
}

int moe_dispatch_layout_noalloc(const moe_shape_t* shape, const int32_t* topk_ids,
                                int32_t* rank_counts, int32_t* rank_offsets,
                                int32_t* expert_counts, int32_t* expert_offsets,
                                int32_t* token_rank_slot, int32_t* pair_row, int32_t* err_word,
                                void* stream) {
  if (!shape_ok(shape)) return MOE_ERR_ARG;
  const size_t need = layout_workspace_bytes(layout_geometry(*shape));
  if (need > MOE_LAYOUT_STATIC_WORKSPACE_BYTES) return MOE_ERR_ARG;
  void* ws = nullptr;
  if (need > 0) {
    const int st = static_workspace(&ws);
    if (st != MOE_OK) return st;
  }
  return moe_dispatch_layout(shape, topk_ids, rank_counts, rank_offsets, expert_counts,
                             expert_offsets, token_rank_slot, pair_row, ws,
                             ws ? size_t(MOE_LAYOUT_STATIC_WORKSPACE_BYTES) : 0, err_word,
                             stream);
}

int moe_dispatch_pack(const moe_shape_t* shape, const uint16_t* hidden,
                      const int32_t* token_rank_slot, uint16_t* rank_buf, int32_t* rank_src_token,
                      int64_t cap_rank, int32_t* err_word, void* stream) {
  if (!shape_ok(shape) || cap_rank < 0) return MOE_ERR_ARG;
  if (shape->T == 0) return MOE_OK;
  if (!hidden || !token_rank_slot || (cap_rank > 0 && (!rank_buf || !rank_src_token)))
    return MOE_ERR_ARG;
  if (!aligned16(hidden) || !aligned16(rank_buf)) return MOE_ERR_ARG;
  const int nvec = shape->H / 8;
  const int groups = (nvec + kWave - 1) / kWave;
  const int64_t copy_bytes = int64_t(shape->T) * std::min(shape->k, shape->R) * shape->H * 2;
  if ((shape->T < kFillTokens || copy_bytes > kPackSplitBytes) && groups > 1 &&
      int64_t(shape->T) * groups <= INT32_MAX) {
    // Small batch: one wave per (token, 1 KiB of the row) (decode step 21.9
    // vs 23.0 us). So too when the copies can outgrow the Infinity Cache:
    // their stores then go on to HBM, which takes them faster from one wave
    // per 1 KiB (T=16384 H=7168 k=8: 234 vs 247 us). Below that one wave per
    // token is faster (T=4096 H=5120 k=6, whose copies wait in the cache for
    // the permute: +1.4 us per step with one wave per 1 KiB).
    MOE_LAUNCH(pack_rows_small, dim3(blocks_for(int64_t(shape->T) * groups)),
                       dim3(kBlock), 0, static_cast<hipStream_t>(stream),
                       reinterpret_cast<const vec4*>(hidden), token_rank_slot,
                       reinterpret_cast<vec4*>(rank_buf), rank_src_token, shape->T, shape->R,
                       nvec, groups, cap_rank, err_word);
    return launch_status();
  }
  ByVec<PackLaunch>::run(copy_vec(nvec), dim3(blocks_for(shape->T)),
                         static_cast<hipStream_t>(stream), reinterpret_cast<const vec4*>(hidden),
                         token_rank_slot, reinterpret_cast<vec4*>(rank_buf), rank_src_token,
                         shape->T, shape->R, nvec, cap_rank, err_word);
  return launch_status();
}

int moe_permute_by_expert(const moe_shape_t* shape, const uint16_t* rank_buf,
                          const int32_t* rank_src_token, const int32_t* rank_offsets,
                          const int32_t* topk_ids, const int32_t* pair_row,
                          const int32_t* expert_counts, const int32_t* expert_offsets,
                          int64_t cap_rank, uint16_t* expert_buf, int32_t* expert_src_pair,
                          int64_t cap_expert, int32_t* err_word, void* stream) {
  if (!shape_ok(shape)) return MOE_ERR_ARG;
  return permute_impl(*shape, rank_buf, nullptr, rank_src_token, rank_offsets, topk_ids,
                      pair_row, expert_counts, expert_offsets, cap_rank, expert_buf, nullptr,
                      expert_src_pair, cap_expert, err_word, stream, shape->H / 8, 0);
}

int moe_dispatch(const moe_shape_t* shape, const uint16_t* hidden, const int32_t* topk_ids,
                 int32_t* rank_counts, int32_t* rank_offsets, int32_t* expert_counts,
                 int32_t* expert_offsets, int32_t* token_rank_slot, int32_t* pair_row,
                 uint16_t* rank_buf, int32_t* rank_src_token, int64_t cap_rank,
                 uint16_t* expert_buf, int32_t* expert_src_pair, int64_t cap_expert,
                 void* workspace, size_t workspace_bytes, int32_t* err_word, void* stream) {
  // The checks of the three calls, all made before anything is launched.
  if (!shape_ok(shape) || cap_rank < 0 || cap_expert < 0) return MOE_ERR_ARG;
  const moe_shape_t& sh = *shape;
  // layout
  if (!rank_counts || !rank_offsets || !expert_counts || !expert_offsets) return MOE_ERR_ARG;
  if (sh.T > 0 && (!topk_ids || !token_rank_slot || !pair_row || !aligned16(topk_ids)))
    return MOE_ERR_ARG;
  const size_t need = layout_workspace_bytes(layout_geometry(sh));
  if (workspace && (workspace_bytes < need || !aligned16(workspace))) return MOE_ERR_ARG;
  // pack
  if (sh.T > 0 && (!hidden || (cap_rank > 0 && (!rank_buf || !rank_src_token)) ||
                   !aligned16(hidden) || !aligned16(rank_buf)))
    return MOE_ERR_ARG;
  // permute
  const bool padded = sh.align > 1 || sh.block > 0;
  const int64_t max_rows = std::min<int64_t>(cap_rank, int64_t(sh.T) * std::min(sh.k, sh.R));
  if (max_rows > 0 || (padded && cap_expert > 0)) {
    if (max_rows > 0 && cap_expert > 0 && !expert_buf) return MOE_ERR_ARG;
    if (cap_expert > 0 && !expert_src_pair) return MOE_ERR_ARG;
    if (!aligned16(rank_buf) || !aligned16(expert_buf)) return MOE_ERR_ARG;
  }
  if (dispatch_one_launch(sh)) {
    DispatchSmallArgs a{reinterpret_cast<const vec4*>(hidden), topk_ids, rank_counts,
                        rank_offsets, expert_counts, expert_offsets, token_rank_slot, pair_row,
                        kWireBf16, rank_buf, nullptr, rank_src_token, cap_rank, expert_buf,
                        nullptr, expert_src_pair, cap_expert, err_word};
    launch_dispatch_small(sh, static_cast<hipStream_t>(stream), a);
    return launch_status();
  }
  int st = moe_dispatch_layout(shape, topk_ids, rank_counts, rank_offsets, expert_counts,
                               expert_offsets, token_rank_slot, pair_row, workspace,
                               workspace_bytes, err_word, stream);
  const int nvec = sh.H / 8;
  const int V = std::min(kExpandVec, (nvec + kWave - 1) / kWave);
  const int64_t slices = (nvec + V * kWave - 1) / (V * kWave);
  const int pad_waves = padded && cap_expert > 0 ? sh.E : 0;
  // (an empty batch takes the permute, for the padding marks alone)
  if (st == MOE_OK && sh.T > 0 && g_dispatch_fused &&
      pad_waves + int64_t(sh.T) * slices <= INT32_MAX) {
    ByVec<PackExpandLaunch>::run(
        V, dim3(blocks_for(pad_waves + int64_t(sh.T) * slices)),
        static_cast<hipStream_t>(stream), reinterpret_cast<const vec4*>(hidden), topk_ids,
        token_rank_slot, pair_row, expert_counts, expert_offsets,
        reinterpret_cast<vec4*>(rank_buf), rank_src_token, reinterpret_cast<vec4*>(expert_buf),
        expert_src_pair, sh.T, sh.E, sh.R, sh.k, float(1.0 / double(sh.E / sh.R)), sh.block,
        nvec, int(slices), pad_waves, cap_rank, cap_expert, err_word);
    return launch_status();
  }
  if (st == MOE_OK)
    st = moe_dispatch_pack(shape, hidden, token_rank_slot, rank_buf, rank_src_token, cap_rank,
                           err_word, stream);
  if (st == MOE_OK)
    st = moe_permute_by_expert(shape, rank_buf, rank_src_token, rank_offsets, topk_ids,
                               pair_row, expert_counts, expert_offsets, cap_rank, expert_buf,
                               expert_src_pair, cap_expert, err_word, stream);
  return st;
}

int moe_dispatch_pack_mxfp8(const moe_shape_t* shape, const uint16_t* hidden,
                            const int32_t* token_rank_slot, uint8_t* rank_q,
                            uint8_t* rank_scale, int32_t* rank_src_token, int64_t cap_rank,
                            int32_t* err_word, void* stream) {
  return pack_mx_impl(8, false, shape, hidden, token_rank_slot, rank_q, rank_scale,
                      rank_src_token, cap_rank, err_word, stream);
}

int moe_dispatch_pack_mxfp4(const moe_shape_t* shape, const uint16_t* hidden,
                            const int32_t* token_rank_slot, uint8_t* rank_q,
                            uint8_t* rank_scale, int32_t* rank_src_token, int64_t cap_rank,
                            int32_t* err_word, void* stream) {
  return pack_mx_impl(4, false, shape, hidden, token_rank_slot, rank_q, rank_scale,
                      rank_src_token, cap_rank, err_word, stream);
}

int moe_dispatch_pack_nvfp4(const moe_shape_t* shape, const uint16_t* hidden,
                            const int32_t* token_rank_slot, uint8_t* rank_q,
                            uint8_t* rank_scale, int32_t* rank_src_token, int64_t cap_rank,
                            int32_t* err_word, void* stream) {
  return pack_mx_impl(4, true, shape, hidden, token_rank_slot, rank_q, rank_scale,
                      rank_src_token, cap_rank, err_word, stream);
}

// The permute of quantised rows: codes of nvec vec4 and scales of nvec_s vec4
// per row move together.
int permute_q_impl(const moe_shape_t* shape, const uint8_t* rank_q, const uint8_t* rank_scale,
                   const int32_t* rank_src_token, const int32_t* rank_offsets,
                   const int32_t* topk_ids, const int32_t* pair_row,
                   const int32_t* expert_counts, const int32_t* expert_offsets,
                   int64_t cap_rank, uint8_t* expert_q, uint8_t* expert_scale,
                   int32_t* expert_src_pair, int64_t cap_expert, int32_t* err_word,
                   void* stream, int nvec, int nvec_s) {
  if (!shape_ok(shape) || shape->H % kMxRowQuantum != 0) return MOE_ERR_ARG;
  const int64_t max_rows =
      std::min<int64_t>(cap_rank, int64_t(shape->T) * std::min(shape->k, shape->R));
  if (max_rows > 0 && !rank_scale) return MOE_ERR_ARG;
  if (cap_expert > 0 && max_rows > 0 && !expert_scale) return MOE_ERR_ARG;
  if (!aligned16(rank_scale) || !aligned16(expert_scale)) return MOE_ERR_ARG;
  // a non-null marker selects the two-row kernel even when nothing is moved
  const void* rs = rank_scale ? rank_scale : static_cast<const void*>(rank_q);
  return permute_impl(*shape, rank_q, rs, rank_src_token, rank_offsets, topk_ids, pair_row,
                      expert_counts, expert_offsets, cap_rank, expert_q, expert_scale,
                      expert_src_pair, cap_expert, err_word, stream, nvec, nvec_s);
}

int moe_permute_by_expert_mxfp8(const moe_shape_t* shape, const uint8_t* rank_q,
                                const uint8_t* rank_scale, const int32_t* rank_src_token,
                                const int32_t* rank_offsets, const int32_t* topk_ids,
                                const int32_t* pair_row, const int32_t* expert_counts,
                                const int32_t* expert_offsets, int64_t cap_rank,
                                uint8_t* expert_q, uint8_t* expert_scale,
                                int32_t* expert_src_pair, int64_t cap_expert, int32_t* err_word,
                                void* stream) {
  if (!shape) return MOE_ERR_ARG;
  return permute_q_impl(shape, rank_q, rank_scale, rank_src_token, rank_offsets, topk_ids,
                        pair_row, expert_counts, expert_offsets, cap_rank, expert_q,
                        expert_scale, expert_src_pair, cap_expert, err_word, stream,
                        shape->H / 16, shape->H / 512);
}

int moe_permute_by_expert_mxfp4(const moe_shape_t* shape, const uint8_t* rank_q,
                                const uint8_t* rank_scale, const int32_t* rank_src_token,
                                const int32_t* rank_offsets, const int32_t* topk_ids,
                                const int32_t* pair_row, const int32_t* expert_counts,
                                const int32_t* expert_offsets, int64_t cap_rank,
                                uint8_t* expert_q, uint8_t* expert_scale,
                                int32_t* expert_src_pair, int64_t cap_expert, int32_t* err_word,
                                void* stream) {
  if (!shape) return MOE_ERR_ARG;
  return permute_q_impl(shape, rank_q, rank_scale, rank_src_token, rank_offsets, topk_ids,
                        pair_row, expert_counts, expert_offsets, cap_rank, expert_q,
                        expert_scale, expert_src_pair, cap_expert, err_word, stream,
                        shape->H / 32, shape->H / 512);
}

int moe_permute_by_expert_nvfp4(const moe_shape_t* shape, const uint8_t* rank_q,
                                const uint8_t* rank_scale, const int32_t* rank_src_token,
                                const int32_t* rank_offsets, const int32_t* topk_ids,
                                const int32_t* pair_row, const int32_t* expert_counts,
                                const int32_t* expert_offsets, int64_t cap_rank,
                                uint8_t* expert_q, uint8_t* expert_scale,
                                int32_t* expert_src_pair, int64_t cap_expert, int32_t* err_word,
                                void* stream) {
  if (!shape) return MOE_ERR_ARG;
  return permute_q_impl(shape, rank_q, rank_scale, rank_src_token, rank_offsets, topk_ids,
                        pair_row, expert_counts, expert_offsets, cap_rank, expert_q,
                        expert_scale, expert_src_pair, cap_expert, err_word, stream,
                        shape->H / 32, shape->H / 256);
}

int moe_dispatch_quantised(const moe_shape_t* shape, int format, const uint16_t* hidden,
                           const int32_t* topk_ids, int32_t* rank_counts, int32_t* rank_offsets,
                           int32_t* expert_counts, int32_t* expert_offsets,
                           int32_t* token_rank_slot, int32_t* pair_row, uint8_t* rank_q,
                           uint8_t* rank_scale, int32_t* rank_src_token, int64_t cap_rank,
                           uint8_t* expert_q, uint8_t* expert_scale, int32_t* expert_src_pair,
                           int64_t cap_expert, void* workspace, size_t workspace_bytes,
                           int32_t* err_word, void* stream) {
  // The checks of the three calls, all made before anything is launched.
  if (format != MOE_WIRE_MXFP8 && format != MOE_WIRE_MXFP4 && format != MOE_WIRE_NVFP4)
    return MOE_ERR_ARG;
  if (!shape_ok(shape) || shape->H % kMxRowQuantum != 0 || cap_rank < 0 || cap_expert < 0)
    return MOE_ERR_ARG;
  const moe_shape_t& sh = *shape;
  // layout
  if (!rank_counts || !rank_offsets || !expert_counts || !expert_offsets) return MOE_ERR_ARG;
  if (sh.T > 0 && (!topk_ids || !token_rank_slot || !pair_row || !aligned16(topk_ids)))
    return MOE_ERR_ARG;
  const size_t need = layout_workspace_bytes(layout_geometry(sh));
  if (workspace && (workspace_bytes < need || !aligned16(workspace))) return MOE_ERR_ARG;
  // quantise-and-pack
  if (sh.T > 0 && (!hidden || (cap_rank > 0 && (!rank_q || !rank_scale || !rank_src_token)) ||
                   !aligned16(hidden) || !aligned16(rank_q) || !aligned16(rank_scale)))
    return MOE_ERR_ARG;
  // permute of the codes and scales
  const bool padded = sh.align > 1 || sh.block > 0;
  const int64_t max_rows = std::min<int64_t>(cap_rank, int64_t(sh.T) * std::min(sh.k, sh.R));
  if (max_rows > 0 && !rank_scale) return MOE_ERR_ARG;
  if (cap_expert > 0 && max_rows > 0 && !expert_scale) return MOE_ERR_ARG;
  if (!aligned16(rank_scale) || !aligned16(expert_scale)) return MOE_ERR_ARG;
  if (max_rows > 0 || (padded && cap_expert > 0)) {
    if (max_rows > 0 && cap_expert > 0 && !expert_q) return MOE_ERR_ARG;
    if (cap_expert > 0 && !expert_src_pair) return MOE_ERR_ARG;
    if (!aligned16(rank_q) || !aligned16(expert_q)) return MOE_ERR_ARG;
  }
  if (dispatch_one_launch(sh)) {
    const int fmt = format == MOE_WIRE_MXFP8 ? kWireMxfp8
                    : format == MOE_WIRE_MXFP4 ? kWireMxfp4 : kWireNvfp4;
    DispatchSmallArgs a{reinterpret_cast<const vec4*>(hidden), topk_ids, rank_counts,
                        rank_offsets, expert_counts, expert_offsets, token_rank_slot, pair_row,
                        fmt, rank_q, rank_scale, rank_src_token, cap_rank, expert_q,
                        expert_scale, expert_src_pair, cap_expert, err_word};
    launch_dispatch_small(sh, static_cast<hipStream_t>(stream), a);
    return launch_status();
  }
  int st = moe_dispatch_layout(shape, topk_ids, rank_counts, rank_offsets, expert_counts,
                               expert_offsets, token_rank_slot, pair_row, workspace,
                               workspace_bytes, err_word, stream);
  if (st != MOE_OK) return st;
  const int groups = sh.H / 512;  // 1 KiB of bf16 per wave
  const int pad_waves = padded && cap_expert > 0 ? sh.E : 0;
  // (an empty batch takes the permute, for the padding marks alone)
  if (sh.T > 0 && g_dispatch_fused && pad_waves + int64_t(sh.T) * groups <= INT32_MAX) {
    const dim3 grid(blocks_for(pad_waves + int64_t(sh.T) * groups));
    const float inv_m = float(1.0 / double(sh.E / sh.R));
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    const vec4* hid = reinterpret_cast<const vec4*>(hidden);
#define MOE_EXPAND_Q(F)                                                                          \
  MOE_LAUNCH((pack_expand_q<F>), grid, dim3(kBlock), 0, hs, hid, topk_ids, token_rank_slot,      \
             pair_row, expert_counts, expert_offsets, rank_q, rank_scale, rank_src_token,         \
             expert_q, expert_scale, expert_src_pair, sh.T, sh.E, sh.R, sh.k, inv_m, sh.block,    \
             sh.H / 8, groups, pad_waves, cap_rank, cap_expert, err_word)
    if (format == MOE_WIRE_MXFP8)
      MOE_EXPAND_Q(kWireMxfp8);
    else if (format == MOE_WIRE_MXFP4)
      MOE_EXPAND_Q(kWireMxfp4);
    else
      MOE_EXPAND_Q(kWireNvfp4);
#undef MOE_EXPAND_Q
    return launch_status();
  }
  const int bits = format == MOE_WIRE_MXFP8 ? 8 : 4;
  const bool e4m3 = format == MOE_WIRE_NVFP4;
  st = pack_mx_impl(bits, e4m3, shape, hidden, token_rank_slot, rank_q, rank_scale,
                    rank_src_token, cap_rank, err_word, stream);
  if (st != MOE_OK) return st;
  const int nvec = bits == 8 ? sh.H / 16 : sh.H / 32;
  const int nvec_s = e4m3 ? sh.H / 256 : sh.H / 512;
  return permute_q_impl(shape, rank_q, rank_scale, rank_src_token, rank_offsets, topk_ids,
                        pair_row, expert_counts, expert_offsets, cap_rank, expert_q,
                        expert_scale, expert_src_pair, cap_expert, err_word, stream, nvec,
                        nvec_s);
}

int moe_combine(const moe_shape_t* shape, const uint16_t* expert_out, const int32_t* pair_row,
                const float* topk_weights, int64_t cap_expert, uint16_t* out, float* out_f32,
                int32_t* err_word, void* stream) {
  if (!shape_ok(shape) || cap_expert < 0) return MOE_ERR_ARG;
  if (shape->T == 0) return MOE_OK;
  if (!pair_row || !topk_weights || !out || (cap_expert > 0 && !expert_out)) return MOE_ERR_ARG;
  if (!aligned16(expert_out) || !aligned16(out) || !aligned16(out_f32)) return MOE_ERR_ARG;
  const int nvec = shape->H / 8;
  int v = 1, slices = 1;
  combine_tiling(nvec, shape->T, combine_groups(shape), &v, &slices);
  // Small batches: one 1 KiB group per wave and every slot requested at once.
  ByVec<CombineLaunch>::run(v, shape->T < kFillTokens && v <= 2,
                            dim3(blocks_for(int64_t(shape->T) * slices)),
                            static_cast<hipStream_t>(stream),
                            reinterpret_cast<const vec4*>(expert_out), pair_row, topk_weights,
                            reinterpret_cast<vec4*>(out), reinterpret_cast<vec4*>(out_f32),
                            shape->T, shape->k, nvec, slices, cap_expert, err_word);
  return launch_status();
}

int moe_combine_rank_partial(const moe_shape_t* shape, const uint16_t* expert_out,
                             const int32_t* rank_src_token, const int32_t* rank_offsets,
                             const int32_t* topk_ids, const int32_t* pair_row,
                             const float* topk_weights, int64_t cap_expert, int64_t cap_rank,
                             uint16_t* partial, float* partial_f32, int32_t* err_word,
                             void* stream) {
  if (!shape_ok(shape) || cap_rank < 0 || cap_expert < 0) return MOE_ERR_ARG;
  if (!rank_offsets) return MOE_ERR_ARG;
  const int64_t max_rows =
      std::min<int64_t>(cap_rank, int64_t(shape->T) * std::min(shape->k, shape->R));
  if (shape->T == 0 || max_rows == 0) return MOE_OK;
  if (!rank_src_token || !topk_ids || !pair_row || !topk_weights || !partial ||
      (cap_expert > 0 && !expert_out))
    return MOE_ERR_ARG;
  if (!aligned16(expert_out) || !aligned16(partial) || !aligned16(partial_f32))
    return MOE_ERR_ARG;
  const int nvec = shape->H / 8;
  int v = 1, slices = 1;
  combine_tiling(nvec, max_rows, kPartialGroups, &v, &slices);
  ByVec<RankPartialLaunch>::run(
      v, dim3(blocks_for(max_rows * slices)),
      static_cast<hipStream_t>(stream),
      reinterpret_cast<const vec4*>(expert_out), rank_src_token, rank_offsets, topk_ids, pair_row,
      topk_weights, reinterpret_cast<vec4*>(partial), reinterpret_cast<vec4*>(partial_f32),
      shape->T, shape->E, shape->R, shape->k, shape->E / shape->R, nvec, slices, cap_rank,
      cap_expert, err_word);
  return launch_status();
}

int moe_combine_ranks(const moe_shape_t* shape, const uint16_t* partial,
                      const int32_t* token_rank_slot, int64_t cap_rank, uint16_t* out,
                      float* out_f32, int32_t* err_word, void* stream) {
  if (!shape_ok(shape) || cap_rank < 0) return MOE_ERR_ARG;
  if (shape->T == 0) return MOE_OK;
  if (!token_rank_slot || !out || (cap_rank > 0 && !partial)) return MOE_ERR_ARG;
  if (!aligned16(partial) || !aligned16(out) || !aligned16(out_f32)) return MOE_ERR_ARG;
  const int nvec = shape->H / 8;
  int v = 1, slices = 1;
  combine_tiling(nvec, shape->T, kRankSumGroups, &v, &slices);
  ByVec<RankSumLaunch>::run(v, dim3(blocks_for(int64_t(shape->T) * slices)),
                            static_cast<hipStream_t>(stream),
                            reinterpret_cast<const vec4*>(partial), token_rank_slot,
                            reinterpret_cast<vec4*>(out), reinterpret_cast<vec4*>(out_f32),
                            shape->T, shape->R, nvec, slices, cap_rank, err_word);
  return launch_status();
}

}  // extern "C"
