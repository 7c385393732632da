// MoE token dispatch and combine for one GPU's share of an expert-parallel
// layer: HIP kernels for CDNA4 (gfx950, wave64) behind the C ABI declared in
// include/moe_dispatch.h.
//
// Pages cited (title, section):
//  [A2A]  "A2A backends" page, vincentzed.com/writing/a2a-backends
//  [GPUs] "How GPUs Talk to Each Other During LLM Inference"
//
// Kernels
//  layout_tiles     per tile of tokens: wavefront-ballot stable ranks and LDS
//                   histograms per expert and per rank ([A2A] sec 3.2 step 1)
//  layout_finalize  per block: tile prefix from the per-tile histograms,
//                   exclusive scans over experts and ranks, absolute rows
//                   ([A2A] sec 5.1: offsets list on the GPU, no CPU wait)
//  pack             one wave per token: read the row once, write one copy per
//                   distinct rank ([A2A] sec 1.3 third answer)
//  permute          one wave per rank-buffer row: read once, write once per
//                   local expert ([A2A] sec 3.3, sec 5.1 do_expand)
//  combine          one wave per token: k row gathers, fp32 FMA in slot
//                   order, bf16 round-to-nearest-even ([A2A] sec 1.1, 7.1;
//                   [GPUs] sec 3.3 fixed addition order)
// Row copies move 16 bytes per lane (global_load/store_dwordx4), 1 KiB per
// wave instruction; nothing here is a dense contraction, so no MFMA.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "moe_dispatch.h"

namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;                 // 4 waves per workgroup
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kSubTile = kBlock;            // tokens per layout sub-tile: one per thread
constexpr int kMaxTiles = 64;               // layout tiles per call (tile size grows with T)
constexpr int kMaxExperts = 1024;
constexpr int kMaxRanks = 64;
constexpr int kMaxK = 32;
constexpr int kExpertBits = 10;             // packed (wave rank << 10 | expert) in LDS
constexpr int kMaxVec = 16;                 // uint4 per lane held in registers per pass

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanes_below() {
  return (uint64_t(1) << lane_id()) - 1;  // lane 63: 2^63 - 1
}

__device__ __forceinline__ int read_lane(int v, int lane) {
  return __builtin_amdgcn_readlane(v, lane);
}

__device__ __forceinline__ void flag_error(int32_t* err_word, int bit) {
  if (err_word) atomicOr(err_word, bit);
}

// ---------------------------------------------------------------------------
// Layout

struct LayoutGeom {
  int T, E, R, k, m;   // m = experts per rank
  int ncols;           // E expert columns followed by R rank columns
  int tile_tokens;     // multiple of kSubTile
  int ntiles;
};

// Per tile: for every valid pair, its rank among the tile's pairs of the same
// expert (in (token, slot) order), and for every (token, rank) copy its rank
// among the tile's tokens with a copy on that rank; both are written into the
// output arrays, relative to the tile. The tile's per-column totals go to
// tile_counts[tile][col].
__global__ __launch_bounds__(kBlock) void layout_tiles(LayoutGeom g, const int32_t* __restrict__ ids,
                                                       int32_t* __restrict__ pair_row,
                                                       int32_t* __restrict__ token_rank_slot,
                                                       int32_t* __restrict__ tile_counts,
                                                       int32_t* err_word) {
  extern __shared__ int32_t smem[];
  int32_t* s_pack = smem;                              // [kSubTile * k]
  int32_t* s_cnt = s_pack + kSubTile * g.k;            // [kWavesPerBlock][ncols]
  int32_t* s_base = s_cnt + kWavesPerBlock * g.ncols;  // [ncols] running tile totals

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = lane_id();
  const int tile = blockIdx.x;
  const int ebits = 32 - __clz(g.E > 1 ? g.E - 1 : 1);  // bits that tell experts apart
  bool bad_id = false;

  for (int c = tid; c < g.ncols; c += kBlock) s_base[c] = 0;

  const int tile_t0 = tile * g.tile_tokens;
  const int tile_t1 = min(g.T, tile_t0 + g.tile_tokens);
  for (int t0 = tile_t0; t0 < tile_t1; t0 += kSubTile) {
    const int nt = min(kSubTile, tile_t1 - t0);
    const int npairs = nt * g.k;
    __syncthreads();  // previous sub-tile done with s_pack / s_cnt
    for (int p = tid; p < kSubTile * g.k; p += kBlock)
      s_pack[p] = p < npairs ? ids[(int64_t)t0 * g.k + p] : -1;
    for (int c = tid; c < kWavesPerBlock * g.ncols; c += kBlock) s_cnt[c] = 0;
    __syncthreads();

    // Expert ranks. Wave w owns tokens [64w, 64w+64) of the sub-tile, i.e. the
    // contiguous pairs [64wk, 64(w+1)k); it walks them 64 at a time in order.
    // Lanes holding the same expert find each other with one ballot per id
    // bit; the rank is the number of such lanes below plus the wave's running
    // count for that expert.
    int32_t* cnt_w = s_cnt + wave * g.ncols;
    for (int ch = 0; ch < g.k; ++ch) {
      const int pl = wave * kWave * g.k + ch * kWave + lane;
      const int e = s_pack[pl];
      const bool valid = e >= 0 && e < g.E;
      bad_id |= (e != -1) && !valid;
      uint64_t peers = __ballot(valid);
      for (int b = 0; b < ebits; ++b) {
        const uint64_t ones = __ballot(valid && ((e >> b) & 1));
        peers &= ((e >> b) & 1) ? ones : ~ones;
      }
      if (valid) {
        const int below = __popcll(peers & lanes_below());
        const int base = cnt_w[e];
        s_pack[pl] = ((base + below) << kExpertBits) | e;
        if (below == 0) cnt_w[e] = base + __popcll(peers);
      } else {
        s_pack[pl] = -1;
      }
    }
    __syncthreads();

    // Rank masks: one token per thread.
    const int tl = tid;
    uint64_t mask = 0;
    for (int j = 0; j < g.k; ++j) {
      const int v = s_pack[tl * g.k + j];
      if (v >= 0) mask |= uint64_t(1) << ((v & ((1 << kExpertBits) - 1)) / g.m);
    }
    for (int r = 0; r < g.R; ++r) {
      const uint64_t on = __ballot((mask >> r) & 1);
      if (lane == 0) cnt_w[g.E + r] = __popcll(on);
    }
    __syncthreads();

    // Per column: wave bases inside this sub-tile, on top of the tile's
    // running total; then advance the running total.
    for (int c = tid; c < g.ncols; c += kBlock) {
      int run = s_base[c];
      for (int w = 0; w < kWavesPerBlock; ++w) {
        const int v = s_cnt[w * g.ncols + c];
        s_cnt[w * g.ncols + c] = run;
        run += v;
      }
      s_base[c] = run;
    }
    __syncthreads();

    // Write tile-relative positions.
    for (int ch = 0; ch < g.k; ++ch) {
      const int pl = wave * kWave * g.k + ch * kWave + lane;
      if (pl < npairs) {
        const int v = s_pack[pl];
        int out = -1;
        if (v >= 0) out = cnt_w[v & ((1 << kExpertBits) - 1)] + (v >> kExpertBits);
        pair_row[(int64_t)t0 * g.k + pl] = out;
      }
    }
    for (int r = 0; r < g.R; ++r) {
      const uint64_t on = __ballot((mask >> r) & 1);
      if (tl < nt) {
        const int out = ((mask >> r) & 1) ? cnt_w[g.E + r] + __popcll(on & lanes_below()) : -1;
        token_rank_slot[(int64_t)(t0 + tl) * g.R + r] = out;
      }
    }
  }
  __syncthreads();
  for (int c = tid; c < g.ncols; c += kBlock) tile_counts[(int64_t)tile * g.ncols + c] = s_base[c];
  if (__ballot(bad_id) && lane == 0) flag_error(err_word, MOE_ERRBIT_BAD_ID);
}

// Exclusive scan of s[0..n) in place, by one workgroup; returns the total.
__device__ int block_exclusive_scan(int32_t* s, int n, int32_t* s_tmp /* [kWavesPerBlock] */) {
  const int tid = threadIdx.x;
  const int per = (n + kBlock - 1) / kBlock;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += s[i];
  // inclusive scan of per-thread sums across the wave
  int x = sum;
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d, kWave);
    if (lane_id() >= d) x += y;
  }
  const int wave = tid / kWave;
  if (lane_id() == kWave - 1) s_tmp[wave] = x;
  __syncthreads();
  int wave_base = 0, total = 0;
  for (int w = 0; w < kWavesPerBlock; ++w) {
    if (w < wave) wave_base += s_tmp[w];
    total += s_tmp[w];
  }
  int run = wave_base + x - sum;
  for (int i = lo; i < hi; ++i) {
    const int v = s[i];
    s[i] = run;
    run += v;
  }
  __syncthreads();
  return total;
}

// Absolute rows: tile prefix (sum of the earlier tiles' counts) plus the
// column's exclusive offset (experts scanned in id order, ranks in rank order).
__global__ __launch_bounds__(kBlock) void layout_finalize(
    LayoutGeom g, const int32_t* __restrict__ ids, const int32_t* __restrict__ tile_counts,
    int32_t* __restrict__ pair_row, int32_t* __restrict__ token_rank_slot,
    int32_t* __restrict__ rank_counts, int32_t* __restrict__ rank_offsets,
    int32_t* __restrict__ expert_counts, int32_t* __restrict__ expert_offsets) {
  __shared__ int32_t s_tot[kMaxExperts + kMaxRanks];
  __shared__ int32_t s_pre[kMaxExperts + kMaxRanks];
  __shared__ int32_t s_tmp[kWavesPerBlock];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kSubTile;
  const int my_tile = t0 / g.tile_tokens;

  for (int c = tid; c < g.ncols; c += kBlock) {
    int tot = 0, pre = 0;
    for (int i = 0; i < g.ntiles; ++i) {
      const int v = tile_counts[(int64_t)i * g.ncols + c];
      tot += v;
      pre += (i < my_tile) ? v : 0;
    }
    s_tot[c] = tot;
    s_pre[c] = pre;
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int c = tid; c < g.E; c += kBlock) expert_counts[c] = s_tot[c];
    for (int c = tid; c < g.R; c += kBlock) rank_counts[c] = s_tot[g.E + c];
  }
  __syncthreads();
  const int nexp = block_exclusive_scan(s_tot, g.E, s_tmp);
  const int ncopy = block_exclusive_scan(s_tot + g.E, g.R, s_tmp);
  if (blockIdx.x == 0) {
    for (int c = tid; c < g.E; c += kBlock) expert_offsets[c] = s_tot[c];
    for (int c = tid; c < g.R; c += kBlock) rank_offsets[c] = s_tot[g.E + c];
    if (tid == 0) {
      expert_offsets[g.E] = nexp;
      rank_offsets[g.R] = ncopy;
    }
  }
  for (int c = tid; c < g.ncols; c += kBlock) s_pre[c] += s_tot[c];
  __syncthreads();

  const int nt = min(kSubTile, g.T - t0);
  if (nt <= 0) return;
  const int64_t p0 = (int64_t)t0 * g.k;
  for (int p = tid; p < nt * g.k; p += kBlock) {
    const int v = pair_row[p0 + p];
    if (v >= 0) pair_row[p0 + p] = v + s_pre[ids[p0 + p]];
  }
  const int64_t s0 = (int64_t)t0 * g.R;
  for (int s = tid; s < nt * g.R; s += kBlock) {
    const int v = token_rank_slot[s0 + s];
    if (v >= 0) token_rank_slot[s0 + s] = v + s_pre[g.E + s % g.R];
  }
}

LayoutGeom layout_geometry(const moe_shape_t& sh) {
  LayoutGeom g;
  g.T = sh.T;
  g.E = sh.E;
  g.R = sh.R;
  g.k = sh.k;
  g.m = sh.E / sh.R;
  g.ncols = sh.E + sh.R;
  const int64_t per_tile = (int64_t(sh.T) + kMaxTiles - 1) / kMaxTiles;
  const int64_t subs = (per_tile + kSubTile - 1) / kSubTile;
  g.tile_tokens = int(std::max<int64_t>(1, subs) * kSubTile);
  g.ntiles = int((int64_t(sh.T) + g.tile_tokens - 1) / g.tile_tokens);
  return g;
}

size_t layout_smem_bytes(const LayoutGeom& g) {
  return sizeof(int32_t) * (size_t(kSubTile) * g.k + size_t(kWavesPerBlock) * g.ncols + g.ncols);
}

// ---------------------------------------------------------------------------
// Row movers. A row is `nvec` uint4 (8 bf16 each). A wave moves a row in
// passes of 64*V uint4: lane l holds columns c0 + l, c0 + 64 + l, ..., so each
// wave instruction touches 1 KiB of contiguous bytes, and all V loads of a
// pass are in flight before the first store. Columns past the last full pass
// (only when H is not a multiple of 512*V) go one uint4 per lane at a time.

// Copies the row at `src` to every row dst_row(d) for d in the lane mask
// `dests`, where dst_row(d) = readlane(row_of_lane, d).
template <int V>
__device__ __forceinline__ void fan_out_row(const uint4* src, uint4* dst_base,
                                            int row_of_lane, uint64_t dests, int nvec) {
  const int lane = lane_id();
  int c0 = 0;
  for (; c0 + kWave * V <= nvec; c0 += kWave * V) {
    uint4 v[V];
#pragma unroll
    for (int q = 0; q < V; ++q) v[q] = src[c0 + q * kWave + lane];
    uint64_t d = dests;
    while (d) {
      const int which = __ffsll((unsigned long long)d) - 1;
      d &= d - 1;
      uint4* dst = dst_base + (int64_t)read_lane(row_of_lane, which) * nvec;
#pragma unroll
      for (int q = 0; q < V; ++q) dst[c0 + q * kWave + lane] = v[q];
    }
  }
  for (int c = c0 + lane; c < nvec; c += kWave) {
    const uint4 v = src[c];
    uint64_t d = dests;
    while (d) {
      const int which = __ffsll((unsigned long long)d) - 1;
      d &= d - 1;
      dst_base[(int64_t)read_lane(row_of_lane, which) * nvec + c] = v;
    }
  }
}

template <int V>
__global__ __launch_bounds__(kBlock) void pack_rows(const uint4* hidden,
                                                    const int32_t* __restrict__ token_rank_slot,
                                                    uint4* rank_buf,
                                                    int32_t* __restrict__ rank_src_token, int T,
                                                    int R, int nvec, int64_t cap_rank,
                                                    int32_t* err_word) {
  const int lane = lane_id();
  const int t = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  if (t >= T) return;
  const int slot = lane < R ? token_rank_slot[(int64_t)t * R + lane] : -1;
  const bool ok = slot >= 0 && slot < cap_rank;
  if (__ballot(slot >= 0 && !ok) && lane == 0) flag_error(err_word, MOE_ERRBIT_RANK_CAP);
  if (ok) rank_src_token[slot] = t;
  const uint64_t dests = __ballot(ok);
  if (dests) fan_out_row<V>(hidden + (int64_t)t * nvec, rank_buf, slot, dests, nvec);
}

template <int V>
__global__ __launch_bounds__(kBlock) void permute_rows(
    const uint4* rank_buf, const int32_t* __restrict__ rank_src_token,
    const int32_t* __restrict__ rank_offsets, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ pair_row, uint4* expert_buf,
    int32_t* __restrict__ expert_src_pair, int T, int E, int R, int k, int m, int nvec,
    int64_t cap_rank, int64_t cap_expert, int32_t* err_word) {
  const int lane = lane_id();
  const int64_t i = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  const int64_t rows = min((int64_t)rank_offsets[R], cap_rank);
  if (i >= rows) return;
  // segment of row i: number of segment ends at or below i
  const int end = lane < R ? rank_offsets[lane + 1] : 0x7FFFFFFF;
  const int r = __popcll(__ballot(lane < R && end <= i));
  const int t = rank_src_token[i];
  if (t < 0 || t >= T) return;
  const int e = lane < k ? ids[(int64_t)t * k + lane] : -1;
  const bool here = e >= 0 && e < E && e / m == r;
  const int p = here ? pair_row[(int64_t)t * k + lane] : -1;
  const bool ok = here && p >= 0 && p < cap_expert;
  if (__ballot(here && !ok) && lane == 0) flag_error(err_word, MOE_ERRBIT_EXPERT_CAP);
  if (ok) expert_src_pair[p] = t * k + lane;
  const uint64_t dests = __ballot(ok);
  if (dests) fan_out_row<V>(rank_buf + i * nvec, expert_buf, p, dests, nvec);
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;  // NaN stays quiet NaN
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void fma_bf16x8(float (&acc)[8], float w, const uint4& y) {
  const uint32_t h[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] = __builtin_fmaf(w, __uint_as_float(h[i] << 16), acc[2 * i]);
    acc[2 * i + 1] = __builtin_fmaf(w, __uint_as_float(h[i] & 0xFFFF0000u), acc[2 * i + 1]);
  }
}

__device__ __forceinline__ void store_sum(const float (&acc)[8], uint4* __restrict__ out,
                                          float4* __restrict__ out_f32, int64_t at) {
  uint4 o;
  o.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
  o.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
  o.z = f32_to_bf16_rne(acc[4]) | (f32_to_bf16_rne(acc[5]) << 16);
  o.w = f32_to_bf16_rne(acc[6]) | (f32_to_bf16_rne(acc[7]) << 16);
  out[at] = o;
  if (out_f32) {
    out_f32[2 * at] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    out_f32[2 * at + 1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

template <int V>
__global__ __launch_bounds__(kBlock) void combine_rows(
    const uint4* expert_out, const int32_t* __restrict__ pair_row,
    const float* __restrict__ weights, uint4* __restrict__ out, float4* __restrict__ out_f32,
    int T, int k, int nvec, int64_t cap_expert, int32_t* err_word) {
  const int lane = lane_id();
  const int t = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  if (t >= T) return;
  const int p = lane < k ? pair_row[(int64_t)t * k + lane] : -1;
  const float wt = lane < k ? weights[(int64_t)t * k + lane] : 0.0f;
  const bool ok = p >= 0 && p < cap_expert;
  if (__ballot(p >= 0 && !ok) && lane == 0) flag_error(err_word, MOE_ERRBIT_EXPERT_CAP);
  const uint64_t slots = __ballot(ok);
  const int64_t row0 = (int64_t)t * nvec;

  int c0 = 0;
  for (; c0 + kWave * V <= nvec; c0 += kWave * V) {
    float acc[V][8];
#pragma unroll
    for (int q = 0; q < V; ++q)
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[q][x] = 0.0f;
    uint64_t s = slots;
    while (s) {  // ascending slot order
      const int j = __ffsll((unsigned long long)s) - 1;
      s &= s - 1;
      const uint4* src = expert_out + (int64_t)read_lane(p, j) * nvec + c0 + lane;
      const float w = __int_as_float(read_lane(__float_as_int(wt), j));
      uint4 y[V];
#pragma unroll
      for (int q = 0; q < V; ++q) y[q] = src[q * kWave];
#pragma unroll
      for (int q = 0; q < V; ++q) fma_bf16x8(acc[q], w, y[q]);
    }
#pragma unroll
    for (int q = 0; q < V; ++q) store_sum(acc[q], out, out_f32, row0 + c0 + q * kWave + lane);
  }
  for (int c = c0 + lane; c < nvec; c += kWave) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    uint64_t s = slots;
    while (s) {
      const int j = __ffsll((unsigned long long)s) - 1;
      s &= s - 1;
      const float w = __int_as_float(read_lane(__float_as_int(wt), j));
      fma_bf16x8(acc, w, expert_out[(int64_t)read_lane(p, j) * nvec + c]);
    }
    store_sum(acc, out, out_f32, row0 + c);
  }
}

// ---------------------------------------------------------------------------
// Host side

bool shape_ok(const moe_shape_t* s) {
  if (!s) return false;
  if (s->T < 0 || s->H <= 0 || s->H % 8 != 0) return false;
  if (s->R < 1 || s->R > kMaxRanks || s->E < 1 || s->E > kMaxExperts || s->E % s->R != 0)
    return false;
  if (s->k < 1 || s->k > kMaxK) return false;
  if (int64_t(s->T) * s->k >= (int64_t(1) << 30)) return false;
  if (int64_t(s->T) * s->R >= (int64_t(1) << 31)) return false;
  return true;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int launch_status() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Register tile V (uint4 per lane per pass): the whole row in one pass when
// it has at most 16 groups of 64 uint4, else a divisor of the group count in
// [8, 16] if there is one (no tail), else 16.
int vec_per_lane(int nvec) {
  const int groups = nvec / kWave;
  if (groups <= 1) return 1;
  if (groups <= kMaxVec) return groups;
  for (int v = kMaxVec; v >= 8; --v)
    if (groups % v == 0) return v;
  return kMaxVec;
}

int blocks_for(int64_t waves) { return int((waves + kWavesPerBlock - 1) / kWavesPerBlock); }

// Picks the instantiation whose per-lane register tile V covers the row in
// as few passes as possible.
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
  static void go(dim3 grid, hipStream_t st, const uint4* hid, const int32_t* slots, uint4* rb,
                 int32_t* src, int T, int R, int nvec, int64_t cap, int32_t* err) {
    hipLaunchKernelGGL(pack_rows<V>, grid, dim3(kBlock), 0, st, hid, slots, rb, src, T, R, nvec,
                       cap, err);
  }
};

template <int V>
struct PermuteLaunch {
  static void go(dim3 grid, hipStream_t st, const uint4* rb, const int32_t* src,
                 const int32_t* roff, const int32_t* ids, const int32_t* prow, uint4* eb,
                 int32_t* esrc, int T, int E, int R, int k, int m, int nvec, int64_t cap_rank,
                 int64_t cap_expert, int32_t* err) {
    hipLaunchKernelGGL(permute_rows<V>, grid, dim3(kBlock), 0, st, rb, src, roff, ids, prow, eb,
                       esrc, T, E, R, k, m, nvec, cap_rank, cap_expert, err);
  }
};

template <int V>
struct CombineLaunch {
  static void go(dim3 grid, hipStream_t st, const uint4* eo, const int32_t* prow,
                 const float* w, uint4* out, float4* out32, int T, int k, int nvec,
                 int64_t cap_expert, int32_t* err) {
    hipLaunchKernelGGL(combine_rows<V>, grid, dim3(kBlock), 0, st, eo, prow, w, out, out32, T, k,
                       nvec, cap_expert, err);
  }
};

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_DISPATCH_ABI_VERSION; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument";
    case MOE_ERR_HIP: return "HIP launch failure";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

size_t moe_layout_workspace_bytes(const moe_shape_t* shape) {
  if (!shape_ok(shape)) return 0;
  const LayoutGeom g = layout_geometry(*shape);
  return sizeof(int32_t) * size_t(std::max(g.ntiles, 1)) * size_t(g.ncols);
}

int moe_dispatch_layout(const moe_shape_t* shape, const int32_t* topk_ids, int32_t* rank_counts,
                        int32_t* rank_offsets, int32_t* expert_counts, int32_t* expert_offsets,
                        int32_t* token_rank_slot, int32_t* pair_row, void* workspace,
                        size_t workspace_bytes, int32_t* err_word, void* stream) {
  if (!shape_ok(shape)) return MOE_ERR_ARG;
  if (!rank_counts || !rank_offsets || !expert_counts || !expert_offsets) return MOE_ERR_ARG;
  if (shape->T > 0 && (!topk_ids || !token_rank_slot || !pair_row)) return MOE_ERR_ARG;
  const size_t need = moe_layout_workspace_bytes(shape);
  if (!workspace || workspace_bytes < need) return MOE_ERR_WORKSPACE;
  const LayoutGeom g = layout_geometry(*shape);
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* tile_counts = static_cast<int32_t*>(workspace);
  if (g.ntiles > 0) {
    hipLaunchKernelGGL(layout_tiles, dim3(g.ntiles), dim3(kBlock), layout_smem_bytes(g), st, g,
                       topk_ids, pair_row, token_rank_slot, tile_counts, err_word);
    if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  }
  const int fin_blocks = std::max(1, (g.T + kSubTile - 1) / kSubTile);
  hipLaunchKernelGGL(layout_finalize, dim3(fin_blocks), dim3(kBlock), 0, st, g, topk_ids,
                     tile_counts, pair_row, token_rank_slot, rank_counts, rank_offsets,
                     expert_counts, expert_offsets);
  return launch_status();
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
  ByVec<PackLaunch>::run(vec_per_lane(nvec), dim3(blocks_for(shape->T)),
                         static_cast<hipStream_t>(stream),
                         reinterpret_cast<const uint4*>(hidden), token_rank_slot,
                         reinterpret_cast<uint4*>(rank_buf), rank_src_token, shape->T, shape->R,
                         nvec, cap_rank, err_word);
  return launch_status();
}

int moe_permute_by_expert(const moe_shape_t* shape, const uint16_t* rank_buf,
                          const int32_t* rank_src_token, const int32_t* rank_offsets,
                          const int32_t* topk_ids, const int32_t* pair_row, int64_t cap_rank,
                          uint16_t* expert_buf, int32_t* expert_src_pair, int64_t cap_expert,
                          int32_t* err_word, void* stream) {
  if (!shape_ok(shape) || cap_rank < 0 || cap_expert < 0) return MOE_ERR_ARG;
  if (!rank_offsets) return MOE_ERR_ARG;
  const int64_t max_rows =
      std::min<int64_t>(cap_rank, int64_t(shape->T) * std::min(shape->k, shape->R));
  if (shape->T == 0 || max_rows == 0) return MOE_OK;
  if (!rank_buf || !rank_src_token || !topk_ids || !pair_row ||
      (cap_expert > 0 && (!expert_buf || !expert_src_pair)))
    return MOE_ERR_ARG;
  if (!aligned16(rank_buf) || !aligned16(expert_buf)) return MOE_ERR_ARG;
  const int nvec = shape->H / 8;
  ByVec<PermuteLaunch>::run(vec_per_lane(nvec), dim3(blocks_for(max_rows)),
                            static_cast<hipStream_t>(stream),
                            reinterpret_cast<const uint4*>(rank_buf), rank_src_token,
                            rank_offsets, topk_ids, pair_row,
                            reinterpret_cast<uint4*>(expert_buf), expert_src_pair, shape->T,
                            shape->E, shape->R, shape->k, shape->E / shape->R, nvec, cap_rank,
                            cap_expert, err_word);
  return launch_status();
}

int moe_combine(const moe_shape_t* shape, const uint16_t* expert_out, const int32_t* pair_row,
                const float* topk_weights, int64_t cap_expert, uint16_t* out, float* out_f32,
                int32_t* err_word, void* stream) {
  if (!shape_ok(shape) || cap_expert < 0) return MOE_ERR_ARG;
  if (shape->T == 0) return MOE_OK;
  if (!pair_row || !topk_weights || !out || (cap_expert > 0 && !expert_out)) return MOE_ERR_ARG;
  if (!aligned16(expert_out) || !aligned16(out) || !aligned16(out_f32)) return MOE_ERR_ARG;
  const int nvec = shape->H / 8;
  ByVec<CombineLaunch>::run(vec_per_lane(nvec), dim3(blocks_for(shape->T)),
                            static_cast<hipStream_t>(stream),
                            reinterpret_cast<const uint4*>(expert_out), pair_row, topk_weights,
                            reinterpret_cast<uint4*>(out), reinterpret_cast<float4*>(out_f32),
                            shape->T, shape->k, nvec, cap_expert, err_word);
  return launch_status();
}

}  // extern "C"
