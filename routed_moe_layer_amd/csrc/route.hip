// Expert routing: a stable counting sort of the flat ids f = t*K + j by expert id.
//
// "torch_npu.npu_moe_init_routing_v2" (section 计算公式): step 1 keyValueSort(expertIdx,
// rowIdx), step 2 the gather map expandedRowIdx[sortedRowIdx[i]] = i, step 3 the
// per-expert histogram as an inclusive prefix sum.  The sort must be stable (equal experts
// keep increasing f) so that the result is unique.  The same page's options are handled
// here too: an active expert range (ids outside it take no part; step 6's
// availableIdxNum is the in-range count), the count and key_value histogram modes, and
// drop/pad slots e*capacity + rank (-1 past the capacity).
//
// Three launches (four above 64 tiles; one for at most kRouteTile ids, see
// route_small_kernel), no host
// readback ("Cake SiTU backend", intro: routing values never take part in host dispatch):
//   hist    : one workgroup per tile of 1024 flat ids; LDS histogram -> tile_hist[tile][e].
//   scan    : per expert, exclusive scan of tile_hist over tiles (in place; above 64 tiles
//             by a column kernel with one workgroup per 64 experts) and the counts; then
//             one workgroup: exclusive/inclusive expert offsets, optionally the grouped-GEMM
//             work lists (small and big token tiles, FC2 runs), and a reset of the SiTU
//             amax stats.
//   scatter : one workgroup per tile; each wave ranks its 256 ids stably with ballot-based
//             key matching (one ballot per key bit), waves are ordered through an LDS
//             per-wave histogram, and every id lands at
//             offset[e] + tile_base[tile][e] + wave_base[w][e] + rank.
#include "common.h"
#include "kernels.h"

namespace rmoe {

constexpr int kIdsPerThread = kRouteTile / kRouteThreads;   // 4
constexpr int kScanBatch = 16;
constexpr size_t kRouteSmallMaxLds = 64 * 1024;   // dynamic LDS of the fused small kernel

// Key of flat id f: its expert id relative to the first routed expert (unsigned wrap, so
// ids below the range come out >= E); -1 past the end of the ids.
__device__ __forceinline__ int route_key(const int32_t* __restrict__ ids, int64_t f, int64_t n,
                                         int e_base) {
  return f < n ? static_cast<int>(static_cast<uint32_t>(ids[f]) - static_cast<uint32_t>(e_base))
               : -1;
}
__device__ __forceinline__ bool key_valid(int e, int E) {
  return static_cast<unsigned>(e) < static_cast<unsigned>(E);
}

__global__ __launch_bounds__(kRouteThreads) void route_hist_kernel(
    const int32_t* __restrict__ ids, int64_t n, int E, int e_base,
    int32_t* __restrict__ tile_hist) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kRouteTile;
  for (int i = threadIdx.x; i < kRouteTile; i += blockDim.x) {
    const int e = route_key(ids, base + i, n, e_base);
    if (key_valid(e, E)) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  int32_t* out = tile_hist + static_cast<int64_t>(blockIdx.x) * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) out[e] = hist[e];
}

// The three per-expert quantities the expert scans need, packed into one 64-bit value so
// that one block scan serves all three: rows (26 bits; at most 2^24 ids per call), small
// tiles or nonzero experts (19 bits; at most 10240 experts), big tiles (19 bits; at most
// 2^20 / kBigRows + 4096 for the layer's 2^20 routed rows over at most 4096 experts).
constexpr int kRowBits = 26, kTileBits = 19;
__device__ __forceinline__ uint64_t pack_counts(int cnt, int n_small, int n_big) {
  return static_cast<uint64_t>(cnt) | (static_cast<uint64_t>(n_small) << kRowBits) |
         (static_cast<uint64_t>(n_big) << (kRowBits + kTileBits));
}
__device__ __forceinline__ int field(uint64_t v, int i) {
  const int shift = i == 0 ? 0 : kRowBits + (i - 1) * kTileBits;
  const int bits = i == 0 ? kRowBits : kTileBits;
  return static_cast<int>((v >> shift) & ((uint64_t{1} << bits) - 1));
}

// One DPP step of a wave scan on a 64-bit value: lane i takes the value of the lane the
// row control selects (zero where that lane lies outside the row or the row is masked).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_take64(uint64_t v) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
      0, static_cast<int>(static_cast<uint32_t>(v)), CTRL, ROW_MASK, 0xF, true));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
      0, static_cast<int>(static_cast<uint32_t>(v >> 32)), CTRL, ROW_MASK, 0xF, true));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Inclusive scan over the 64 lanes of a wave: prefix sums within each row of 16 lanes by
// shifts of 1, 2, 4 and 8 lanes, then lane 15 of rows 0 and 2 added to rows 1 and 3, and
// lane 31 (the total of rows 0-1) to rows 2 and 3.
__device__ __forceinline__ uint64_t wave_incl_scan64(uint64_t x) {
  x += dpp_take64<0x111, 0xF>(x);      // row_shr:1
  x += dpp_take64<0x112, 0xF>(x);      // row_shr:2
  x += dpp_take64<0x114, 0xF>(x);      // row_shr:4
  x += dpp_take64<0x118, 0xF>(x);      // row_shr:8
  x += dpp_take64<0x142, 0xA>(x);      // row_bcast:15 into rows 1 and 3
  x += dpp_take64<0x143, 0xC>(x);      // row_bcast:31 into rows 2 and 3
  return x;
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int lane) {
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), lane));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), lane));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Block-wide exclusive scan of one uint64 per thread (any multiple of 64 threads up to
// 1024); returns the exclusive prefix and writes the total to *total.
__device__ uint64_t block_excl_scan64(uint64_t v, uint64_t* sh, uint64_t* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
  const int nw = blockDim.x / kWave;
  const uint64_t incl = wave_incl_scan64(v);
  if (lane == kWave - 1) sh[w] = incl;
  __syncthreads();
  // every wave scans the (at most 16) wave totals itself
  const uint64_t x = wave_incl_scan64(lane < nw ? sh[lane] : 0);
  const uint64_t wave_excl = w == 0 ? 0 : readlane64(x, w - 1);
  *total = readlane64(x, nw - 1);
  __syncthreads();                                // sh is free for the next scan
  return wave_excl + incl - v;
}

// Token tiles of one expert with `cnt` rows: (number of tiles, rows per tile but the last).
// With small_only every tile is a small one (at most kSmallRows rows).
__device__ __forceinline__ void expert_tiles(int cnt, bool small_only, int* n_small,
                                             int* n_big, int* base) {
  *n_small = 0; *n_big = 0; *base = 0;
  if (cnt <= 0) return;
  if (cnt <= kSmallRows) { *n_small = 1; *base = cnt; return; }
  if (small_only) {
    *n_small = (cnt + kSmallRows - 1) / kSmallRows;
    *base = kSmallRows;
    return;
  }
  const int nb = (cnt + kBigTileRows - 1) / kBigTileRows;
  const int b = min(kBigTileRows, ((cnt + nb - 1) / nb + 15) / 16 * 16);
  *base = b;
  *n_big = (cnt + b - 1) / b;
}

// One round of the expert scan over experts e0 .. e0 + blockDim.x - 1; thread e - e0 holds
// expert e's count `cnt` (0 for e >= E).  Writes the expert offsets (also to off_sh when
// given), the inclusive cumsum, and either the grouped-GEMM tile lists or the key-value
// pairs, and when asked the FC2 runs (up to kRunTiles consecutive big tiles of one
// expert).  carry[0..3] are the running totals of rows, small tiles (or nonzero experts),
// big tiles and runs; they are updated for the next round.
__device__ void scan_experts_round(const RouteBuffers& b, int E, int e, int cnt, uint64_t* sh,
                                   int* carry, int32_t* off_sh) {
  const bool lists = b.tiles_small != nullptr;
  int n_small, n_big, base;
  expert_tiles(lists ? cnt : 0, b.small_only != 0, &n_small, &n_big, &base);
  if (b.key_value) n_small = cnt > 0 ? 1 : 0;
  uint64_t tot;
  const uint64_t ex = block_excl_scan64(pack_counts(cnt, n_small, n_big), sh, &tot);
  const int total = field(tot, 0), stotal = field(tot, 1), btotal = field(tot, 2);
  const int sexcl = field(ex, 1), bexcl = field(ex, 2);
  const int off = carry[0] + field(ex, 0);
  if (e < E) {
    b.offsets[e] = off;
    if (off_sh) off_sh[e] = off;
    if (b.cumsum) b.cumsum[e] = off + cnt;
    if (n_small) {
      const int slot = carry[1] + sexcl;
      if (lists) {
        for (int j = 0; j < n_small; ++j)
          b.tiles_small[slot + j] = TileDesc{e, off + j * base, min(base, cnt - j * base), 0};
      } else {
        b.key_value[2 * slot] = e + b.e_base;
        b.key_value[2 * slot + 1] = cnt;
      }
    }
    for (int j = 0; j < n_big; ++j)
      b.tiles_big[carry[2] + bexcl + j] = TileDesc{e, off + j * base, min(base, cnt - j * base), 0};
  }
  int rtotal = 0;
  if (b.runs) {
    const int n_runs = (n_big + kRunTiles - 1) / kRunTiles;
    uint64_t rtot;
    const int rexcl = static_cast<int>(block_excl_scan64(static_cast<uint64_t>(n_runs), sh, &rtot));
    rtotal = static_cast<int>(rtot);
    if (e < E)
      for (int j = 0; j < n_runs; ++j) {
        const int r0 = j * kRunTiles * base;
        b.runs[carry[3] + rexcl + j] = TileDesc{e, off + r0, min(kRunTiles * base, cnt - r0), 0};
      }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    carry[0] += total; carry[1] += stotal; carry[2] += btotal; carry[3] += rtotal;
  }
  __syncthreads();
}

// After the last round: the total, the tile counts, and the zero rows of the key-value
// output past the nonzero experts.
__device__ void scan_experts_finish(const RouteBuffers& b, int E, const int* carry) {
  if (threadIdx.x == 0) {
    b.offsets[E] = carry[0];
    if (b.available) b.available[0] = carry[0];
    if (b.num_tiles) {
      b.num_tiles[0] = carry[1];
      b.num_tiles[1] = carry[2];
      b.num_tiles[2] = b.runs ? carry[3] : 0;
    }
  }
  if (b.key_value)
    for (int i = carry[1] + threadIdx.x; i < b.kv_rows; i += blockDim.x) {
      b.key_value[2 * i] = 0;
      b.key_value[2 * i + 1] = 0;
    }
}

// Column scan for many tiles: workgroup c owns experts [64c, 64c + 64) (one per lane); its
// 16 waves split the tiles into 16 contiguous ranges, sum them, take the exclusive prefix
// over waves in LDS, and rewrite their tile histograms in place as per-tile bases
// (exclusive over tiles) while the last wave writes the expert counts.  Each thread has
// one batch of loads in flight per range pass, where one workgroup walking all the tiles
// of every expert waits ntiles / kScanBatch memory latencies.
constexpr int kScanExperts = 64, kScanWaves = 16;
constexpr int kColumnScanTiles = 64;        // above this many tiles the column scan runs

__global__ __launch_bounds__(kScanExperts * kScanWaves) void route_colscan_kernel(
    RouteBuffers b, int ntiles, int E) {
  __shared__ int part[kScanWaves][kScanExperts];
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int e = blockIdx.x * kScanExperts + lane;
  const int per = (ntiles + kScanWaves - 1) / kScanWaves;
  const int t0 = min(ntiles, w * per), t1 = min(ntiles, t0 + per);
  int32_t* __restrict__ col = b.tile_hist + e;
  int sum = 0;
  int v[kScanBatch];
  if (e < E) {
    for (int tb = t0; tb < t1; tb += kScanBatch) {
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i)
        v[i] = tb + i < t1 ? col[static_cast<int64_t>(tb + i) * E] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) sum += v[i];
    }
  }
  part[w][lane] = sum;
  __syncthreads();
  if (e >= E) return;
  int base = 0;
  for (int i = 0; i < w; ++i) base += part[i][lane];
  if (t1 - t0 <= kScanBatch) {
    // one batch: its values are still in v
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i)
      if (t0 + i < t1) {
        col[static_cast<int64_t>(t0 + i) * E] = base;
        base += v[i];
      }
  } else {
    for (int tb = t0; tb < t1; tb += kScanBatch) {
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i)
        v[i] = tb + i < t1 ? col[static_cast<int64_t>(tb + i) * E] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i)
        if (tb + i < t1) {
          col[static_cast<int64_t>(tb + i) * E] = base;
          base += v[i];
        }
    }
  }
  if (w == kScanWaves - 1) {
    b.counts[e] = base;
    if (b.amax_reset) b.amax_reset[e] = 0.0f;
  }
}

// The expert scan (one workgroup).  With `counted` the column scan has already turned the
// tile histograms into bases and written the counts; otherwise each thread scans its
// expert's tiles here first.
__global__ __launch_bounds__(1024) void route_scan_kernel(RouteBuffers b, int ntiles, int E,
                                                          int counted) {
  __shared__ uint64_t sh[16];
  __shared__ int carry[4];
  if (threadIdx.x == 0) { carry[0] = 0; carry[1] = 0; carry[2] = 0; carry[3] = 0; }
  __syncthreads();
  int32_t* __restrict__ tile_hist = b.tile_hist;
  // Experts are handled in rounds of 1024.
  for (int e0 = 0; e0 < E; e0 += blockDim.x) {
    const int e = e0 + threadIdx.x;
    int cnt = 0;
    if (e < E && counted) {
      cnt = b.counts[e];
    } else if (e < E) {
      // exclusive over tiles, in place; kScanBatch independent loads in flight per step
      for (int t0 = 0; t0 < ntiles; t0 += kScanBatch) {
        int v[kScanBatch];
#pragma unroll
        for (int i = 0; i < kScanBatch; ++i)
          v[i] = t0 + i < ntiles ? tile_hist[static_cast<int64_t>(t0 + i) * E + e] : 0;
#pragma unroll
        for (int i = 0; i < kScanBatch; ++i) {
          if (t0 + i < ntiles) tile_hist[static_cast<int64_t>(t0 + i) * E + e] = cnt;
          cnt += v[i];
        }
      }
      b.counts[e] = cnt;
      if (b.amax_reset) b.amax_reset[e] = 0.0f;
    }
    scan_experts_round(b, E, e, cnt, sh, carry, nullptr);
  }
  scan_experts_finish(b, E, carry);
}

// Stable ranking of one wave's kIdsPerThread*64 consecutive flat ids (from wave_base):
// in rounds of 64, an id's rank is the number of equal keys in earlier rounds of this
// wave (my_hist, the wave's running per-expert count in LDS) plus the equal keys on
// lower lanes of its round (ballot-based key matching).  key[r] is the expert key (-1 for
// no id) and rank[r] the rank of round r's id.
__device__ __forceinline__ void rank_wave_ids(const int32_t* __restrict__ ids, int64_t n, int E,
                                              int nbits, int e_base, int64_t wave_base,
                                              int lane, int32_t* my_hist,
                                              int32_t* expanded_row_idx,
                                              int (&key)[kIdsPerThread],
                                              int (&rank)[kIdsPerThread]) {
  // all of the wave's id loads in flight together (unconditional, index clamped)
  int keys[kIdsPerThread];
#pragma unroll
  for (int r = 0; r < kIdsPerThread; ++r) {
    const int64_t f = wave_base + r * kWave + lane;
    const uint32_t raw = n > 0 ? static_cast<uint32_t>(ids[min(f, n - 1)]) : 0u;
    keys[r] = f < n ? static_cast<int>(raw - static_cast<uint32_t>(e_base)) : -1;
  }
  for (int r = 0; r < kIdsPerThread; ++r) {
    const int64_t f = wave_base + r * kWave + lane;
    int e = keys[r];
    // An id outside the routed range is dropped (never counted, never scattered) and its
    // position-map entry is -1, so no kernel indexes with it.
    const bool valid = key_valid(e, E);
    if (f < n && !valid) expanded_row_idx[f] = -1;
    if (!valid) e = 0;
    const uint64_t active = __ballot(valid);
    const uint64_t peers = match_key(static_cast<uint32_t>(e), nbits, active);
    const int before = valid ? my_hist[e] : 0;
    const int rk = before + __popcll(peers & lanemask_lt());
    // the lowest lane of each group of equal keys bumps the wave histogram
    if (valid && (peers & lanemask_lt()) == 0) my_hist[e] = before + __popcll(peers);
    key[r] = valid ? e : -1;
    rank[r] = rk;
    __builtin_amdgcn_wave_barrier();
  }
}

// Final placement of in-range flat id f of expert key e, rank r_in within its expert and
// expert offset off.
__device__ __forceinline__ int32_t place_id(const RouteBuffers& b, int e, int64_t f, int off,
                                            int r_in) {
  const int pos = off + r_in;
  if (b.sorted_ids) b.sorted_ids[pos] = e + b.e_base;
  if (b.sorted_row_idx) b.sorted_row_idx[pos] = static_cast<int32_t>(f);
  const int32_t m = b.capacity > 0 ? (r_in < b.capacity ? e * b.capacity + r_in : -1) : pos;
  b.expanded_row_idx[f] = m;
  return m;
}

// Sorted positions at and past the in-range total hold no id: -1.
__device__ __forceinline__ void fill_tail(const RouteBuffers& b, int64_t f, int64_t n,
                                          int total) {
  if (f < n && f >= total) {
    if (b.sorted_ids) b.sorted_ids[f] = -1;
    if (b.sorted_row_idx) b.sorted_row_idx[f] = -1;
  }
}

// Many experts (per-wave histograms of more than kScatterWaveHistMaxE experts would not fit
// in LDS): the tile's waves rank their ids in turn against one running histogram of the
// tile ([E] in LDS), so each rank already counts the earlier waves' ids of its expert.
constexpr int kScatterWaveHistMaxE = 4096;

__global__ __launch_bounds__(kRouteThreads) void route_scatter_seq_kernel(
    const int32_t* __restrict__ ids, int64_t n, int E, int nbits, RouteBuffers b) {
  extern __shared__ int32_t hist[];                // [E]
  const int nw = kRouteThreads / kWave;
  for (int i = threadIdx.x; i < E; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int64_t wave_base = static_cast<int64_t>(blockIdx.x) * kRouteTile + w * (kRouteTile / nw);
  int key[kIdsPerThread];
  int rank[kIdsPerThread];
  for (int turn = 0; turn < nw; ++turn) {
    if (w == turn)
      rank_wave_ids(ids, n, E, nbits, b.e_base, wave_base, lane, hist, b.expanded_row_idx, key,
                    rank);
    __syncthreads();
  }
  const int32_t* th = b.tile_hist + static_cast<int64_t>(blockIdx.x) * E;
  const int total = b.offsets[E];
  for (int r = 0; r < kIdsPerThread; ++r) {
    const int64_t f = wave_base + r * kWave + lane;
    fill_tail(b, f, n, total);
    const int e = key[r];
    if (e < 0) continue;
    place_id(b, e, f, b.offsets[e], th[e] + rank[r]);
  }
}

// Workgroups past the router tiles (when the layer passes its token quantization along)
// quantize kRouteThreads 16-value blocks each: the two are independent, so they share the
// launch instead of running back to back.
__global__ __launch_bounds__(kRouteThreads) void route_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t n, int E, int nbits, RouteBuffers b,
    QuantizeArgs qa) {
  extern __shared__ int32_t wave_hist[];           // [4][E]
  const int64_t ntiles = (n + kRouteTile - 1) / kRouteTile;
  if (static_cast<int64_t>(blockIdx.x) >= ntiles) {  // uniform over the workgroup
    const int64_t blk = static_cast<int64_t>(blockIdx.x - ntiles) * kRouteThreads + threadIdx.x;
    if (blk < qa.nblocks)
      quantize_nvfp4_block(qa.src, blk, qa.blocks_per_row, qa.rows_per_group, qa.q, qa.codes,
                           qa.scales, qa.decoded);
    return;
  }
  const int nw = kRouteThreads / kWave;
  for (int i = threadIdx.x; i < nw * E; i += blockDim.x) wave_hist[i] = 0;
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int64_t wave_base = static_cast<int64_t>(blockIdx.x) * kRouteTile + w * (kRouteTile / nw);
  int key[kIdsPerThread];
  int rank[kIdsPerThread];
  int32_t* my_hist = wave_hist + w * E;
  rank_wave_ids(ids, n, E, nbits, b.e_base, wave_base, lane, my_hist, b.expanded_row_idx, key,
                rank);
  __syncthreads();
  // Exclusive scan over the waves, per expert.
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int s = 0;
    for (int ww = 0; ww < nw; ++ww) {
      int v = wave_hist[ww * E + e];
      wave_hist[ww * E + e] = s;
      s += v;
    }
  }
  __syncthreads();
  const int32_t* th = b.tile_hist + static_cast<int64_t>(blockIdx.x) * E;
  const int total = b.offsets[E];
  for (int r = 0; r < kIdsPerThread; ++r) {
    const int64_t f = wave_base + r * kWave + lane;
    fill_tail(b, f, n, total);
    const int e = key[r];
    if (e < 0) continue;
    place_id(b, e, f, b.offsets[e], th[e] + my_hist[e] + rank[r]);
  }
}

// At most kRouteTile flat ids: the three passes fused in one workgroup of 1024 threads (no
// tile histograms, no handoff between launches).  The first four waves rank the ids (256
// each, as in the scatter kernel); all sixteen scan the experts.  LDS: the per-wave
// histograms [4][E] (after the ranking, exclusive over waves) and the expert offsets [E].
constexpr int kRouteSmallThreads = 1024;

__device__ __forceinline__ void route_small_body(const int32_t* __restrict__ ids, int64_t n,
                                                 int E, int nbits, const RouteBuffers& b,
                                                 int32_t* lds, uint64_t* sh, int* carry,
                                                 int32_t* map_lds = nullptr) {
  constexpr int nw = kRouteThreads / kWave;            // ranking waves
  int32_t* wave_hist = lds;
  int32_t* off_sh = lds + nw * E;
  for (int i = threadIdx.x; i < nw * E; i += blockDim.x) wave_hist[i] = 0;
  if (threadIdx.x == 0) { carry[0] = 0; carry[1] = 0; carry[2] = 0; carry[3] = 0; }
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int64_t wave_base = static_cast<int64_t>(w) * (kRouteTile / nw);
  int key[kIdsPerThread];
  int rank[kIdsPerThread];
  if (w < nw)
    rank_wave_ids(ids, n, E, nbits, b.e_base, wave_base, lane, wave_hist + w * E,
                  b.expanded_row_idx, key, rank);
  __syncthreads();
  for (int e0 = 0; e0 < E; e0 += blockDim.x) {
    const int e = e0 + threadIdx.x;
    int cnt = 0;
    if (e < E) {
      for (int ww = 0; ww < nw; ++ww) {
        const int v = wave_hist[ww * E + e];
        wave_hist[ww * E + e] = cnt;                   // exclusive over waves
        cnt += v;
      }
      b.counts[e] = cnt;
      if (b.amax_reset) b.amax_reset[e] = 0.0f;
    }
    scan_experts_round(b, E, e, cnt, sh, carry, off_sh);
  }
  scan_experts_finish(b, E, carry);
  __syncthreads();                                      // off_sh complete
  if (w >= nw) return;
  const int total = carry[0];
  for (int r = 0; r < kIdsPerThread; ++r) {
    const int64_t f = wave_base + r * kWave + lane;
    fill_tail(b, f, n, total);
    const int e = key[r];
    if (e < 0) continue;
    const int32_t m = place_id(b, e, f, off_sh[e], wave_hist[w * E + e] + rank[r]);
    if (map_lds) map_lds[f] = m;
  }
}

__global__ __launch_bounds__(kRouteSmallThreads) void route_small_kernel(
    const int32_t* __restrict__ ids, int64_t n, int E, int nbits, RouteBuffers b) {
  extern __shared__ int32_t lds[];
  __shared__ uint64_t sh[16];
  __shared__ int carry[4];
  route_small_body(ids, n, E, nbits, b, lds, sh, carry);
}

// Small batches: the token quantization and the single-workgroup router in one launch
// (they are independent).  Workgroup 0 routes; workgroups 1.. quantize 1024 blocks each.
__global__ __launch_bounds__(kRouteSmallThreads) void quantize_route_small_kernel(
    QuantizeArgs qa, const int32_t* __restrict__ ids, int64_t n, int E, int nbits,
    RouteBuffers b) {
  extern __shared__ int32_t lds[];
  __shared__ uint64_t sh[16];
  __shared__ int carry[4];
  if (blockIdx.x == 0) {
    route_small_body(ids, n, E, nbits, b, lds, sh, carry);
    return;
  }
  const int64_t blk = static_cast<int64_t>(blockIdx.x - 1) * kRouteSmallThreads + threadIdx.x;
  if (blk < qa.nblocks)
    quantize_nvfp4_block(qa.src, blk, qa.blocks_per_row, qa.rows_per_group, qa.q, qa.codes,
                         qa.scales, qa.decoded);
}

// Routing primitive on a few tokens (the page's case of small shapes: loading, sorting
// and moving in one kernel): the single-workgroup router, which also keeps every id's
// row-map entry in LDS, then the token rows moved by the same workgroup, one token at a
// time, each row held in registers (up to kFusedCache 16-byte vectors per thread).
constexpr int kFusedMaxTokens = 8;
constexpr int kFusedCache = 8;

__global__ __launch_bounds__(kRouteSmallThreads) void route_permute_small_kernel(
    const int32_t* __restrict__ ids, int64_t n, int E, int nbits, RouteBuffers b,
    PermuteArgs p) {
  extern __shared__ int32_t lds[];
  __shared__ uint64_t sh[16];
  __shared__ int carry[4];
  __shared__ float red[kRouteSmallThreads / kWave];
  __shared__ int32_t dst[64];
  int32_t* map = lds + (kRouteThreads / kWave + 1) * E;
  for (int f = threadIdx.x; f < n; f += blockDim.x) map[f] = -1;   // ordered by the body's barrier
  route_small_body(ids, n, E, nbits, b, lds, sh, carry, map);
  __syncthreads();
  const int nvec = p.H / 8;
  const float s_st = p.quant == 2 ? p.static_scale[0] : 0.0f;
  const float o_st = p.quant == 2 ? p.static_offset[0] : 0.0f;
  for (int t = 0; t < p.N; ++t) {
    if (threadIdx.x < p.K) {
      const int32_t d = map[t * p.K + threadIdx.x];
      dst[threadIdx.x] = (d >= 0 && d < p.limit) ? d : -1;
    }
    __syncthreads();
    bool any = false;
    for (int j = 0; j < p.K; ++j) any |= dst[j] >= 0;
    if (any) {                                           // uniform over the workgroup
      const uint4* xr = reinterpret_cast<const uint4*>(p.x + static_cast<int64_t>(t) * p.H);
      uint4 r[kFusedCache];
#pragma unroll
      for (int i = 0; i < kFusedCache; ++i) {
        const int v = threadIdx.x + i * kRouteSmallThreads;
        r[i] = v < nvec ? xr[v] : make_uint4(0u, 0u, 0u, 0u);
      }
      float scale = 0.0f;
      if (p.quant == 1) {
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < kFusedCache; ++i) {
          const uint32_t w4[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            amax = fmaxf(amax, fabsf(__uint_as_float(w4[q] << 16)));
            amax = fmaxf(amax, fabsf(__uint_as_float(w4[q] & 0xFFFF0000u)));
          }
        }
        scale = block_max(amax, red) / 127.0f;
      }
#pragma unroll
      for (int i = 0; i < kFusedCache; ++i) {
        const int v = threadIdx.x + i * kRouteSmallThreads;
        if (v >= nvec) continue;
        if (p.quant == 0) {
          for (int j = 0; j < p.K; ++j)
            if (dst[j] >= 0)
              reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.expanded_x) +
                                       static_cast<int64_t>(dst[j]) * p.H)[v] = r[i];
          continue;
        }
        const uint2 pv =
            p.quant == 2 ? quant8(r[i], [=](float xv) { return static_int8(xv, s_st, o_st); })
                         : quant8(r[i], [=](float xv) {
                             const float qf = (scale == 0.0f) ? 0.0f : rintf(xv / scale);
                             return fminf(fmaxf(qf, -127.0f), 127.0f);
                           });
        for (int j = 0; j < p.K; ++j)
          if (dst[j] >= 0)
            reinterpret_cast<uint2*>(static_cast<int8_t*>(p.expanded_x) +
                                     static_cast<int64_t>(dst[j]) * p.H)[v] = pv;
      }
      if (threadIdx.x < p.K && dst[threadIdx.x] >= 0 && p.expanded_scale) {
        if (p.quant == 1) p.expanded_scale[dst[threadIdx.x]] = scale;
        else if (p.quant == 0 && p.row_scale) p.expanded_scale[dst[threadIdx.x]] = p.row_scale[t];
      }
    }
    __syncthreads();                                     // dst[] and red[] are reused
  }
}

bool route_permute_fits_one_workgroup(int64_t n, int E, int64_t N, int H) {
  const size_t lds = (kRouteThreads / kWave + 1) * static_cast<size_t>(E) * sizeof(int32_t) +
                     static_cast<size_t>(n) * sizeof(int32_t);
  return route_tiles(n) == 1 && lds <= kRouteSmallMaxLds && N <= kFusedMaxTokens &&
         H / 8 <= kFusedCache * kRouteSmallThreads;
}

hipError_t launch_route_permute_small(const int32_t* ids, int64_t n, int E, const RouteBuffers& b,
                                      const PermuteArgs& p, hipStream_t stream) {
  const size_t lds = (kRouteThreads / kWave + 1) * static_cast<size_t>(E) * sizeof(int32_t) +
                     static_cast<size_t>(n) * sizeof(int32_t);
  route_permute_small_kernel<<<dim3(1), dim3(kRouteSmallThreads), lds, stream>>>(
      ids, n, E, bits_for(E), b, p);
  return hipGetLastError();
}

bool route_fits_one_workgroup(int64_t n, int E) {
  const size_t small_lds = (kRouteThreads / kWave + 1) * static_cast<size_t>(E) * sizeof(int32_t);
  return route_tiles(n) == 1 && small_lds <= kRouteSmallMaxLds;
}

hipError_t launch_quantize_route_small(const QuantizeArgs& qa, const int32_t* ids, int64_t n,
                                       int E, const RouteBuffers& b, hipStream_t stream) {
  const size_t small_lds = (kRouteThreads / kWave + 1) * static_cast<size_t>(E) * sizeof(int32_t);
  const int64_t qblocks = (qa.nblocks + kRouteSmallThreads - 1) / kRouteSmallThreads;
  quantize_route_small_kernel<<<dim3(static_cast<unsigned>(1 + qblocks)), dim3(kRouteSmallThreads),
                                small_lds, stream>>>(qa, ids, n, E, bits_for(E), b);
  return hipGetLastError();
}

hipError_t launch_route(const int32_t* ids, int64_t n, int E, const RouteBuffers& b,
                        hipStream_t stream, const QuantizeArgs* fused) {
  const int nt = route_tiles(n);
  if (nt == 0) return hipSuccess;
  // the token quantization rides along with the scatter launch (the many-expert scatter
  // and the one-workgroup router run it as a launch of its own first)
  QuantizeArgs qa{};
  const bool fuse = fused != nullptr && fused->nblocks > 0 && !route_fits_one_workgroup(n, E) &&
                    E <= kScatterWaveHistMaxE;
  if (fused != nullptr && fused->nblocks > 0 && !fuse) {
    const int64_t rows = fused->nblocks / fused->blocks_per_row;
    const hipError_t e = launch_quantize_nvfp4(
        fused->src, rows / fused->rows_per_group, fused->rows_per_group,
        fused->blocks_per_row * kGroup, fused->q, fused->codes, fused->scales, fused->decoded,
        stream);
    if (e != hipSuccess) return e;
  }
  if (fuse) qa = *fused;
  const int64_t qgroups = (qa.nblocks + kRouteThreads - 1) / kRouteThreads;
  const size_t small_lds = (kRouteThreads / kWave + 1) * static_cast<size_t>(E) * sizeof(int32_t);
  if (route_fits_one_workgroup(n, E)) {
    route_small_kernel<<<dim3(1), dim3(kRouteSmallThreads), small_lds, stream>>>(
        ids, n, E, bits_for(E), b);
    return hipGetLastError();
  }
  route_hist_kernel<<<dim3(nt), dim3(kRouteThreads), E * sizeof(int32_t), stream>>>(
      ids, n, E, b.e_base, b.tile_hist);
  const int counted = nt > kColumnScanTiles ? 1 : 0;
  if (counted)
    route_colscan_kernel<<<dim3((E + kScanExperts - 1) / kScanExperts),
                           dim3(kScanExperts * kScanWaves), 0, stream>>>(b, nt, E);
  route_scan_kernel<<<dim3(1), dim3(1024), 0, stream>>>(b, nt, E, counted);
  if (E <= kScatterWaveHistMaxE)
    route_scatter_kernel<<<dim3(static_cast<unsigned>(nt + qgroups)), dim3(kRouteThreads),
                           (kRouteThreads / kWave) * E * sizeof(int32_t), stream>>>(
        ids, n, E, bits_for(E), b, qa);
  else
    route_scatter_seq_kernel<<<dim3(nt), dim3(kRouteThreads), E * sizeof(int32_t), stream>>>(
        ids, n, E, bits_for(E), b);
  return hipGetLastError();
}

}  // namespace rmoe
