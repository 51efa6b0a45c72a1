// Expert routing: a stable counting sort of the flat ids f = t*K + j by expert id.
//
// "torch_npu.npu_moe_init_routing_v2" (section 计算公式): step 1 keyValueSort(expertIdx,
// rowIdx), step 2 the gather map expandedRowIdx[sortedRowIdx[i]] = i, step 3 the
// per-expert histogram as an inclusive prefix sum.  The sort must be stable (equal experts
// keep increasing f) so that the result is unique.
//
// Three launches, no host readback ("Cake SiTU backend", intro: routing values never take
// part in host dispatch):
//   hist    : one workgroup per tile of 1024 flat ids; LDS histogram -> tile_hist[tile][e].
//   scan    : one workgroup; per expert, exclusive scan of tile_hist over tiles (in place),
//             counts, exclusive/inclusive expert offsets; optionally the two grouped-GEMM
//             work lists (small and big token tiles) and a reset of the SiTU amax stats.
//   scatter : one workgroup per tile; each wave ranks its 256 ids stably with ballot-based
//             key matching (one ballot per key bit), waves are ordered through an LDS
//             per-wave histogram, and every id lands at
//             offset[e] + tile_base[tile][e] + wave_base[w][e] + rank.
#include "common.h"
#include "kernels.h"

namespace rmoe {

constexpr int kIdsPerThread = kRouteTile / kRouteThreads;   // 4

__global__ __launch_bounds__(kRouteThreads) void route_hist_kernel(
    const int32_t* __restrict__ ids, int64_t n, int E, int32_t* __restrict__ tile_hist) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kRouteTile;
  for (int i = threadIdx.x; i < kRouteTile; i += blockDim.x) {
    int64_t f = base + i;
    if (f < n) {
      const int e = ids[f];
      if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  int32_t* out = tile_hist + static_cast<int64_t>(blockIdx.x) * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) out[e] = hist[e];
}

// Block-wide exclusive scan of one int per thread (1024 threads); returns the exclusive
// prefix and writes the total to *total.
__device__ int block_excl_scan(int v, int* sh, int* total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  int incl = v;
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) sh[w] = incl;
  __syncthreads();
  if (w == 0) {
    int nw = blockDim.x / kWave;
    int s = lane < nw ? sh[lane] : 0;
    for (int off = 1; off < kWave; off <<= 1) {
      int o = __shfl_up(s, off);
      if (lane >= off) s += o;
    }
    if (lane < nw) sh[lane] = s;     // inclusive over waves
  }
  __syncthreads();
  int wave_excl = w == 0 ? 0 : sh[w - 1];
  *total = sh[blockDim.x / kWave - 1];
  __syncthreads();
  return wave_excl + incl - v;
}

// Token tiles of one expert with `cnt` rows: (number of tiles, rows per tile but the last).
__device__ __forceinline__ void expert_tiles(int cnt, int* n_small, int* n_big, int* base) {
  *n_small = 0; *n_big = 0; *base = 0;
  if (cnt <= 0) return;
  if (cnt <= kSmallRows) { *n_small = 1; *base = cnt; return; }
  const int nb = (cnt + kBigRows - 1) / kBigRows;
  const int b = min(kBigRows, ((cnt + nb - 1) / nb + 15) / 16 * 16);
  *base = b;
  *n_big = (cnt + b - 1) / b;
}

__global__ __launch_bounds__(1024) void route_scan_kernel(
    int32_t* __restrict__ tile_hist, int ntiles, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ cumsum,
    TileDesc* __restrict__ tiles_small, TileDesc* __restrict__ tiles_big,
    int32_t* __restrict__ num_tiles, float* __restrict__ amax_reset) {
  __shared__ int sh[16];
  __shared__ int carry[3];
  if (threadIdx.x == 0) { carry[0] = 0; carry[1] = 0; carry[2] = 0; }
  __syncthreads();
  const bool lists = tiles_small != nullptr;
  // Experts are handled in rounds of 1024 (E <= 4096).
  for (int e0 = 0; e0 < E; e0 += blockDim.x) {
    const int e = e0 + threadIdx.x;
    int cnt = 0;
    if (e < E) {
      for (int t = 0; t < ntiles; ++t) {
        int32_t* p = tile_hist + static_cast<int64_t>(t) * E + e;
        int v = *p;
        *p = cnt;                       // exclusive over tiles
        cnt += v;
      }
      counts[e] = cnt;
      if (amax_reset) amax_reset[e] = 0.0f;
    }
    int n_small, n_big, base;
    expert_tiles(lists ? cnt : 0, &n_small, &n_big, &base);
    int total, stotal, btotal;
    const int excl = block_excl_scan(cnt, sh, &total);
    const int sexcl = block_excl_scan(n_small, sh, &stotal);
    const int bexcl = block_excl_scan(n_big, sh, &btotal);
    const int off = carry[0] + excl;
    if (e < E) {
      offsets[e] = off;
      if (cumsum) cumsum[e] = off + cnt;
      if (n_small) tiles_small[carry[1] + sexcl] = TileDesc{e, off, cnt, 0};
      for (int j = 0; j < n_big; ++j)
        tiles_big[carry[2] + bexcl + j] = TileDesc{e, off + j * base, min(base, cnt - j * base), 0};
    }
    __syncthreads();
    if (threadIdx.x == 0) { carry[0] += total; carry[1] += stotal; carry[2] += btotal; }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    offsets[E] = carry[0];
    if (num_tiles) { num_tiles[0] = carry[1]; num_tiles[1] = carry[2]; }
  }
}

__global__ __launch_bounds__(kRouteThreads) void route_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t n, int E, int nbits,
    const int32_t* __restrict__ tile_hist, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ sorted_row_idx,
    int32_t* __restrict__ expanded_row_idx) {
  extern __shared__ int32_t wave_hist[];           // [4][E]
  const int nw = kRouteThreads / kWave;
  for (int i = threadIdx.x; i < nw * E; i += blockDim.x) wave_hist[i] = 0;
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int64_t wave_base = static_cast<int64_t>(blockIdx.x) * kRouteTile + w * (kRouteTile / nw);
  int key[kIdsPerThread];
  int rank[kIdsPerThread];
  int32_t* my_hist = wave_hist + w * E;
  // Rounds of 64 consecutive ids, in order: rank within the round among equal keys plus
  // the count of equal keys in earlier rounds of this wave.
  for (int r = 0; r < kIdsPerThread; ++r) {
    int64_t f = wave_base + r * kWave + lane;
    int e = f < n ? ids[f] : -1;
    // An id outside [0, E) breaks the caller's contract; it is dropped (never counted,
    // never scattered) and its gather-map entry is -1, so no kernel indexes with it.
    bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(E);
    if (f < n && !valid) expanded_row_idx[f] = -1;
    if (!valid) e = 0;
    uint64_t active = __ballot(valid);
    uint64_t peers = match_key(static_cast<uint32_t>(e), nbits, active);
    int before = valid ? my_hist[e] : 0;
    int rk = before + __popcll(peers & lanemask_lt());
    // the lowest lane of each group of equal keys bumps the wave histogram
    if (valid && (peers & lanemask_lt()) == 0) my_hist[e] = before + __popcll(peers);
    key[r] = valid ? e : -1;
    rank[r] = rk;
    __builtin_amdgcn_wave_barrier();
  }
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
  const int32_t* th = tile_hist + static_cast<int64_t>(blockIdx.x) * E;
  for (int r = 0; r < kIdsPerThread; ++r) {
    int e = key[r];
    if (e < 0) continue;
    int64_t f = wave_base + r * kWave + lane;
    int pos = offsets[e] + th[e] + my_hist[e] + rank[r];
    if (sorted_ids) sorted_ids[pos] = e;
    if (sorted_row_idx) sorted_row_idx[pos] = static_cast<int32_t>(f);
    expanded_row_idx[f] = pos;
  }
}

hipError_t launch_route(const int32_t* ids, int64_t n, int E, const RouteBuffers& b,
                        hipStream_t stream) {
  const int nt = route_tiles(n);
  if (nt == 0) return hipSuccess;
  route_hist_kernel<<<dim3(nt), dim3(kRouteThreads), E * sizeof(int32_t), stream>>>(
      ids, n, E, b.tile_hist);
  route_scan_kernel<<<dim3(1), dim3(1024), 0, stream>>>(
      b.tile_hist, nt, E, b.counts, b.offsets, b.cumsum, b.tiles_small, b.tiles_big, b.num_tiles,
      b.amax_reset);
  route_scatter_kernel<<<dim3(nt), dim3(kRouteThreads),
                         (kRouteThreads / kWave) * E * sizeof(int32_t), stream>>>(
      ids, n, E, bits_for(E), b.tile_hist, b.offsets, b.sorted_ids, b.sorted_row_idx,
      b.expanded_row_idx);
  return hipGetLastError();
}

}  // namespace rmoe
