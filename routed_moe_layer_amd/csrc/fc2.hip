// FC2 grouped GEMM with the whole token tile resident in LDS.
//
// "Cake SiTU backend" (intro; section "Prepared weights and scales"):
//   o[r, h] = alpha2[e] * sum_i ahat[r, i] * w2hat[e, h, i],  i < I
// with ahat the requantized SiTU output (NVFP4, decoded exactly to f16) and w2hat the FC2
// weights; the result is stored as f16 rows scaled by a power of two per expert
// (store_out_block) for the finalization.
//
// FC2's reduction is short (I = 384 at the page's shape), so a workgroup decodes its token
// tile's full K range into LDS once, with a single barrier, and then sweeps a group of
// weight slabs over it: no further barriers, the weight fragments of the next (slab,
// chunk) stream into registers two steps ahead, and each slab's output rows are stored as
// soon as its K loop ends.  Each wave owns WRG 16-row MFMA groups of every slab.
#include <type_traits>

#include "common.h"
#include "fc2_tile.h"
#include "gemm_util.h"
#include "kernels.h"

namespace rmoe {

// grid: (token sub-tile, slab group) pairs; slab group = SPW consecutive slabs.  A work
// list tile of up to kBigRows rows is taken as SPLIT sub-tiles of BN rows (BN < kBigRows
// keeps the LDS tile small enough for several workgroups per CU).
template <int NW, int WRG, int BN, int SPW, int SPLIT>
__global__ __launch_bounds__(NW * 64) void fc2_kernel(LayerArgs a, int big) {
  __shared__ _Float16 s_tok[BN * kFc2LdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t s_out[NW * 16 * out_lds_stride<WRG>()];
  const TileDesc* tiles = big ? a.tiles_big : a.tiles_small;
  const int ntiles = a.num_tiles[big];
  const int n_slabs = a.H / (NW * WRG * 16);
  const int n_groups = (n_slabs + SPW - 1) / SPW;
  int ts, grp;
  map_workgroup(blockIdx.x, n_groups, a.xcds, &ts, &grp);
  const int tt = ts / SPLIT, part = ts % SPLIT;
  if (tt >= ntiles) return;
  TileDesc td = tiles[tt];
  // a tile of more than BN rows is split into SPLIT sub-tiles of about equal size (whole
  // 16-row blocks), so that no sub-tile streams all of the expert's weights for a few rows
  const int blocks = (td.nrows + 15) / 16;
  const int per = blocks * 16 <= BN ? BN / 16 : (blocks + SPLIT - 1) / SPLIT;
  td.row_start += part * per * 16;
  td.nrows = min(per * 16, td.nrows - part * per * 16);
  if (td.nrows <= 0) return;
  // decode the tile's codes, columns [0, Ip), rows below 16*ncb, into LDS (zero past I)
  const int ncb = (td.nrows + 15) / 16;
  fc2_stage_tile(a, td, ncb, s_tok, threadIdx.x, NW * 64);
  __syncthreads();
  const int slab0 = grp * SPW;
  const int nslabs = min(SPW, n_slabs - slab0);
  // compile-time token blocks (uniform branch per workgroup) and chunks per slab
  auto run = [&](auto ncba) {
    constexpr int NCBA = decltype(ncba)::value;
    switch (a.Ip / kChunk) {
      case 1: fc2_tile<NW, WRG, BN, NCBA, 1>(a, td, slab0, nslabs, s_tok, s_out); break;
      case 2: fc2_tile<NW, WRG, BN, NCBA, 2>(a, td, slab0, nslabs, s_tok, s_out); break;
      default: fc2_tile<NW, WRG, BN, NCBA, 3>(a, td, slab0, nslabs, s_tok, s_out); break;
    }
  };
  using std::integral_constant;
  if constexpr (BN == 32) {
    if (ncb == 1) run(integral_constant<int, 1>{});
    else run(integral_constant<int, 2>{});
  } else if constexpr (BN == 64) {
    switch (ncb) {
      case 1: run(integral_constant<int, 1>{}); break;
      case 2: run(integral_constant<int, 2>{}); break;
      case 3: run(integral_constant<int, 3>{}); break;
      default: run(integral_constant<int, 4>{}); break;
    }
  } else {
    switch (ncb) {
      case 1: run(integral_constant<int, 1>{}); break;
      case 2: run(integral_constant<int, 2>{}); break;
      case 3: run(integral_constant<int, 3>{}); break;
      case 4: run(integral_constant<int, 4>{}); break;
      case 5: run(integral_constant<int, 5>{}); break;
      case 6: run(integral_constant<int, 6>{}); break;
      case 7: run(integral_constant<int, 7>{}); break;
      default: run(integral_constant<int, 8>{}); break;
    }
  }
}

// Weight-stationary FC2 for big tiles when there are many routed rows.
//
// Work items are (run, slab) pairs.  A run is up to kRunTiles consecutive big tiles of one
// expert (a contiguous range of its sorted rows, listed by the router), and a slab is
// NW*WRG*16 output columns.  For an item, the slab's weight codes and scales for the whole
// reduction (NCH chunks of 128) stay in registers, and the run's token rows pass through
// one LDS tile kFc2PassRows at a time: the next pass's codes are loaded into registers
// while the current pass's MFMAs run, and are decoded into LDS between two barriers.  An
// expert's weights are thus read once per run rather than once per 64-row sub-tile.
// The kernel is persistent (two workgroups per CU, each taking items at a fixed stride), so
// the grid never holds workgroups with no work; the items of run r go to the workgroups
// of XCD r % xcds, the slabs of one run to consecutive workgroups there, so the run's token
// rows are fetched from HBM once and reread by the other slabs from that XCD's L2.
constexpr int kFc2PassRows = 64;
constexpr int kFc2StationaryRows = 2 * kFc2PassRows;
// Two workgroups on each compute unit, a whole number per XCD.
inline int fc2_stationary_grid(const LayerArgs& a) {
  return static_cast<int>(round_up(2 * static_cast<int64_t>(a.cus), a.xcds));
}

template <int NW, int WRG, int NCH>
__global__ __launch_bounds__(NW * 64, 2) void fc2_stationary_kernel(LayerArgs a) {
  constexpr int kSlabGroups = NW * WRG;
  constexpr int kThreads = NW * 64;

  __shared__ __attribute__((aligned(16))) _Float16 s_tok[kFc2PassRows * kFc2LdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t s_out[NW * 16 * out_lds_stride<WRG>()];

  const int n_slabs = a.H / (kSlabGroups * 16);
  const int n_runs = a.num_tiles[2];
  const int xcds = a.xcds;                       // gridDim.x is a multiple of it
  const int xcd = blockIdx.x % xcds, per_xcd = gridDim.x / xcds;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4;
  const int code_bytes = a.I / 2, scale_cols = a.I / 16;
  const _Float16* xrow = s_tok + (lane & 15) * kFc2LdsRow + 8 * g;
  uint16_t* wave_out = s_out + w * 16 * out_lds_stride<WRG>();

  // Token rows [p0, p0 + nr) of the run (rows past nr repeat the last one; they are not
  // stored).  Four threads per row, each NCH 16-byte pieces of codes (32 values) and the
  // two scale bytes of each piece.
  static_assert(kThreads == 4 * kFc2PassRows, "four threads per staged row");
  const int st_row = tid >> 2, st_part = (tid & 3) * NCH;   // piece index within the row
  u32x4 pc[NCH];
  uint32_t ps[NCH];
  auto fetch = [&](int p0, int nr) {
    const int64_t row = p0 + min(st_row, nr - 1);
    const u32x4* codes = reinterpret_cast<const u32x4*>(a.a_codes + row * code_bytes) + st_part;
    const uint16_t* scales = reinterpret_cast<const uint16_t*>(a.a_scales + row * scale_cols) + st_part;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      pc[j] = codes[j];
      ps[j] = scales[j];
    }
  };
  auto stage = [&]() {
    f16x8* dst = reinterpret_cast<f16x8*>(s_tok + st_row * kFc2LdsRow) + 4 * st_part;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const f16x2 s0 = scale_f16x2_of(ps[j], 0), s1 = scale_f16x2_of(ps[j], 1);
      dst[4 * j + 0] = decode8(pc[j][0], s0);
      dst[4 * j + 1] = decode8(pc[j][1], s0);
      dst[4 * j + 2] = decode8(pc[j][2], s1);
      dst[4 * j + 3] = decode8(pc[j][3], s1);
    }
  };

  for (int k = blockIdx.x / xcds;; k += per_xcd) {
    const int run = xcd + xcds * (k / n_slabs);
    if (run >= n_runs) break;
    const int slab = k - (k / n_slabs) * n_slabs;
    const TileDesc rd = a.runs[run];
    const int e = rd.expert, row_end = rd.row_start + rd.nrows;

    W2Regs<WRG> wr[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) fc2_load<NW, WRG, kBigRows>(a, e, w, lane, slab, c, NCH, wr[c]);
    // the block scales of K-steps (0, 1) and (2, 3) of every chunk and row group, as f16
    f16x2 wsc[NCH][WRG][2];
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int r = 0; r < WRG; ++r) scales4_f16(wr[c].s[r], &wsc[c][r][0], &wsc[c][r][1]);

    const OutScale osc = out_scale(a.alpha2[e], a.I);
    const int col0 = 16 * (slab * kSlabGroups + w * WRG);
    int32_t flat[kFc2PassRows / 16];
    int p0 = rd.row_start;
    int nr = min(kFc2PassRows, row_end - p0);

    // One pass over NCB 16-token blocks: all K-steps from the resident weights, then the
    // output rows (stored at their flat ids through the per-wave LDS staging).
    auto pass = [&](auto ncb_c) {
      constexpr int NCB = decltype(ncb_c)::value;
      f32x4 acc[WRG][NCB];
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          // The decoded weights are the same in every pass: an opaque 1.0 as the
          // conversion's scale (a scalar register, no vector work) keeps the compiler from
          // hoisting all of them (NCH*4*WRG*4 registers) out of the pass loop.
          uint32_t one_bits = 0x3F800000u;
          asm volatile("" : "+s"(one_bits));
          const float one = __uint_as_float(one_bits);
          f16x8 xf[NCB];
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            xf[cb] = *reinterpret_cast<const f16x8*>(xrow + cb * 16 * kFc2LdsRow + c * kChunk + 32 * s);
#pragma unroll
          for (int r = 0; r < WRG; ++r) {
            const uint4& cc = wr[c].c[r];
            const uint32_t cw = s == 0 ? cc.x : s == 1 ? cc.y : s == 2 ? cc.z : cc.w;
            const f16x8 wf = decode8(cw, bcast_f16x2(wsc[c][r][s >> 1], s & 1), one);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
              acc[r][cb] = mfma16x16x32(wf, xf[cb],
                                        (c == 0 && s == 0) ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[r][cb]);
          }
          __builtin_amdgcn_sched_barrier(0);   // bounds the live decoded weights to one K-step
        }
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        f32x4 blk[WRG];
#pragma unroll
        for (int r = 0; r < WRG; ++r) blk[r] = acc[r][cb];
        store_out_block<WRG>(blk, osc, wave_out, lane, flat[cb], nr - cb * 16, a.o_rows, a.o_exp,
                             a.H, col0);
      }
    };

    fetch(p0, nr);
    stage();
    __syncthreads();
    using std::integral_constant;
    for (;;) {
      // flat ids of this pass's rows (lane l: block row l % 16), loaded before the next
      // pass's codes so that waiting for them does not wait for those
#pragma unroll
      for (int cb = 0; cb < kFc2PassRows / 16; ++cb)
        flat[cb] = a.sorted_row_idx[p0 + min(cb * 16 + (lane & 15), nr - 1)];
      const int next = p0 + kFc2PassRows;
      const bool more = next < row_end;
      const int nr_next = more ? min(kFc2PassRows, row_end - next) : 0;
      if (more) fetch(next, nr_next);
      switch ((nr + 15) / 16) {
        case 1: pass(integral_constant<int, 1>{}); break;
        case 2: pass(integral_constant<int, 2>{}); break;
        case 3: pass(integral_constant<int, 3>{}); break;
        default: pass(integral_constant<int, 4>{}); break;
      }
      __syncthreads();      // the tile is read; the next pass or item overwrites it
      if (!more) break;
      stage();
      __syncthreads();
      p0 = next;
      nr = nr_next;
    }
  }
}

template <int NW, int WRG, int NCH>
static void launch_fc2_stationary(const LayerArgs& a, hipStream_t stream) {
  fc2_stationary_kernel<NW, WRG, NCH>
      <<<dim3(static_cast<unsigned>(fc2_stationary_grid(a))), dim3(NW * 64), 0, stream>>>(a);
}

template <int NW, int WRG, int BN, int SPW, int SPLIT = 1>
static void launch_fc2_variant(const LayerArgs& a, int64_t max_tiles, int big,
                               hipStream_t stream) {
  const int n_slabs = a.H / (NW * WRG * 16);
  const int n_groups = (n_slabs + SPW - 1) / SPW;
  const int64_t grid =
      round_up(round_up(max_tiles * SPLIT, kTileGroup) * n_groups, a.xcds * kXcdRun);
  if (grid > 0)
    fc2_kernel<NW, WRG, BN, SPW, SPLIT>
        <<<dim3(static_cast<unsigned>(grid)), dim3(NW * 64), 0, stream>>>(a, big);
}

// Small tiles: 256-column slabs in groups of 7 (two workgroups per tile at H = 3584, each
// staging the token tile once: fewer stagings than smaller groups, twice the workgroups
// of one group of 14), 128-column slabs when H is not a multiple of 256;
// big tiles: the weight-stationary kernel on 256-column slabs (H a multiple of 256, I of
// 128, long runs), else the token-resident kernel on 256-column slabs (128 when H is not a
// multiple of 256), all slabs in one group.
bool fc2_resident_fits(const LayerArgs& a) { return a.Ip <= kFc2MaxIp; }

void launch_fc2_resident_small(const LayerArgs& a, hipStream_t stream) {
  if (a.H % 256 == 0) launch_fc2_variant<4, 4, kSmallRows, 7>(a, a.max_small, 0, stream);
  else launch_fc2_variant<4, 2, kSmallRows, 7>(a, a.max_small, 0, stream);
}

// Big tiles of a mid-size batch (fewer routed rows than many_rows): 64-row sub-tiles in
// two groups of 7 slabs, so that each tile spreads over four workgroups (H a multiple of
// 256).
void launch_fc2_resident_big_spread(const LayerArgs& a, hipStream_t stream) {
  launch_fc2_variant<4, 4, kBigRows / 2, 7, 2>(a, a.max_big, 1, stream);
}

void launch_fc2_resident_big(const LayerArgs& a, hipStream_t stream) {
  // The stationary kernel loads a slab's weights once per run, so it pays off when runs
  // span several passes: experts with at least kFc2StationaryRows routed rows on average.
  const bool long_runs = static_cast<int64_t>(a.T) * a.k >=
                         static_cast<int64_t>(kFc2StationaryRows) * a.E;
  if (a.H % 256 == 0 && a.I == a.Ip && long_runs) {
    switch (a.Ip / kChunk) {
      case 1: launch_fc2_stationary<4, 4, 1>(a, stream); break;
      case 2: launch_fc2_stationary<4, 4, 2>(a, stream); break;
      default: launch_fc2_stationary<4, 4, 3>(a, stream); break;
    }
  } else if (a.H % 256 == 0) {
    launch_fc2_variant<4, 4, kBigRows / 2, 1 << 20, 2>(a, a.max_big, 1, stream);
  } else {
    launch_fc2_variant<4, 2, kBigRows / 2, 1 << 20, 2>(a, a.max_big, 1, stream);
  }
}

}  // namespace rmoe
