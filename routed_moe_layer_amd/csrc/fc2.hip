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
#include "gemm_util.h"
#include "kernels.h"

namespace rmoe {

constexpr int kFc2MaxIp = 384;                  // padded K the LDS tile is sized for
constexpr int kFc2LdsRow = kFc2MaxIp + 8;       // f16 per staged token row (+16 B pad)

template <int WRG>
struct W2Regs {
  uint4 c[WRG];
  uint32_t s[WRG];
};

// A wave's weight fragments of (slab j, chunk c): WRG 16-row groups x 16 code bytes and
// one scale dword per lane.
template <int NW, int WRG>
__device__ __forceinline__ void fc2_load(const LayerArgs& a, int e, int w, int lane, int j,
                                         int c, int nchunks, W2Regs<WRG>& dst) {
  constexpr int kSlabGroups = NW * WRG;
  const uint4* __restrict__ wcodes = reinterpret_cast<const uint4*>(a.w2_codes);
  const uint32_t* __restrict__ wscales = reinterpret_cast<const uint32_t*>(a.w2_scales);
  const int64_t chunk0 = prepared_chunk(e, c, j * kSlabGroups + w * WRG, nchunks, a.H / 16);
#pragma unroll
  for (int r = 0; r < WRG; ++r) {
    dst.c[r] = wcodes[(chunk0 + r) * 64 + lane];
    dst.s[r] = wscales[prepared_scale_index(chunk0 + r, lane)];
  }
}

// The slabs [slab0, slab0 + nslabs) of one token tile; NCH = Ip/128 chunks per slab.
// Steps q = (slab, chunk) run in order; step q decodes its register set, refills it with
// step q+2 (two sets alternate, so no register copies of in-flight loads), runs the MFMAs
// over the LDS-resident token tile and, after a slab's last chunk, stores the slab's
// output rows.  Two slabs per loop trip keep the chunk index, the register set and the
// epilogue compile-time; a slab's first K-step starts from a zero accumulator.
// The output of one wave for one 16-token block and one slab passes through a per-wave LDS
// buffer (store_out_block): each lane then holds consecutive columns of one token row, so
// the global stores are whole 16-byte pieces of consecutive columns (the rows are
// scattered over the FC2 output, so longer runs per store instruction cut the memory
// transactions).
template <int NW, int WRG, int BN, int NCBA, int NCH>
__device__ __forceinline__ void fc2_tile(const LayerArgs& a, const TileDesc& td, int slab0,
                                         int nslabs, const _Float16* __restrict__ s_tok,
                                         uint16_t* __restrict__ s_out) {
  constexpr int kSlabGroups = NW * WRG;                 // 16-row groups per slab
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4;
  const int e = td.expert;
  const int last = slab0 + nslabs - 1;
  const OutScale osc = out_scale(a.alpha2[e], a.I);
  const _Float16* xrow = s_tok + (lane & 15) * kFc2LdsRow + 8 * g;
  // FC2 rows are stored at their flat id t*k + j, so that the finalization reads each
  // token's k rows as one contiguous run; lane l holds the flat id of block row l % 16
  int32_t flat_cb[NCBA];
#pragma unroll
  for (int cb = 0; cb < NCBA; ++cb) {
    const int n = min(cb * 16 + (lane & 15), td.nrows - 1);
    flat_cb[cb] = a.sorted_row_idx[td.row_start + n];
  }
  uint16_t* wave_out = s_out + w * 16 * out_lds_stride<WRG>();
  f32x4 acc[WRG][NCBA];

  auto decode = [&](const W2Regs<WRG>& cur, const int s, f16x8 (&wf)[WRG]) {
#pragma unroll
    for (int r = 0; r < WRG; ++r) {
      const uint32_t cw = s == 0 ? cur.c[r].x : s == 1 ? cur.c[r].y : s == 2 ? cur.c[r].z : cur.c[r].w;
      wf[r] = decode8(cw, scale_f16x2_of(cur.s[r], s));
    }
  };
  auto step = [&](const int j, const int c, W2Regs<WRG>& cur) {
    // Software pipeline over the four 32-column K-steps: the weight fragments of step s+1
    // are decoded while the MFMAs of step s run (interleaved: per 16-token block one LDS
    // operand read, then each MFMA followed by two VALU instructions).  After the last
    // decode the set is refilled with step q+2 (slab clamped: surplus loads past the last
    // slab are unused and unconditional, so the compiler's load counters stay exact).
    f16x8 wf[2][WRG];
    decode(cur, 0, wf[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) decode(cur, s + 1, wf[(s + 1) & 1]);
      else fc2_load<NW, WRG>(a, e, w, lane, min(j + (c + 2) / NCH, last), (c + 2) % NCH, NCH, cur);
      // token operand of block cb+1 is read while block cb's MFMAs run
      const _Float16* xs = xrow + c * kChunk + 32 * s;
      f16x8 xf = *reinterpret_cast<const f16x8*>(xs);
#pragma unroll
      for (int cb = 0; cb < NCBA; ++cb) {
        const f16x8 xn = cb + 1 < NCBA
            ? *reinterpret_cast<const f16x8*>(xs + (cb + 1) * 16 * kFc2LdsRow) : xf;
#pragma unroll
        for (int r = 0; r < WRG; ++r)
          acc[r][cb] = mfma16x16x32(wf[s & 1][r], xf,
                                    (c == 0 && s == 0) ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[r][cb]);
        xf = xn;
      }
      if (s < 3) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        // LDS read, block 0
#pragma unroll
        for (int cb = 0; cb < NCBA; ++cb) {
          if (cb + 1 < NCBA) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // block cb+1
#pragma unroll
          for (int r = 0; r < WRG; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);    // VALU (next decode)
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (c == NCH - 1) {
      const int G0 = j * kSlabGroups + w * WRG;
#pragma unroll
      for (int cb = 0; cb < NCBA; ++cb) {
        f32x4 blk[WRG];
#pragma unroll
        for (int r = 0; r < WRG; ++r) blk[r] = acc[r][cb];
        store_out_block<WRG>(blk, osc, wave_out, lane, flat_cb[cb], td.nrows - cb * 16, a.o_rows,
                             a.o_exp, a.H, 16 * G0);
      }
      // the next slab's MFMAs (fresh accumulators) stay after these stores, so the two
      // accumulator sets are never live together
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  W2Regs<WRG> setA, setB;
  fc2_load<NW, WRG>(a, e, w, lane, slab0, 0, NCH, setA);
  fc2_load<NW, WRG>(a, e, w, lane, min(slab0 + 1 / NCH, last), 1 % NCH, NCH, setB);
  int j = slab0;
  for (; j + 1 <= last; j += 2) {
#pragma unroll
    for (int q = 0; q < 2 * NCH; ++q) step(j + q / NCH, q % NCH, (q & 1) ? setB : setA);
  }
  if (j == last) {
#pragma unroll
    for (int q = 0; q < NCH; ++q) step(j, q, (q & 1) ? setB : setA);
  }
}

// grid: (token sub-tile, slab group) pairs; slab group = SPW consecutive slabs.  A work
// list tile of up to kBigRows rows is taken as SPLIT sub-tiles of BN rows (BN < kBigRows
// keeps the LDS tile small enough for several workgroups per CU).
template <int NW, int WRG, int BN, int SPW, int SPLIT>
__global__ __launch_bounds__(NW * 64) void fc2_kernel(LayerArgs a, int big) {
  __shared__ _Float16 s_tok[BN * kFc2LdsRow];
  __shared__ int64_t s_row[BN];
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
  td.row_start += part * BN;
  td.nrows = min(BN, td.nrows - part * BN);
  if (td.nrows <= 0) return;
  const int tid = threadIdx.x;
  if (tid < BN) s_row[tid] = td.row_start + min(tid, td.nrows - 1);
  __syncthreads();
  // decode the tile's codes, columns [0, Ip), rows below 16*ncb, into LDS (zero past I)
  const int ncb = (td.nrows + 15) / 16;
  const int dw_per_row = a.Ip / 8;
  const int code_bytes = a.I / 2;
  for (int idx = tid; idx < 16 * ncb * dw_per_row; idx += NW * 64) {
    const int r = idx / dw_per_row, d = idx - r * dw_per_row;
    uint32_t cw = 0, sb = 0;
    if (4 * d < code_bytes) {
      cw = *reinterpret_cast<const uint32_t*>(a.a_codes + s_row[r] * code_bytes + 4 * d);
      sb = a.a_scales[s_row[r] * (a.I / 16) + d / 2];
    }
    *reinterpret_cast<f16x8*>(s_tok + r * kFc2LdsRow + 8 * d) = decode8(cw, scale_f16x2(sb));
  }
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
    for (int c = 0; c < NCH; ++c) fc2_load<NW, WRG>(a, e, w, lane, slab, c, NCH, wr[c]);
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

// Small tiles: 128-row slabs in groups of 4 (enough workgroups for decode-size batches);
// big tiles: the weight-stationary kernel on 256-column slabs (H a multiple of 256, I of
// 128, long runs), else the token-resident kernel on 256-column slabs (128 when H is not a
// multiple of 256), all slabs in one group.
bool fc2_resident_fits(const LayerArgs& a) { return a.Ip <= kFc2MaxIp; }

void launch_fc2_resident_small(const LayerArgs& a, hipStream_t stream) {
  launch_fc2_variant<4, 2, kSmallRows, 4>(a, a.max_small, 0, stream);
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
