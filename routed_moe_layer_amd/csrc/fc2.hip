// FC2 grouped GEMM with the whole token tile resident in LDS.
//
// "Cake SiTU backend" (intro; section "Prepared weights and scales"):
//   o[r, h] = alpha2[e] * sum_i ahat[r, i] * w2hat[e, h, i],  i < I
// with ahat the requantized SiTU output (NVFP4, decoded exactly to f16) and w2hat the FC2
// weights; the result is stored as BF16 rows for the finalization.
//
// FC2's reduction is short (I = 384 at the page's shape), so a workgroup decodes its token
// tile's full K range into LDS once, with a single barrier, and then sweeps a group of
// weight slabs over it: no further barriers, the weight fragments of the next (slab,
// chunk) stream into registers two steps ahead, and each slab's BF16 rows are stored as
// soon as its K loop ends.  Each wave owns WRG 16-row MFMA groups of every slab.
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

template <int NW, int WRG, int BN, int NCBA>
__device__ __forceinline__ void fc2_tile(const LayerArgs& a, const TileDesc& td, int slab0,
                                         int nslabs, const _Float16* __restrict__ s_tok) {
  constexpr int kSlabGroups = NW * WRG;         // 16-row groups per slab
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4;
  const int e = td.expert;
  const int nchunks = a.Ip / kChunk;
  const int RG = a.H / 16;
  const int total = nslabs * nchunks;
  const uint4* __restrict__ wcodes = reinterpret_cast<const uint4*>(a.w2_codes);
  const uint32_t* __restrict__ wscales = reinterpret_cast<const uint32_t*>(a.w2_scales);

  auto load = [&](int q, W2Regs<WRG>& dst) {
    const int j = slab0 + q / nchunks, c = q % nchunks;
    const int64_t slot = static_cast<int64_t>(e) * RG + j * kSlabGroups + w * WRG;
#pragma unroll
    for (int r = 0; r < WRG; ++r) {
      dst.c[r] = wcodes[((slot + r) * nchunks + c) * 64 + lane];
      dst.s[r] = wscales[prepared_scale_index(slot + r, nchunks, c, lane)];
    }
  };

  f32x4 acc[WRG][NCBA];
#pragma unroll
  for (int i = 0; i < WRG; ++i)
#pragma unroll
    for (int j = 0; j < NCBA; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One (slab, chunk) step q: decode the fragments in `cur` (freeing it), reload `cur`
  // with step q + 2, run the MFMAs, and store the slab's rows after its last chunk.
  // Two register sets alternate by the parity of q, so every load lands in the set that
  // is decoded two steps later (no register copies of in-flight loads).
  const float al = a.alpha2[e];
  auto step = [&](int q, W2Regs<WRG>& cur) {
    const int c = q % nchunks;
    f16x8 wf[4][WRG];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int r = 0; r < WRG; ++r) {
        const uint32_t cw = s == 0 ? cur.c[r].x : s == 1 ? cur.c[r].y : s == 2 ? cur.c[r].z : cur.c[r].w;
        wf[s][r] = decode8(cw, scale_f16x2((cur.s[r] >> (8 * s)) & 0xFFu));
      }
    if (q + 2 < total) load(q + 2, cur);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int cb = 0; cb < NCBA; ++cb) {
        const f16x8 xf = *reinterpret_cast<const f16x8*>(
            s_tok + (cb * 16 + (lane & 15)) * kFc2LdsRow + c * kChunk + 32 * s + 8 * g);
#pragma unroll
        for (int r = 0; r < WRG; ++r) acc[r][cb] = mfma16x16x32(wf[s][r], xf, acc[r][cb]);
      }
    if (c == nchunks - 1) {
      const int j = slab0 + q / nchunks;
      const int G0 = j * kSlabGroups + w * WRG;
#pragma unroll
      for (int cb = 0; cb < NCBA; ++cb) {
        const int n = cb * 16 + (lane & 15);
        const int64_t row = td.row_start + n;
#pragma unroll
        for (int r = 0; r < WRG; ++r) {
          const f32x4 o = acc[r][cb];
          acc[r][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (n < td.nrows) {
            const int h0 = 16 * (G0 + r) + 4 * g;
            uint2 v;
            v.x = static_cast<uint32_t>(f32_to_bf16_rne(o[0] * al)) |
                  (static_cast<uint32_t>(f32_to_bf16_rne(o[1] * al)) << 16);
            v.y = static_cast<uint32_t>(f32_to_bf16_rne(o[2] * al)) |
                  (static_cast<uint32_t>(f32_to_bf16_rne(o[3] * al)) << 16);
            *reinterpret_cast<uint2*>(a.o_rows + row * a.H + h0) = v;
          }
        }
      }
    }
  };

  W2Regs<WRG> setA, setB;
  load(0, setA);
  if (total > 1) load(1, setB);
  int q = 0;
  for (; q + 1 < total; q += 2) {
    step(q, setA);
    step(q + 1, setB);
  }
  if (q < total) step(q, setA);
}

// grid: (token tile, slab group) pairs; slab group = SPW consecutive slabs.
template <int NW, int WRG, int BN, int SPW>
__global__ __launch_bounds__(NW * 64) void fc2_kernel(LayerArgs a, int big) {
  __shared__ _Float16 s_tok[BN * kFc2LdsRow];
  __shared__ int64_t s_row[BN];
  const TileDesc* tiles = big ? a.tiles_big : a.tiles_small;
  const int ntiles = a.num_tiles[big];
  const int n_slabs = a.H / (NW * WRG * 16);
  const int n_groups = (n_slabs + SPW - 1) / SPW;
  int tt, grp;
  map_workgroup(blockIdx.x, n_groups, &tt, &grp);
  if (tt >= ntiles) return;
  const TileDesc td = tiles[tt];
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
  if constexpr (BN == 32) {
    if (ncb == 1) fc2_tile<NW, WRG, BN, 1>(a, td, slab0, nslabs, s_tok);
    else fc2_tile<NW, WRG, BN, 2>(a, td, slab0, nslabs, s_tok);
  } else {
    switch (ncb) {
      case 1: fc2_tile<NW, WRG, BN, 1>(a, td, slab0, nslabs, s_tok); break;
      case 2: fc2_tile<NW, WRG, BN, 2>(a, td, slab0, nslabs, s_tok); break;
      case 3: fc2_tile<NW, WRG, BN, 3>(a, td, slab0, nslabs, s_tok); break;
      case 4: fc2_tile<NW, WRG, BN, 4>(a, td, slab0, nslabs, s_tok); break;
      case 5: fc2_tile<NW, WRG, BN, 5>(a, td, slab0, nslabs, s_tok); break;
      case 6: fc2_tile<NW, WRG, BN, 6>(a, td, slab0, nslabs, s_tok); break;
      case 7: fc2_tile<NW, WRG, BN, 7>(a, td, slab0, nslabs, s_tok); break;
      default: fc2_tile<NW, WRG, BN, 8>(a, td, slab0, nslabs, s_tok); break;
    }
  }
}

template <int NW, int WRG, int BN, int SPW>
static void launch_fc2_variant(const LayerArgs& a, int64_t max_tiles, int big,
                               hipStream_t stream) {
  const int n_slabs = a.H / (NW * WRG * 16);
  const int n_groups = (n_slabs + SPW - 1) / SPW;
  const int64_t grid = round_up(round_up(max_tiles, kTileGroup) * n_groups, kXcds * kXcdRun);
  if (grid > 0)
    fc2_kernel<NW, WRG, BN, SPW><<<dim3(static_cast<unsigned>(grid)), dim3(NW * 64), 0, stream>>>(a, big);
}

// Small tiles: 128-row slabs in groups of 4 (enough workgroups for decode-size batches);
// big tiles: 256-row slabs (128 when H is not a multiple of 256), all slabs in one group.
bool fc2_resident_fits(const LayerArgs& a) { return a.Ip <= kFc2MaxIp; }

void launch_fc2_resident_small(const LayerArgs& a, hipStream_t stream) {
  launch_fc2_variant<4, 2, kSmallRows, 4>(a, a.max_small, 0, stream);
}

void launch_fc2_resident_big(const LayerArgs& a, hipStream_t stream) {
  if (a.H % 256 == 0)
    launch_fc2_variant<4, 4, kBigRows, 1 << 20>(a, a.max_big, 1, stream);
  else
    launch_fc2_variant<4, 2, kBigRows, 1 << 20>(a, a.max_big, 1, stream);
}

}  // namespace rmoe
