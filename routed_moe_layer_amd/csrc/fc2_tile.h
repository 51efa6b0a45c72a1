// FC2's token-resident tile body, shared by the FC2 kernels and the fused small-batch
// layer kernel: a token tile decoded into LDS once and a group of weight slabs swept over
// it ("Cake SiTU backend", intro; section "Prepared weights and scales":
//   o[r, h] = alpha2[e] * sum_i ahat[r, i] * w2hat[e, h, i]).
#pragma once

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
// (TILE_ROWS: the token tile's capacity, which sets the cache policy, weight_load_policy)
template <int NW, int WRG, int TILE_ROWS>
__device__ __forceinline__ void fc2_load(const LayerArgs& a, int e, int w, int lane, int j,
                                         int c, int nchunks, W2Regs<WRG>& dst) {
  constexpr int kSlabGroups = NW * WRG;
  const u32x4* __restrict__ wcodes = reinterpret_cast<const u32x4*>(a.w2_codes);
  const uint32_t* __restrict__ wscales = reinterpret_cast<const uint32_t*>(a.w2_scales);
  const int64_t chunk0 = prepared_chunk(e, c, j * kSlabGroups + w * WRG, nchunks, a.H / 16);
#pragma unroll
  for (int r = 0; r < WRG; ++r) {
    const u32x4* pc = wcodes + (chunk0 + r) * 64 + lane;
    const uint32_t* ps = wscales + prepared_scale_index(chunk0 + r, lane);
    if constexpr (weight_load_policy(TILE_ROWS) == kNontemporal) {
      const u32x4 v = __builtin_nontemporal_load(pc);
      dst.c[r] = uint4{v[0], v[1], v[2], v[3]};
      dst.s[r] = __builtin_nontemporal_load(ps);
    } else {
      const u32x4 v = *pc;
      dst.c[r] = uint4{v[0], v[1], v[2], v[3]};
      dst.s[r] = *ps;
    }
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
    // operand read, two blocks ahead, then each MFMA followed by two VALU instructions).
    // After the last decode the set is refilled with step q+2 (slab clamped: surplus loads
    // past the last slab are unused and unconditional, so the compiler's load counters stay
    // exact).
    f16x8 wf[2][WRG];
    decode(cur, 0, wf[0]);
    // the token operands of the chunk's 4*NCBA (K-step, block) items, in order, are read
    // two items ahead of their MFMAs
    constexpr int kItems = 4 * NCBA;
    auto frag_of = [&](int i) {
      return *reinterpret_cast<const f16x8*>(xrow + c * kChunk + 32 * (i / NCBA) +
                                             (i % NCBA) * 16 * kFc2LdsRow);
    };
    f16x8 xf = frag_of(0);
    f16x8 x1 = kItems > 1 ? frag_of(1) : xf;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) decode(cur, s + 1, wf[(s + 1) & 1]);
      else fc2_load<NW, WRG, BN>(a, e, w, lane, min(j + (c + 2) / NCH, last), (c + 2) % NCH, NCH, cur);
#pragma unroll
      for (int cb = 0; cb < NCBA; ++cb) {
        const int i = s * NCBA + cb;
        const f16x8 x2 = i + 2 < kItems ? frag_of(i + 2) : x1;
#pragma unroll
        for (int r = 0; r < WRG; ++r)
          acc[r][cb] = mfma16x16x32(wf[s & 1][r], xf,
                                    (c == 0 && s == 0) ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[r][cb]);
        xf = x1;
        x1 = x2;
      }
      if (s < 3) {
#pragma unroll
        for (int cb = 0; cb < NCBA; ++cb) {
          if (s * NCBA + cb + 2 < kItems) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
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
  fc2_load<NW, WRG, BN>(a, e, w, lane, slab0, 0, NCH, setA);
  fc2_load<NW, WRG, BN>(a, e, w, lane, min(slab0 + 1 / NCH, last), 1 % NCH, NCH, setB);
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

// Decode rows [row_start, row_start + 16*ncb) of the requantized SiTU output (codes and
// scales in sorted-row order; rows past nrows repeat the last one) into the LDS tile, all
// Ip columns (zero past I), by all nthreads threads of the workgroup.
__device__ __forceinline__ void fc2_stage_tile(const LayerArgs& a, const TileDesc& td, int ncb,
                                               _Float16* __restrict__ s_tok, int tid,
                                               int nthreads) {
  const int dw_per_row = a.Ip / 8;
  const int code_bytes = a.I / 2;
  for (int idx = tid; idx < 16 * ncb * dw_per_row; idx += nthreads) {
    const int r = idx / dw_per_row, d = idx - r * dw_per_row;
    const int64_t row = td.row_start + min(r, td.nrows - 1);
    uint32_t cw = 0, sb = 0;
    if (4 * d < code_bytes) {
      cw = *reinterpret_cast<const uint32_t*>(a.a_codes + row * code_bytes + 4 * d);
      sb = a.a_scales[row * (a.I / 16) + d / 2];
    }
    *reinterpret_cast<f16x8*>(s_tok + r * kFc2LdsRow + 8 * d) = decode8(cw, scale_f16x2(sb));
  }
}

}  // namespace rmoe
