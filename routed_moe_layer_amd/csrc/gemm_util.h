// Helpers shared by the grouped-GEMM kernels: the workgroup -> (token tile, weight slab)
// mapping and buffer-resource constants.
#pragma once

#include "common.h"
#include "kernels.h"

namespace rmoe {

// Workgroup -> (token tile, weight slab).  Workgroups are dealt to the device's XCDs
// round-robin by id (xcds of them; 8 on an MI355X in its single-partition mode); kXcdRun
// consecutive logical ids are kept on one XCD (and in flight together), and logical ids
// run over kTileGroup consecutive token tiles of one slab before moving to the next slab.
// The token tiles of an expert are adjacent in the work list, so the workgroups that read
// the same weight slab share that XCD's L2, and a group of token tiles is reread across
// slabs while it is still cached.  Grids are whole multiples of xcds * kXcdRun.
constexpr int kXcdRun = 4, kTileGroup = 4;

// (run: the number of consecutive logical ids kept on one XCD, kXcdRun unless given)
__device__ __forceinline__ void map_workgroup(int b, int n_wt, int xcds, int* tt, int* wt,
                                              int run = kXcdRun) {
  const int xcd = b % xcds, slot = b / xcds;
  const int L = ((slot / run) * xcds + xcd) * run + slot % run;
  const int per_group = n_wt * kTileGroup;
  *tt = (L / per_group) * kTileGroup + L % kTileGroup;
  *wt = (L / kTileGroup) % n_wt;
}

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Word 3 of a raw (unformatted, stride 0) buffer resource on gfx9-family targets: 32-bit
// data format, so dword loads of any width are taken as raw bytes; reads at or beyond
// num_records return zero.
constexpr int kBufferFlags = 0x00020000;

// Cache policy of a weight stream.  Small token tiles (at most kSmallRows rows, one per
// lightly used expert) read each weight once per layer call, so their streams are
// nontemporal (the "nt" bit of a buffer load): a CU streams such loads about 15% faster
// than plain ones (27.6 against 24-25 GB/s per CU on the MI355X).  Big tiles keep the
// default policy: the several tiles of a heavily used expert reread its weights from the
// L2, which nontemporal loads would give up.
constexpr int kNontemporal = 2;
constexpr int weight_load_policy(int tile_rows) { return tile_rows <= kSmallRows ? kNontemporal : 0; }

// FC2 output rows (workspace "o_rows"): routed row f = t*k + j's FC2 output O[f, h] =
// alpha2 * acc is kept as the f16 value of O * 2^s, with one exponent s per expert, stored
// as an int8 in o_exp[f] for the finalization (which recovers O by an exact multiplication
// with 2^-s).  s comes from a bound rather than from the data: every decoded NVFP4 value is
// at most 6 * 448 = 2688 in magnitude, so |acc| <= I * 2688^2; with E the biased exponent
// of p = fp32(|alpha2| * I * 2688^2), s = 141 - E puts p * 2^s below 2^15, so no stored
// value overflows f16, and every |O| * 2^s of at least 2^-14 (every |acc| above
// I * 2688^2 * 2^-29, e.g. above 5.2 at I = 384) keeps f16's 11 significant bits.  Nonzero
// accumulators are sums of products of decoded values (multiples of 2^-20), and a row
// with any nonzero intermediate code is far above that floor unless its products cancel.
// s is clamped to [-126, 126] so that 2^s and 2^-s are normal floats.
struct OutScale {
  float c;                // alpha2 * 2^s
  int s;
};
__device__ __forceinline__ OutScale out_scale(float al, int I) {
  const float p = fabsf(al) * (static_cast<float>(I) * 7225344.0f);   // 2688^2
  const int ep = static_cast<int>((__float_as_uint(p) >> 23) & 0xFFu);
  const int s = min(max(141 - ep, -126), 126);
  return OutScale{al * __uint_as_float(static_cast<uint32_t>(127 + s) << 23), s};
}

// Halves per token row of a wave's output staging buffer (16 rows, padded by 8).
template <int WRG>
constexpr int out_lds_stride() { return 16 * WRG + 8; }

// Store one wave's 16-token block of FC2 output.  acc[r] holds, in the MFMA output layout,
// columns col0 + 16r + 4(lane/16) + i of block token lane % 16.  The scaled f16 values
// pass through the wave's LDS buffer `lds` (16 * out_lds_stride<WRG>() halves) so that the
// global stores are whole 16-byte pieces of consecutive columns: one store instruction
// covers 64/(2*WRG) token rows with 32*WRG contiguous bytes each (the rows are scattered
// over the output, so longer runs per store instruction cut the memory transactions).
// flat_lane is the flat id t*k + j (output row) of token lane % 16; tokens >= ntok are not
// stored.  The wave that holds column 0 also stores the rows' exponent.
template <int WRG>
__device__ __forceinline__ void store_out_block(const f32x4 (&acc)[WRG], const OutScale& sc,
                                                uint16_t* lds, int lane, int32_t flat_lane,
                                                int ntok, uint16_t* __restrict__ o_rows,
                                                int8_t* __restrict__ o_exp, int H, int col0) {
  constexpr int S = out_lds_stride<WRG>();
  const int g = lane >> 4, n16 = lane & 15;
  const float c = sc.c;
#pragma unroll
  for (int r = 0; r < WRG; ++r) {
    const f32x4 o = acc[r];
    u32x2 v;
    v[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{o[0] * c, o[1] * c}, f16x2));
    v[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{o[2] * c, o[3] * c}, f16x2));
    *reinterpret_cast<u32x2*>(lds + n16 * S + 16 * r + 4 * g) = v;
  }
  __builtin_amdgcn_wave_barrier();
  constexpr int kPieces = 2 * WRG;                 // 16-byte pieces per row
  constexpr int kRowsPerPass = 64 / kPieces;
  constexpr int kPasses = 16 / kRowsPerPass;
  // every pass's LDS read and row id first, then the stores: one wait for all of them
  u32x4 v[kPasses];
  uint32_t flat[kPasses];
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int row = pass * kRowsPerPass + lane / kPieces, piece = lane % kPieces;
    v[pass] = *reinterpret_cast<const u32x4*>(lds + row * S + 8 * piece);
    flat[pass] = static_cast<uint32_t>(__shfl(flat_lane, row));
  }
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int row = pass * kRowsPerPass + lane / kPieces, piece = lane % kPieces;
    // the row's 16-byte piece index, flat * H/8 + ..., in 32 bits from one 24-bit multiply
    // (a flat id is below 2^20 and H/8 at most 2^11; H and col0 are multiples of 8)
    const uint32_t q = __umul24(flat[pass], static_cast<uint32_t>(H / 8)) +
                       static_cast<uint32_t>(col0 / 8 + piece);
    if (row < ntok) reinterpret_cast<u32x4*>(o_rows)[q] = v[pass];
  }
  __builtin_amdgcn_wave_barrier();                 // (the wave's LDS operations run in order)
  if (col0 == 0 && g == 0 && n16 < ntok) o_exp[flat_lane] = static_cast<int8_t>(sc.s);
}

}  // namespace rmoe
