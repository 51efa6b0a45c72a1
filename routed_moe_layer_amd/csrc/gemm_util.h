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

__device__ __forceinline__ void map_workgroup(int b, int n_wt, int xcds, int* tt, int* wt) {
  const int xcd = b % xcds, slot = b / xcds;
  const int L = ((slot / kXcdRun) * xcds + xcd) * kXcdRun + slot % kXcdRun;
  const int per_group = n_wt * kTileGroup;
  *tt = (L / per_group) * kTileGroup + L % kTileGroup;
  *wt = (L / kTileGroup) % n_wt;
}

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Word 3 of a raw (unformatted, stride 0) buffer resource on gfx9-family targets: 32-bit
// data format, so dword loads of any width are taken as raw bytes; reads at or beyond
// num_records return zero.
constexpr int kBufferFlags = 0x00020000;

// FC2 output rows (workspace "o_rows"): routed row f = t*k + j's FC2 output O[f, h] =
// alpha2 * acc is kept as the f16 value of O * 2^s, with one exponent s per kOutSeg
// consecutive columns stored as an int8 in o_exp[t, h / kOutSeg, j] (token-major, so the
// finalization reads a segment's k exponents as one run).  s puts the largest |O| of the
// wave's columns into [2^13, 2^15], so every stored value keeps f16's 11 significant bits
// relative to it (BF16 would keep 8) and the finalization recovers O by an exact
// multiplication with 2^-s.
constexpr int kOutSeg = 32;

// Output scaling of one expert (uniform).  For a segment whose largest raw accumulator
// magnitude is m, p = fp32(m * |al|) is (up to rounding) its largest |O|; with E = p's
// biased exponent, s = 141 - E and c = al * 2^s, so the scaled values lie below 2^15
// (no f16 overflow) and the largest at or above 2^13.  E is clamped from below at
// max(15, Ea - 21) (Ea = al's biased exponent): this keeps s <= 126 and c finite for an
// all-zero segment (m = 0, values stay 0) and never binds otherwise, since nonzero
// accumulators are sums of multiples of 2^-20 (decoded NVFP4 products).
struct OutScale {
  float al, al_abs;
  uint32_t e_min;         // lower clamp of E, as exponent bits
};
__device__ __forceinline__ OutScale out_scale_of(float al) {
  const int ea = static_cast<int>((__float_as_uint(al) >> 23) & 0xFFu);
  OutScale o;
  o.al = al;
  o.al_abs = fabsf(al);
  o.e_min = static_cast<uint32_t>(max(15, ea - 21)) << 23;
  return o;
}
constexpr uint32_t kOutPowBase = static_cast<uint32_t>(127 + 141) << 23;   // 2^s = kOutPowBase - E<<23

// Bits of the largest magnitude among N floats, with integer max only (a float max
// would first quiet each input for NaN): as unsigned integers every negative float ranks
// above every positive one and among negatives the larger magnitude ranks higher, so the
// unsigned max is the largest-magnitude negative when there is one; as signed integers
// the max is the largest positive when there is one.  The larger magnitude of the two is
// the answer (a signed max, since a negative signed result lies below any magnitude).
template <int N>
__device__ __forceinline__ uint32_t max_abs_bits(const float (&v)[N]) {
  uint32_t u = __float_as_uint(v[0]);
  int32_t i = __float_as_int(v[0]);
#pragma unroll
  for (int n = 1; n < N; ++n) {
    u = max(u, __float_as_uint(v[n]));
    i = max(i, __float_as_int(v[n]));
  }
  return static_cast<uint32_t>(max(i, static_cast<int32_t>(u & 0x7FFFFFFFu)));
}

// Largest of v over lanes l, l^16, l^32, l^48 (gfx950's row-swap instructions: no LDS).
__device__ __forceinline__ float max_over_lane_rows(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t m = max(a[0], a[1]);               // non-negative floats order as bits
  const auto b = __builtin_amdgcn_permlane32_swap(m, m, false, false);
  return __uint_as_float(max(b[0], b[1]));
}

// Halves per token row of a wave's output staging buffer (16 rows, padded by 8).
template <int WRG>
constexpr int out_lds_stride() { return 16 * WRG + 8; }

// Store one wave's 16-token block of FC2 output.  acc[r] holds, in the MFMA output layout,
// columns col0 + 16r + 4(lane/16) + i of block token lane % 16, so the wave's 16*WRG
// columns of a token lie in lanes n, n+16, n+32, n+48.  The exponent is taken over all of
// them (the same value in each of the wave's 32-column slots of o_exp): the 4*WRG values of
// each lane and one max over those lanes.  The scaled f16 values pass through the wave's
// LDS buffer `lds` (16 * out_lds_stride<WRG>() halves) so that the global stores are whole
// 16-byte pieces of consecutive columns: one store instruction covers 64/(2*WRG) token rows
// with 32*WRG contiguous bytes each (the rows are scattered over the output, so longer runs
// per instruction cut the memory transactions).  flat_lane is the flat id t*k + j (output
// row) of token lane % 16; tokens >= ntok are not stored.
template <int WRG>
__device__ __forceinline__ void store_out_block(const f32x4 (&acc)[WRG], const OutScale& sc,
                                                uint16_t* lds, int lane, int32_t flat_lane,
                                                int ntok, uint16_t* __restrict__ o_rows,
                                                int8_t* __restrict__ o_exp, int H, int k,
                                                uint64_t k_inv, int col0) {
  static_assert(WRG == 2 || WRG == 4, "whole 32-column slots per wave");
  constexpr int S = out_lds_stride<WRG>();
  const int g = lane >> 4, n16 = lane & 15;
  float vals[4 * WRG];
#pragma unroll
  for (int r = 0; r < WRG; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) vals[4 * r + i] = acc[r][i];
  const float m = __uint_as_float(max_abs_bits(vals));
  const uint32_t eb =
      max(__float_as_uint(max_over_lane_rows(m) * sc.al_abs) & 0x7F800000u, sc.e_min);
  const float c = sc.al * __uint_as_float(kOutPowBase - eb);
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
#pragma unroll
  for (int pass = 0; pass < 16 / kRowsPerPass; ++pass) {
    const int row = pass * kRowsPerPass + lane / kPieces, piece = lane % kPieces;
    const u32x4 v = *reinterpret_cast<const u32x4*>(lds + row * S + 8 * piece);
    const int64_t flat = __shfl(flat_lane, row);
    if (row < ntok) *reinterpret_cast<u32x4*>(o_rows + flat * H + col0 + 8 * piece) = v;
  }
  __builtin_amdgcn_wave_barrier();                 // (the wave's LDS operations run in order)
  if (g < WRG / 2 && n16 < ntok) {
    const int8_t se = static_cast<int8_t>(141 - static_cast<int>(eb >> 23));
    // t = flat / k by the multiplicative inverse (exact for flat ids below 2^26)
    const int t = static_cast<int>((static_cast<uint64_t>(flat_lane) * k_inv) >> 32);
    const int j = flat_lane - t * k;
    o_exp[(static_cast<int64_t>(t) * (H / kOutSeg) + col0 / kOutSeg + g) * k + j] = se;
  }
}

}  // namespace rmoe
