// Helpers shared by the grouped-GEMM kernels: the workgroup -> (token tile, weight slab)
// mapping and buffer-resource constants.
#pragma once

#include "common.h"
#include "kernels.h"

namespace rmoe {

// Workgroup -> (token tile, weight slab).  Workgroups are dealt to the 8 XCDs round-robin
// by id; kXcdRun consecutive logical ids are kept on one XCD (and in flight together),
// and logical ids run over kTileGroup consecutive token tiles of one slab before moving to
// the next slab.  The token tiles of an expert are adjacent in the work list, so the
// workgroups that read the same weight slab share that XCD's L2, and a group of token
// tiles is reread across slabs while it is still cached.
constexpr int kXcds = 8, kXcdRun = 4, kTileGroup = 4;

__device__ __forceinline__ void map_workgroup(int b, int n_wt, int* tt, int* wt) {
  const int xcd = b % kXcds, slot = b / kXcds;
  const int L = ((slot / kXcdRun) * kXcds + xcd) * kXcdRun + slot % kXcdRun;
  const int per_group = n_wt * kTileGroup;
  *tt = (L / per_group) * kTileGroup + L % kTileGroup;
  *wt = (L / kTileGroup) % n_wt;
}

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Word 3 of a raw (unformatted, stride 0) buffer resource on gfx9-family targets: 32-bit
// data format, so dword loads of any width are taken as raw bytes; reads at or beyond
// num_records return zero.
constexpr int kBufferFlags = 0x00020000;

// FC2 output rows (workspace "o_rows"): routed row f's FC2 output O[f, h] = alpha2 * acc
// is kept as the f16 value of O * 2^s, with one exponent s per kOutSeg consecutive columns
// stored as an int8 in o_exp[f, h / kOutSeg].  s puts the segment's largest |O| into
// [2^14, 2^15), so every stored value keeps f16's 11 significant bits (BF16 would keep 8)
// and the finalization recovers O by an exact multiplication with 2^-s.
constexpr int kOutSeg = 32;

// Scale c = alpha2 * 2^s of a segment whose largest raw accumulator magnitude is mraw, and
// its exponent s (0 for an all-zero or NaN segment).  alpha2 * 2^s is exact: nonzero
// accumulators are sums of multiples of 2^-20 (decoded NVFP4 products), so |c| stays in
// the normal range; s is clamped to [-126, 126] so that 2^s and 2^-s are normal floats.
__device__ __forceinline__ float out_seg_scale(float mraw, float al, int* s_out) {
  const float m = mraw * fabsf(al);
  int s = 0;
  if (m > 0.0f) {
    const int e = static_cast<int>(__float_as_uint(m) >> 23) - 127;   // floor(log2 m)
    s = min(max(14 - e, -126), 126);
  }
  *s_out = s;
  return al * __uint_as_float(static_cast<uint32_t>(127 + s) << 23);
}

// The value of lane l^1 or l^2 (a DPP quad permutation: no LDS traffic).
__device__ __forceinline__ float lane_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}

// Floats per token row of a wave's output staging buffer (16 rows).
template <int WRG>
constexpr int out_lds_stride() { return 16 * WRG + 4; }

// Store one wave's 16-token block of FC2 output.  acc[r] holds, in the MFMA output layout,
// columns col0 + 16r + 4(lane/16) + i of block token lane % 16.  The raw accumulators pass
// through the wave's LDS buffer `lds` (16 * out_lds_stride<WRG>() floats) so that lane l
// then holds the 4*WRG consecutive columns col0 + 4*WRG*(l%4) .. of token l/4: a 32-column
// segment lies in 32/(4*WRG) adjacent lanes, which agree on its exponent with one or two
// lane exchanges.  flat_lane is the flat id (output row) of token lane % 16; tokens with
// ntok <= l/4 are not stored.
template <int WRG>
__device__ __forceinline__ void store_out_block(const f32x4 (&acc)[WRG], float al, float* lds,
                                                int lane, int32_t flat_lane, int ntok,
                                                uint16_t* __restrict__ o_rows,
                                                int8_t* __restrict__ o_exp, int H, int col0) {
  static_assert(WRG == 2 || WRG == 4, "a 32-column segment spans 4 or 2 lanes");
  constexpr int S = out_lds_stride<WRG>();
  constexpr int V = 4 * WRG;                     // consecutive columns per lane
#pragma unroll
  for (int r = 0; r < WRG; ++r)
    *reinterpret_cast<f32x4*>(lds + (lane & 15) * S + 16 * r + 4 * (lane >> 4)) = acc[r];
  __builtin_amdgcn_wave_barrier();
  const int n = lane >> 2, q = lane & 3;
  float v[V];
#pragma unroll
  for (int i = 0; i < V; i += 4) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(lds + n * S + q * V + i);
    v[i] = t[0]; v[i + 1] = t[1]; v[i + 2] = t[2]; v[i + 3] = t[3];
  }
  __builtin_amdgcn_wave_barrier();               // (the wave's LDS operations run in order)
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < V; ++i) m = fmaxf(m, fabsf(v[i]));
  m = fmaxf(m, lane_xor1(m));
  if constexpr (V == 8) m = fmaxf(m, lane_xor2(m));
  int s;
  const float c = out_seg_scale(m, al, &s);
  uint32_t h[V / 2];
#pragma unroll
  for (int i = 0; i < V / 2; ++i)
    h[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(
                                            f32x2{v[2 * i] * c, v[2 * i + 1] * c}, f16x2));
  const int64_t flat = __shfl(flat_lane, n);
  if (n < ntok) {
    const int col = col0 + q * V;
    u32x4* dst = reinterpret_cast<u32x4*>(o_rows + flat * H + col);
#pragma unroll
    for (int i = 0; i < V / 8; ++i) dst[i] = u32x4{h[4 * i], h[4 * i + 1], h[4 * i + 2], h[4 * i + 3]};
    if (col % kOutSeg == 0) o_exp[flat * (H / kOutSeg) + col / kOutSeg] = static_cast<int8_t>(s);
  }
}

}  // namespace rmoe
