// Helpers shared by the grouped-GEMM kernels: token-code loads, their decode into LDS
// f16 rows, and the workgroup -> (token tile, weight slab) mapping.
#pragma once

#include "common.h"
#include "kernels.h"

namespace rmoe {

// Loads, for chunk c, the code dwords and scale bytes one thread decodes.  Columns past
// the row's real length read as zero codes with a zero scale.
template <int NDW>
__device__ __forceinline__ void load_token_chunk(const uint8_t* __restrict__ codes_row,
                                                 const uint8_t* __restrict__ scales_row,
                                                 int c, int part, int valid_code_bytes,
                                                 uint32_t (&w)[NDW], uint32_t& sc) {
  static_assert(NDW <= 2 || NDW % 4 == 0, "a thread decodes 1, 2 or a multiple of 4 dwords");
  const int byte0 = c * 64 + part * NDW * 4;           // first code byte of this thread
  if constexpr (NDW == 1) {
    w[0] = byte0 < valid_code_bytes ? *reinterpret_cast<const uint32_t*>(codes_row + byte0) : 0u;
  } else if constexpr (NDW == 2) {
    if (byte0 < valid_code_bytes) {
      const uint2 v = *reinterpret_cast<const uint2*>(codes_row + byte0);
      w[0] = v.x; w[1] = v.y;
    } else {
      w[0] = 0; w[1] = 0;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NDW; i += 4) {
      if (byte0 + 4 * i < valid_code_bytes) {
        const uint4 v = *reinterpret_cast<const uint4*>(codes_row + byte0 + 4 * i);
        w[i] = v.x; w[i + 1] = v.y; w[i + 2] = v.z; w[i + 3] = v.w;
      } else {
        w[i] = 0; w[i + 1] = 0; w[i + 2] = 0; w[i + 3] = 0;
      }
    }
  }
  // NDW dwords = 8*NDW codes = NDW/2 blocks; scale bytes of this thread
  const int sbyte0 = byte0 / 8;
  sc = 0;
  if (byte0 < valid_code_bytes) {
    if constexpr (NDW >= 8) {
      sc = *reinterpret_cast<const uint32_t*>(scales_row + sbyte0);
    } else {
#pragma unroll
      for (int b = 0; b < (NDW + 1) / 2; ++b)
        sc |= static_cast<uint32_t>(scales_row[sbyte0 + b]) << (8 * b);
    }
  }
}

template <int NDW>
__device__ __forceinline__ void store_token_chunk(_Float16* __restrict__ dst,
                                                  const uint32_t (&w)[NDW], uint32_t sc) {
#pragma unroll
  for (int i = 0; i < NDW; ++i) {
    const f16x8 v = decode8(w[i], scale_f16x2((sc >> (8 * (i >> 1))) & 0xFFu));
    *reinterpret_cast<f16x8*>(dst + 8 * i) = v;
  }
}

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

}  // namespace rmoe
