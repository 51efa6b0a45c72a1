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

}  // namespace rmoe
