// Internal launcher declarations shared by the C-ABI host code and the kernel files.
// Every launcher enqueues on `stream` and returns the hipGetLastError() of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rmoe {

// One entry of the grouped-GEMM work list: `nrows` consecutive expert-sorted rows starting
// at `row_start`, all routed to expert `expert`.
struct TileDesc {
  int32_t expert;
  int32_t row_start;
  int32_t nrows;
  int32_t pad;
};

// Router geometry: flat ids are processed in tiles of kRouteTile by workgroups of 256.
constexpr int kRouteTile = 1024;
constexpr int kRouteThreads = 256;
// Grouped-GEMM token tiles (the N side of both FC kernels).  An expert with at most
// kSmallRows routed rows gets one "small" tile; a larger expert is split into
// nb = ceil(cnt / kBigTileRows) "big" tiles of near-equal size (a multiple of 16 rows, the
// last one shorter).  The two lists feed two variants of the GEMM kernels, whose big-tile
// LDS tiles are kBigRows rows; big tiles hold at most seven 16-row blocks, so the kernels
// need no accumulators for an eighth.
constexpr int kSmallRows = 32;
constexpr int kBigRows = 128;
constexpr int kBigTileRows = 112;
// FC2 for many routed rows works on runs of up to kRunTiles consecutive big tiles of one
// expert (a contiguous range of its sorted rows).
constexpr int kRunTiles = 4;
// From two big tiles per compute unit on (2 * cus * kBigRows routed rows, 65536 on the
// 256-CU MI355X), FC1 stages every token tile as NVFP4 codes and the layer does not write
// the f16 copy of x (x_dec).
inline bool many_rows(int64_t R, int cus) { return R >= int64_t{2} * cus * kBigRows; }
inline bool layer_writes_x_dec(int64_t R, int cus) { return !many_rows(R, cus); }

inline int route_tiles(int64_t n) { return static_cast<int>((n + kRouteTile - 1) / kRouteTile); }
inline int bits_for(int E) { int b = 1; while ((1 << b) < E) ++b; return b; }
// Upper bounds of the list lengths for R routed rows over E experts.
// Batches of at most kSmallOnlyRows routed rows take small tiles only (an expert with more
// than kSmallRows rows gets several), so their GEMMs need no big-tile launches.
constexpr int64_t kSmallOnlyRows = 1024;
inline int64_t max_small_tiles(int64_t R, int E) {
  // (the second term stays at its largest value above kSmallOnlyRows, so the bound, and
  // the workspace, never shrink as R grows)
  return (R < E ? R : E) + (R < kSmallOnlyRows ? R : kSmallOnlyRows) / kSmallRows;
}
inline int64_t max_big_tiles(int64_t R, int E) {
  const int64_t big_experts = R / (kSmallRows + 1);
  return R / kBigTileRows + (big_experts < E ? big_experts : E);
}

hipError_t launch_quantize_nvfp4(const uint16_t* src, int64_t groups, int64_t rows_per_group,
                                 int K, const float* q, uint8_t* codes, uint8_t* scales,
                                 uint16_t* decoded, hipStream_t stream);

// Routing: histogram, scan (+ optional GEMM tile list and stats reset), stable scatter.
// The E experts routed are ids e_base .. e_base + E - 1 (an active expert range); other
// ids take no part.  Positions i of the sort run over the in-range ids only.
struct RouteBuffers {
  int32_t* tile_hist;        // [route_tiles(n), E]
  int32_t* counts;           // [E]
  int32_t* offsets;          // [E + 1] exclusive; offsets[E] = number of in-range ids
  int32_t* cumsum;           // [E] inclusive (may be null)
  int32_t* sorted_ids;       // [n] absolute expert ids; entries >= offsets[E] are -1 (or null)
  int32_t* sorted_row_idx;   // [n] flat ids; entries >= offsets[E] are -1 (or null)
  int32_t* expanded_row_idx; // [n] position map: sorted position of f, -1 out of range
  TileDesc* tiles_small;     // [max_small_tiles] or null
  TileDesc* tiles_big;       // [max_big_tiles] or null
  TileDesc* runs;            // [max_big_tiles] FC2 runs (needs the tile lists) or null
  int small_only;            // every tile a small one (layer batches of <= kSmallOnlyRows rows)
  int32_t* num_tiles;        // [2] small, big (or [3] with runs); or null
  float* amax_reset;         // [E] zeroed by the scan kernel, or null
  int32_t* key_value;        // [kv_rows, 2]: (expert id, count) of the experts with a
                             // nonzero count in increasing id, then zero rows; or null.
                             // Never together with the tile lists.
  int32_t* available;        // [1] number of in-range ids, or null
  int32_t kv_rows;
  int32_t e_base;
  int32_t capacity;          // > 0: the position map holds slot e*capacity + rank within
                             // the expert, or -1 when rank >= capacity
};


// The layer's token quantization as extra workgroups of a router launch: with the
// single-workgroup router (route_fits_one_workgroup; launch_quantize_route_small) or with
// the scatter of the tiled router (launch_route with `fused`).
struct QuantizeArgs {
  const uint16_t* src;       // BF16 rows
  int64_t nblocks;           // 16-value blocks in all rows
  int blocks_per_row;
  int64_t rows_per_group;
  const float* q;            // encoding scale per group of rows
  uint8_t* codes;
  uint8_t* scales;
  uint16_t* decoded;         // or null
};
// The routing pipeline; with `fused`, the token quantization it describes runs in the
// same launches (the scatter's extra workgroups), else nothing more.
hipError_t launch_route(const int32_t* ids, int64_t n, int E, const RouteBuffers& b,
                        hipStream_t stream, const QuantizeArgs* fused = nullptr);
bool route_fits_one_workgroup(int64_t n, int E);

// Routing primitive on a few tokens: routing and token movement in one workgroup (see
// launch_route_permute for the modes).  Applies when route_permute_fits_one_workgroup.
struct PermuteArgs {
  const uint16_t* x;
  int64_t N;
  int H, K, quant;
  int64_t limit;
  const float* row_scale;
  const float* static_scale;
  const float* static_offset;
  void* expanded_x;
  float* expanded_scale;
};
bool route_permute_fits_one_workgroup(int64_t n, int E, int64_t N, int H);
hipError_t launch_route_permute_small(const int32_t* ids, int64_t n, int E, const RouteBuffers& b,
                                      const PermuteArgs& p, hipStream_t stream);
hipError_t launch_quantize_route_small(const QuantizeArgs& qa, const int32_t* ids, int64_t n,
                                       int E, const RouteBuffers& b, hipStream_t stream);

// Token movement of the routing primitive: token row t goes to rows map[t*K + j] (skipped
// when negative or >= limit).  may_skip: some tokens may have no row to go to (an expert
// range, capacity or row limit); such tokens are then not read.  quant 0: BF16 copy (plus row_scale[t] to expanded_scale
// when both are given); 1: dynamic int8 with its scale; 2: static int8 with the device
// scalars *static_scale and *static_offset.
hipError_t launch_route_permute(const uint16_t* x, int64_t N, int H, int K, int quant,
                                const int32_t* map, int64_t limit, bool may_skip,
                                const float* row_scale,
                                const float* static_scale, const float* static_offset,
                                void* expanded_x, float* expanded_scale, hipStream_t stream);
// NVFP4 token movement: token row t quantized once (group 16, device scalar *qx) and its
// codes [H/2] and E4M3 scales [H/16] written to rows map[t*K + j] (skipped when negative).
hipError_t launch_route_permute_nvfp4(const uint16_t* x, int64_t N, int H, int K,
                                      const int32_t* map, const float* qx, uint8_t* codes,
                                      uint8_t* scales, hipStream_t stream);
// Drop/pad: zero the slots of expert e at and past counts[e] (rows of row_bytes bytes,
// a multiple of 8; scale 0 when expanded_scale is given), for E experts of C slots each.
hipError_t launch_route_pad_fill(const int32_t* counts, int E, int C, int64_t row_bytes,
                                 void* expanded_x, float* expanded_scale, hipStream_t stream);

// Streamed front end (stream.hip): one 64-byte counter record per ring slot.
struct RingSlot {
  uint32_t route_ready;    // generation the routing producer last published
  uint32_t layout_ready;   // generation the layout producer last published
  uint32_t consumed;       // generation the consumer last finished
  uint32_t route_seq;      // routing producer's sequence
  uint32_t layout_seq;     // layout producer's sequence
  uint32_t consumer_seq;   // consumer's sequence
  uint32_t pad[10];
};
static_assert(sizeof(RingSlot) == 64, "one counter record per 64 bytes");
hipError_t launch_ring_init(uint32_t* words, int n, hipStream_t stream);
hipError_t launch_ring_wait(const uint32_t* a, const uint32_t* b, const uint32_t* seq,
                            uint32_t add, int64_t ticks, uint32_t* status, uint32_t code,
                            hipStream_t stream);
hipError_t launch_ring_publish(uint32_t* gen, uint32_t* seq, hipStream_t stream);
// Device copy of `bytes` (even) bytes on `stream`, 2-byte aligned pointers.
hipError_t launch_slot_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream);
// Copy of n expert ids, or n times -1 when *status (the ring's status word) is nonzero.
hipError_t launch_slot_ids(int32_t* dst, const int32_t* src, int64_t n, const uint32_t* status,
                           hipStream_t stream);

// Top-k expert selection with softmax weights over the picks (topk.hip): logits f32
// [T, E] (E <= 4096), k <= 64 -> ids i32 [T, k], BF16 weights [T, k].
hipError_t launch_topk_softmax(const float* logits, int64_t T, int E, int k, int32_t* ids,
                               uint16_t* weights, hipStream_t stream);

hipError_t launch_prepare_weights(int H, int I, int E, const uint8_t* w13,
                                  const uint8_t* w13_sf, const uint8_t* w2,
                                  const uint8_t* w2_sf, uint8_t* prepared, hipStream_t stream);

struct LayerArgs {
  int H, I, Ip, E, k, T;
  int cus, xcds;               // compute units and XCDs (L2 domains) of the device
  const uint8_t* x_codes;      // [T, H/2]
  const uint8_t* x_scales;     // [T, H/16]
  const uint16_t* x_dec;       // [T, H] f16: code times block scale
  const int32_t* sorted_row_idx;
  const int32_t* expanded_row_idx;
  const TileDesc* tiles_small;
  const TileDesc* tiles_big;
  const TileDesc* runs;        // FC2 runs (list length max_big_tiles)
  const int32_t* num_tiles;    // [3]: small tiles, big tiles, runs
  int64_t max_small, max_big;
  const uint8_t* w13_codes;    // prepared
  const uint8_t* w13_scales;
  const uint8_t* w2_codes;
  const uint8_t* w2_scales;
  const float* alpha1;
  const float* qa;
  const float* alpha2;
  const float* beta;           // may be null
  const float* lam;            // may be null
  uint8_t* a_codes;            // [T*k, I/2]
  uint8_t* a_scales;           // [T*k, I/16]
  float* a_amax;               // [E]
  uint16_t* o_rows;            // [T*k, H] f16 O * 2^s, row t*k + j (flat id order)
  int8_t* o_exp;               // [T*k] exponent s of each FC2 output row (its expert's)
  const uint16_t* route_weights;
  uint16_t* out;               // [T, H]
};
hipError_t launch_fc1(const LayerArgs& a, hipStream_t stream);
// FC1 and FC2 in one launch when every routed row can have a CU of its own
// (layer_small_fused_fits); launch_fc1 + launch_fc2 otherwise.
bool layer_small_fused_fits(const LayerArgs& a);
hipError_t launch_layer_small_fused(const LayerArgs& a, hipStream_t stream);
hipError_t launch_fc2(const LayerArgs& a, hipStream_t stream);
// FC2 with the whole token tile resident in LDS (when the padded I fits; fc2.hip).
bool fc2_resident_fits(const LayerArgs& a);
void launch_fc2_resident_small(const LayerArgs& a, hipStream_t stream);
void launch_fc2_resident_big(const LayerArgs& a, hipStream_t stream);
void launch_fc2_resident_big_spread(const LayerArgs& a, hipStream_t stream);
hipError_t launch_finalize(const LayerArgs& a, hipStream_t stream);

// Prepared-weight layout (private).  For a matrix of R rows (multiple of 16) and K columns
// padded to Kp (multiple of 128), per expert: codes [Kp/128][R/16][64 lanes][16 B] and
// scales [Kp/128][R/16][2][16][4 B] -- chunk-major, so the row groups a workgroup reads
// for one 128-column chunk are one contiguous run.  Lane l of row group G, chunk c holds
// row 16G + l%16,
// and its dword s (s = 0..3) holds the 8 codes k = 128c + 32s + 8(l/16) + [0..7]
// (the f16 16x16x32 MFMA operand for K-step s).  Those 8 codes lie in block
// 8c + 2s + (l/16)/2, so lanes l and l+16 share a block: the scale dword of lane l is
// dword (l/32)*16 + l%16 of the chunk, byte s of it being the scale of K-step s.  Both
// parts are exactly as large as the canonical codes and scales.
// FC1 rows are reordered so that row 2j of group G is gate row 8G+j and row 2j+1 is up
// row 8G+j: each lane then holds g and u of the same intermediate channels.
inline size_t prepared_codes_bytes(int R, int Kp) { return static_cast<size_t>(R) * Kp / 2; }
inline size_t prepared_scales_bytes(int R, int Kp) { return static_cast<size_t>(R) * Kp / 16; }
// Index of the 16-row x 128-column chunk (expert e, chunk c, row group G) among a
// matrix's chunks (groups = R/16 row groups, nchunks = Kp/128 chunks per expert): its
// codes are the 1024 bytes at 1024 * index, its scales the 32 dwords at 32 * index.
__host__ __device__ inline int64_t prepared_chunk(int64_t e, int c, int G, int nchunks,
                                                  int groups) {
  return (e * nchunks + c) * groups + G;
}
// Index of lane `lane`'s scale dword of chunk `chunk`, in uint32 units.
__host__ __device__ inline int64_t prepared_scale_index(int64_t chunk, int lane) {
  return chunk * 32 + (lane >> 5) * 16 + (lane & 15);
}

}  // namespace rmoe
