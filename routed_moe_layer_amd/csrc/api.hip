// C ABI of the routed-MoE library: argument validation, workspace carving and launches.
// Declarations and the contract of every entry point are in include/routed_moe.h.
#include "routed_moe.h"

#include <algorithm>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace {

using namespace rmoe;

constexpr size_t kAlign = 256;
// The routing primitive's expert-count limits ("torch_npu.npu_moe_init_routing_v2",
// parameter expert_num: at most 10240, at most 5120 with the key_value histogram); the
// whole layer takes at most 4096 experts.
constexpr int kRouteMaxExperts = 10240, kRouteMaxExpertsKeyValue = 5120;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, kAlign);
    return o;
  }
};

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

moe_status_t check_dims(const moe_dims_t& d) {
  if (d.hidden <= 0 || d.inter <= 0 || d.num_experts <= 0 || d.top_k <= 0)
    return MOE_ERR_INVALID_ARG;
  if (d.hidden % 128 || d.inter % 64) return MOE_ERR_UNSUPPORTED;
  if (d.hidden < 128 || d.hidden > 16384 || d.inter < 64 || d.inter > 4096)
    return MOE_ERR_UNSUPPORTED;
  if (d.num_experts > 4096 || d.top_k > 64) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// The FC2 row stores index 16-byte pieces of the row output in 32 bits (flat id times
// H/8 through a 24-bit multiply): the limits above keep both factors and the index in range.
static_assert(int64_t{MOE_MAX_TOKENS} * 64 <= (int64_t{1} << 20), "flat ids below 2^20");
static_assert(int64_t{MOE_MAX_TOKENS} * 64 * (16384 / 8) <= (int64_t{1} << 31),
              "FC2 row piece indices fit 32 bits");

int padded_inter(int I) { return (I + kChunk - 1) / kChunk * kChunk; }

// Streamed front end: ring carving and the device wall-clock rate for wait deadlines.
moe_status_t ring_layout(const moe_dims_t& d, int32_t S, int32_t C, moe_ring_layout_t* L) {
  moe_status_t st = check_dims(d);
  if (st != MOE_OK) return st;
  if (S < 1 || S > 4096 || C < 1 || C > MOE_MAX_TOKENS) return MOE_ERR_INVALID_ARG;
  const size_t slot_tokens = static_cast<size_t>(S) * C;
  Carver c;
  L->x = c.take(slot_tokens * d.hidden * 2);
  L->expert_ids = c.take(slot_tokens * d.top_k * 4);
  L->route_weights = c.take(slot_tokens * d.top_k * 2);
  L->counters = c.take(static_cast<size_t>(S) * sizeof(RingSlot));
  L->status = c.take(4);
  L->total = c.off;
  return MOE_OK;
}

moe_status_t check_ring(const moe_dims_t& d, const moe_ring_t* r, moe_ring_layout_t* L) {
  if (!r || !r->base) return MOE_ERR_INVALID_ARG;
  moe_status_t st = ring_layout(d, r->num_slots, r->tokens_per_slot, L);
  if (st != MOE_OK) return st;
  if (!aligned(r->base, kAlign)) return MOE_ERR_INVALID_ARG;
  if (r->bytes < L->total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return MOE_OK;
}

RingSlot* ring_slots(const moe_ring_t* r, const moe_ring_layout_t& L) {
  return reinterpret_cast<RingSlot*>(static_cast<uint8_t*>(r->base) + L.counters);
}

uint32_t* ring_status(const moe_ring_t* r, const moe_ring_layout_t& L) {
  return reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(r->base) + L.status);
}

// Wall-clock ticks of a timeout (0 = the default), on the current device.
constexpr uint32_t kDefaultRingTimeoutUs = 1000000;
bool ring_ticks(uint32_t timeout_us, int64_t* ticks) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
    return false;
  const uint64_t us = timeout_us ? timeout_us : kDefaultRingTimeoutUs;
  *ticks = static_cast<int64_t>(us * static_cast<uint64_t>(khz) / 1000u);
  return true;
}

struct Layout {
  moe_workspace_layout_t pub;
  size_t offsets, tile_hist, tiles_small, tiles_big, runs, num_tiles;
};

Layout make_layout(const moe_dims_t& d, int64_t T) {
  const int64_t H = d.hidden, I = d.inter, E = d.num_experts, R = T * d.top_k;
  Carver c;
  Layout L{};
  L.pub.x_codes = c.take(T * H / 2);
  L.pub.x_scales = c.take(T * H / 16);
  L.pub.x_dec = c.take(T * H * 2);
  L.pub.sorted_ids = c.take(R * 4);
  L.pub.sorted_row_idx = c.take(R * 4);
  L.pub.expanded_row_idx = c.take(R * 4);
  L.pub.expert_counts = c.take(E * 4);
  L.offsets = c.take((E + 1) * 4);
  L.pub.expert_cumsum = c.take(E * 4);
  L.tile_hist = c.take(static_cast<size_t>(route_tiles(R)) * E * 4);
  L.tiles_small = c.take(static_cast<size_t>(max_small_tiles(R, static_cast<int>(E))) * sizeof(TileDesc));
  L.tiles_big = c.take(static_cast<size_t>(max_big_tiles(R, static_cast<int>(E))) * sizeof(TileDesc));
  L.runs = c.take(static_cast<size_t>(max_big_tiles(R, static_cast<int>(E))) * sizeof(TileDesc));
  L.num_tiles = c.take(16);
  L.pub.a_codes = c.take(R * I / 2);
  L.pub.a_scales = c.take(R * I / 16);
  L.pub.o_rows = c.take(R * H * 2);
  L.pub.o_exp = c.take(R);
  L.pub.a_amax = c.take(E * 4);
  L.pub.total = c.off;
  return L;
}

size_t prepared_bytes(const moe_dims_t& d) {
  const int H = d.hidden, I = d.inter, Ip = padded_inter(I);
  return static_cast<size_t>(d.num_experts) *
         (prepared_codes_bytes(2 * I, H) + prepared_scales_bytes(2 * I, H) +
          prepared_codes_bytes(H, Ip) + prepared_scales_bytes(H, Ip));
}

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Compute units and XCDs of the current device, queried once per device: the persistent
// grids and the XCD-aware workgroup order follow the device (a partitioned GPU exposes
// fewer of both than the whole MI355X's 256 CUs in 8 XCDs).
struct DeviceShape {
  int cus, xcds;
};
std::mutex g_shape_mu;
DeviceShape g_shape[64] = {};

moe_status_t device_shape(DeviceShape* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= 64) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_shape_mu);
  DeviceShape& sh = g_shape[dev];
  if (sh.cus == 0) {
    int cus = 0, xcds = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      return MOE_ERR_HIP;
    if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess ||
        xcds <= 0 || xcds > cus)
      xcds = 1;                   // no XCD count: treat the device as one L2 domain
    sh.xcds = xcds;
    sh.cus = cus;
  }
  *out = sh;
  return MOE_OK;
}

// Dimensions moe_route uses: hidden (a multiple of 8, of 16 for NVFP4), experts, top-k.
moe_status_t route_dims_ok(const moe_dims_t& d, moe_quant_t q) {
  if (d.hidden <= 0 || d.num_experts <= 0 || d.top_k <= 0) return MOE_ERR_INVALID_ARG;
  if (d.hidden % (q == MOE_QUANT_NVFP4_G16 ? 16 : 8) || d.hidden > 65536)
    return MOE_ERR_UNSUPPORTED;
  if (d.num_experts > kRouteMaxExperts || d.top_k > 64) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported dimensions";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

moe_status_t moe_workspace_size(moe_dims_t d, int32_t max_tokens, moe_quant_t q,
                                size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  if (q != MOE_QUANT_NONE && q != MOE_QUANT_INT8_ROW_DYNAMIC && q != MOE_QUANT_NVFP4_G16)
    return MOE_ERR_INVALID_ARG;
  size_t route = 0;
  moe_status_t st = route_dims_ok(d, q);
  if (st != MOE_OK) return st;
  st = moe_route_workspace_size(max_tokens, d.top_k, d.num_experts, &route);
  if (st != MOE_OK) return st;
  if (q != MOE_QUANT_NVFP4_G16) {
    *bytes = route;
    return MOE_OK;
  }
  // the layer's quantization: moe_forward's workspace, which also serves moe_route
  st = check_dims(d);
  if (st != MOE_OK) return st;
  if (max_tokens < 1 || max_tokens > MOE_MAX_TOKENS) return MOE_ERR_INVALID_ARG;
  *bytes = std::max(route, make_layout(d, max_tokens).pub.total);
  return MOE_OK;
}

moe_status_t moe_prepared_weights_size(moe_dims_t d, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  moe_status_t st = check_dims(d);
  if (st != MOE_OK) return st;
  *bytes = prepared_bytes(d);
  return MOE_OK;
}

moe_status_t moe_workspace_layout(moe_dims_t d, int32_t T, moe_workspace_layout_t* out) {
  if (!out) return MOE_ERR_INVALID_ARG;
  moe_status_t st = check_dims(d);
  if (st != MOE_OK) return st;
  if (T < 1 || T > MOE_MAX_TOKENS) return MOE_ERR_INVALID_ARG;
  *out = make_layout(d, T).pub;
  return MOE_OK;
}

moe_status_t moe_route_workspace_size(int32_t num_rows, int32_t top_k, int32_t num_experts,
                                      size_t* bytes) {
  if (!bytes || num_rows < 1 || top_k < 1 || num_experts < 1) return MOE_ERR_INVALID_ARG;
  if (top_k > 64 || num_experts > kRouteMaxExperts) return MOE_ERR_UNSUPPORTED;
  const int64_t n = static_cast<int64_t>(num_rows) * top_k;
  if (n > (int64_t{1} << 24)) return MOE_ERR_UNSUPPORTED;
  Carver c;
  c.take(static_cast<size_t>(route_tiles(n)) * num_experts * 4);   // tile histograms
  c.take(static_cast<size_t>(num_experts) * 4);                     // counts
  c.take(static_cast<size_t>(num_experts + 1) * 4);                 // offsets
  c.take(static_cast<size_t>(n) * 4);                               // position map (v2)
  *bytes = c.off;
  return MOE_OK;
}

moe_status_t moe_quantize_nvfp4(const uint16_t* src, int64_t groups, int64_t rows_per_group,
                                int32_t K, const float* q, uint8_t* codes, uint8_t* scales,
                                moe_stream_t stream) {
  if (!src || !q || !codes || !scales) return MOE_ERR_INVALID_ARG;
  if (groups < 1 || rows_per_group < 1 || K < 16 || K % 16 || K > 65536)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(src, 16) || !aligned(codes, 8) || !aligned(q, 4)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_quantize_nvfp4(src, groups, rows_per_group, K, q, codes, scales, nullptr,
                                          reinterpret_cast<hipStream_t>(stream)));
}

moe_status_t moe_prepare_weights(moe_dims_t d, const uint8_t* w13, const uint8_t* w13_sf,
                                 const uint8_t* w2, const uint8_t* w2_sf, void* prepared,
                                 size_t prepared_size, moe_stream_t stream) {
  moe_status_t st = check_dims(d);
  if (st != MOE_OK) return st;
  if (!w13 || !w13_sf || !w2 || !w2_sf || !prepared) return MOE_ERR_INVALID_ARG;
  if (!aligned(w13, 4) || !aligned(w2, 4) || !aligned(prepared, kAlign))
    return MOE_ERR_INVALID_ARG;
  if (prepared_size < prepared_bytes(d)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return hip_status(launch_prepare_weights(d.hidden, d.inter, d.num_experts, w13, w13_sf, w2,
                                           w2_sf, static_cast<uint8_t*>(prepared),
                                           reinterpret_cast<hipStream_t>(stream)));
}

moe_status_t moe_route(moe_dims_t d, int32_t T, const uint16_t* x, const int32_t* expert_ids,
                       moe_quant_t q, const float* qx, int32_t* sorted_expert_ids,
                       int32_t* sorted_row_idx, int32_t* expanded_row_idx,
                       int32_t* expert_cumsum, void* expanded_x, void* expanded_sf_or_scale,
                       void* workspace, size_t workspace_bytes, moe_stream_t stream) {
  if (q != MOE_QUANT_NONE && q != MOE_QUANT_INT8_ROW_DYNAMIC && q != MOE_QUANT_NVFP4_G16)
    return MOE_ERR_INVALID_ARG;
  moe_status_t st = route_dims_ok(d, q);
  if (st != MOE_OK) return st;
  size_t need = 0;
  st = moe_route_workspace_size(T, d.top_k, d.num_experts, &need);
  if (st != MOE_OK) return st;
  const int H = d.hidden, E = d.num_experts, K = d.top_k;
  if (!x || !expert_ids || !expanded_x || !expanded_row_idx || !expert_cumsum || !workspace)
    return MOE_ERR_INVALID_ARG;
  if ((q == MOE_QUANT_INT8_ROW_DYNAMIC || q == MOE_QUANT_NVFP4_G16) && !expanded_sf_or_scale)
    return MOE_ERR_INVALID_ARG;
  if (q == MOE_QUANT_NVFP4_G16 && !qx) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(expanded_x, 16) || !aligned(workspace, kAlign) ||
      !aligned(expert_ids, 4) || !aligned(expanded_row_idx, 4))
    return MOE_ERR_INVALID_ARG;
  if (q == MOE_QUANT_NVFP4_G16 && !aligned(qx, 4)) return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  const int64_t n = static_cast<int64_t>(T) * K;
  Carver c;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  RouteBuffers b{};
  b.tile_hist = reinterpret_cast<int32_t*>(ws + c.take(static_cast<size_t>(route_tiles(n)) * E * 4));
  b.counts = reinterpret_cast<int32_t*>(ws + c.take(static_cast<size_t>(E) * 4));
  b.offsets = reinterpret_cast<int32_t*>(ws + c.take(static_cast<size_t>(E + 1) * 4));
  b.cumsum = expert_cumsum;
  b.sorted_ids = sorted_expert_ids;
  b.sorted_row_idx = sorted_row_idx;
  b.expanded_row_idx = expanded_row_idx;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (q == MOE_QUANT_NVFP4_G16) {
    if (launch_route(expert_ids, n, E, b, s) != hipSuccess) return MOE_ERR_HIP;
    return hip_status(launch_route_permute_nvfp4(
        x, T, H, K, expanded_row_idx, qx, static_cast<uint8_t*>(expanded_x),
        static_cast<uint8_t*>(expanded_sf_or_scale), s));
  }
  float* expanded_scale = static_cast<float*>(expanded_sf_or_scale);
  if (route_permute_fits_one_workgroup(n, E, T, H)) {
    const PermuteArgs p{x, T, H, K, static_cast<int>(q), INT64_MAX, nullptr, nullptr, nullptr,
                        expanded_x, expanded_scale};
    return hip_status(launch_route_permute_small(expert_ids, n, E, b, p, s));
  }
  hipError_t e = launch_route(expert_ids, n, E, b, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = launch_route_permute(x, T, H, K, static_cast<int>(q), expanded_row_idx, INT64_MAX, false,
                           nullptr, nullptr, nullptr, expanded_x, expanded_scale, s);
  return hip_status(e);
}

moe_status_t moe_route_v2(int32_t num_rows, int32_t hidden, int32_t num_experts, int32_t top_k,
                          const uint16_t* x, const int32_t* expert_idx, const float* scale,
                          const float* offset, const moe_route_options_t* opts,
                          void* expanded_x, int32_t* expanded_row_idx, int32_t* expert_tokens,
                          float* expanded_scale, int32_t* available_idx_num, void* workspace,
                          size_t workspace_bytes, moe_stream_t stream) {
  size_t need = 0;
  moe_status_t st = moe_route_workspace_size(num_rows, top_k, num_experts, &need);
  if (st != MOE_OK) return st;
  if (!opts) return MOE_ERR_INVALID_ARG;
  if (hidden < 8 || hidden % 8 || hidden > 65536) return MOE_ERR_UNSUPPORTED;
  const moe_route_options_t o = *opts;
  int start = o.expert_start, end = o.expert_end;
  if (start == 0 && end == 0) end = num_experts;
  if (start < 0 || end <= start || end > num_experts) return MOE_ERR_INVALID_ARG;
  if (o.row_idx_type != 0 && o.row_idx_type != 1) return MOE_ERR_INVALID_ARG;
  if (o.expert_tokens_num_type < 0 || o.expert_tokens_num_type > 2) return MOE_ERR_INVALID_ARG;
  if (o.expert_tokens_num_type == 2 && num_experts > kRouteMaxExpertsKeyValue)
    return MOE_ERR_UNSUPPORTED;
  if (o.quant_mode < -1 || o.quant_mode > 1) return MOE_ERR_INVALID_ARG;
  if (o.drop_pad_mode != 0 && o.drop_pad_mode != 1) return MOE_ERR_INVALID_ARG;
  const int64_t n = static_cast<int64_t>(num_rows) * top_k;
  const bool drop_pad = o.drop_pad_mode == 1;
  if (drop_pad) {
    if (start != 0 || end != num_experts || o.row_idx_type != 0 || o.active_num > 0)
      return MOE_ERR_INVALID_ARG;
    if (o.expert_capacity < 1 || o.expert_capacity > n) return MOE_ERR_INVALID_ARG;
    if (static_cast<int64_t>(num_experts) * o.expert_capacity > INT32_MAX)
      return MOE_ERR_UNSUPPORTED;
  }
  if (!x || !expert_idx || !expanded_x || !expanded_row_idx || !workspace)
    return MOE_ERR_INVALID_ARG;
  if (o.quant_mode == 0 && (!scale || !offset)) return MOE_ERR_INVALID_ARG;
  if (o.quant_mode == 1 && !expanded_scale) return MOE_ERR_INVALID_ARG;
  if (o.quant_mode == -1 && scale && !expanded_scale) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(expanded_x, 16) || !aligned(workspace, kAlign) ||
      !aligned(expert_idx, 4) || !aligned(expanded_row_idx, 4))
    return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  const int E_act = end - start;
  Carver c;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  RouteBuffers b{};
  b.tile_hist = reinterpret_cast<int32_t*>(ws + c.take(static_cast<size_t>(route_tiles(n)) * num_experts * 4));
  b.counts = reinterpret_cast<int32_t*>(ws + c.take(static_cast<size_t>(num_experts) * 4));
  b.offsets = reinterpret_cast<int32_t*>(ws + c.take(static_cast<size_t>(num_experts + 1) * 4));
  int32_t* map = reinterpret_cast<int32_t*>(ws + c.take(static_cast<size_t>(n) * 4));
  b.e_base = start;
  b.capacity = drop_pad ? o.expert_capacity : 0;
  b.available = available_idx_num;
  if (o.row_idx_type == 1) {
    b.sorted_row_idx = expanded_row_idx;      // the scatter index
  } else {
    map = expanded_row_idx;                   // the gather index is the position map
  }
  b.expanded_row_idx = map;
  if (expert_tokens) {
    if (o.expert_tokens_num_type == 0) b.cumsum = expert_tokens;
    else if (o.expert_tokens_num_type == 1) b.counts = expert_tokens;
    else { b.key_value = expert_tokens; b.kv_rows = num_experts; }
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int quant = o.quant_mode == -1 ? 0 : (o.quant_mode == 1 ? 1 : 2);
  const int64_t limit = drop_pad ? static_cast<int64_t>(num_experts) * o.expert_capacity
                                 : (o.active_num > 0 ? o.active_num : INT64_MAX);
  const float* row_scale = o.quant_mode == -1 ? scale : nullptr;
  hipError_t e;
  if (route_permute_fits_one_workgroup(n, E_act, num_rows, hidden)) {
    const PermuteArgs p{x, num_rows, hidden, top_k, quant, limit, row_scale, scale, offset,
                        expanded_x, expanded_scale};
    e = launch_route_permute_small(expert_idx, n, E_act, b, p, s);
  } else {
    e = launch_route(expert_idx, n, E_act, b, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    const bool may_skip = E_act != num_experts || drop_pad || o.active_num > 0;
    e = launch_route_permute(x, num_rows, hidden, top_k, quant, map, limit, may_skip,
                             row_scale, scale, offset, expanded_x, expanded_scale, s);
  }
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (drop_pad) {
    const int64_t row_bytes = static_cast<int64_t>(hidden) * (quant == 0 ? 2 : 1);
    e = launch_route_pad_fill(b.counts, num_experts, o.expert_capacity, row_bytes, expanded_x,
                              quant == 1 || (quant == 0 && scale) ? expanded_scale : nullptr, s);
  }
  return hip_status(e);
}

static moe_status_t forward_impl(moe_dims_t d, int32_t T, const uint16_t* x,
                                 const int32_t* expert_ids, const uint16_t* route_weights,
                                 const void* prepared, const float* qx, const float* alpha1,
                                 const float* qa, const float* alpha2, const float* situ_beta,
                                 const float* situ_linear_beta, void* workspace,
                                 size_t workspace_bytes, uint16_t* out, moe_stream_t stream,
                                 void* const* events, bool quantized = false) {
  moe_status_t st = check_dims(d);
  if (st != MOE_OK) return st;
  if (T < 1 || T > MOE_MAX_TOKENS) return MOE_ERR_INVALID_ARG;
  // quantized: x's codes and scales (and, below 65536 routed rows, its f16 copy) are
  // already in the workspace; x and qx are not used
  if ((!quantized && (!x || !qx)) || !expert_ids || !route_weights || !prepared || !alpha1 ||
      !qa || !alpha2 || !workspace || !out)
    return MOE_ERR_INVALID_ARG;
  if ((!quantized && !aligned(x, 16)) || !aligned(out, 16) || !aligned(prepared, kAlign) ||
      !aligned(workspace, kAlign) || !aligned(expert_ids, 4) || !aligned(route_weights, 2))
    return MOE_ERR_INVALID_ARG;
  const Layout L = make_layout(d, T);
  if (workspace_bytes < L.pub.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int H = d.hidden, I = d.inter, E = d.num_experts, k = d.top_k;
  const int64_t R = static_cast<int64_t>(T) * k;

  LayerArgs a{};
  DeviceShape shape;
  st = device_shape(&shape);
  if (st != MOE_OK) return st;
  a.H = H; a.I = I; a.Ip = padded_inter(I); a.E = E; a.k = k; a.T = T;
  a.cus = shape.cus; a.xcds = shape.xcds;
  a.x_codes = ws + L.pub.x_codes;
  a.x_scales = ws + L.pub.x_scales;
  a.x_dec = reinterpret_cast<const uint16_t*>(ws + L.pub.x_dec);
  int32_t* sorted_ids = reinterpret_cast<int32_t*>(ws + L.pub.sorted_ids);
  int32_t* sorted_row_idx = reinterpret_cast<int32_t*>(ws + L.pub.sorted_row_idx);
  int32_t* expanded_row_idx = reinterpret_cast<int32_t*>(ws + L.pub.expanded_row_idx);
  a.sorted_row_idx = sorted_row_idx;
  a.expanded_row_idx = expanded_row_idx;
  a.tiles_small = reinterpret_cast<TileDesc*>(ws + L.tiles_small);
  a.tiles_big = reinterpret_cast<TileDesc*>(ws + L.tiles_big);
  a.num_tiles = reinterpret_cast<int32_t*>(ws + L.num_tiles);
  a.runs = reinterpret_cast<TileDesc*>(ws + L.runs);
  a.max_small = max_small_tiles(R, E);
  a.max_big = max_big_tiles(R, E);
  const uint8_t* p = static_cast<const uint8_t*>(prepared);
  a.w13_codes = p;
  a.w13_scales = a.w13_codes + static_cast<size_t>(E) * prepared_codes_bytes(2 * I, H);
  a.w2_codes = a.w13_scales + static_cast<size_t>(E) * prepared_scales_bytes(2 * I, H);
  a.w2_scales = a.w2_codes + static_cast<size_t>(E) * prepared_codes_bytes(H, a.Ip);
  a.alpha1 = alpha1; a.qa = qa; a.alpha2 = alpha2;
  a.beta = situ_beta; a.lam = situ_linear_beta;
  a.a_codes = ws + L.pub.a_codes;
  a.a_scales = ws + L.pub.a_scales;
  a.a_amax = reinterpret_cast<float*>(ws + L.pub.a_amax);
  a.o_rows = reinterpret_cast<uint16_t*>(ws + L.pub.o_rows);
  a.o_exp = reinterpret_cast<int8_t*>(ws + L.pub.o_exp);
  a.route_weights = route_weights;
  a.out = out;

  auto mark = [&](int i) -> bool {
    return events == nullptr ||
           hipEventRecord(static_cast<hipEvent_t>(events[i]), s) == hipSuccess;
  };
  if (!mark(0)) return MOE_ERR_HIP;
  RouteBuffers b{};
  b.tile_hist = reinterpret_cast<int32_t*>(ws + L.tile_hist);
  b.counts = reinterpret_cast<int32_t*>(ws + L.pub.expert_counts);
  b.offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  b.cumsum = reinterpret_cast<int32_t*>(ws + L.pub.expert_cumsum);
  b.sorted_ids = sorted_ids;
  b.sorted_row_idx = sorted_row_idx;
  b.expanded_row_idx = expanded_row_idx;
  b.tiles_small = reinterpret_cast<TileDesc*>(ws + L.tiles_small);
  b.tiles_big = reinterpret_cast<TileDesc*>(ws + L.tiles_big);
  b.num_tiles = reinterpret_cast<int32_t*>(ws + L.num_tiles);
  b.small_only = R <= kSmallOnlyRows ? 1 : 0;
  // FC2's runs group big tiles; a batch of small tiles only has none (and skips their scan)
  b.runs = b.small_only ? nullptr : reinterpret_cast<TileDesc*>(ws + L.runs);
  b.amax_reset = a.a_amax;
  uint8_t* x_codes = ws + L.pub.x_codes;
  uint8_t* x_scales = ws + L.pub.x_scales;
  uint16_t* x_dec = reinterpret_cast<uint16_t*>(ws + L.pub.x_dec);
  if (!quantized && route_fits_one_workgroup(R, E)) {
    // small batch: quantization and routing in one launch (both stage marks after it)
    const QuantizeArgs qa{x, static_cast<int64_t>(T) * (H / kGroup), H / kGroup, T, qx,
                          x_codes, x_scales, x_dec};
    if (launch_quantize_route_small(qa, expert_ids, R, E, b, s) != hipSuccess || !mark(1) ||
        !mark(2))
      return MOE_ERR_HIP;
  } else {
    // the quantization runs in the router's scatter launch (both stage marks after it)
    const QuantizeArgs qa{x, static_cast<int64_t>(T) * (H / kGroup), H / kGroup, T, qx,
                          x_codes, x_scales, layer_writes_x_dec(R, a.cus) ? x_dec : nullptr};
    if (launch_route(expert_ids, R, E, b, s, quantized ? nullptr : &qa) != hipSuccess ||
        !mark(1) || !mark(2))
      return MOE_ERR_HIP;
  }
  if (layer_small_fused_fits(a)) {
    // FC1 and FC2 in one launch (both stage marks after it)
    if (launch_layer_small_fused(a, s) != hipSuccess || !mark(3) || !mark(4)) return MOE_ERR_HIP;
  } else {
    if (launch_fc1(a, s) != hipSuccess || !mark(3)) return MOE_ERR_HIP;
    if (launch_fc2(a, s) != hipSuccess || !mark(4)) return MOE_ERR_HIP;
  }
  if (launch_finalize(a, s) != hipSuccess || !mark(5)) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status_t moe_forward(moe_dims_t d, int32_t T, const uint16_t* x, const int32_t* expert_ids,
                         const uint16_t* route_weights, const void* prepared, const float* qx,
                         const float* alpha1, const float* qa, const float* alpha2,
                         const float* situ_beta, const float* situ_linear_beta,
                         void* workspace, size_t workspace_bytes, uint16_t* out,
                         moe_stream_t stream) {
  return forward_impl(d, T, x, expert_ids, route_weights, prepared, qx, alpha1, qa, alpha2,
                      situ_beta, situ_linear_beta, workspace, workspace_bytes, out, stream,
                      nullptr);
}

moe_status_t moe_forward_timed(moe_dims_t d, int32_t T, const uint16_t* x,
                               const int32_t* expert_ids, const uint16_t* route_weights,
                               const void* prepared, const float* qx, const float* alpha1,
                               const float* qa, const float* alpha2, const float* situ_beta,
                               const float* situ_linear_beta, void* workspace,
                               size_t workspace_bytes, uint16_t* out, moe_stream_t stream,
                               void* const* events) {
  if (!events) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < MOE_FORWARD_STAGES + 1; ++i)
    if (!events[i]) return MOE_ERR_INVALID_ARG;
  return forward_impl(d, T, x, expert_ids, route_weights, prepared, qx, alpha1, qa, alpha2,
                      situ_beta, situ_linear_beta, workspace, workspace_bytes, out, stream,
                      events);
}

moe_status_t moe_ring_layout(moe_dims_t d, int32_t num_slots, int32_t tokens_per_slot,
                             moe_ring_layout_t* out) {
  if (!out) return MOE_ERR_INVALID_ARG;
  return ring_layout(d, num_slots, tokens_per_slot, out);
}

moe_status_t moe_ring_init(moe_dims_t d, const moe_ring_t* ring, moe_stream_t stream) {
  moe_ring_layout_t L;
  moe_status_t st = check_ring(d, ring, &L);
  if (st != MOE_OK) return st;
  // the counter records and the status word are contiguous
  const int words = static_cast<int>((L.total - L.counters) / 4);
  return hip_status(launch_ring_init(reinterpret_cast<uint32_t*>(ring_slots(ring, L)), words,
                                     reinterpret_cast<hipStream_t>(stream)));
}

moe_status_t moe_ring_acquire(moe_dims_t d, const moe_ring_t* ring, int32_t slot,
                              moe_ring_role_t role, uint32_t timeout_us, moe_stream_t stream) {
  moe_ring_layout_t L;
  moe_status_t st = check_ring(d, ring, &L);
  if (st != MOE_OK) return st;
  if (slot < 0 || slot >= ring->num_slots) return MOE_ERR_INVALID_ARG;
  if (role != MOE_RING_ROUTE && role != MOE_RING_LAYOUT) return MOE_ERR_INVALID_ARG;
  int64_t ticks = 0;
  if (!ring_ticks(timeout_us, &ticks)) return MOE_ERR_HIP;
  RingSlot* rs = ring_slots(ring, L) + slot;
  const uint32_t* seq = role == MOE_RING_ROUTE ? &rs->route_seq : &rs->layout_seq;
  // free for this producer once the consumer has finished its last publish of the slot
  return hip_status(launch_ring_wait(&rs->consumed, nullptr, seq, 0u, ticks,
                                     ring_status(ring, L), MOE_RING_PRODUCER_TIMEOUT,
                                     reinterpret_cast<hipStream_t>(stream)));
}

moe_status_t moe_ring_publish(moe_dims_t d, const moe_ring_t* ring, int32_t slot,
                              moe_ring_role_t role, moe_stream_t stream) {
  moe_ring_layout_t L;
  moe_status_t st = check_ring(d, ring, &L);
  if (st != MOE_OK) return st;
  if (slot < 0 || slot >= ring->num_slots) return MOE_ERR_INVALID_ARG;
  if (role != MOE_RING_ROUTE && role != MOE_RING_LAYOUT) return MOE_ERR_INVALID_ARG;
  RingSlot* rs = ring_slots(ring, L) + slot;
  return hip_status(role == MOE_RING_ROUTE
                        ? launch_ring_publish(&rs->route_ready, &rs->route_seq,
                                              reinterpret_cast<hipStream_t>(stream))
                        : launch_ring_publish(&rs->layout_ready, &rs->layout_seq,
                                              reinterpret_cast<hipStream_t>(stream)));
}

moe_status_t moe_forward_streamed(moe_dims_t d, const moe_ring_t* ring, int32_t total_tokens,
                                  int32_t first_chunk, int32_t num_chunks,
                                  const void* prepared, const float* qx, const float* alpha1,
                                  const float* qa, const float* alpha2, const float* situ_beta,
                                  const float* situ_linear_beta, uint32_t timeout_us,
                                  void* workspace, size_t workspace_bytes, uint16_t* out,
                                  moe_stream_t stream) {
  moe_ring_layout_t L;
  moe_status_t st = check_ring(d, ring, &L);
  if (st != MOE_OK) return st;
  const int64_t C = ring->tokens_per_slot, S = ring->num_slots;
  if (total_tokens < 1 || first_chunk < 0 || num_chunks < 1) return MOE_ERR_INVALID_ARG;
  const int64_t chunks = (total_tokens + C - 1) / C;
  if (static_cast<int64_t>(first_chunk) + num_chunks > chunks) return MOE_ERR_INVALID_ARG;
  if (!out || !aligned(out, 16)) return MOE_ERR_INVALID_ARG;
  size_t need = 0;
  st = moe_workspace_size(d, static_cast<int32_t>(C), MOE_QUANT_NVFP4_G16, &need);
  if (st != MOE_OK) return st;
  if (!workspace || workspace_bytes < need) return workspace ? MOE_ERR_WORKSPACE_TOO_SMALL
                                                             : MOE_ERR_INVALID_ARG;
  int64_t ticks = 0;
  if (!ring_ticks(timeout_us, &ticks)) return MOE_ERR_HIP;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint8_t* base = static_cast<uint8_t*>(ring->base);
  const int H = d.hidden, k = d.top_k;
  for (int64_t n = first_chunk; n < first_chunk + num_chunks; ++n) {
    const int64_t slot = n % S;
    const int32_t valid = static_cast<int32_t>(std::min<int64_t>(C, total_tokens - n * C));
    RingSlot* rs = ring_slots(ring, L) + slot;
    if (launch_ring_wait(&rs->route_ready, &rs->layout_ready, &rs->consumer_seq, 1u, ticks,
                         ring_status(ring, L), MOE_RING_CONSUMER_TIMEOUT, s) != hipSuccess)
      return MOE_ERR_HIP;
    const uint16_t* x = reinterpret_cast<const uint16_t*>(base + L.x) + slot * C * H;
    const int32_t* ids = reinterpret_cast<const int32_t*>(base + L.expert_ids) + slot * C * k;
    const uint16_t* w = reinterpret_cast<const uint16_t*>(base + L.route_weights) + slot * C * k;
    // The chunk's ids go through the workspace's FC2-row area (the router reads them there
    // before FC2 writes that area): after a failed wait they are all dropped, so the chunk
    // computes nothing from the slot and its output rows are zero.
    int32_t* ids_ws = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) +
                                                 make_layout(d, valid).pub.o_rows);
    if (launch_slot_ids(ids_ws, ids, static_cast<int64_t>(valid) * k, ring_status(ring, L),
                        s) != hipSuccess)
      return MOE_ERR_HIP;
    st = forward_impl(d, valid, x, ids_ws, w, prepared, qx, alpha1, qa, alpha2, situ_beta,
                      situ_linear_beta, workspace, workspace_bytes, out + n * C * H, stream,
                      nullptr);
    if (st != MOE_OK) return st;
    if (launch_ring_publish(&rs->consumed, &rs->consumer_seq, s) != hipSuccess)
      return MOE_ERR_HIP;
  }
  return MOE_OK;
}

// Workspace of the sealed front end for a stream of `tokens` tokens: the layer's workspace
// for that many tokens, then the stream's expert ids and route weights.
struct SealedLayout {
  size_t layer_bytes, ids, weights, total;   // the layer's part starts at offset 0
};
static moe_status_t sealed_layout(moe_dims_t d, int32_t tokens, SealedLayout* out) {
  if (tokens < 1 || tokens > MOE_MAX_TOKENS) return MOE_ERR_INVALID_ARG;
  size_t layer = 0;
  moe_status_t st = moe_workspace_size(d, tokens, MOE_QUANT_NVFP4_G16, &layer);
  if (st != MOE_OK) return st;
  Carver c;
  c.take(layer);
  out->layer_bytes = layer;
  out->ids = c.take(static_cast<size_t>(tokens) * d.top_k * 4);
  out->weights = c.take(static_cast<size_t>(tokens) * d.top_k * 2);
  out->total = c.off;
  return MOE_OK;
}

moe_status_t moe_sealed_workspace_size(moe_dims_t d, int32_t total_tokens, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  SealedLayout S;
  moe_status_t st = sealed_layout(d, total_tokens, &S);
  if (st == MOE_OK) *bytes = S.total;
  return st;
}

static moe_status_t check_sealed_workspace(moe_dims_t d, int32_t total_tokens,
                                           const void* workspace, size_t workspace_bytes,
                                           SealedLayout* S) {
  moe_status_t st = sealed_layout(d, total_tokens, S);
  if (st != MOE_OK) return st;
  if (!workspace || !aligned(workspace, kAlign)) return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < S->total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return MOE_OK;
}

moe_status_t moe_forward_absorb(moe_dims_t d, const moe_ring_t* ring, int32_t total_tokens,
                                int32_t first_chunk, int32_t num_chunks, const float* qx,
                                uint32_t timeout_us, void* workspace, size_t workspace_bytes,
                                moe_stream_t stream) {
  moe_ring_layout_t RL;
  moe_status_t st = check_ring(d, ring, &RL);
  if (st != MOE_OK) return st;
  const int64_t C = ring->tokens_per_slot, S = ring->num_slots;
  if (total_tokens < 1 || first_chunk < 0 || num_chunks < 1 || !qx) return MOE_ERR_INVALID_ARG;
  const int64_t chunks = (total_tokens + C - 1) / C;
  if (static_cast<int64_t>(first_chunk) + num_chunks > chunks) return MOE_ERR_INVALID_ARG;
  SealedLayout SL;
  st = check_sealed_workspace(d, total_tokens, workspace, workspace_bytes, &SL);
  if (st != MOE_OK) return st;
  int64_t ticks = 0;
  if (!ring_ticks(timeout_us, &ticks)) return MOE_ERR_HIP;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint8_t* base = static_cast<uint8_t*>(ring->base);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const Layout L = make_layout(d, total_tokens);
  const int H = d.hidden, k = d.top_k;
  DeviceShape shape;
  st = device_shape(&shape);
  if (st != MOE_OK) return st;
  const bool with_dec = layer_writes_x_dec(static_cast<int64_t>(total_tokens) * k, shape.cus);
  for (int64_t n = first_chunk; n < first_chunk + num_chunks; ++n) {
    const int64_t slot = n % S;
    const int32_t valid = static_cast<int32_t>(std::min<int64_t>(C, total_tokens - n * C));
    RingSlot* rs = ring_slots(ring, RL) + slot;
    if (launch_ring_wait(&rs->route_ready, &rs->layout_ready, &rs->consumer_seq, 1u, ticks,
                         ring_status(ring, RL), MOE_RING_CONSUMER_TIMEOUT, s) != hipSuccess)
      return MOE_ERR_HIP;
    const uint16_t* x = reinterpret_cast<const uint16_t*>(base + RL.x) + slot * C * H;
    const int32_t* ids = reinterpret_cast<const int32_t*>(base + RL.expert_ids) + slot * C * k;
    const uint16_t* w = reinterpret_cast<const uint16_t*>(base + RL.route_weights) + slot * C * k;
    const int64_t t0 = n * C;
    // the chunk's tokens are rows t0 .. of the stream's batch: quantized in place, and
    // their ids and route weights copied out of the slot before it is released
    uint16_t* dec = with_dec ? reinterpret_cast<uint16_t*>(ws + L.pub.x_dec) + t0 * H : nullptr;
    if (launch_quantize_nvfp4(x, 1, valid, H, qx, ws + L.pub.x_codes + t0 * (H / 2),
                              ws + L.pub.x_scales + t0 * (H / kGroup), dec, s) != hipSuccess)
      return MOE_ERR_HIP;
    // (after a failed wait the ids are all dropped: the chunk's output rows are zero)
    if (launch_slot_ids(reinterpret_cast<int32_t*>(ws + SL.ids) + t0 * k, ids,
                        static_cast<int64_t>(valid) * k, ring_status(ring, RL), s) != hipSuccess ||
        launch_slot_copy(ws + SL.weights + t0 * k * 2, w, static_cast<int64_t>(valid) * k * 2,
                         s) != hipSuccess)
      return MOE_ERR_HIP;
    if (launch_ring_publish(&rs->consumed, &rs->consumer_seq, s) != hipSuccess)
      return MOE_ERR_HIP;
  }
  return MOE_OK;
}

moe_status_t moe_forward_seal(moe_dims_t d, int32_t total_tokens, const void* prepared,
                              const float* alpha1, const float* qa, const float* alpha2,
                              const float* situ_beta, const float* situ_linear_beta,
                              void* workspace, size_t workspace_bytes, uint16_t* out,
                              moe_stream_t stream) {
  SealedLayout SL;
  moe_status_t st = check_sealed_workspace(d, total_tokens, workspace, workspace_bytes, &SL);
  if (st != MOE_OK) return st;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  return forward_impl(d, total_tokens, nullptr, reinterpret_cast<const int32_t*>(ws + SL.ids),
                      reinterpret_cast<const uint16_t*>(ws + SL.weights), prepared, nullptr,
                      alpha1, qa, alpha2, situ_beta, situ_linear_beta, workspace, SL.layer_bytes, out,
                      stream, nullptr, /*quantized=*/true);
}

}  // extern "C"

// Workspace of moe_forward_noalloc: a fixed array in each GPU's global memory, held for the
// life of the process.  Host code never uses the array's name as an address (on the host it
// names a stand-in, not device memory): the device address comes from hipGetSymbolAddress,
// once per device with that device current, and is kept per device.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status_t scratch_on_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

extern "C" {

moe_status_t moe_forward_noalloc(moe_dims_t d, int32_t T, const uint16_t* x,
                                 const int32_t* expert_ids, const uint16_t* route_weights,
                                 const void* prepared, const float* qx, const float* alpha1,
                                 const float* qa, const float* alpha2, const float* situ_beta,
                                 const float* situ_linear_beta, uint16_t* out,
                                 moe_stream_t stream) {
  moe_status_t st = check_dims(d);
  if (st != MOE_OK) return st;
  if (T < 1 || T > MOE_MAX_TOKENS) return MOE_ERR_INVALID_ARG;
  if (make_layout(d, T).pub.total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_UNSUPPORTED;
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != MOE_OK) return st;
  // the layer's kernels need no zeroed workspace (every value they read is written
  // earlier in the same call), so the array's previous contents are harmless
  return forward_impl(d, T, x, expert_ids, route_weights, prepared, qx, alpha1, qa, alpha2,
                      situ_beta, situ_linear_beta, ws, MOE_NOALLOC_SCRATCH_BYTES, out, stream,
                      nullptr);
}

moe_status_t moe_topk_softmax(int32_t T, int32_t num_experts, int32_t top_k,
                              const float* logits, int32_t* expert_ids, uint16_t* route_weights,
                              moe_stream_t stream) {
  if (T < 1 || num_experts < 1 || top_k < 1 || top_k > num_experts) return MOE_ERR_INVALID_ARG;
  if (num_experts > 4096 || top_k > 64) return MOE_ERR_UNSUPPORTED;
  if (!logits || !expert_ids || !route_weights) return MOE_ERR_INVALID_ARG;
  if (!aligned(logits, 4) || !aligned(expert_ids, 4) || !aligned(route_weights, 2))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_topk_softmax(logits, T, num_experts, top_k, expert_ids, route_weights,
                                        reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
