// Top-k expert selection with softmax route weights: the step before the layer, turning
// router logits [T, E] into the layer's expert_ids [T, k] and BF16 route_weights [T, k].
// The pages take expert ids and route weights as given ("Cake SiTU backend", intro) and do
// not define the gate; the reading here: a token's k largest logits in decreasing order
// (equal logits in increasing expert id), weights = softmax over those k logits only,
// computed in fp32 and rounded to BF16 (nearest even).
//
// One wavefront per token.  Lane l holds the keys of logits l, l + 64, ... in registers
// (PER_LANE of them), sorted in decreasing order within the lane; each of the k rounds
// takes the wavefront's maximum of the lanes' first keys with DPP moves (no LDS traffic),
// and the winning lane shifts its keys down by one.
#include "common.h"
#include "kernels.h"

namespace rmoe {

constexpr int kTopkWaves = 4;

// Candidate key: the logit mapped to an unsigned integer of the same order in the high
// half, the complement of the expert id in the low half, so that the unsigned maximum is
// the larger logit and, among equal logits, the lower expert id.  0 = no candidate.
__device__ __forceinline__ uint64_t topk_key(float v, int e) {
  const uint32_t u = __float_as_uint(v + 0.0f);         // -0 and +0 are equal logits
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(o) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(e));
}
__device__ __forceinline__ float topk_key_value(uint64_t key) {
  const uint32_t o = static_cast<uint32_t>(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ int topk_key_id(uint64_t key) {
  return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key));
}

// Move a 64-bit value across lanes with one DPP control on both halves; lanes outside
// ROW_MASK keep their own value.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp64(uint64_t x) {
  const int lo = static_cast<int>(static_cast<uint32_t>(x));
  const int hi = static_cast<int>(static_cast<uint32_t>(x >> 32));
  const uint32_t mlo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xF, false));
  const uint32_t mhi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xF, false));
  return (static_cast<uint64_t>(mhi) << 32) | mlo;
}

// Unsigned 64-bit maximum over the wavefront, returned to every lane: within quads, then
// half rows and rows by mirroring, across rows by the row broadcasts, read from lane 63.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
  auto mx = [](uint64_t a, uint64_t b) { return a > b ? a : b; };
  x = mx(x, dpp64<0xB1, 0xF>(x));            // quad_perm [1,0,3,2]
  x = mx(x, dpp64<0x4E, 0xF>(x));            // quad_perm [2,3,0,1]
  x = mx(x, dpp64<0x141, 0xF>(x));           // row_half_mirror
  x = mx(x, dpp64<0x140, 0xF>(x));           // row_mirror
  x = mx(x, dpp64<0x142, 0xA>(x));           // row_bcast:15 into rows 1, 3
  x = mx(x, dpp64<0x143, 0xC>(x));           // row_bcast:31 into rows 2, 3
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(x), 63);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(x >> 32), 63);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

template <int PER_LANE>
__global__ __launch_bounds__(kTopkWaves * 64) void topk_softmax_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k, int32_t* __restrict__ ids,
    uint16_t* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTopkWaves + (threadIdx.x >> 6);
  if (t >= T) return;                                   // whole wavefronts
  const float* z = logits + t * E;
  uint64_t key[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? topk_key(z[e], e) : 0;
  }
  // each lane's keys in decreasing order (bitonic network over register indices)
#pragma unroll
  for (int size = 2; size <= PER_LANE; size *= 2) {
#pragma unroll
    for (int stride = size / 2; stride > 0; stride /= 2) {
#pragma unroll
      for (int i = 0; i < PER_LANE; ++i) {
        const int l = i ^ stride;
        if (l > i) {
          const bool desc = (i & size) == 0;
          const uint64_t a = key[i], b = key[l];
          if ((a < b) == desc) { key[i] = b; key[l] = a; }
        }
      }
    }
  }
  uint64_t pick = 0;                                    // lane j: the j-th pick
  for (int j = 0; j < k; ++j) {
    const uint64_t w = wave_max_u64(key[0]);
    if (lane == j) pick = w;
    if (key[0] == w) {                                  // the winner's lane (keys are unique)
#pragma unroll
      for (int i = 0; i + 1 < PER_LANE; ++i) key[i] = key[i + 1];
      key[PER_LANE - 1] = 0;
    }
  }
  // softmax over the k picks; the first pick is the maximum
  const float v = topk_key_value(pick);
  const float m = __shfl(v, 0);
  const float p = lane < k ? expf(v - m) : 0.0f;
  float s = p;
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (lane < k) {
    ids[t * k + lane] = topk_key_id(pick);
    weights[t * k + lane] = f32_to_bf16_rne(p / s);
  }
}

hipError_t launch_topk_softmax(const float* logits, int64_t T, int E, int k, int32_t* ids,
                               uint16_t* weights, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>((T + kTopkWaves - 1) / kTopkWaves);
  const int per_lane = (E + 63) / 64;
#define RMOE_TOPK(P) \
  topk_softmax_kernel<P><<<dim3(grid), dim3(kTopkWaves * 64), 0, stream>>>(logits, T, E, k, ids, weights)
  if (per_lane <= 4) RMOE_TOPK(4);
  else if (per_lane <= 8) RMOE_TOPK(8);
  else if (per_lane <= 16) RMOE_TOPK(16);
  else if (per_lane <= 32) RMOE_TOPK(32);
  else RMOE_TOPK(64);
#undef RMOE_TOPK
  return hipGetLastError();
}

}  // namespace rmoe
