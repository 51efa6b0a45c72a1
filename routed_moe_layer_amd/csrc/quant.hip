// Token quantization kernels.
//
//  * quantize_nvfp4_kernel: group-16 NVFP4 quantization of BF16 rows ("Cake SiTU
//    backend", intro: group-16 NVFP4 input quantization with the fp32 scale qX).  One
//    thread per 16-value block: a 32-byte load, 8 bytes of codes and 1 scale byte out,
//    and optionally the block's decoded values (code times block scale, exact in f16;
//    32 bytes), which FC1 stages as its operand.  HBM-bound (41 or 73 bytes per block).
//  * route_permute_kernel: the token movement of "torch_npu.npu_moe_init_routing_v2"
//    (section 计算公式, steps 4-5): per-row dynamic int8 quantization (or a BF16 copy),
//    each token row written to its K expert-sorted positions through the gather map.
//    One workgroup per token row: the row is read once and written K times.
//  * route_permute_nvfp4_kernel: the same movement with the layer's group-16 NVFP4
//    quantization (codes and E4M3 block scales written to each of the K rows).
#include "common.h"
#include "kernels.h"

namespace rmoe {

__global__ __launch_bounds__(256) void quantize_nvfp4_kernel(
    const uint16_t* __restrict__ src, int64_t nblocks, int blocks_per_row,
    int64_t rows_per_group, const float* __restrict__ q, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, uint16_t* __restrict__ decoded) {
  const int64_t b = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (b < nblocks)
    quantize_nvfp4_block(src, b, blocks_per_row, rows_per_group, q, codes, scales, decoded);
}

hipError_t launch_quantize_nvfp4(const uint16_t* src, int64_t groups, int64_t rows_per_group,
                                 int K, const float* q, uint8_t* codes, uint8_t* scales,
                                 uint16_t* decoded, hipStream_t stream) {
  int64_t nblocks = groups * rows_per_group * (K / kGroup);
  if (nblocks == 0) return hipSuccess;
  int64_t grid = (nblocks + 255) / 256;
  quantize_nvfp4_kernel<<<dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream>>>(
      src, nblocks, K / kGroup, rows_per_group, q, codes, scales, decoded);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Token movement for the routing primitive ("torch_npu.npu_moe_init_routing_v2", section
// 计算公式 steps 4-5).  One workgroup per token row t; the row goes to rows map[t*K + j]
// (skipped when negative or >= limit).
//   quant 0: BF16 copy; with row_scale, expanded_scale[row] = row_scale[t].
//   quant 1: dynamic int8 per row, scale = fp32(row_max|x| / 127),
//            q = clip(rint(fp32(x / scale)), -127, 127) (0 when scale is 0).
//   quant 2: static int8, q = clip(rint(fp32(fp32(x * s) + o)), -128, 127).
// ---------------------------------------------------------------------------------------
// Up to kPermCache 16-byte vectors per thread of the current row chunk are held in
// registers: all of a chunk's loads are in flight together, and a row of at most
// kPermThreads * kPermCache vectors (H <= 8192) is read from memory once even in the
// dynamic mode, whose scale needs the whole row before the first code.
constexpr int kPermThreads = 256;
constexpr int kPermCache = 4;

__global__ __launch_bounds__(kPermThreads) void route_permute_kernel(
    const uint16_t* __restrict__ x, int H, int K, int quant, const int32_t* __restrict__ map,
    int64_t limit, bool may_skip, const float* __restrict__ row_scale,
    const float* __restrict__ static_scale, const float* __restrict__ static_offset,
    void* __restrict__ expanded_x, float* __restrict__ expanded_scale) {
  __shared__ float red[kPermThreads / kWave];
  __shared__ int32_t dst[64];
  const int64_t t = blockIdx.x;
  const uint4* xr = reinterpret_cast<const uint4*>(x + t * H);
  const int nvec = H / 8;                   // 16-byte vectors of 8 BF16
  const int per_chunk = kPermThreads * kPermCache;
  uint4 r[kPermCache];
  auto load_chunk = [&](int base) {
#pragma unroll
    for (int i = 0; i < kPermCache; ++i) {
      const int v = base + threadIdx.x + i * kPermThreads;
      r[i] = v < nvec ? xr[v] : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  if (threadIdx.x < K) {
    const int32_t d = map[t * K + threadIdx.x];
    dst[threadIdx.x] = (d >= 0 && d < limit) ? d : -1;
  }
  // Without an expert range, capacity or row limit every token is moved: its first
  // chunk is loaded while the row map arrives.
  if (!may_skip) load_chunk(0);
  __syncthreads();
  if (may_skip) {
    // A token none of whose ids is moved is not read at all (uniform over the workgroup).
    bool any = false;
    for (int j = 0; j < K; ++j) any |= dst[j] >= 0;
    if (!any) return;
    load_chunk(0);
  }
  float scale = 0.0f;
  if (quant == 1) {
    float amax = 0.0f;
    for (int base = 0; base < nvec; base += per_chunk) {
      if (base > 0) load_chunk(base);
#pragma unroll
      for (int i = 0; i < kPermCache; ++i) {
        const uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          amax = fmaxf(amax, fabsf(__uint_as_float(w[q] << 16)));
          amax = fmaxf(amax, fabsf(__uint_as_float(w[q] & 0xFFFF0000u)));
        }
      }
    }
    amax = block_max(amax, red);
    scale = amax / 127.0f;
    if (nvec > per_chunk) load_chunk(0);      // the row did not stay in registers
  }
  const float s_st = quant == 2 ? static_scale[0] : 0.0f;
  const float o_st = quant == 2 ? static_offset[0] : 0.0f;
  for (int base = 0; base < nvec; base += per_chunk) {
    if (base > 0) load_chunk(base);
#pragma unroll
    for (int i = 0; i < kPermCache; ++i) {
      const int v = base + threadIdx.x + i * kPermThreads;
      if (v >= nvec) continue;
      if (quant == 0) {
        for (int j = 0; j < K; ++j) {
          if (dst[j] < 0) continue;
          uint16_t* o = static_cast<uint16_t*>(expanded_x) + static_cast<int64_t>(dst[j]) * H;
          reinterpret_cast<uint4*>(o)[v] = r[i];
        }
        continue;
      }
      const uint2 pv =
          quant == 2 ? quant8(r[i], [=](float xv) { return static_int8(xv, s_st, o_st); })
                     : quant8(r[i], [=](float xv) {
                         const float qf = (scale == 0.0f) ? 0.0f : rintf(xv / scale);
                         return fminf(fmaxf(qf, -127.0f), 127.0f);
                       });
      for (int j = 0; j < K; ++j) {
        if (dst[j] < 0) continue;
        int8_t* o = static_cast<int8_t*>(expanded_x) + static_cast<int64_t>(dst[j]) * H;
        reinterpret_cast<uint2*>(o)[v] = pv;
      }
    }
  }
  if (threadIdx.x < K && dst[threadIdx.x] >= 0 && expanded_scale) {
    if (quant == 1) expanded_scale[dst[threadIdx.x]] = scale;
    else if (quant == 0 && row_scale) expanded_scale[dst[threadIdx.x]] = row_scale[t];
  }
}

hipError_t launch_route_permute(const uint16_t* x, int64_t N, int H, int K, int quant,
                                const int32_t* map, int64_t limit, bool may_skip,
                                const float* row_scale,
                                const float* static_scale, const float* static_offset,
                                void* expanded_x, float* expanded_scale, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  route_permute_kernel<<<dim3(static_cast<unsigned>(N)), dim3(kPermThreads), 0, stream>>>(
      x, H, K, quant, map, limit, may_skip, row_scale, static_scale, static_offset, expanded_x,
      expanded_scale);
  return hipGetLastError();
}

// Quantized token movement with group-16 NVFP4 ("torch_npu.npu_moe_init_routing_v2",
// section 计算公式 step 5, with the layer's input quantization of "Cake SiTU backend",
// intro): token row t is quantized once -- per 16-value block s = E4M3(min(fp32(fp32(amax *
// qx)/6), 448)), codes E2M1(fp32(v * qx/s)) -- and its codes [H/2] and scales [H/16] are
// written to its K expert-sorted rows map[t*K + j] (skipped when negative).  One workgroup
// per token row, one thread per 16-value block: the row's 32-byte reads and every
// destination's 8-byte code and 1-byte scale writes are contiguous across the threads.
__global__ __launch_bounds__(kPermThreads) void route_permute_nvfp4_kernel(
    const uint16_t* __restrict__ x, int H, int K, const int32_t* __restrict__ map,
    const float* __restrict__ qx, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  __shared__ int32_t dst[64];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < K) dst[threadIdx.x] = map[t * K + threadIdx.x];
  __syncthreads();
  const float q = qx[0];
  const int nb = H / kGroup;
  for (int b = threadIdx.x; b < nb; b += blockDim.x) {
    uint2 c;
    const uint32_t sb = nvfp4_quantize16(x + t * H + b * kGroup, q, &c);
    for (int j = 0; j < K; ++j) {
      const int64_t r = dst[j];
      if (r < 0) continue;
      reinterpret_cast<uint2*>(codes + r * (H / 2))[b] = c;
      scales[r * nb + b] = static_cast<uint8_t>(sb);
    }
  }
}

hipError_t launch_route_permute_nvfp4(const uint16_t* x, int64_t N, int H, int K,
                                      const int32_t* map, const float* qx, uint8_t* codes,
                                      uint8_t* scales, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  route_permute_nvfp4_kernel<<<dim3(static_cast<unsigned>(N)), dim3(kPermThreads), 0, stream>>>(
      x, H, K, map, qx, codes, scales);
  return hipGetLastError();
}

// Drop/pad ("torch_npu.npu_moe_init_routing_v2", step 5: experts with fewer rows than the
// capacity are filled with zeros).  Workgroup (x, e) zeroes slots counts[e] + x,
// counts[e] + x + gridDim.x, ... of expert e.
__global__ __launch_bounds__(256) void route_pad_fill_kernel(const int32_t* __restrict__ counts,
                                                             int C, int64_t row_bytes,
                                                             void* __restrict__ expanded_x,
                                                             float* __restrict__ expanded_scale) {
  const int e = blockIdx.y;
  const int first = min(max(counts[e], 0), C);
  const int64_t words = row_bytes / 8;
  for (int s = first + static_cast<int>(blockIdx.x); s < C; s += gridDim.x) {
    const int64_t slot = static_cast<int64_t>(e) * C + s;
    uint2* row = reinterpret_cast<uint2*>(static_cast<uint8_t*>(expanded_x) + slot * row_bytes);
    for (int64_t v = threadIdx.x; v < words; v += blockDim.x) row[v] = make_uint2(0u, 0u);
    if (expanded_scale && threadIdx.x == 0) expanded_scale[slot] = 0.0f;
  }
}

hipError_t launch_route_pad_fill(const int32_t* counts, int E, int C, int64_t row_bytes,
                                 void* expanded_x, float* expanded_scale, hipStream_t stream) {
  if (E == 0 || C == 0) return hipSuccess;
  const unsigned gx = static_cast<unsigned>(C < 64 ? C : 64);
  route_pad_fill_kernel<<<dim3(gx, static_cast<unsigned>(E)), dim3(256), 0, stream>>>(
      counts, C, row_bytes, expanded_x, expanded_scale);
  return hipGetLastError();
}

}  // namespace rmoe
