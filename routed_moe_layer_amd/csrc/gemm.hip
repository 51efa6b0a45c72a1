// Grouped GEMMs of the routed MoE layer on the f16 MFMA (16x16x32, fp32 accumulate) and
// the BF16 weighted finalization.
//
// "Cake SiTU backend" (intro; section "Prepared weights and scales"):
//   FC1: h[r, n] = alpha1[e] * sum_k xhat[r, k] * w13hat[e, n, k]    n in [0, 2I)
//   SiTU: a = (beta*tanh(g/beta)*sigmoid(g)) * (lambda*tanh(u/lambda)), g = h[.., i],
//         u = h[.., I + i]; then group-16 NVFP4 requantization with qA[e]
//   FC2: o[r, h] = alpha2[e] * sum_i ahat[r, i] * w2hat[e, h, i]
//   out[t] = BF16(sum_j w[t, j] * o[row(t, j)])
// where xhat, what, ahat are NVFP4 values decoded exactly (E2M1 code times E4M3 block
// scale: at most 6 significant bits, so exact in f16), and alpha multiplies the fp32
// accumulator after block dequantization ("Nvfp4 Tensor": the global scale is applied
// after block dequantization).
//
// Work decomposition: the router writes a list of token tiles (up to kTokTile expert-sorted
// rows of one expert).  A workgroup (4 waves) takes one token tile and 128 weight rows;
// each wave owns 32 weight rows (two 16-row MFMA groups) and all tokens of the tile.
// Weight fragments stream straight from HBM into registers in the prepared layout (one
// 16-byte load per lane per 128-column chunk); the token tile is staged in LDS and shared
// by the four waves.  Both operands are decoded to f16 in registers right before the MFMA.
// The FC1 epilogue fuses alpha1, SiTU, the group-16 requantization (each wave's 32 rows
// are 16 intermediate channels = one NVFP4 group) and the per-expert amax statistic.
#include "common.h"
#include "kernels.h"

namespace rmoe {

constexpr int kLdsStride = 17;      // dwords per staged token row (16 + 1 pad)

__device__ __forceinline__ float situ(float g, float u, float beta, float inv_beta,
                                      float lam, float inv_lam) {
  float sig = 1.0f / (1.0f + __expf(-g));
  float gate = beta * tanhf(g * inv_beta) * sig;
  return gate * (lam * tanhf(u * inv_lam));
}

// Main loop shared by FC1 and FC2.  Token rows come from `tok_codes` (row stride
// tok_stride bytes, scales tok_sstride bytes) at the row indices in s_row[]; valid_bytes
// limits the row (columns past the real K read as zero codes with zero scales).
template <int BN>
__device__ __forceinline__ void mainloop(const uint4* __restrict__ wcodes,
                                         const uint32_t* __restrict__ wscales, int64_t slot,
                                         int nchunks,
                                         const uint8_t* __restrict__ tok_codes,
                                         const uint8_t* __restrict__ tok_scales,
                                         int64_t tok_stride, int64_t tok_sstride,
                                         int valid_code_bytes, int valid_scale_bytes,
                                         const int64_t* s_row, uint32_t* s_codes,
                                         uint32_t* s_scales, int ncb,
                                         f32x4 (&acc)[2][BN / 16]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = lane >> 4;
  for (int c = 0; c < nchunks; ++c) {
    for (int i = tid; i < BN * 16; i += blockDim.x) {
      const int r = i >> 4, d = i & 15;
      const int byte = c * 64 + 4 * d;
      uint32_t v = 0;
      if (byte < valid_code_bytes)
        v = *reinterpret_cast<const uint32_t*>(tok_codes + s_row[r] * tok_stride + byte);
      s_codes[r * kLdsStride + d] = v;
    }
    for (int i = tid; i < BN * 2; i += blockDim.x) {
      const int r = i >> 1, d = i & 1;
      const int byte = c * 8 + 4 * d;
      uint32_t v = 0;
      if (byte < valid_scale_bytes)
        v = *reinterpret_cast<const uint32_t*>(tok_scales + s_row[r] * tok_sstride + byte);
      s_scales[r * 2 + d] = v;
    }
    const uint4 wc0 = wcodes[(slot * nchunks + c) * 64 + lane];
    const uint4 wc1 = wcodes[((slot + 1) * nchunks + c) * 64 + lane];
    const uint32_t ws0 = wscales[prepared_scale_index(slot, nchunks, c, lane)];
    const uint32_t ws1 = wscales[prepared_scale_index(slot + 1, nchunks, c, lane)];
    __syncthreads();
    const uint32_t wcw[2][4] = {{wc0.x, wc0.y, wc0.z, wc0.w}, {wc1.x, wc1.y, wc1.z, wc1.w}};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f16x8 w0 = decode8(wcw[0][s], scale_f16x2((ws0 >> (8 * s)) & 0xFFu));
      const f16x8 w1 = decode8(wcw[1][s], scale_f16x2((ws1 >> (8 * s)) & 0xFFu));
      const int sbyte = 2 * s + (g >> 1);            // block of this lane's 8 columns
#pragma unroll
      for (int cb = 0; cb < BN / 16; ++cb) {
        if (cb < ncb) {
          const int n = cb * 16 + (lane & 15);
          const uint32_t xw = s_codes[n * kLdsStride + 4 * s + g];
          const uint32_t xs = (s_scales[n * 2 + (sbyte >> 2)] >> (8 * (sbyte & 3))) & 0xFFu;
          const f16x8 xf = decode8(xw, scale_f16x2(xs));
          acc[0][cb] = mfma16x16x32(w0, xf, acc[0][cb]);
          acc[1][cb] = mfma16x16x32(w1, xf, acc[1][cb]);
        }
      }
    }
    __syncthreads();
  }
}

template <int BN>
__global__ __launch_bounds__(256) void fc1_kernel(LayerArgs a) {
  const int tt = blockIdx.y;
  if (tt >= *a.num_tiles) return;
  const TileDesc td = a.tiles[tt];
  const int e = td.expert;
  __shared__ uint32_t s_codes[BN * kLdsStride];
  __shared__ uint32_t s_scales[BN * 2];
  __shared__ int64_t s_row[BN];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4;
  if (tid < BN) {
    const int r = min(tid, td.nrows - 1);
    s_row[tid] = a.sorted_row_idx[td.row_start + r] / a.k;     // token of the routed row
  }
  __syncthreads();
  const int nchunks = a.H / kChunk;
  const int RG = 2 * a.I / 16;
  const int G0 = blockIdx.x * 8 + 2 * w;
  const int64_t slot = static_cast<int64_t>(e) * RG + G0;     // first of the wave's 2 groups
  f32x4 acc[2][BN / 16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < BN / 16; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int ncb = (td.nrows + 15) / 16;
  mainloop<BN>(reinterpret_cast<const uint4*>(a.w13_codes),
               reinterpret_cast<const uint32_t*>(a.w13_scales), slot, nchunks, a.x_codes,
               a.x_scales, a.H / 2, a.H / 16, a.H / 2, a.H / 16, s_row, s_codes, s_scales, ncb,
               acc);
  // Epilogue: lane holds rows 4g..4g+3 of each group = (gate i, up i, gate i+1, up i+1).
  const float al = a.alpha1[e];
  const float qa = a.qa[e];
  const float beta = a.beta ? a.beta[e] : 4.0f;
  const float lam = a.lam ? a.lam[e] : 25.0f;
  const float ib = 1.0f / beta, il = 1.0f / lam;
  const int blk = G0 >> 1;                       // NVFP4 group of 16 intermediates
  float wave_amax = 0.0f;
#pragma unroll
  for (int cb = 0; cb < BN / 16; ++cb) {
    if (cb >= ncb) break;
    const int n = cb * 16 + (lane & 15);
    const bool valid = n < td.nrows;
    float av[4];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const f32x4 h = acc[rg][cb];
      av[2 * rg] = situ(h[0] * al, h[1] * al, beta, ib, lam, il);
      av[2 * rg + 1] = situ(h[2] * al, h[3] * al, beta, ib, lam, il);
    }
    float m = fmaxf(fmaxf(fabsf(av[0]), fabsf(av[1])), fmaxf(fabsf(av[2]), fabsf(av[3])));
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    if (valid) wave_amax = fmaxf(wave_amax, m);
    float enc;
    const uint32_t sb = nvfp4_block_scale(m, qa, &enc);
    const uint32_t b0 = e2m1_encode(av[0] * enc) | (e2m1_encode(av[1] * enc) << 4);
    const uint32_t b1 = e2m1_encode(av[2] * enc) | (e2m1_encode(av[3] * enc) << 4);
    if (valid) {
      const int64_t row = td.row_start + n;
      uint8_t* ac = a.a_codes + row * (a.I / 2) + 8 * blk;
      ac[g] = static_cast<uint8_t>(b0);
      ac[4 + g] = static_cast<uint8_t>(b1);
      if (g == 0) a.a_scales[row * (a.I / 16) + blk] = static_cast<uint8_t>(sb);
    }
  }
  for (int off = 32; off > 0; off >>= 1) wave_amax = fmaxf(wave_amax, __shfl_xor(wave_amax, off));
  if (lane == 0 && wave_amax > 0.0f)
    atomicMax(reinterpret_cast<unsigned int*>(a.a_amax + e), __float_as_uint(wave_amax));
}

template <int BN>
__global__ __launch_bounds__(256) void fc2_kernel(LayerArgs a) {
  const int tt = blockIdx.y;
  if (tt >= *a.num_tiles) return;
  const TileDesc td = a.tiles[tt];
  const int e = td.expert;
  __shared__ uint32_t s_codes[BN * kLdsStride];
  __shared__ uint32_t s_scales[BN * 2];
  __shared__ int64_t s_row[BN];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4;
  if (tid < BN) s_row[tid] = td.row_start + min(tid, td.nrows - 1);
  __syncthreads();
  const int nchunks = a.Ip / kChunk;
  const int RG = a.H / 16;
  const int G0 = blockIdx.x * 8 + 2 * w;
  const int64_t slot = static_cast<int64_t>(e) * RG + G0;     // first of the wave's 2 groups
  f32x4 acc[2][BN / 16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < BN / 16; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int ncb = (td.nrows + 15) / 16;
  mainloop<BN>(reinterpret_cast<const uint4*>(a.w2_codes),
               reinterpret_cast<const uint32_t*>(a.w2_scales), slot, nchunks, a.a_codes,
               a.a_scales, a.I / 2, a.I / 16, a.I / 2, a.I / 16, s_row, s_codes, s_scales, ncb,
               acc);
  const float al = a.alpha2[e];
#pragma unroll
  for (int cb = 0; cb < BN / 16; ++cb) {
    if (cb >= ncb) break;
    const int n = cb * 16 + (lane & 15);
    if (n >= td.nrows) continue;
    const int64_t row = td.row_start + n;
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const f32x4 o = acc[rg][cb];
      const int h0 = 16 * (G0 + rg) + 4 * g;
      uint2 v;
      v.x = static_cast<uint32_t>(f32_to_bf16_rne(o[0] * al)) |
            (static_cast<uint32_t>(f32_to_bf16_rne(o[1] * al)) << 16);
      v.y = static_cast<uint32_t>(f32_to_bf16_rne(o[2] * al)) |
            (static_cast<uint32_t>(f32_to_bf16_rne(o[3] * al)) << 16);
      *reinterpret_cast<uint2*>(a.o_rows + row * a.H + h0) = v;
    }
  }
}

// out[t, 8v..8v+7] = BF16(sum_j w[t, j] * o[expanded_row_idx[t*k + j], 8v..8v+7]), j in
// order, fp32 fused multiply-add.  One thread per 8 outputs; 16-byte loads and stores.
__global__ __launch_bounds__(256) void finalize_kernel(LayerArgs a) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int nv = a.H / 8;
  if (idx >= static_cast<int64_t>(a.T) * nv) return;
  const int64_t t = idx / nv;
  const int v = static_cast<int>(idx % nv);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < a.k; ++j) {
    const float wt = bf16_to_f32(a.route_weights[t * a.k + j]);
    const int64_t pos = a.expanded_row_idx[t * a.k + j];
    if (pos < 0) continue;                      // dropped (expert id out of range)
    const uint4 d = reinterpret_cast<const uint4*>(a.o_rows + pos * a.H)[v];
    const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = fmaf(wt, __uint_as_float(dw[i] << 16), acc[2 * i]);
      acc[2 * i + 1] = fmaf(wt, __uint_as_float(dw[i] & 0xFFFF0000u), acc[2 * i + 1]);
    }
  }
  uint4 o;
  o.x = f32_to_bf16_rne(acc[0]) | (static_cast<uint32_t>(f32_to_bf16_rne(acc[1])) << 16);
  o.y = f32_to_bf16_rne(acc[2]) | (static_cast<uint32_t>(f32_to_bf16_rne(acc[3])) << 16);
  o.z = f32_to_bf16_rne(acc[4]) | (static_cast<uint32_t>(f32_to_bf16_rne(acc[5])) << 16);
  o.w = f32_to_bf16_rne(acc[6]) | (static_cast<uint32_t>(f32_to_bf16_rne(acc[7])) << 16);
  reinterpret_cast<uint4*>(a.out + t * a.H)[v] = o;
}

hipError_t launch_fc1(const LayerArgs& a, hipStream_t stream) {
  dim3 grid(2 * a.I / kWRows, static_cast<unsigned>(a.max_tiles));
  fc1_kernel<kTokTile><<<grid, dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_fc2(const LayerArgs& a, hipStream_t stream) {
  dim3 grid(a.H / kWRows, static_cast<unsigned>(a.max_tiles));
  fc2_kernel<kTokTile><<<grid, dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_finalize(const LayerArgs& a, hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(a.T) * (a.H / 8);
  finalize_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace rmoe
