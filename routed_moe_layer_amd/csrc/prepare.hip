// One-time re-layout of canonical NVFP4 expert weights into the MFMA-fragment layout
// ("Cake SiTU backend", section "Prepared weights and scales": the weights are prepared
// once, FC1 gate/up rows are permuted together and the block scales travel with the
// packed bytes).  The layout itself is this library's own (see kernels.h): a wave loads
// one 16-row x 128-column chunk as 64 lanes x 16 contiguous bytes of codes plus 128
// bytes of scales, already in the lane order of the 16x16x32 MFMA operand.
#include "common.h"
#include "kernels.h"

namespace rmoe {

// fc1 != 0: rows are the 2I FC1 rows, reordered so that row 2j of each 16-row group G is
// gate row 8G+j and row 2j+1 is up row 8G+j.
__global__ __launch_bounds__(256) void prepare_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ sf, int R, int K, int Kp,
    int I, int fc1, int64_t total, uint8_t* __restrict__ out_codes,
    uint8_t* __restrict__ out_scales) {
  int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  // idx = 64 * prepared_chunk(e, c, G) + lane
  const int lane = static_cast<int>(idx & 63);
  int64_t rest = idx >> 6;
  const int nchunks = Kp / kChunk;
  const int groups = R / 16;
  const int G = static_cast<int>(rest % groups);
  rest /= groups;
  const int c = static_cast<int>(rest % nchunks);
  const int64_t e = rest / nchunks;
  const int pr = 16 * G + (lane & 15);
  int row = pr;
  if (fc1) {
    const int j = pr & 15, i = 8 * G + (j >> 1);
    row = (j & 1) ? I + i : i;
  }
  const uint8_t* crow = codes + (e * R + row) * static_cast<int64_t>(K / 2);
  const uint8_t* srow = sf + (e * R + row) * static_cast<int64_t>(K / 16);
  const int g = lane >> 4;
  uint32_t w[4];
  uint32_t sc = 0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int k0 = kChunk * c + 32 * s + 8 * g;
    if (k0 < K) {
      w[s] = *reinterpret_cast<const uint32_t*>(crow + k0 / 2);
      sc |= static_cast<uint32_t>(srow[k0 / 16]) << (8 * s);
    } else {
      w[s] = 0;
    }
  }
  reinterpret_cast<uint4*>(out_codes)[idx] = make_uint4(w[0], w[1], w[2], w[3]);
  // lanes l and l+16 carry the same block scales; the even lane-group stores them
  if ((g & 1) == 0)
    reinterpret_cast<uint32_t*>(out_scales)[prepared_scale_index(idx >> 6, lane)] = sc;
}

hipError_t launch_prepare_weights(int H, int I, int E, const uint8_t* w13,
                                  const uint8_t* w13_sf, const uint8_t* w2,
                                  const uint8_t* w2_sf, uint8_t* prepared, hipStream_t stream) {
  const int Ip = (I + kChunk - 1) / kChunk * kChunk;
  uint8_t* c1 = prepared;
  uint8_t* s1 = c1 + static_cast<size_t>(E) * prepared_codes_bytes(2 * I, H);
  uint8_t* c2 = s1 + static_cast<size_t>(E) * prepared_scales_bytes(2 * I, H);
  uint8_t* s2 = c2 + static_cast<size_t>(E) * prepared_codes_bytes(H, Ip);
  int64_t t1 = static_cast<int64_t>(E) * (2 * I / 16) * (H / kChunk) * 64;
  int64_t t2 = static_cast<int64_t>(E) * (H / 16) * (Ip / kChunk) * 64;
  prepare_kernel<<<dim3(static_cast<unsigned>((t1 + 255) / 256)), dim3(256), 0, stream>>>(
      w13, w13_sf, 2 * I, H, H, I, 1, t1, c1, s1);
  prepare_kernel<<<dim3(static_cast<unsigned>((t2 + 255) / 256)), dim3(256), 0, stream>>>(
      w2, w2_sf, H, I, Ip, I, 0, t2, c2, s2);
  return hipGetLastError();
}

}  // namespace rmoe
