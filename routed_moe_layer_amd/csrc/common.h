// Device helpers shared by the routed-MoE kernels (gfx950 / CDNA4, wave64).
//
// Number formats ("Cake SiTU backend", section "Prepared weights and scales"; "Nvfp4
// Tensor", struct NVFP4Tensor): NVFP4 = E2M1 codes (sign bit 3, magnitudes
// {0,.5,1,1.5,2,3,4,6}) in groups of 16 sharing one float8_e4m3fn scale (bias 7, max 448,
// no Inf), with an fp32 global scale applied after block dequantization.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rmoe {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kGroup = 16;          // NVFP4 block length
constexpr int kChunk = 128;         // K elements per prepared-weight chunk (4 MFMA K-steps)

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> BF16 bits (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values as packed BF16 (lo in bits 0..15), rounded to nearest even by the
// hardware conversion (same result as f32_to_bf16_rne for finite values).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// fp32 value of an E4M3 byte (the byte's sign is ignored: block scales are >= 0).
// gfx950's fp8 conversion is the OCP E4M3 ("fn") format.
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(byte & 0x7Fu), false);
  return v[0];
}

// E2M1 codes of two fp32 values into byte SEL of w (the first value in the low nibble):
// the nearest of {0,.5,1,1.5,2,3,4,6}, ties to the even code, saturating at 6 (also for
// infinities), the sign in bit 3 (-0 and small negatives give 0x8).  gfx950's packed
// conversion with scale 1 implements this rule; tests/test_gpu_codec_edges.py pins it
// against the oracle on every midpoint between two E2M1 magnitudes (both signs) and one
// and two float steps either side, under block scales from 2^-9 to 2^8.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pack2(uint32_t w, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, SEL);
}

// Group-16 NVFP4 quantization of one block with global encoding scale q:
// s = E4M3(min(fp32(fp32(amax*q)/6), 448)); enc = q/s (0 if s == 0);
// code_i = E2M1(fp32(v_i*enc)).  Returns the scale byte; codes packed two per byte,
// element 2b in the low nibble of byte b (codes_lo: elements 0..7, codes_hi: 8..15).
// The E4M3 byte rounds to nearest even after the clamp to 448 (subnormals in steps of
// 2^-9): gfx950's fp32 -> E4M3 conversion does that on [0, 448]; tests/test_gpu_codec_edges.py
// pins it against the oracle on every midpoint between two E4M3 values (and one float step
// either side) from the subnormal range to saturation.  The quotient by 6 is RN(1/6) times
// amax*q with one FMA correction of the residual: over every non-negative finite float it
// differs from the IEEE quotient only below 2^-100, where the scale byte is 0 either way
// (tests/c/scale_division.c, run by tests/test_nvfp4_scale_division.py).
__device__ __forceinline__ uint32_t nvfp4_scale_byte(float amax, float q) {
  constexpr float kSixth = 0.16666667163372040f;      // RN(1/6)
  const float x = amax * q;
  const float q0 = x * kSixth;
  const float s32 = __builtin_fmaf(__builtin_fmaf(-6.0f, q0, x), kSixth, q0);
  return static_cast<uint32_t>(
      __builtin_amdgcn_cvt_pk_fp8_f32(fminf(s32, 448.0f), 0.0f, 0, false)) & 0xFFu;
}

// The encode factor q/s of scale byte sb (0 when s is 0).
__device__ __forceinline__ float nvfp4_encode_factor(uint32_t sb, float q) {
  const float s = e4m3_to_f32(sb);
  return (s == 0.0f) ? 0.0f : q / s;
}

__device__ __forceinline__ uint32_t nvfp4_block_scale(float amax, float q, float* enc_out) {
  const uint32_t sb = nvfp4_scale_byte(amax, q);
  *enc_out = nvfp4_encode_factor(sb, q);
  return sb;
}

__device__ __forceinline__ uint32_t pack8_codes(const float* v, float enc) {
  uint32_t w = 0;
  w = e2m1_pack2<0>(w, v[0] * enc, v[1] * enc);
  w = e2m1_pack2<1>(w, v[2] * enc, v[3] * enc);
  w = e2m1_pack2<2>(w, v[4] * enc, v[5] * enc);
  w = e2m1_pack2<3>(w, v[6] * enc, v[7] * enc);
  return w;
}

// Decode 8 NVFP4 codes (one 32-bit word, element i in nibble i) times the block scale
// into the f16x8 operand of a 16x16x32 f16 MFMA.  The conversion instruction applies only
// a power-of-two scale, so it runs with scale 1 (exact E2M1 values) and the E4M3 scale
// (at most 4 significant bits, range 2^-9..448) multiplies in f16: every product has at
// most 6 significant bits and lies in [2^-10, 2688], so it is exact in f16.
// `one` is the conversion's scale operand: any value in [1, 2) gives the same result (only
// its power of two is applied); a loop-variant one keeps a decode inside its loop.
__device__ __forceinline__ f16x8 decode8(uint32_t w, f16x2 scale2, float one = 1.0f) {
  f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, one, 0);
  f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, one, 1);
  f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, one, 2);
  f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, one, 3);
  a *= scale2; b *= scale2; c *= scale2; d *= scale2;
  f16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ __forceinline__ f16x2 scale_f16x2(uint32_t e4m3_byte) {
  _Float16 h = static_cast<_Float16>(e4m3_to_f32(e4m3_byte));   // exact: E4M3 fits f16
  f16x2 r; r[0] = h; r[1] = h;
  return r;
}

// The four E4M3 scale bytes of one dword as f16 (exact; sign bits ignored like
// e4m3_to_f32): lo = {byte 0, byte 1}, hi = {byte 2, byte 3}.
__device__ __forceinline__ void scales4_f16(uint32_t w, f16x2* lo, f16x2* hi) {
  const uint32_t m = w & 0x7F7F7F7Fu;
  *lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(m, 1.0f, false);
  *hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(m, 1.0f, true);
}

// Element i of a scale pair in both halves.
__device__ __forceinline__ f16x2 bcast_f16x2(f16x2 pair, int i) {
  f16x2 r;
  r[0] = pair[i];
  r[1] = pair[i];
  return r;
}

// scale_f16x2 of byte b of a dword of E4M3 scales, by one packed conversion of the byte
// pair that holds it (b is a compile-time constant after unrolling).
__device__ __forceinline__ f16x2 scale_f16x2_of(uint32_t w, int b) {
  const uint32_t m = w & 0x7F7F7F7Fu;
  const f16x2 pair = b >= 2 ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(m, 1.0f, true)
                            : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(m, 1.0f, false);
  return bcast_f16x2(pair, b & 1);
}

__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Lane-mask of lanes whose value of `key` equals this lane's (keys < 2^nbits), among
// `active` lanes, via one ballot per key bit.
__device__ __forceinline__ uint64_t match_key(uint32_t key, int nbits, uint64_t active) {
  uint64_t peers = active;
  for (int b = 0; b < nbits; ++b) {
    uint32_t bit = (key >> b) & 1u;
    uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  uint32_t lane = __lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Group-16 NVFP4 quantization of the 16 BF16 values at src (32-byte aligned) with global
// encoding scale q: returns the E4M3 scale byte; *codes receives the 8 code bytes (element
// 2i in the low nibble of byte i).
__device__ __forceinline__ uint32_t nvfp4_quantize16(const uint16_t* __restrict__ src, float q,
                                                     uint2* codes) {
  // read once: nontemporal (a CU streams such loads faster, and they leave the caches to
  // the data that is reread)
  const u32x4* p = reinterpret_cast<const u32x4*>(src);
  const u32x4 lo = __builtin_nontemporal_load(p), hi = __builtin_nontemporal_load(p + 1);
  const uint32_t wv[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  float v[16];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = __uint_as_float(wv[i] << 16);
    v[2 * i + 1] = __uint_as_float(wv[i] & 0xFFFF0000u);
    amax = fmaxf(amax, fmaxf(fabsf(v[2 * i]), fabsf(v[2 * i + 1])));
  }
  float enc;
  const uint32_t sb = nvfp4_block_scale(amax, q, &enc);
  codes->x = pack8_codes(v, enc);
  codes->y = pack8_codes(v + 8, enc);
  return sb;
}

// Group-16 NVFP4 quantization of 16-value block b of BF16 rows (blocks_per_row blocks per
// row, one encoding scale q[row / rows_per_group] per group of rows): 8 bytes of codes, the
// E4M3 block scale and, when `decoded` is given, the block's decoded values in f16 (code
// times block scale, exact).  Shared by the quantization kernel and the fused
// quantize-and-route kernel.
__device__ __forceinline__ void quantize_nvfp4_block(const uint16_t* __restrict__ src, int64_t b,
                                                     int blocks_per_row, int64_t rows_per_group,
                                                     const float* __restrict__ q,
                                                     uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales,
                                                     uint16_t* __restrict__ decoded) {
  const int64_t row = b / blocks_per_row;
  uint2 out;
  const uint32_t sb = nvfp4_quantize16(src + b * kGroup, q[row / rows_per_group], &out);
  reinterpret_cast<uint2*>(codes)[b] = out;
  scales[b] = static_cast<uint8_t>(sb);
  if (decoded) {
    const f16x2 sc = scale_f16x2(sb);
    f16x8* d = reinterpret_cast<f16x8*>(decoded + b * kGroup);
    d[0] = decode8(out.x, sc);
    d[1] = decode8(out.y, sc);
  }
}

// Routing-primitive int8 helpers (shared by the permute kernel and the fused small
// route-and-permute kernel).
// Maximum of v over the workgroup (red: one float per wave in LDS).
__device__ __forceinline__ float block_max(float v, float* red) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
  __syncthreads();
  float m = red[0];
  for (int i = 1; i < static_cast<int>(blockDim.x / kWave); ++i) m = fmaxf(m, red[i]);
  return m;
}

// Static quantization of one value: the product and the sum are rounded to fp32 one at a
// time (no fused multiply-add), then rounded half to even and saturated.
__device__ __forceinline__ float static_int8(float x, float s, float o) {
#pragma clang fp contract(off)
  const float y = x * s + o;
  return fminf(fmaxf(rintf(y), -128.0f), 127.0f);
}

// Eight BF16 values (one 16-byte vector) to eight int8 codes through q().
template <class Q>
__device__ __forceinline__ uint2 quant8(uint4 d, Q q) {
  const uint32_t w[4] = {d.x, d.y, d.z, d.w};
  uint32_t packed[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t bits = (i & 1) ? (w[i >> 1] & 0xFFFF0000u) : (w[i >> 1] << 16);
    const float qf = q(__uint_as_float(bits));
    packed[i >> 2] |= (static_cast<uint32_t>(static_cast<int32_t>(qf)) & 0xFFu) << (8 * (i & 3));
  }
  return make_uint2(packed[0], packed[1]);
}

}  // namespace rmoe
